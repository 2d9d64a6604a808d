"""Expert counts on both sides of one wavefront. Below 64 groups the GEMM
kernels hold the group table in every wave's registers (lane g for group g,
lane E for the tail; prefix sums by DPP, which crosses 16-lane rows at
lanes 16, 32 and 48); from 64 on they build it in LDS 64 groups at a time
(prefix sums carried across passes), up to the ABI's 1024. With 1 to 1024
ragged groups, many of them empty, every grouped entry point is checked
against the oracle bit for bit: the operands are small integers under
power-of-two scales, which the MFMA sums exactly (and the bf16
wgrad_with_hp sums exactly in float32 before its one rounding)."""

import numpy as np
import pytest
import torch

from _helpers import bf16_host, dev, host, k128, plain, to_dev
from oracle import mx as O
from quantize_grouped_gemm_amd import mx, synth

pytestmark = pytest.mark.gpu


def _int_mx(shape, seed):
    """Codes of 0, +-1 .. +-8 and scale bytes 127..130: exact MFMA sums."""
    rng = np.random.default_rng(seed)
    vals = np.array([0, 1, 2, 3, 4, 6, 8, -1, -2, -3, -4, -6, -8], np.float64)
    q = O.e4m3_encode(rng.choice(vals, shape))
    s = rng.integers(127, 131, shape[:-1] + (shape[-1] // 32,)).astype(np.uint8)
    return q, s


def _mx_dev(q, s):
    return to_dev(q), to_dev(k128(s))


def _slots(E, seed, p_empty):
    """Per-group slots in 128-row units: empty with probability p_empty, else
    1..3 slots; the last group is forced non-empty."""
    rng = np.random.default_rng(seed)
    n = np.where(rng.random(E) < p_empty, 0, rng.integers(1, 4, E))
    n[-1] = max(n[-1], 1)
    return (n * 128).astype(np.int64)


@pytest.mark.parametrize("E,p_empty", [(1, 0.0), (17, 0.35), (33, 0.35), (63, 0.35), (64, 0.35), (200, 0.35),
                                       (1024, 0.8)])
def test_many_groups_fwd_dgrad(gpu, E, p_empty):
    N, K = 256, 128
    offs = np.cumsum(_slots(E, E, p_empty)).astype(np.int32)
    Tcap = int(offs[-1]) + 256
    qa, sa = _int_mx((Tcap, K), 1)
    qw, sw = _int_mx((E, N, K), 2)
    ref = O.grouped_mm(qa, sa, qw, sw, offs)
    for fn in (mx.grouped_mm_fwd, mx.grouped_mm_dgrad):
        err = torch.zeros(1, dtype=torch.int32, device=dev())
        out = torch.full((Tcap, N), float("nan"), dtype=torch.float32, device=dev())
        got = fn(*_mx_dev(qa, sa), *_mx_dev(qw, sw), to_dev(offs), torch.float32, out=out, dev_err=err)
        np.testing.assert_array_equal(host(got).astype(np.float64), ref, err_msg=fn.__name__)
        assert int(err.item()) == 0


@pytest.mark.parametrize("E", [17, 63, 64, 200, 1024])
def test_many_groups_token_order_and_pad_quantize(gpu, E):
    """Routed tokens with ragged sizes (empty experts included): fused pad +
    quantize against the oracle, then the token-order forward against the
    oracle's padded result unpadded."""
    rng = np.random.default_rng(E + 1)
    sizes = np.where(rng.random(E) < 0.4, 0, rng.integers(1, 200, E)).astype(np.int32)
    T = int(sizes.sum())
    Tcap = synth.capacity(T, E)
    D, N = 128, 256
    xb = synth.bits(synth.normal_bf16((T, D), 1.0, synth.generator(E)))
    x = to_dev(xb.view(np.int16)).view(torch.bfloat16)
    err = torch.zeros(1, dtype=torch.int32, device=dev())
    got = mx.pad_quantize(x, to_dev(sizes), Tcap, "rceil", True, False, dev_err=err)
    ref = O.pad_quantize(xb, sizes, 128, Tcap, "rceil", True, False)
    np.testing.assert_array_equal(host(got["offs"]), ref["offs"])
    np.testing.assert_array_equal(host(got["src_row"]), ref["src_row"])
    np.testing.assert_array_equal(host(got["q_row"]), ref["q_row"])
    np.testing.assert_array_equal(plain(host(got["s_row"])), ref["s_row"])
    assert int(err.item()) == 0
    # token-order forward on exact operands: equals the oracle's padded
    # product with the pad rows and the tail dropped
    qa, sa = _int_mx((Tcap, D), 3)
    qw, sw = _int_mx((E, N, D), 4)
    padded = O.grouped_mm(qa, sa, qw, sw, ref["offs"])
    src = ref["src_row"]
    want = np.zeros((T, N))
    want[src[src >= 0]] = padded[src >= 0]
    got_t = mx.grouped_mm_fwd_unpad(*_mx_dev(qa, sa), *_mx_dev(qw, sw), got["offs"], to_dev(sizes), T,
                                    torch.float32, dev_err=err)
    np.testing.assert_array_equal(host(got_t).astype(np.float64), want)
    assert int(err.item()) == 0


@pytest.mark.parametrize("E,p_empty", [(1, 0.0), (17, 0.35), (33, 0.35), (63, 0.35), (64, 0.35), (200, 0.35),
                                       (1024, 0.8)])
def test_many_groups_wgrad(gpu, E, p_empty):
    N, K = 128, 160
    offs = np.cumsum(_slots(E, E + 2, p_empty)).astype(np.int32)
    Tcap = int(offs[-1]) + 128
    qg, sg = _int_mx((N, Tcap), 5)
    qx, sx = _int_mx((K, Tcap), 6)
    out = torch.full((E, N, K), float("nan"), dtype=torch.float32, device=dev())
    got = mx.grouped_mm_wgrad(*_mx_dev(qg, sg), *_mx_dev(qx, sx), to_dev(offs), torch.float32, out=out)
    np.testing.assert_array_equal(host(got).astype(np.float64), O.grouped_mm_wgrad(qg, sg, qx, sx, offs))


@pytest.mark.parametrize("E", [63, 64, 200])
def test_many_groups_wgrad_hp(gpu, E):
    """bf16 operands that are small integers: the float32 sums are exact, so
    the one bf16 rounding matches the oracle's."""
    N, K = 96, 128
    offs = np.cumsum(_slots(E, 9, 0.35)).astype(np.int32)
    Tcap = int(offs[-1]) + 128
    rng = np.random.default_rng(7)
    g = torch.from_numpy(rng.integers(-8, 9, (Tcap, N)).astype(np.float32)).to(torch.bfloat16)
    x = torch.from_numpy(rng.integers(-8, 9, (Tcap, K)).astype(np.float32)).to(torch.bfloat16)
    out = torch.full((E, N, K), float("nan"), dtype=torch.bfloat16, device=dev())
    got = mx.grouped_mm_wgrad_hp(g.to(dev()), x.to(dev()), to_dev(offs), out=out)
    ref = O.grouped_mm_wgrad_hp(synth.bits(g), synth.bits(x), offs)
    np.testing.assert_array_equal(bf16_host(got).view(np.uint16), O.f64_to_bf16(ref))


@pytest.mark.parametrize("E", [3, 63, 64, 70])
def test_bad_offsets_flag_dev_err_both_tables(gpu, E):
    """Offsets that are not multiples of 128, that decrease, or that pass
    Tcap raise bit 0 of dev_err in the forward and the weight gradient, with
    the table in registers (E < 64) and in LDS; valid ones raise nothing."""
    N, K = 128, 128
    good = np.cumsum(_slots(E, E + 5, 0.3)).astype(np.int32)
    Tcap = int(good[-1]) + 128
    qa, sa = _int_mx((Tcap, K), 11)
    qw, sw = _int_mx((E, N, K), 12)
    qg, sg = _int_mx((N, Tcap), 13)
    qx, sx = _int_mx((K, Tcap), 14)
    bads = []
    b = good.copy(); b[E // 2] += 64; bads.append(b)                              # not a multiple of 128
    if E > 1:
        b = good.copy(); b[E - 2] = b[E - 1] + 128; bads.append(b)                 # decreasing
    b = good.copy(); b[-1] = Tcap + 128; bads.append(b)                            # past Tcap
    for offs in [good] + bads:
        want = 0 if offs is good else 1
        for run in ("fwd", "wgrad"):
            err = torch.zeros(1, dtype=torch.int32, device=dev())
            if run == "fwd":
                mx.grouped_mm_fwd(*_mx_dev(qa, sa), *_mx_dev(qw, sw), to_dev(offs), torch.float32, dev_err=err)
            else:
                mx.grouped_mm_wgrad(*_mx_dev(qg, sg), *_mx_dev(qx, sx), to_dev(offs), torch.float32, dev_err=err)
            torch.cuda.synchronize()
            assert (int(err.item()) & 1) == want, (run, offs.tolist())


@pytest.mark.parametrize("seed", range(12))
def test_random_shapes_bit_exact(gpu, seed):
    """Seeded random shapes around the tile edges: 1..80 groups (empty ones
    included, so both group tables run), N and the weight gradient's K any
    multiple of 16 up to 640 (partial column tiles), K 128..640 (one to five
    K steps, odd counts included), a tail of 0..2 slots. Forward, dgrad,
    weight gradient and the token-order forward, bit for bit against the
    oracle on exact operands."""
    rng = np.random.default_rng(1000 + seed)
    E = int(rng.integers(1, 81))
    N = 16 * int(rng.integers(1, 41))
    K = 128 * int(rng.integers(1, 6))
    Kw = 16 * int(rng.integers(1, 41))
    offs = np.cumsum(_slots(E, 2000 + seed, float(rng.uniform(0.0, 0.6)))).astype(np.int32)
    Tcap = int(offs[-1]) + 128 * int(rng.integers(0, 3))
    print(f"seed {seed}: E={E} N={N} K={K} Kw={Kw} Tcap={Tcap}", flush=True)
    qa, sa = _int_mx((Tcap, K), 3 * seed)
    qw, sw = _int_mx((E, N, K), 3 * seed + 1)
    ref = O.grouped_mm(qa, sa, qw, sw, offs)
    err = torch.zeros(1, dtype=torch.int32, device=dev())
    for fn in (mx.grouped_mm_fwd, mx.grouped_mm_dgrad):
        out = torch.full((Tcap, N), float("nan"), dtype=torch.float32, device=dev())
        got = fn(*_mx_dev(qa, sa), *_mx_dev(qw, sw), to_dev(offs), torch.float32, out=out, dev_err=err)
        np.testing.assert_array_equal(host(got).astype(np.float64), ref, err_msg=fn.__name__)
    # token order: each group's first n_g padded rows are its tokens
    slot = np.diff(np.concatenate([[0], offs]))
    sizes = np.minimum(slot, rng.integers(0, 129, E) + np.maximum(slot - 128, 0)).astype(np.int32)
    T = int(sizes.sum())
    if T:
        rows = np.concatenate([np.arange(s, s + n) for s, n in zip(offs - slot, sizes)]).astype(np.int64)
        got_t = mx.grouped_mm_fwd_unpad(*_mx_dev(qa, sa), *_mx_dev(qw, sw), to_dev(offs), to_dev(sizes), T,
                                        torch.float32, dev_err=err)
        np.testing.assert_array_equal(host(got_t).astype(np.float64), ref[rows])
    qg, sg = _int_mx((N, Tcap), 3 * seed + 2)
    qx, sx = _int_mx((Kw, Tcap), 3 * seed + 3)
    out = torch.full((E, N, Kw), float("nan"), dtype=torch.float32, device=dev())
    got = mx.grouped_mm_wgrad(*_mx_dev(qg, sg), *_mx_dev(qx, sx), to_dev(offs), torch.float32, out=out,
                              dev_err=err)
    np.testing.assert_array_equal(host(got).astype(np.float64), O.grouped_mm_wgrad(qg, sg, qx, sx, offs))
    assert int(err.item()) == 0


@pytest.mark.parametrize("seed", range(6))
def test_random_shapes_wgrad_hp(gpu, seed):
    """wgrad_with_hp on seeded random shapes: 1..80 groups, N and K any
    multiple of 16 up to 640, a tail of 0..2 slots; small-integer bf16
    operands, so the float32 sums are exact and the one bf16 rounding must
    match the oracle's bit for bit."""
    rng = np.random.default_rng(7000 + seed)
    E = int(rng.integers(1, 81))
    N = 16 * int(rng.integers(1, 41))
    K = 16 * int(rng.integers(1, 41))
    offs = np.cumsum(_slots(E, 8000 + seed, float(rng.uniform(0.0, 0.6)))).astype(np.int32)
    Tcap = int(offs[-1]) + 128 * int(rng.integers(0, 3))
    print(f"seed {seed}: E={E} N={N} K={K} Tcap={Tcap}", flush=True)
    g = torch.from_numpy(rng.integers(-8, 9, (Tcap, N)).astype(np.float32)).to(torch.bfloat16)
    x = torch.from_numpy(rng.integers(-8, 9, (Tcap, K)).astype(np.float32)).to(torch.bfloat16)
    out = torch.full((E, N, K), float("nan"), dtype=torch.bfloat16, device=dev())
    err = torch.zeros(1, dtype=torch.int32, device=dev())
    got = mx.grouped_mm_wgrad_hp(g.to(dev()), x.to(dev()), to_dev(offs), out=out, dev_err=err)
    ref = O.grouped_mm_wgrad_hp(synth.bits(g), synth.bits(x), offs)
    np.testing.assert_array_equal(bf16_host(got).view(np.uint16), O.f64_to_bf16(ref))
    assert int(err.item()) == 0
