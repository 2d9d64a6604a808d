"""GPU parity of the fused SwiGLU + dual MX quantization kernels (forward and
backward) against the oracle, plus the fused-vs-standalone contract: the
fused forward's codes equal the standalone quantization of the bf16 h that
the same kernel materializes on request."""

import numpy as np
import pytest
import torch

from _helpers import bf16_host, code_tolerance, dev, host, plain, to_dev
from oracle import mx as O
from quantize_grouped_gemm_amd import mx, synth

pytestmark = pytest.mark.gpu


def _inputs(T, H, seed, scale=2.0):
    g = synth.generator(seed)
    z = synth.normal_bf16((T, 2 * H), scale, g)      # the w13 output: [a | b]
    dh = synth.normal_bf16((T, H), 1.0, g)
    return synth.bits(z), synth.bits(dh)


def _dev_bf16(b):
    return to_dev(b.view(np.int16)).view(torch.bfloat16)


def _scales(t, layout):
    return plain(host(t)) if layout == "k128" else host(t)


SHAPES = [(64, 96, "plain"), (160, 224, "plain"), (256, 384, "k128"), (2048, 2048, "k128")]


def _assert_close_codes(got, ref, what, frac=1e-5):
    ndiff, nbeyond, n, nscale = code_tolerance(got[0], got[1], ref[0], ref[1])
    assert nbeyond == 0, f"{what}: {nbeyond} elements beyond one E4M3 code"
    assert ndiff <= max(frac * n, 0), f"{what}: {ndiff}/{n} elements differ"


@pytest.mark.parametrize("mode", ["rceil", "floor"])
@pytest.mark.parametrize("T,H,layout", SHAPES)
def test_swiglu_fwd(gpu, mode, T, H, layout):
    zb, _ = _inputs(T, H, seed=T + H)
    z = _dev_bf16(zb)
    got = mx.swiglu_quant_fwd(z[:, :H], z[:, H:], mode, want_h=True, layout=layout)
    ref = O.swiglu_quant_fwd(zb[:, :H], zb[:, H:], mode)
    _assert_close_codes((host(got["q_row"]), _scales(got["s_row"], layout)), (ref["q_row"], ref["s_row"]), "row")
    _assert_close_codes((host(got["q_col"]), _scales(got["s_col"], layout)), (ref["q_col"], ref["s_col"]), "col")
    # the materialized bf16 h: within one bf16 ulp of the correctly rounded value
    hg = O.bf16_to_f64(bf16_host(got["h"]))
    hr = O.bf16_to_f64(ref["h"])
    ulp = np.exp2(np.maximum(np.floor(np.log2(np.where(hr != 0, np.abs(hr), 1.0))), -126) - 7)
    assert np.all(np.abs(hg - hr) <= ulp)
    assert np.mean(hg != hr) < 1e-3
    # fused vs standalone: quantizing the kernel's own bf16 h gives the same bytes
    st = mx.quantize(got["h"], mode, True, True, layout=layout)
    for k in ("q_row", "s_row", "q_col", "s_col"):
        assert torch.equal(st[k], got[k]), k


@pytest.mark.parametrize("mode", ["rceil", "floor"])
@pytest.mark.parametrize("T,H,layout", SHAPES)
def test_swiglu_bwd(gpu, mode, T, H, layout):
    zb, dhb = _inputs(T, H, seed=3 * T + H)
    z = _dev_bf16(zb)
    dh = _dev_bf16(dhb)
    got = mx.swiglu_quant_bwd(dh, z[:, :H], z[:, H:], mode, want_dab=True, layout=layout)
    ref = O.swiglu_quant_bwd(dhb, zb[:, :H], zb[:, H:], mode)
    _assert_close_codes((host(got["q_row"]), _scales(got["s_row"], layout)), (ref["q_row"], ref["s_row"]), "row")
    _assert_close_codes((host(got["q_col"]), _scales(got["s_col"], layout)), (ref["q_col"], ref["s_col"]), "col")
    dg = O.bf16_to_f64(bf16_host(got["dab"]))
    dr = O.bf16_to_f64(ref["dab"])
    ulp = np.exp2(np.maximum(np.floor(np.log2(np.where(dr != 0, np.abs(dr), 1.0))), -126) - 7)
    assert np.all(np.abs(dg - dr) <= ulp)
    st = mx.quantize(got["dab"], mode, True, True, layout=layout)
    for k in ("q_row", "s_row", "q_col", "s_col"):
        assert torch.equal(st[k], got[k]), k


@pytest.mark.parametrize("seed", range(6))
def test_swiglu_random_shapes(gpu, seed):
    """Seeded random shapes off the tile grid (T and H multiples of 32, or of
    128 for k128 scales), a and b with a row stride wider than 2H (views of
    a wider z), dh with its own wider stride: forward and backward against
    the oracle, and the fused-vs-standalone bytes."""
    rng = np.random.default_rng(5000 + seed)
    layout = ["plain", "k128"][seed % 2]
    mode = ["rceil", "floor"][int(rng.integers(0, 2))]
    m = 128 if layout == "k128" else 32
    T = m * int(rng.integers(1, 1 + 512 // m))
    H = m * int(rng.integers(1, 1 + 512 // m))
    pad_z = 8 * int(rng.integers(0, 4))
    pad_dh = 8 * int(rng.integers(0, 4))
    print(f"seed {seed}: {layout} {mode} T={T} H={H} pad_z={pad_z} pad_dh={pad_dh}", flush=True)
    g = synth.generator(6000 + seed)
    zb = synth.bits(synth.normal_bf16((T, 2 * H + pad_z), 2.0, g))
    dhb = synth.bits(synth.normal_bf16((T, H + pad_dh), 1.0, g))
    z = _dev_bf16(zb)
    dh = _dev_bf16(dhb)[:, :H]
    za, zbb = zb[:, :H], zb[:, H:2 * H]
    got = mx.swiglu_quant_fwd(z[:, :H], z[:, H:2 * H], mode, want_h=True, layout=layout)
    ref = O.swiglu_quant_fwd(np.ascontiguousarray(za), np.ascontiguousarray(zbb), mode)
    _assert_close_codes((host(got["q_row"]), _scales(got["s_row"], layout)), (ref["q_row"], ref["s_row"]), "fwd row")
    _assert_close_codes((host(got["q_col"]), _scales(got["s_col"], layout)), (ref["q_col"], ref["s_col"]), "fwd col")
    st = mx.quantize(got["h"], mode, True, True, layout=layout)
    for k in ("q_row", "s_row", "q_col", "s_col"):
        assert torch.equal(st[k], got[k]), k
    got = mx.swiglu_quant_bwd(dh, z[:, :H], z[:, H:2 * H], mode, want_dab=True, layout=layout)
    ref = O.swiglu_quant_bwd(np.ascontiguousarray(dhb[:, :H]), np.ascontiguousarray(za), np.ascontiguousarray(zbb),
                             mode)
    _assert_close_codes((host(got["q_row"]), _scales(got["s_row"], layout)), (ref["q_row"], ref["s_row"]), "bwd row")
    _assert_close_codes((host(got["q_col"]), _scales(got["s_col"], layout)), (ref["q_col"], ref["s_col"]), "bwd col")
    st = mx.quantize(got["dab"], mode, True, True, layout=layout)
    for k in ("q_row", "s_row", "q_col", "s_col"):
        assert torch.equal(st[k], got[k]), k


def test_swiglu_special_values(gpu):
    """Zero gate or up halves give exact zeros; large |a| saturates silu."""
    T, H = 64, 64
    zb, dhb = _inputs(T, H, seed=1)
    zb[:, :32] = 0                                  # a = 0 -> h = 0, dB = 0
    zb[:8, H:] = 0                                  # b = 0 -> h = 0
    zb[8:16, 32:H] = 0xC47A                         # a = -1000
    zb[16:24, 32:H] = 0x447A                        # a = +1000
    z = _dev_bf16(zb)
    got = mx.swiglu_quant_fwd(z[:, :H], z[:, H:], "rceil", want_h=True, layout="plain")
    ref = O.swiglu_quant_fwd(zb[:, :H], zb[:, H:], "rceil")
    np.testing.assert_array_equal(bf16_host(got["h"]) & 0x7FFF, ref["h"] & 0x7FFF)
    for k in ("q_row", "s_row", "q_col", "s_col"):
        np.testing.assert_array_equal(host(got[k]) & (0x7F if k[0] == "q" else 0xFF),
                                      ref[k] & (0x7F if k[0] == "q" else 0xFF))


@pytest.mark.parametrize("direction", ["fwd", "bwd"])
def test_swiglu_full_size_sampled(gpu, direction):
    """The MoE Scout SwiGLU boundary in the benchmark's launch configuration
    (z = [a | b] of [18432, 16384], h of [18432, 8192]): 32 sampled rows
    of the row-wise output and 32 sampled columns of the column-wise output
    against the oracle, which evaluates only those rows / columns."""
    T, H = 18432, 8192
    g = synth.generator(21 if direction == "fwd" else 22, dev())
    z = synth.normal_bf16((T, 2 * H), 2.0, g, dev())
    a, b = z[:, :H], z[:, H:]
    dh = synth.normal_bf16((T, H), 1.0, g, dev())
    rng = np.random.default_rng(4)
    # 32 of each: the oracle's dual quantization blocks both axes by 32
    rows = torch.as_tensor(np.sort(rng.choice(T, 32, replace=False)), device=dev())
    hcols = np.sort(rng.choice(H, 32, replace=False))
    if direction == "fwd":
        got = mx.swiglu_quant_fwd(a, b, "rceil")
        ref_r = O.swiglu_quant_fwd(bf16_host(a[rows]), bf16_host(b[rows]), "rceil")
        c = torch.as_tensor(hcols, device=dev())
        ref_c = O.swiglu_quant_fwd(bf16_host(a[:, c]), bf16_host(b[:, c]), "rceil")
        col_rows = hcols
    else:
        got = mx.swiglu_quant_bwd(dh, a, b, "rceil")
        ref_r = O.swiglu_quant_bwd(bf16_host(dh[rows]), bf16_host(a[rows]), bf16_host(b[rows]), "rceil")
        c = torch.as_tensor(hcols, device=dev())
        ref_c = O.swiglu_quant_bwd(bf16_host(dh[:, c]), bf16_host(a[:, c]), bf16_host(b[:, c]), "rceil")
        col_rows = np.concatenate([hcols, H + hcols])   # dA columns, then dB columns of [dA | dB]
    _assert_close_codes((host(got["q_row"][rows]), plain(host(got["s_row"][:, rows]))),
                        (ref_r["q_row"], ref_r["s_row"]), "row")
    qc = host(got["q_col"][torch.as_tensor(col_rows, device=dev())])
    sc = plain(host(got["s_col"][:, torch.as_tensor(col_rows, device=dev())]))
    _assert_close_codes((qc, sc), (ref_c["q_col"], ref_c["s_col"]), "col")


def _every_finite_bf16():
    """All 65536 bf16 bit patterns as a [256, 256] tile, with the 512 Inf and
    NaN patterns (exponent all ones) replaced by zero."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    bits[(bits & 0x7F80) == 0x7F80] = 0
    return bits.reshape(256, 256)


def _within_one_bf16_ulp(got_bits, ref_bits, what):
    g, r = O.bf16_to_f64(got_bits), O.bf16_to_f64(ref_bits)
    ulp = np.exp2(np.maximum(np.floor(np.log2(np.where(r != 0, np.abs(r), 1.0))), -126) - 7)
    bad = np.abs(g - r) > ulp
    assert not bad.any(), f"{what}: {int(bad.sum())} values beyond one bf16 ulp, e.g. a bits " \
                          f"{np.argwhere(bad)[:4].tolist()}"


def test_swiglu_every_bf16_gate_value(gpu):
    """Every finite bf16 gate value a, with b = dh = 1: h = silu(a) and
    [dA | dB] = [s (1 + a (1 - s)), a s] each within one bf16 ulp of the
    oracle's correctly rounded value. This covers the sigmoid over its whole
    range: saturation at both ends, and the gate values near -87 .. -103
    where e^a is a float32 subnormal while silu(a) is still a bf16 number."""
    ab = _every_finite_bf16()
    ones = np.full_like(ab, 0x3F80)
    zb = np.concatenate([ab, ones], axis=1)
    z = _dev_bf16(zb)
    H = ab.shape[1]
    fwd = mx.swiglu_quant_fwd(z[:, :H], z[:, H:], "rceil", want_h=True, layout="plain")
    ref = O.swiglu_quant_fwd(ab, ones, "rceil")
    _within_one_bf16_ulp(bf16_host(fwd["h"]), ref["h"], "h")
    bwd = mx.swiglu_quant_bwd(_dev_bf16(ones), z[:, :H], z[:, H:], "rceil", want_dab=True, layout="plain")
    refb = O.swiglu_quant_bwd(ones, ab, ones, "rceil")
    _within_one_bf16_ulp(bf16_host(bwd["dab"]), refb["dab"], "dA | dB")
    # the codes: never more than one E4M3 code from the oracle's
    for got, want in ((fwd, ref), (bwd, refb)):
        for ax in ("row", "col"):
            _, nbeyond, _, _ = code_tolerance(host(got["q_" + ax]), host(got["s_" + ax]),
                                              want["q_" + ax], want["s_" + ax])
            assert nbeyond == 0, ax
