"""GPU parity of the MXFP8 scaled GEMM, the grouped GEMMs (forward, input
gradient, weight gradient) and the bf16 wgrad_with_hp GEMM against the
oracle's float64 results: bit-exact on operands the MFMA sums exactly (this
pins the operand layout and every scale), within the MFMA accumulation model
(see _helpers) otherwise; at small sizes spanning several tiles with ragged
edges, empty groups and tails, and at the full MLP / MoE shapes on sampled
outputs."""

import numpy as np
import pytest
import torch

from _helpers import (FROB_MFMA, bf16_host, check_gemm, dev, host, hp_bound, k128, mfma_bound, rand_mx, real_mx,
                      to_dev)
from oracle import mx as O
from quantize_grouped_gemm_amd import mx, synth

pytestmark = pytest.mark.gpu


def _mx_dev(q, s):
    """Oracle operand (plain scales) -> device codes and k128 scales."""
    return to_dev(q), to_dev(k128(s))


def _got(got):
    """Device GEMM output -> float64 host values."""
    if got.dtype == torch.float32:
        return host(got).astype(np.float64)
    return O.bf16_to_f64(bf16_host(got))


def _check(got, A, B, ref, out_dtype, what="", frob=FROB_MFMA):
    """got vs the oracle's float64 ref = A B^T (A, B dequantized): within the
    MFMA model's bound elementwise (see _helpers.check_gemm); float32 outputs
    also within `frob` relative Frobenius error."""
    kind = "f32" if out_dtype == torch.float32 else "bf16"
    stats = check_gemm(_got(got), ref, mfma_bound(A, B), kind, what)
    if kind == "f32" and frob is not None:
        assert stats["frob"] <= frob, f"{what}: relative Frobenius error {stats['frob']}"
    return stats


def _int_mx(shape, seed):
    """Integer-valued MX operand the MFMA sums exactly: codes for 0, +-1, +-2,
    +-3, +-4, +-6, +-8 and scale bytes 127..130 (x1..x8)."""
    rng = np.random.default_rng(seed)
    vals = np.array([0, 1, 2, 3, 4, 6, 8, -1, -2, -3, -4, -6, -8], np.float64)
    q = O.e4m3_encode(rng.choice(vals, shape))
    s = rng.integers(127, 131, shape[:-1] + (shape[-1] // 32,)).astype(np.uint8)
    return q, s


@pytest.mark.parametrize("M,N,K", [(256, 256, 512), (300, 200, 384), (512, 768, 1024), (16, 48, 128)])
def test_scaled_mm_exact_with_scales(gpu, M, N, K):
    """Products lie within 2^12 of each other in every 16-group and sums stay
    below 2^24: the float32 result must equal the exact one bit for bit."""
    qa, sa = _int_mx((M, K), M + K)
    qb, sb = _int_mx((N, K), N + K + 1)
    got = mx.scaled_mm(*_mx_dev(qa, sa), *_mx_dev(qb, sb), torch.float32)
    ref = O.scaled_mm(qa, sa, qb, sb)
    np.testing.assert_array_equal(host(got).astype(np.float64), ref)


@pytest.mark.parametrize("seed", range(8))
def test_scaled_mm_random_shapes_exact(gpu, seed):
    """Seeded random shapes around the tile edges (M any, N a multiple of 16,
    K one to six 128-wide steps), written into a wider output (row stride
    above N): exact operands, bit for bit, and the columns past N untouched."""
    rng = np.random.default_rng(3000 + seed)
    M = int(rng.integers(1, 700))
    N = 16 * int(rng.integers(1, 45))
    K = 128 * int(rng.integers(1, 7))
    ld = N + 16 * int(rng.integers(0, 3))
    print(f"seed {seed}: M={M} N={N} K={K} ld={ld}", flush=True)
    qa, sa = _int_mx((M, K), 2 * seed)
    qb, sb = _int_mx((N, K), 2 * seed + 1)
    wide = torch.full((M, ld), 7.0, dtype=torch.float32, device=dev())
    got = mx.scaled_mm(*_mx_dev(qa, sa), *_mx_dev(qb, sb), out=wide[:, :N])
    np.testing.assert_array_equal(host(got).astype(np.float64), O.scaled_mm(qa, sa, qb, sb))
    assert torch.all(wide[:, N:] == 7.0)


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("M,N,K", [(256, 256, 512), (300, 200, 384), (512, 768, 1024), (16, 48, 128)])
def test_scaled_mm_realistic(gpu, M, N, K, out_dtype):
    qa, sa, _ = real_mx((M, K), 1.0, M + K)
    qb, sb, _ = real_mx((N, K), 0.02, N + K + 1)
    got = mx.scaled_mm(*_mx_dev(qa, sa), *_mx_dev(qb, sb), out_dtype)
    _check(got, O.dequantize(qa, sa), O.dequantize(qb, sb), O.scaled_mm(qa, sa, qb, sb), out_dtype,
           f"{M}x{N}x{K}")


def test_scaled_mm_wide_dynamic_range(gpu):
    """Codes uniform over all finite E4M3 values (products spanning ~2^36):
    elementwise within the MFMA bound."""
    qa, sa = rand_mx((256, 512), 1)
    qb, sb = rand_mx((320, 512), 2)
    got = mx.scaled_mm(*_mx_dev(qa, sa), *_mx_dev(qb, sb), torch.float32)
    _check(got, O.dequantize(qa, sa), O.dequantize(qb, sb), O.scaled_mm(qa, sa, qb, sb), torch.float32,
           frob=1e-4)


def test_scaled_mm_linear_workload(gpu):
    """The single MXFP8 linear: bf16 x [256,512] ~ N(0,1), W [256,512] ~
    N(0,0.02), RCEIL row-wise quantization on the GPU (bit-exact against the
    oracle), then the scaled GEMM to bf16."""
    x, w = synth.linear_inputs(seed=0, device=dev())
    qx = mx.quantize(x, "rceil")
    qw = mx.quantize(w, "rceil")
    ox = O.quantize_bf16(bf16_host(x), "rceil")
    ow = O.quantize_bf16(bf16_host(w), "rceil")
    np.testing.assert_array_equal(host(qx["q_row"]), ox["q_row"])
    np.testing.assert_array_equal(host(qw["q_row"]), ow["q_row"])
    for dt in (torch.bfloat16, torch.float32):
        y = mx.scaled_mm(qx["q_row"], qx["s_row"], qw["q_row"], qw["s_row"], dt)
        _check(y, O.dequantize(ox["q_row"], ox["s_row"]), O.dequantize(ow["q_row"], ow["s_row"]),
               O.scaled_mm(ox["q_row"], ox["s_row"], ow["q_row"], ow["s_row"]), dt)


def _offsets(slots):
    return np.cumsum(slots).astype(np.int32)


def test_grouped_exact_with_scales(gpu):
    E, N, K = 5, 320, 256
    slots = np.array([128, 0, 384, 256, 128])
    offs = _offsets(slots)
    Tcap = int(offs[-1]) + 256
    qa, sa = _int_mx((Tcap, K), 1)
    qw, sw = _int_mx((E, N, K), 2)
    ref = O.grouped_mm(qa, sa, qw, sw, offs)
    for fn in (mx.grouped_mm_fwd, mx.grouped_mm_dgrad):
        out = torch.full((Tcap, N), float("nan"), dtype=torch.float32, device=dev())
        got = fn(*_mx_dev(qa, sa), *_mx_dev(qw, sw), to_dev(offs), torch.float32, out=out)
        np.testing.assert_array_equal(host(got).astype(np.float64), ref)
    qg, sg = _int_mx((N, Tcap), 3)
    qx, sx = _int_mx((K, Tcap), 4)
    out = torch.full((E, N, K), float("nan"), dtype=torch.float32, device=dev())
    got = mx.grouped_mm_wgrad(*_mx_dev(qg, sg), *_mx_dev(qx, sx), to_dev(offs), torch.float32, out=out)
    np.testing.assert_array_equal(host(got).astype(np.float64), O.grouped_mm_wgrad(qg, sg, qx, sx, offs))


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_grouped_fwd_and_dgrad(gpu, out_dtype):
    E, N, K = 5, 320, 256
    slots = np.array([128, 0, 384, 256, 128])           # empty group, half tiles
    offs = _offsets(slots)
    Tcap = int(offs[-1]) + 256                          # a tail of 256 rows
    qa, sa, _ = real_mx((Tcap, K), 1.0, 1)
    qw, sw, _ = real_mx((E, N, K), 0.02, 2)
    ref = O.grouped_mm(qa, sa, qw, sw, offs)
    A = O.dequantize(qa, sa)
    for fn in (mx.grouped_mm_fwd, mx.grouped_mm_dgrad):
        out = torch.full((Tcap, N), float("nan"), dtype=out_dtype, device=dev())
        got = fn(*_mx_dev(qa, sa), *_mx_dev(qw, sw), to_dev(offs), out_dtype, out=out)
        assert torch.all(got[int(offs[-1]):] == 0)
        start = 0
        for g in range(E):
            end = int(offs[g])
            if end > start:
                _check(got[start:end], A[start:end], O.dequantize(qw[g], sw[g]), ref[start:end], out_dtype,
                       f"{fn.__name__} group {g}")
            start = end


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("sizes", [[250, 0, 300, 50], [128, 256, 1], [0, 0, 5], [700, 0, 0, 300, 129]])
def test_grouped_token_order_equals_unpadded(gpu, sizes, out_dtype):
    """The token-order fwd / dgrad write exactly the bytes that unpadding the
    padded result gives (all rows of the output), and nothing for pad rows."""
    sizes = np.array(sizes, np.int32)
    E, T = len(sizes), int(sizes.sum())
    Tcap = synth.capacity(T, E)
    offs = _offsets(-(-sizes // 128) * 128)
    N, K = 320, 256
    src = O.pad_groups(np.zeros((T, 1), np.uint16), sizes, 128, Tcap)[2]
    qa, sa, _ = real_mx((Tcap, K), 1.0, 7)
    qw, sw, _ = real_mx((E, N, K), 0.05, 8)
    args = (*_mx_dev(qa, sa), *_mx_dev(qw, sw), to_dev(offs))
    for fn, fn_unpad in ((mx.grouped_mm_fwd, mx.grouped_mm_fwd_unpad),
                         (mx.grouped_mm_dgrad, mx.grouped_mm_dgrad_unpad)):
        padded = fn(*args, out_dtype)
        ref = mx.unpad_groups(padded, to_dev(src), T)
        err = torch.zeros(1, dtype=torch.int32, device=dev())
        out = torch.full((T, N), float("nan"), dtype=out_dtype, device=dev())
        got = fn_unpad(*args, to_dev(sizes), T, out_dtype, out=out, dev_err=err)
        assert torch.equal(got, ref), fn.__name__
        assert int(err.item()) == 0
    # sizes that exceed their padded slot are reported
    bad = sizes.copy()
    bad[np.argmax(bad)] += 128
    err = torch.zeros(1, dtype=torch.int32, device=dev())
    mx.grouped_mm_fwd_unpad(*args, to_dev(bad), T, out_dtype, dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) & 4


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_grouped_wgrad_many_group_sizes_exact(gpu, out_dtype):
    """Whole 256 x 256 dW tiles (N, K multiples of 256) over 70 groups of 0 to
    9 token steps: odd and even step counts, one-step groups and empty groups
    in between, so tiles of every length and the zero tiles of empty groups
    share one launch. Bit-exact against the oracle on integer operands
    (float32 output; bf16 output is its round-to-nearest-even)."""
    rng = np.random.default_rng(17)
    steps = rng.integers(0, 10, 70)
    steps[[3, 11, 40]] = 0
    steps[[5, 6, 7]] = 1
    offs = _offsets(steps * 128)
    Tcap = int(offs[-1]) + 256
    E, N, K = len(steps), 1024, 1024
    qg, sg = _int_mx((N, Tcap), 21)
    qx, sx = _int_mx((K, Tcap), 22)
    out = torch.full((E, N, K), float("nan"), dtype=out_dtype, device=dev())
    got = mx.grouped_mm_wgrad(*_mx_dev(qg, sg), *_mx_dev(qx, sx), to_dev(offs), out_dtype, out=out)
    ref = O.grouped_mm_wgrad(qg, sg, qx, sx, offs)
    if out_dtype == torch.float32:
        np.testing.assert_array_equal(host(got).astype(np.float64), ref)
    else:
        np.testing.assert_array_equal(bf16_host(got), O.f64_to_bf16(ref))


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_grouped_wgrad(gpu, out_dtype):
    E, N, K = 4, 272, 320
    slots = np.array([256, 0, 640, 128])
    offs = _offsets(slots)
    Tcap = int(offs[-1]) + 128
    qg, sg, _ = real_mx((Tcap, N), 1.0, 3, colwise=True)     # dY column-wise: [N, Tcap]
    qx, sx, _ = real_mx((Tcap, K), 1.0, 4, colwise=True)     # X column-wise:  [K, Tcap]
    out = torch.full((E, N, K), float("nan"), dtype=out_dtype, device=dev())
    got = mx.grouped_mm_wgrad(*_mx_dev(qg, sg), *_mx_dev(qx, sx), to_dev(offs), out_dtype, out=out)
    ref = O.grouped_mm_wgrad(qg, sg, qx, sx, offs)
    G, X = O.dequantize(qg, sg), O.dequantize(qx, sx)
    start = 0
    for g in range(E):
        end = int(offs[g])
        if end == start:
            assert torch.all(got[g] == 0)
        else:
            _check(got[g], G[:, start:end], X[:, start:end], ref[g], out_dtype, f"group {g}")
        start = end


def test_grouped_wgrad_hp(gpu):
    E, N, K = 3, 144, 208
    slots = np.array([384, 0, 256])
    offs = _offsets(slots)
    Tcap = int(offs[-1]) + 128
    gen = synth.generator(6)
    g = synth.normal_bf16((Tcap, N), 1.0, gen)
    x = synth.normal_bf16((Tcap, K), 1.0, gen)
    out = torch.full((E, N, K), float("nan"), dtype=torch.bfloat16, device=dev())
    got = mx.grouped_mm_wgrad_hp(g.to(dev()), x.to(dev()), to_dev(offs), out=out)
    ref = O.grouped_mm_wgrad_hp(synth.bits(g), synth.bits(x), offs)
    assert torch.all(got[1] == 0)
    G, X = O.bf16_to_f64(synth.bits(g)), O.bf16_to_f64(synth.bits(x))
    start = 0
    for e in range(E):
        end = int(offs[e])
        if end > start:
            check_gemm(_got(got[e]), ref[e], hp_bound(G[start:end], X[start:end]), "bf16", f"hp group {e}")
        start = end


def test_invalid_offsets_flag_dev_err(gpu):
    E, N, K, Tcap = 3, 64, 128, 512
    qa, sa = rand_mx((Tcap, K), 7)
    qw, sw = rand_mx((E, N, K), 8)
    for bad in ([128, 100, 512], [256, 128, 384], [128, 256, 640]):
        err = torch.zeros(1, dtype=torch.int32, device=dev())
        mx.grouped_mm_fwd(*_mx_dev(qa, sa), *_mx_dev(qw, sw), to_dev(np.array(bad, np.int32)),
                          dev_err=err)
        torch.cuda.synchronize()
        assert int(err.item()) & 1, bad
    err = torch.zeros(1, dtype=torch.int32, device=dev())
    mx.grouped_mm_fwd(*_mx_dev(qa, sa), *_mx_dev(qw, sw), to_dev(np.array([128, 256, 512], np.int32)),
                      dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0


def test_abi_rejects_bad_arguments(gpu):
    qa, sa = rand_mx((128, 96), 1)
    q, s = to_dev(qa), to_dev(sa)
    with pytest.raises(mx.MXError):
        mx.scaled_mm(q, s, q, s)                                  # K = 96 not a multiple of 128
    with pytest.raises(mx.MXError):
        mx.quantize(torch.zeros((64, 48), dtype=torch.bfloat16, device=dev()))   # cols % 32
    x = torch.zeros((64, 136), dtype=torch.bfloat16, device=dev())
    with pytest.raises(mx.MXError, match="16-byte aligned"):
        mx.quantize(x[:, 4:132])                                  # rows start 8 bytes into a 16-byte unit
    with pytest.raises(mx.MXError, match="q_row: "):              # output smaller than the sizes passed
        mx.quantize(x[:, :128], out={"q_row": torch.empty((64, 96), dtype=torch.uint8, device=dev())})


# ---------------------------------------------------------------- full shapes

def _oracle_rows(x_dev, rows):
    """The oracle's row-wise quantization of selected rows of a device bf16
    tensor (the input, copied to the host)."""
    q = O.quantize_bf16(bf16_host(x_dev[rows]), "rceil")
    return q["q_row"], q["s_row"]


@pytest.mark.parametrize("M,N,K", [(8192, 28672, 4096), (8192, 4096, 14336), (28672, 4096, 8192)])
def test_dense_mlp_gemm_shapes_sampled(gpu, M, N, K):
    """Dense SwiGLU MLP GEMM shapes (w13 forward, w2 forward, w13 weight
    gradient): N(0,1) x N(0,0.02) bf16 operands drawn on the GPU, quantized
    there, GEMM'd in the benchmark's launch configuration; 192 x 192 sampled
    outputs against the oracle, which quantizes the sampled rows itself."""
    g = synth.generator(M + N + K, dev())
    a = synth.normal_bf16((M, K), 1.0, g, dev())
    b = synth.normal_bf16((N, K), 0.02, g, dev())
    qa = mx.quantize(a, "rceil")
    qb = mx.quantize(b, "rceil")
    got = mx.scaled_mm(qa["q_row"], qa["s_row"], qb["q_row"], qb["s_row"], torch.bfloat16)
    rng = np.random.default_rng(0)
    rows = torch.as_tensor(np.sort(rng.choice(M, 192, replace=False)), device=dev())
    cols = torch.as_tensor(np.sort(rng.choice(N, 192, replace=False)), device=dev())
    oa = _oracle_rows(a, rows)
    ob = _oracle_rows(b, cols)
    np.testing.assert_array_equal(host(qa["q_row"][rows]), oa[0])
    A, B = O.dequantize(*oa), O.dequantize(*ob)
    _check(got[rows][:, cols], A, B, A @ B.T, torch.bfloat16)


def test_moe_grouped_shapes_sampled(gpu):
    """Routed-experts shapes (E=16, D=5120, H=8192, 16384 Zipf-routed tokens
    padded to 128): padded N(0,1) tokens and N(0,0.02) expert weights on the
    GPU, quantized there, grouped w13 forward; 16 sampled rows of every
    non-empty group x 128 sampled columns against the oracle."""
    E, D, H, T = 16, 5120, 8192, 16384
    sizes = synth.zipf_group_sizes(T, E, 14)
    Tcap = synth.capacity(T, E)
    N, K = 2 * H, D
    g = synth.generator(3, dev())
    x = synth.normal_bf16((T, K), 1.0, g, dev())
    w = synth.normal_bf16((E, N, K), 0.02, g, dev())
    x_pad, offs_d, _ = mx.pad_groups(x, to_dev(sizes.astype(np.int32)), Tcap)
    qx = mx.quantize(x_pad, "rceil")
    qw = mx.quantize(w, "rceil")
    got = mx.grouped_mm_fwd(qx["q_row"], qx["s_row"], qw["q_row"], qw["s_row"], offs_d, torch.bfloat16)
    offs = host(offs_d)
    assert torch.all(got[int(offs[-1]):] == 0)
    rng = np.random.default_rng(1)
    cols = torch.as_tensor(np.sort(rng.choice(N, 128, replace=False)), device=dev())
    start = 0
    for e in range(E):
        end = int(offs[e])
        if end > start:
            rows = torch.as_tensor(np.sort(rng.choice(np.arange(start, end), 16, replace=False)), device=dev())
            A, B = O.dequantize(*_oracle_rows(x_pad, rows)), O.dequantize(*_oracle_rows(w[e], cols))
            _check(got[rows][:, cols], A, B, A @ B.T, torch.bfloat16, f"group {e}")
        start = end



def _moe_scout_groups():
    E, T = 16, 16384
    sizes = synth.zipf_group_sizes(T, E, 14)
    Tcap = synth.capacity(T, E)
    slots = -(-sizes // 128) * 128
    return E, Tcap, _offsets(slots)


def _oracle_cols(t_dev, cols):
    """The oracle's quantization along dim 0 (tokens) of selected columns of
    a device bf16 [Tcap, C] tensor: row-wise quantization of those rows of
    its transpose (the column-wise layout's rows)."""
    q = O.quantize_bf16(bf16_host(t_dev[:, cols].T.contiguous()), "rceil")
    return q["q_row"], q["s_row"]


def test_moe_wgrad_full_size_sampled(gpu):
    """The MoE Scout w13 weight gradient in the benchmark's launch
    configuration: dW [16, 16384, 5120] float32 from column-wise MXFP8
    dZ [18432, 16384] and X [18432, 5120] over the Zipf groups (2 empty).
    Empty groups' dW is exactly zero; 24 x 24 sampled entries of every other
    group match the oracle, which quantizes the sampled rows of dZ^T and X^T
    along the tokens itself and contracts over the group's tokens."""
    E, Tcap, offs = _moe_scout_groups()
    N, K = 16384, 5120
    g = synth.generator(11, dev())
    dz = synth.normal_bf16((Tcap, N), 1.0, g, dev())
    x = synth.normal_bf16((Tcap, K), 1.0, g, dev())
    qg = mx.quantize(dz, "rceil", rowwise=False, colwise=True)
    qx = mx.quantize(x, "rceil", rowwise=False, colwise=True)
    got = mx.grouped_mm_wgrad(qg["q_col"], qg["s_col"], qx["q_col"], qx["s_col"], to_dev(offs), torch.float32)
    rng = np.random.default_rng(2)
    rows = torch.as_tensor(np.sort(rng.choice(N, 24, replace=False)), device=dev())
    cols = torch.as_tensor(np.sort(rng.choice(K, 24, replace=False)), device=dev())
    qa, sa = _oracle_cols(dz, rows)
    qb, sb = _oracle_cols(x, cols)
    np.testing.assert_array_equal(host(qg["q_col"][rows]), qa)
    start = 0
    for e in range(E):
        end = int(offs[e])
        if end == start:
            assert torch.all(got[e] == 0), f"empty group {e}"
            continue
        A = (qa[:, start:end], sa[:, start // 32:end // 32])
        B = (qb[:, start:end], sb[:, start // 32:end // 32])
        ref = O.scaled_mm(*A, *B)
        _check(got[e][rows][:, cols], O.dequantize(*A), O.dequantize(*B), ref, torch.float32, f"group {e}")
        start = end


def test_moe_dgrad_full_size_sampled(gpu):
    """The MoE Scout w13 input gradient: dX [18432, 5120] bf16 from row-wise
    MXFP8 dZ [18432, 16384] and the experts' w13 quantized along 2H
    ([16, 5120, 16384] column-wise), Zipf groups; the tail is zero and 16
    sampled rows of every non-empty group x 96 sampled columns match the
    oracle."""
    E, Tcap, offs = _moe_scout_groups()
    N, K = 5120, 16384                      # output columns (D), contraction (2H)
    g = synth.generator(12, dev())
    dz = synth.normal_bf16((Tcap, K), 1.0, g, dev())
    w = synth.normal_bf16((E, K, N), 0.02, g, dev())     # w13 [E, 2H, D]
    qd = mx.quantize(dz, "rceil")
    qw = mx.quantize(w, "rceil", rowwise=False, colwise=True)  # [E, D, 2H]
    got = mx.grouped_mm_dgrad(qd["q_row"], qd["s_row"], qw["q_col"], qw["s_col"], to_dev(offs), torch.bfloat16)
    assert torch.all(got[int(offs[-1]):] == 0)
    rng = np.random.default_rng(3)
    cols = torch.as_tensor(np.sort(rng.choice(N, 96, replace=False)), device=dev())
    start = 0
    for e in range(E):
        end = int(offs[e])
        if end > start:
            rows = torch.as_tensor(np.sort(rng.choice(np.arange(start, end), 16, replace=False)), device=dev())
            A, B = O.dequantize(*_oracle_rows(dz, rows)), O.dequantize(*_oracle_cols(w[e], cols))
            _check(got[rows][:, cols], A, B, A @ B.T, torch.bfloat16, f"group {e}")
        start = end


def test_dsv3_full_size_sampled(gpu):
    """The DeepSeek-V3-like expert share in the benchmark's launch
    configuration (32 experts, 65536 routed token slots with Dirichlet(0.3)
    group sizes padded to 128, D=7168, H=2048): the grouped w13 forward on
    sampled rows of every non-empty group, and the w2 weight gradient both in
    MXFP8 (float32 dW) and as wgrad_with_hp (bf16 operands, bf16 dW) on
    sampled entries of every group. The oracle evaluates the same GEMMs on
    the sampled rows / columns only."""
    E, D, H, T = 32, 7168, 2048, 65536
    sizes = synth.dirichlet_group_sizes(T, E, 0.3)
    Tcap = synth.capacity(T, E)
    offs = _offsets(-(-sizes // 128) * 128)
    offs_d = to_dev(offs)
    g = synth.generator(13, dev())
    rng = np.random.default_rng(5)
    # w13 forward: [Tcap, D] x [E, 2H, D]
    x = synth.normal_bf16((Tcap, D), 1.0, g, dev())
    w = synth.normal_bf16((E, 2 * H, D), 0.02, g, dev())
    qx, qw = mx.quantize(x, "rceil"), mx.quantize(w, "rceil")
    got = mx.grouped_mm_fwd(qx["q_row"], qx["s_row"], qw["q_row"], qw["s_row"], offs_d, torch.bfloat16)
    assert torch.all(got[int(offs[-1]):] == 0)
    cols = torch.as_tensor(np.sort(rng.choice(2 * H, 64, replace=False)), device=dev())
    start = 0
    for e in range(E):
        end = int(offs[e])
        if end > start:
            rows = torch.as_tensor(np.sort(rng.choice(np.arange(start, end), 8, replace=False)), device=dev())
            A, B = O.dequantize(*_oracle_rows(x, rows)), O.dequantize(*_oracle_rows(w[e], cols))
            _check(got[rows][:, cols], A, B, A @ B.T, torch.bfloat16, f"fwd group {e}")
        start = end
    del x, w, qx, qw, got
    # w2 weight gradient: dW2[g] = dY_g^T h_g, [E, D, H]
    dy = synth.normal_bf16((Tcap, D), 1.0, g, dev())
    h = synth.normal_bf16((Tcap, H), 1.0, g, dev())
    rows = torch.as_tensor(np.sort(rng.choice(D, 24, replace=False)), device=dev())
    cols = torch.as_tensor(np.sort(rng.choice(H, 24, replace=False)), device=dev())
    qd = mx.quantize(dy, "rceil", rowwise=False, colwise=True)
    qh = mx.quantize(h, "rceil", rowwise=False, colwise=True)
    got = mx.grouped_mm_wgrad(qd["q_col"], qd["s_col"], qh["q_col"], qh["s_col"], offs_d, torch.float32)
    qa, sa = _oracle_cols(dy, rows)
    qb, sb = _oracle_cols(h, cols)
    ref = O.grouped_mm_wgrad(qa, sa, qb, sb, offs)
    start = 0
    for e in range(E):
        end = int(offs[e])
        if end == start:
            assert torch.all(got[e] == 0), f"empty group {e}"
        else:
            A = O.dequantize(qa[:, start:end], sa[:, start // 32:end // 32])
            B = O.dequantize(qb[:, start:end], sb[:, start // 32:end // 32])
            _check(got[e][rows][:, cols], A, B, ref[e], torch.float32, f"wgrad group {e}")
        start = end
    del got, qd, qh
    got = mx.grouped_mm_wgrad_hp(dy, h, offs_d)
    Gs, Hs = bf16_host(dy[:, rows]), bf16_host(h[:, cols])
    ref = O.grouped_mm_wgrad_hp(Gs, Hs, offs)
    Gf, Hf = O.bf16_to_f64(Gs), O.bf16_to_f64(Hs)
    start = 0
    for e in range(E):
        end = int(offs[e])
        if end == start:
            assert torch.all(got[e] == 0), f"empty group {e} (hp)"
        else:
            check_gemm(_got(got[e][rows][:, cols]), ref[e], hp_bound(Gf[start:end], Hf[start:end]), "bf16",
                       f"hp wgrad group {e}")
        start = end


@pytest.mark.parametrize("mode", ["rceil", "floor"])
@pytest.mark.parametrize("sizes,H,K", [([250, 0, 300, 50], 256, 256), ([128, 256, 1], 384, 128),
                                       ([0, 0, 5], 128, 256), ([700, 0, 0, 300, 129], 256, 384)])
def test_grouped_swiglu_fused_equals_unfused(gpu, mode, sizes, H, K):
    """The w13 forward with the SwiGLU + dual quantization in its epilogue
    writes the same z, the same h and the same h codes and scales (both
    directions) as the grouped forward followed by the standalone fused
    SwiGLU kernel, including pad rows, the tail and empty groups."""
    sizes = np.array(sizes, np.int32)
    E, T = len(sizes), int(sizes.sum())
    Tcap = synth.capacity(T, E)
    offs = _offsets(-(-sizes // 128) * 128)
    g = synth.generator(T + H + K, dev())
    x = synth.normal_bf16((Tcap, K), 1.0, g, dev())
    w13 = synth.normal_bf16((E, 2 * H, K), 0.05, g, dev())
    qx, qw = mx.quantize(x, mode), mx.quantize(w13, mode)
    offs_d = to_dev(offs)
    fused = mx.grouped_mm_swiglu_fwd(qx["q_row"], qx["s_row"], qw["q_row"], qw["s_row"], offs_d, mode,
                                     want_h=True)
    z = mx.grouped_mm_fwd(qx["q_row"], qx["s_row"], qw["q_row"], qw["s_row"], offs_d, torch.bfloat16)
    ref = mx.swiglu_quant_fwd(z[:, :H], z[:, H:], mode, want_h=True)
    assert torch.equal(fused["z"], z)
    for k in ("h", "q_row", "s_row", "q_col", "s_col"):
        assert torch.equal(fused[k], ref[k]), k


def test_grouped_swiglu_fused_full_size(gpu):
    """The MoE Scout w13 forward (Tcap 18432, 16 experts, D 5120, H 8192)
    fused with its SwiGLU: the same bytes as the unfused pair."""
    E, Tcap, offs = _moe_scout_groups()
    H, K = 8192, 5120
    g = synth.generator(15, dev())
    x = synth.normal_bf16((Tcap, K), 1.0, g, dev())
    w13 = synth.normal_bf16((E, 2 * H, K), 0.02, g, dev())
    qx, qw = mx.quantize(x, "rceil"), mx.quantize(w13, "rceil")
    del w13
    offs_d = to_dev(offs)
    fused = mx.grouped_mm_swiglu_fwd(qx["q_row"], qx["s_row"], qw["q_row"], qw["s_row"], offs_d)
    z = mx.grouped_mm_fwd(qx["q_row"], qx["s_row"], qw["q_row"], qw["s_row"], offs_d, torch.bfloat16)
    assert torch.equal(fused["z"], z)
    ref = mx.swiglu_quant_fwd(z[:, :H], z[:, H:], "rceil")
    for k in ("q_row", "s_row", "q_col", "s_col"):
        assert torch.equal(fused[k], ref[k]), k
