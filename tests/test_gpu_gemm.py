"""GPU parity of the MXFP8 scaled GEMM, the grouped GEMMs (forward, input
gradient, weight gradient) and the bf16 wgrad_with_hp GEMM against the
oracle's float64 results, at small sizes spanning several tiles with ragged
edges, empty groups and tails, and at the full MLP / MoE shapes on sampled
outputs."""

import numpy as np
import pytest
import torch

from _helpers import bf16_host, bf16_ulp_check, dev, frob_rel, host, rand_mx, to_dev
from oracle import mx as O
from quantize_grouped_gemm_amd import mx, synth

pytestmark = pytest.mark.gpu


def _mx_dev(q, s):
    return to_dev(q), to_dev(s)


def _check_out(got, ref, out_dtype, what=""):
    if out_dtype == torch.float32:
        err = frob_rel(host(got), ref)
        assert err <= 1e-5, f"{what}: relative Frobenius error {err}"
    else:
        worst, strict = bf16_ulp_check(bf16_host(got), ref)
        assert worst <= 2.0, f"{what}: {worst} bf16 ulp (strict failures {strict})"


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("M,N,K", [(256, 256, 512), (300, 200, 384), (512, 768, 1024), (16, 48, 128)])
def test_scaled_mm(gpu, M, N, K, out_dtype):
    qa, sa = rand_mx((M, K), M + K)
    qb, sb = rand_mx((N, K), N + K + 1)
    got = mx.scaled_mm(*_mx_dev(qa, sa), *_mx_dev(qb, sb), out_dtype)
    _check_out(got, O.scaled_mm(qa, sa, qb, sb), out_dtype, f"{M}x{N}x{K}")


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
    y = mx.scaled_mm(qx["q_row"], qx["s_row"], qw["q_row"], qw["s_row"], torch.bfloat16)
    _check_out(y, O.scaled_mm(ox["q_row"], ox["s_row"], ow["q_row"], ow["s_row"]), torch.bfloat16)


def test_scaled_mm_unit_scales_exact(gpu):
    """Unit scales and small-integer codes: every partial sum is an integer
    below 2^24, so the float32 result must be exact."""
    rng = np.random.default_rng(4)
    vals = np.array([0.0, 1.0, 2.0, 3.0, -1.0, -2.0, -4.0, 8.0])
    A = rng.choice(vals, (256, 1024))
    B = rng.choice(vals, (128, 1024))
    qa, qb = O.e4m3_encode(A), O.e4m3_encode(B)
    sa = np.full((256, 32), 127, np.uint8)
    sb = np.full((128, 32), 127, np.uint8)
    got = mx.scaled_mm(*_mx_dev(qa, sa), *_mx_dev(qb, sb), torch.float32)
    np.testing.assert_array_equal(host(got), (A @ B.T).astype(np.float32))


def _offsets(sizes_padded):
    return np.cumsum(sizes_padded).astype(np.int32)


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_grouped_fwd_and_dgrad(gpu, out_dtype):
    E, N, K = 5, 320, 256
    slots = np.array([128, 0, 384, 256, 128])           # empty group, half tiles
    offs = _offsets(slots)
    Tcap = int(offs[-1]) + 256                          # a tail of 256 rows
    qa, sa = rand_mx((Tcap, K), 1)
    qw, sw = rand_mx((E, N, K), 2)
    offs_d = to_dev(offs)
    ref = O.grouped_mm(qa, sa, qw, sw, offs)
    for fn in (mx.grouped_mm_fwd, mx.grouped_mm_dgrad):
        out = torch.full((Tcap, N), float("nan"), dtype=out_dtype, device=dev())
        got = fn(*_mx_dev(qa, sa), *_mx_dev(qw, sw), offs_d, out_dtype, out=out)
        _check_out(got, ref, out_dtype, fn.__name__)
        assert torch.all(got[int(offs[-1]):] == 0)


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_grouped_wgrad(gpu, out_dtype):
    E, N, K = 4, 272, 320
    slots = np.array([256, 0, 640, 128])
    offs = _offsets(slots)
    Tcap = int(offs[-1]) + 128
    qg, sg = rand_mx((N, Tcap), 3)
    qx, sx = rand_mx((K, Tcap), 4)
    out = torch.full((E, N, K), float("nan"), dtype=out_dtype, device=dev())
    got = mx.grouped_mm_wgrad(*_mx_dev(qg, sg), *_mx_dev(qx, sx), to_dev(offs), out_dtype, out=out)
    ref = O.grouped_mm_wgrad(qg, sg, qx, sx, offs)
    for g in range(E):
        if slots[g] == 0:
            assert torch.all(got[g] == 0)
        else:
            _check_out(got[g], ref[g], out_dtype, f"group {g}")


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
    for e in (0, 2):
        worst, _ = bf16_ulp_check(bf16_host(got[e]), ref[e])
        assert worst <= 2.0


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
    with pytest.raises(mx.MXError):
        mx.scaled_mm(*_mx_dev(qa, sa), *_mx_dev(qa, sa))          # K = 96 not a multiple of 128
    with pytest.raises(mx.MXError):
        mx.quantize(torch.zeros((64, 48), dtype=torch.bfloat16, device=dev()))   # cols % 32


# ---------------------------------------------------------------- full shapes

def _sampled_gemm_check(got, qa, sa, qb, sb, rows, cols, out_dtype):
    ref = O.scaled_mm(host(qa[rows]), host(sa[rows]), host(qb[cols]), host(sb[cols]))
    g = got[rows][:, cols]
    _check_out(g, ref, out_dtype)


@pytest.mark.parametrize("M,N,K", [(8192, 28672, 4096), (8192, 4096, 14336), (28672, 4096, 8192)])
def test_dense_mlp_gemm_shapes_sampled(gpu, M, N, K):
    """Dense SwiGLU MLP GEMM shapes (w13 forward, w2 forward, w13 weight
    gradient) with synthetic MX operands; 256 x 256 sampled outputs."""
    gen = torch.Generator(device=dev())
    gen.manual_seed(M + N + K)
    qa = torch.randint(0, 0x7F, (M, K), generator=gen, device=dev(), dtype=torch.int32).to(torch.uint8)
    qb = torch.randint(0, 0x7F, (N, K), generator=gen, device=dev(), dtype=torch.int32).to(torch.uint8)
    qa |= (torch.randint(0, 2, (M, K), generator=gen, device=dev(), dtype=torch.int32) << 7).to(torch.uint8)
    qb |= (torch.randint(0, 2, (N, K), generator=gen, device=dev(), dtype=torch.int32) << 7).to(torch.uint8)
    sa = torch.randint(118, 132, (M, K // 32), generator=gen, device=dev(), dtype=torch.int32).to(torch.uint8)
    sb = torch.randint(118, 132, (N, K // 32), generator=gen, device=dev(), dtype=torch.int32).to(torch.uint8)
    got = mx.scaled_mm(qa, sa, qb, sb, torch.bfloat16)
    rng = np.random.default_rng(0)
    rows = torch.as_tensor(np.sort(rng.choice(M, 256, replace=False)), device=dev())
    cols = torch.as_tensor(np.sort(rng.choice(N, 256, replace=False)), device=dev())
    _sampled_gemm_check(got, qa, sa, qb, sb, rows, cols, torch.bfloat16)


def test_moe_grouped_shapes_sampled(gpu):
    """Routed-experts shapes (E=16, D=5120, H=8192, 16384 Zipf-routed tokens
    padded to 128): grouped w13 forward on synthetic MX operands, sampled
    rows of every non-empty group against the oracle."""
    E, D, H, T = 16, 5120, 8192, 16384
    sizes = synth.zipf_group_sizes(T, E, 14)
    slots = (sizes + 127) // 128 * 128
    offs = _offsets(slots)
    Tcap = synth.capacity(T, E)
    N, K = 2 * H, D
    gen = torch.Generator(device=dev())
    gen.manual_seed(3)
    qa = torch.randint(0, 256, (Tcap, K), generator=gen, device=dev(), dtype=torch.int32).to(torch.uint8)
    qa[(qa & 0x7F) == 0x7F] = 0x11
    sa = torch.randint(118, 132, (Tcap, K // 32), generator=gen, device=dev(), dtype=torch.int32).to(torch.uint8)
    qw = torch.randint(0, 256, (E, N, K), generator=gen, device=dev(), dtype=torch.int32).to(torch.uint8)
    qw[(qw & 0x7F) == 0x7F] = 0x22
    sw = torch.randint(118, 132, (E, N, K // 32), generator=gen, device=dev(), dtype=torch.int32).to(torch.uint8)
    got = mx.grouped_mm_fwd(qa, sa, qw, sw, to_dev(offs), torch.bfloat16)
    assert torch.all(got[int(offs[-1]):] == 0)
    rng = np.random.default_rng(1)
    cols = torch.as_tensor(np.sort(rng.choice(N, 128, replace=False)), device=dev())
    start = 0
    for g in range(E):
        end = int(offs[g])
        if end > start:
            rows = torch.as_tensor(np.sort(rng.choice(np.arange(start, end), 16, replace=False)), device=dev())
            ref = O.scaled_mm(host(qa[rows]), host(sa[rows]), host(qw[g][cols]), host(sw[g][cols]))
            _check_out(got[rows][:, cols], ref, torch.bfloat16, f"group {g}")
        start = end
