"""Host-side checks of the Python binding without a GPU: every tensor it
hands to the library is checked against the sizes passed with it (dtype,
element count, layout, device) before any call, so a buffer that does not
match raises instead of being read or written out of bounds."""

import pytest
import torch

from quantize_grouped_gemm_amd import mx

U8, BF, I32 = torch.uint8, torch.bfloat16, torch.int32


def u8(*shape):
    return torch.zeros(shape, dtype=U8)


def i32(*shape):
    return torch.zeros(shape, dtype=I32)


def bf(*shape):
    return torch.zeros(shape, dtype=BF)


def raises(fn, *args, match, **kw):
    with pytest.raises(mx.MXError, match=match):
        fn(*args, **kw)


def test_dense_gemm_buffers():
    M, N, K = 256, 128, 256
    qa, sa, qb, sb = u8(M, K), u8(K // 128, M, 4), u8(N, K), u8(K // 128, N, 4)
    raises(mx.scaled_mm, qa, sa, u8(N, 128), sb, match="K=")
    raises(mx.scaled_mm, qa, u8(K // 128, M, 2), qb, sb, match="sa: ")
    raises(mx.scaled_mm, qa, sa, qb, sb, out=torch.zeros((M, N + 16), dtype=BF), match="out: shape")
    raises(mx.scaled_mm, qa, sa, qb, sb, out=torch.zeros((M, N), dtype=torch.float16), match="out: expected")
    raises(mx.scaled_mm, u8(M, 2 * K)[:, :K], sa, qb, sb, match="qa must be contiguous")
    raises(mx.scaled_mm, qa, sa, qb, sb, out=torch.zeros((N, M), dtype=BF).t(), match="contiguous rows")
    # an output whose rows are spaced wider than N is accepted up to the device check
    raises(mx.scaled_mm, qa, sa, qb, sb, out=torch.zeros((M, N + 32), dtype=BF)[:, :N], match="cuda")
    raises(mx.scaled_mm, qa.to(torch.int8), sa, qb, sb, match="qa: dtype")
    # matching buffers reach the device check, not the library
    raises(mx.scaled_mm, qa, sa, qb, sb, match="cuda")


def test_grouped_gemm_buffers():
    E, Tcap, N, K = 4, 512, 256, 256
    qa, sa = u8(Tcap, K), u8(K // 128, Tcap, 4)
    qw, sw = u8(E, N, K), u8(E, K // 128, N, 4)
    offs = i32(E)
    raises(mx.grouped_mm_fwd, qa, sa, qw, sw, offs.long(), match="offs: dtype")
    raises(mx.grouped_mm_fwd, qa, sa, qw, sw, i32(E - 1), match="offs: 3 elements")
    raises(mx.grouped_mm_fwd, qa, sa, u8(E, N, 128), sw, offs, match="K=")
    raises(mx.grouped_mm_fwd, qa, sa, qw, u8(E - 1, K // 128, N, 4), offs, match="sw: ")
    raises(mx.grouped_mm_dgrad, qa, sa, qw, sw, offs, out=torch.zeros((Tcap - 128, N), dtype=BF),
           match="out: shape")
    raises(mx.grouped_mm_fwd, qa, sa, qw, sw, offs, dev_err=torch.zeros(1, dtype=torch.int64),
           match="dev_err: dtype")
    raises(mx.grouped_mm_fwd_unpad, qa, sa, qw, sw, offs, i32(E + 1), 300, match="sizes: 5 elements")
    raises(mx.grouped_mm_fwd_unpad, qa, sa, qw, sw, offs, i32(E), 300,
           out=torch.zeros((Tcap, N), dtype=BF), match="out: shape")
    raises(mx.grouped_mm_swiglu_fwd, qa, sa, u8(E, 2 * N, K), u8(E, K // 128, 2 * N, 4), offs,
           out={"z": torch.zeros((Tcap, N), dtype=BF)}, match="z: shape")
    raises(mx.grouped_mm_fwd, qa, sa, qw, sw, offs, match="cuda")


def test_weight_gradient_buffers():
    E, Tcap, N, K = 3, 512, 256, 128
    qg, sg = u8(N, Tcap), u8(Tcap // 128, N, 4)
    qx, sx = u8(K, Tcap), u8(Tcap // 128, K, 4)
    offs = i32(E)
    raises(mx.grouped_mm_wgrad, qg, sg, u8(K, Tcap - 128), sx, offs, match="token columns")
    raises(mx.grouped_mm_wgrad, qg, sg, qx, u8(Tcap // 128, K, 2), offs, match="sx: ")
    raises(mx.grouped_mm_wgrad, qg, sg, qx, sx, offs, out=torch.zeros((E, K, N)), match="out: shape")
    raises(mx.grouped_mm_wgrad, qg, sg, qx, sx, i32(E, 1), match="offs: expected")
    raises(mx.grouped_mm_wgrad, qg, sg, qx, sx, offs, match="cuda")
    raises(mx.grouped_mm_wgrad_hp, bf(Tcap, N), bf(Tcap + 128, K), offs, match="rows")
    raises(mx.grouped_mm_wgrad_hp, bf(Tcap, N).float(), bf(Tcap, K), offs, match="g: dtype")
    raises(mx.grouped_mm_wgrad_hp, bf(Tcap, N), bf(Tcap, K), offs, out=bf(E, N, K).float(),
           match="out: dtype")
    raises(mx.grouped_mm_wgrad_hp, bf(Tcap, N), bf(Tcap, K), offs, match="cuda")


def test_quantize_buffers():
    R, C = 256, 128
    x = bf(R, C)
    raises(mx.quantize, x.float(), match="bf16")
    raises(mx.quantize, bf(C, R).t(), match="contiguous rows")
    raises(mx.quantize, x, out={"q_row": u8(R, C - 32)}, match="q_row: ")
    raises(mx.quantize, x, colwise=True, out={"s_col": u8(C // 128, R, 2)}, match="s_col: ")
    # batched: the matrices must follow each other R rows apart
    raises(mx.quantize, bf(3, R, C)[::2], match="apart")
    raises(mx.quantize, x, match="cuda")
    # strided rows are accepted up to the device check
    raises(mx.quantize, bf(R, 2 * C)[:, C:], match="cuda")
    raises(mx.quantize_fp8, x, True, True, offs=i32(2).long(), match="offs: dtype")
    raises(mx.quantize_fp8, x, True, True, out={"q_col": u8(C, R // 2)}, match="q_col: ")
    raises(mx.quantize_fp8_dual_scratch, x, out={"s_row": u8(1)}, match="s_row: ")
    raises(mx.dequantize, u8(R, C), u8(R, C // 32), out=torch.zeros((R, C + 1)), match="out: shape")
    raises(mx.dequantize, u8(R, C), u8(R, C // 64), match="s: ")


def test_swiglu_and_padding_buffers():
    T, H = 256, 128
    z = bf(T, 2 * H)
    raises(mx.swiglu_quant_fwd, z[:, :H], bf(T, H + 32), match="b: shape")
    raises(mx.swiglu_quant_fwd, z[:, :H], bf(T, H), match="row stride")
    raises(mx.swiglu_quant_fwd, z[:, :H], z[:, H:], want_h=True, out={"h": bf(T, 2 * H)}, match="h: shape")
    raises(mx.swiglu_quant_fwd, z[:, :H], z[:, H:], match="cuda")
    raises(mx.swiglu_quant_bwd, bf(T, H + 32), z[:, :H], z[:, H:], match="dh: shape")
    raises(mx.swiglu_quant_bwd, bf(T, H), z[:, :H], z[:, H:], out={"q_row": u8(T, H)}, match="q_row: ")
    raises(mx.swiglu_quant_bwd, bf(T, H), z[:, :H], z[:, H:], match="cuda")
    E, Tcap = 3, 512
    x = bf(T, H)
    raises(mx.pad_groups, x, i32(E).long(), Tcap, match="sizes: dtype")
    raises(mx.pad_groups, x, i32(E), Tcap, out={"x_pad": bf(Tcap - 128, H)}, match="x_pad: shape")
    raises(mx.pad_groups, x, i32(E), Tcap, out={"src_row": i32(T)}, match="src_row: ")
    raises(mx.pad_groups, bf(T, 2 * H)[:, :H], i32(E), Tcap, match="x must be contiguous")
    raises(mx.pad_groups, x, i32(E), Tcap, match="cuda")
    raises(mx.pad_quantize, x, i32(E), Tcap, colwise=True, out={"offs": i32(E + 1)}, match="offs: ")
    raises(mx.pad_quantize, x, i32(E), Tcap, colwise=True, out={"q_col": u8(H, T)}, match="q_col: ")
    raises(mx.pad_quantize, x, i32(E), Tcap, match="cuda")
    raises(mx.unpad_groups, bf(Tcap, H), i32(T), T, match="src_row: ")
    raises(mx.unpad_groups, bf(Tcap, H), i32(Tcap), T, out=bf(T, H // 2), match="out: shape")
    raises(mx.unpad_groups, bf(Tcap, H), i32(Tcap), T, match="cuda")
