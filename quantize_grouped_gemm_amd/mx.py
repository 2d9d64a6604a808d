"""Thin Python binding of libmxfp8.so (C ABI in include/mxfp8.h).

Argument marshalling only: every function checks nothing beyond what ctypes
needs, allocates its outputs with torch (device memory is torch's) and calls
the library on torch's current stream. All arithmetic happens in the HIP
kernels. If the library is missing or cannot run on the current device, the
call raises; there is no fallback.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmxfp8.so")

RCEIL, FLOOR = 0, 1
BF16, F32 = 0, 1
ROWWISE, COLWISE = 1, 2
SCALES_PLAIN, SCALES_K128 = 0, 1
_MODES = {"rceil": RCEIL, "floor": FLOOR, RCEIL: RCEIL, FLOOR: FLOOR}
_LAYOUTS = {"plain": SCALES_PLAIN, "k128": SCALES_K128}
_DT = {torch.bfloat16: BF16, torch.float32: F32, "bf16": BF16, "f32": F32}

_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_SIGS = {
    "mx_abi_version": ([], ctypes.c_int),
    "mx_last_error": ([], ctypes.c_char_p),
    "mx_init": ([], ctypes.c_int),
    "mx_quantize": ([_P, _I64, _I64, _I64, _I64, ctypes.c_int, ctypes.c_uint, ctypes.c_int, _P, _P, _P, _P, _P],
                    ctypes.c_int),
    "mx_dequantize": ([_P, _P, _I64, _I64, ctypes.c_int, ctypes.c_int, _P, _P], ctypes.c_int),
    "mx_swiglu_quant_fwd": ([_P, _P, _I64, _I64, _I64, ctypes.c_int, ctypes.c_int, _P, _P, _P, _P, _P, _P],
                            ctypes.c_int),
    "mx_swiglu_quant_bwd": ([_P, _I64, _P, _P, _I64, _I64, _I64, ctypes.c_int, ctypes.c_int, _P, _P, _P, _P, _P,
                             _P], ctypes.c_int),
    "mx_scaled_mm": ([_P, _P, _P, _P, _I64, _I64, _I64, ctypes.c_int, _P, _I64, _P], ctypes.c_int),
    "mx_scaled_grouped_mm_fwd": ([_P, _P, _P, _P, _P, _I32, _I64, _I64, _I64, ctypes.c_int, _P, _P, _P],
                                 ctypes.c_int),
    "mx_scaled_grouped_mm_dgrad": ([_P, _P, _P, _P, _P, _I32, _I64, _I64, _I64, ctypes.c_int, _P, _P, _P],
                                   ctypes.c_int),
    "mx_scaled_grouped_mm_swiglu_fwd": ([_P, _P, _P, _P, _P, _I32, _I64, _I64, _I64, ctypes.c_int, _P, _P, _P, _P,
                                         _P, _P, _P, _P], ctypes.c_int),
    "mx_scaled_grouped_mm_fwd_unpad": ([_P, _P, _P, _P, _P, _P, _I32, _I64, _I64, _I64, _I64, ctypes.c_int, _P,
                                        _P, _P], ctypes.c_int),
    "mx_scaled_grouped_mm_dgrad_unpad": ([_P, _P, _P, _P, _P, _P, _I32, _I64, _I64, _I64, _I64, ctypes.c_int, _P,
                                          _P, _P], ctypes.c_int),
    "mx_scaled_grouped_mm_wgrad": ([_P, _P, _P, _P, _P, _I32, _I64, _I64, _I64, ctypes.c_int, _P, _P, _P],
                                   ctypes.c_int),
    "mx_grouped_mm_wgrad_hp": ([_P, _P, _P, _I32, _I64, _I64, _I64, _P, _P, _P], ctypes.c_int),
    "mx_pad_groups": ([_P, _P, _I32, _I64, _I64, _I32, _I64, _P, _P, _P, _P, _P], ctypes.c_int),
    "mx_pad_quantize": ([_P, _P, _I32, _I64, _I64, _I32, _I64, ctypes.c_int, ctypes.c_uint, ctypes.c_int, _P, _P,
                         _P, _P, _P, _P, _P, _P], ctypes.c_int),
    "mx_quantize_fp8_rowwise": ([_P, _I64, _I64, _I64, _I64, _P, _P, _P], ctypes.c_int),
    "mx_quantize_fp8_colwise": ([_P, _I64, _I64, _I64, _I64, _P, _I32, _P, _P, _P, _P, _P], ctypes.c_int),
    "mx_quantize_fp8_dual": ([_P, _I64, _I64, _I64, _I64, _P, _I32, _P, _P, _P, _P, _P, _P, _P], ctypes.c_int),
    "mx_quantize_fp8_dual_scratch": ([_P, _I64, _I64, _I64, _I64, _P, _I32, _P, _P, _P, _P, _P, _P], ctypes.c_int),
    "mx_unpad_groups": ([_P, _P, _I64, _I64, _I64, _P, _P], ctypes.c_int),
}
EXPORTS = tuple(_SIGS)


class MXError(RuntimeError):
    pass


def lib():
    """Load libmxfp8.so (once). Raises if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise MXError(f"{LIB_PATH} is missing: build it with python -m quantize_grouped_gemm_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def _check(st, name):
    if st != 0:
        raise MXError(f"{name} failed (status {st}): {lib().mx_last_error().decode()}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _u8(shape, device):
    return torch.empty(shape, dtype=torch.uint8, device=device)


def scale_shape(R, C, layout="k128"):
    """Shape of the scale tensor of an [R, C] code matrix: plain [R, C/32],
    k128 [C/128, R, 4]."""
    return (C // 128, R, 4) if layout == "k128" else (R, C // 32)


def quantize(x, mode="rceil", rowwise=True, colwise=False, layout="k128", out=None):
    """MX-quantize bf16 x [..., R, C] (row stride may exceed C).

    Returns dict with q_row [..., R, C] and s_row (the scales of that [R, C]
    matrix, see scale_shape) and/or q_col [..., C, R] and s_col (uint8)."""
    assert x.dtype == torch.bfloat16 and x.stride(-1) == 1
    R, C = x.shape[-2], x.shape[-1]
    lead = tuple(x.shape[:-2])
    batch = 1
    for d in lead:
        batch *= d
    ld = x.stride(-2)
    if batch > 1:
        assert x.is_contiguous() or all(x.stride(i) == x.stride(i + 1) * x.shape[i + 1] for i in range(len(lead)))
        assert len(lead) == 0 or x.stride(-3) == R * ld
    out = dict(out or {})
    dev = x.device
    if rowwise:
        out.setdefault("q_row", _u8(lead + (R, C), dev))
        out.setdefault("s_row", _u8(lead + scale_shape(R, C, layout), dev))
    if colwise:
        out.setdefault("q_col", _u8(lead + (C, R), dev))
        out.setdefault("s_col", _u8(lead + scale_shape(C, R, layout), dev))
    dirs = (ROWWISE if rowwise else 0) | (COLWISE if colwise else 0)
    st = lib().mx_quantize(_ptr(x), batch, R, C, ld, _MODES[mode], dirs, _LAYOUTS[layout],
                           _ptr(out.get("q_row")), _ptr(out.get("s_row")),
                           _ptr(out.get("q_col")), _ptr(out.get("s_col")), _stream(dev))
    _check(st, "mx_quantize")
    return out


def quantize_fp8(x, rowwise=True, colwise=False, offs=None, out=None, fused=True, dev_err=None):
    """FP8 with one power-of-two scale per row (column-wise: per column, or
    per column and group with offs). x bf16 [..., R, C]; returns the same
    keys and k128 layouts as quantize(). Both directions go through the
    one-read-per-pass entry point unless fused=False. dev_err: optional
    int32 device flag word for bad offsets."""
    assert x.dtype == torch.bfloat16 and x.stride(-1) == 1
    R, C = x.shape[-2], x.shape[-1]
    lead = tuple(x.shape[:-2])
    batch = 1
    for d in lead:
        batch *= d
    ld = x.stride(-2)
    assert batch == 1 or x.stride(-3) == R * ld
    out = dict(out or {})
    dev = x.device
    E = 0 if offs is None else offs.shape[0]
    if rowwise and colwise and fused:
        out.setdefault("q_row", _u8(lead + (R, C), dev))
        out.setdefault("s_row", _u8(lead + scale_shape(R, C), dev))
        out.setdefault("q_col", _u8(lead + (C, R), dev))
        out.setdefault("s_col", _u8(lead + scale_shape(C, R), dev))
        work = torch.empty((batch * ((E + 1) * C + R),), dtype=torch.int32, device=dev)
        st = lib().mx_quantize_fp8_dual(_ptr(x), batch, R, C, ld, _ptr(offs), E, _ptr(out["q_row"]),
                                        _ptr(out["s_row"]), _ptr(out["q_col"]), _ptr(out["s_col"]), _ptr(work),
                                        _ptr(dev_err), _stream(dev))
        _check(st, "mx_quantize_fp8_dual")
        return out
    if rowwise:
        out.setdefault("q_row", _u8(lead + (R, C), dev))
        out.setdefault("s_row", _u8(lead + scale_shape(R, C), dev))
        st = lib().mx_quantize_fp8_rowwise(_ptr(x), batch, R, C, ld, _ptr(out["q_row"]), _ptr(out["s_row"]),
                                           _stream(dev))
        _check(st, "mx_quantize_fp8_rowwise")
    if colwise:
        out.setdefault("q_col", _u8(lead + (C, R), dev))
        out.setdefault("s_col", _u8(lead + scale_shape(C, R), dev))
        work = torch.empty((batch * (E + 1) * C,), dtype=torch.int32, device=dev)
        st = lib().mx_quantize_fp8_colwise(_ptr(x), batch, R, C, ld, _ptr(offs), E, _ptr(out["q_col"]),
                                           _ptr(out["s_col"]), _ptr(work), _ptr(dev_err), _stream(dev))
        _check(st, "mx_quantize_fp8_colwise")
    return out


def quantize_fp8_dual_scratch(x, offs=None, out=None, dev_err=None):
    """quantize_fp8(x, True, True, offs) through the allocation-free entry
    point: the library's own device work area instead of a torch-allocated
    one (outputs are still allocated here unless given in `out`)."""
    assert x.dtype == torch.bfloat16 and x.stride(-1) == 1
    R, C = x.shape[-2], x.shape[-1]
    lead = tuple(x.shape[:-2])
    batch = 1
    for d in lead:
        batch *= d
    ld = x.stride(-2)
    assert batch == 1 or x.stride(-3) == R * ld
    out = dict(out or {})
    dev = x.device
    E = 0 if offs is None else offs.shape[0]
    out.setdefault("q_row", _u8(lead + (R, C), dev))
    out.setdefault("s_row", _u8(lead + scale_shape(R, C), dev))
    out.setdefault("q_col", _u8(lead + (C, R), dev))
    out.setdefault("s_col", _u8(lead + scale_shape(C, R), dev))
    st = lib().mx_quantize_fp8_dual_scratch(_ptr(x), batch, R, C, ld, _ptr(offs), E, _ptr(out["q_row"]),
                                            _ptr(out["s_row"]), _ptr(out["q_col"]), _ptr(out["s_col"]),
                                            _ptr(dev_err), _stream(dev))
    _check(st, "mx_quantize_fp8_dual_scratch")
    return out


def dequantize(q, s, out_dtype=torch.float32, layout=None, out=None):
    """layout defaults to k128 for a 3-D scale tensor, plain for 2-D."""
    R, C = q.shape
    if layout is None:
        layout = "k128" if s.dim() == 3 else "plain"
    if out is None:
        out = torch.empty((R, C), dtype=out_dtype, device=q.device)
    _check(lib().mx_dequantize(_ptr(q), _ptr(s), R, C, _LAYOUTS[layout], _DT[out.dtype], _ptr(out),
                               _stream(q.device)), "mx_dequantize")
    return out


def swiglu_quant_fwd(a, b, mode="rceil", want_h=False, layout="k128", out=None):
    """Fused SwiGLU + dual quantization. a, b: bf16 [T, H] views sharing a row
    stride (e.g. the two halves of the w13 output)."""
    assert a.stride(0) == b.stride(0) and a.stride(1) == 1 and b.stride(1) == 1
    T, H = a.shape
    dev = a.device
    out = dict(out or {})
    out.setdefault("q_row", _u8((T, H), dev))
    out.setdefault("s_row", _u8(scale_shape(T, H, layout), dev))
    out.setdefault("q_col", _u8((H, T), dev))
    out.setdefault("s_col", _u8(scale_shape(H, T, layout), dev))
    if want_h:
        out.setdefault("h", torch.empty((T, H), dtype=torch.bfloat16, device=dev))
    st = lib().mx_swiglu_quant_fwd(_ptr(a), _ptr(b), a.stride(0), T, H, _MODES[mode], _LAYOUTS[layout],
                                   _ptr(out["q_row"]), _ptr(out["s_row"]), _ptr(out["q_col"]),
                                   _ptr(out["s_col"]), _ptr(out.get("h")), _stream(dev))
    _check(st, "mx_swiglu_quant_fwd")
    return out


def swiglu_quant_bwd(dh, a, b, mode="rceil", want_dab=False, layout="k128", out=None):
    assert a.stride(0) == b.stride(0) and dh.stride(1) == 1
    T, H = a.shape
    dev = a.device
    out = dict(out or {})
    out.setdefault("q_row", _u8((T, 2 * H), dev))
    out.setdefault("s_row", _u8(scale_shape(T, 2 * H, layout), dev))
    out.setdefault("q_col", _u8((2 * H, T), dev))
    out.setdefault("s_col", _u8(scale_shape(2 * H, T, layout), dev))
    if want_dab:
        out.setdefault("dab", torch.empty((T, 2 * H), dtype=torch.bfloat16, device=dev))
    st = lib().mx_swiglu_quant_bwd(_ptr(dh), dh.stride(0), _ptr(a), _ptr(b), a.stride(0), T, H,
                                   _MODES[mode], _LAYOUTS[layout], _ptr(out["q_row"]), _ptr(out["s_row"]),
                                   _ptr(out["q_col"]), _ptr(out["s_col"]), _ptr(out.get("dab")),
                                   _stream(dev))
    _check(st, "mx_swiglu_quant_bwd")
    return out


def scaled_mm(qa, sa, qb, sb, out_dtype=torch.bfloat16, out=None):
    """GEMM of two MX operands with k128 scales."""
    M, K = qa.shape
    N = qb.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=qa.device)
    st = lib().mx_scaled_mm(_ptr(qa), _ptr(sa), _ptr(qb), _ptr(sb), M, N, K, _DT[out.dtype],
                            _ptr(out), out.stride(0), _stream(qa.device))
    _check(st, "mx_scaled_mm")
    return out


def _grouped(name, qa, sa, qw, sw, offs, out_dtype, out, dev_err):
    Tcap, K = qa.shape
    E, N = qw.shape[0], qw.shape[1]
    if out is None:
        out = torch.empty((Tcap, N), dtype=out_dtype, device=qa.device)
    st = getattr(lib(), name)(_ptr(qa), _ptr(sa), _ptr(qw), _ptr(sw), _ptr(offs), E, Tcap, N, K,
                              _DT[out.dtype], _ptr(out), _ptr(dev_err), _stream(qa.device))
    _check(st, name)
    return out


def grouped_mm_fwd(qa, sa, qw, sw, offs, out_dtype=torch.bfloat16, out=None, dev_err=None):
    return _grouped("mx_scaled_grouped_mm_fwd", qa, sa, qw, sw, offs, out_dtype, out, dev_err)


def grouped_mm_dgrad(qa, sa, qw, sw, offs, out_dtype=torch.bfloat16, out=None, dev_err=None):
    return _grouped("mx_scaled_grouped_mm_dgrad", qa, sa, qw, sw, offs, out_dtype, out, dev_err)


def grouped_mm_swiglu_fwd(qa, sa, qw13, sw13, offs, mode="rceil", want_h=False, out=None, dev_err=None):
    """The w13 grouped forward fused with SwiGLU + dual quantization.
    qw13 [E, 2H, K] (gate rows first). Returns dict with z [Tcap, 2H] bf16,
    q_row/s_row, q_col/s_col of h (k128 scales) and, if asked, h bf16."""
    Tcap, K = qa.shape
    E, H2 = qw13.shape[0], qw13.shape[1]
    H = H2 // 2
    dev = qa.device
    out = dict(out or {})
    out.setdefault("z", torch.empty((Tcap, H2), dtype=torch.bfloat16, device=dev))
    out.setdefault("q_row", _u8((Tcap, H), dev))
    out.setdefault("s_row", _u8(scale_shape(Tcap, H), dev))
    out.setdefault("q_col", _u8((H, Tcap), dev))
    out.setdefault("s_col", _u8(scale_shape(H, Tcap), dev))
    if want_h:
        out.setdefault("h", torch.empty((Tcap, H), dtype=torch.bfloat16, device=dev))
    st = lib().mx_scaled_grouped_mm_swiglu_fwd(_ptr(qa), _ptr(sa), _ptr(qw13), _ptr(sw13), _ptr(offs), E, Tcap, H,
                                               K, _MODES[mode], _ptr(out["z"]), _ptr(out["q_row"]),
                                               _ptr(out["s_row"]), _ptr(out["q_col"]), _ptr(out["s_col"]),
                                               _ptr(out.get("h")), _ptr(dev_err), _stream(dev))
    _check(st, "mx_scaled_grouped_mm_swiglu_fwd")
    return out


def _grouped_unpad(name, qa, sa, qw, sw, offs, sizes, T, out_dtype, out, dev_err):
    Tcap, K = qa.shape
    E, N = qw.shape[0], qw.shape[1]
    if out is None:
        out = torch.empty((T, N), dtype=out_dtype, device=qa.device)
    st = getattr(lib(), name)(_ptr(qa), _ptr(sa), _ptr(qw), _ptr(sw), _ptr(offs), _ptr(sizes), E, Tcap, T, N, K,
                              _DT[out.dtype], _ptr(out), _ptr(dev_err), _stream(qa.device))
    _check(st, name)
    return out


def grouped_mm_fwd_unpad(qa, sa, qw, sw, offs, sizes, T, out_dtype=torch.bfloat16, out=None, dev_err=None):
    """grouped_mm_fwd with the result in token order [T, N] (sizes: int32
    [E] tokens per group on the device)."""
    return _grouped_unpad("mx_scaled_grouped_mm_fwd_unpad", qa, sa, qw, sw, offs, sizes, T, out_dtype, out,
                          dev_err)


def grouped_mm_dgrad_unpad(qa, sa, qw, sw, offs, sizes, T, out_dtype=torch.bfloat16, out=None, dev_err=None):
    """grouped_mm_dgrad with the result in token order [T, N]."""
    return _grouped_unpad("mx_scaled_grouped_mm_dgrad_unpad", qa, sa, qw, sw, offs, sizes, T, out_dtype, out,
                          dev_err)


def grouped_mm_wgrad(qg, sg, qx, sx, offs, out_dtype=torch.float32, out=None, dev_err=None):
    N, Tcap = qg.shape
    K = qx.shape[0]
    E = offs.shape[0]
    if out is None:
        out = torch.empty((E, N, K), dtype=out_dtype, device=qg.device)
    st = lib().mx_scaled_grouped_mm_wgrad(_ptr(qg), _ptr(sg), _ptr(qx), _ptr(sx), _ptr(offs), E, Tcap,
                                          N, K, _DT[out.dtype], _ptr(out), _ptr(dev_err),
                                          _stream(qg.device))
    _check(st, "mx_scaled_grouped_mm_wgrad")
    return out


def grouped_mm_wgrad_hp(g, x, offs, out=None, dev_err=None):
    Tcap, N = g.shape
    K = x.shape[1]
    E = offs.shape[0]
    if out is None:
        out = torch.empty((E, N, K), dtype=torch.bfloat16, device=g.device)
    st = lib().mx_grouped_mm_wgrad_hp(_ptr(g), _ptr(x), _ptr(offs), E, Tcap, N, K, _ptr(out),
                                      _ptr(dev_err), _stream(g.device))
    _check(st, "mx_grouped_mm_wgrad_hp")
    return out


def pad_groups(x, sizes, Tcap, multiple=128, out=None, dev_err=None):
    """x [T, ...] rows grouped by expert; sizes int32 [E] on the device.
    Returns (x_pad [Tcap, ...], offs int32 [E], src_row int32 [Tcap])."""
    T = x.shape[0]
    row_bytes = x[0].numel() * x.element_size() if T else x.stride(0) * x.element_size()
    E = sizes.shape[0]
    dev = x.device
    out = dict(out or {})
    x_pad = out.get("x_pad")
    if x_pad is None:
        x_pad = torch.empty((Tcap,) + tuple(x.shape[1:]), dtype=x.dtype, device=dev)
    offs = out.get("offs")
    if offs is None:
        offs = torch.empty((E,), dtype=torch.int32, device=dev)
    src = out.get("src_row")
    if src is None:
        src = torch.empty((Tcap,), dtype=torch.int32, device=dev)
    st = lib().mx_pad_groups(_ptr(x), _ptr(sizes), E, T, row_bytes, multiple, Tcap, _ptr(x_pad),
                             _ptr(offs), _ptr(src), _ptr(dev_err), _stream(dev))
    _check(st, "mx_pad_groups")
    return x_pad, offs, src


def pad_quantize(x, sizes, Tcap, mode="rceil", rowwise=True, colwise=False, layout="k128", multiple=128,
                 out=None, dev_err=None):
    """Padding fused with MX quantization: the outputs of
    quantize(pad_groups(x, sizes, Tcap)[0]) without the bf16 x_pad.

    x bf16 [T, C] contiguous; sizes int32 [E] on the device. Returns dict with
    q_row/s_row and/or q_col/s_col of the padded [Tcap, C] tensor, plus offs
    int32 [E] and src_row int32 [Tcap]."""
    assert x.dtype == torch.bfloat16 and x.dim() == 2 and x.is_contiguous()
    T, C = x.shape
    E = sizes.shape[0]
    dev = x.device
    out = dict(out or {})
    if rowwise:
        out.setdefault("q_row", _u8((Tcap, C), dev))
        out.setdefault("s_row", _u8(scale_shape(Tcap, C, layout), dev))
    if colwise:
        out.setdefault("q_col", _u8((C, Tcap), dev))
        out.setdefault("s_col", _u8(scale_shape(C, Tcap, layout), dev))
    if out.get("offs") is None:
        out["offs"] = torch.empty((E,), dtype=torch.int32, device=dev)
    if out.get("src_row") is None:
        out["src_row"] = torch.empty((Tcap,), dtype=torch.int32, device=dev)
    dirs = (ROWWISE if rowwise else 0) | (COLWISE if colwise else 0)
    st = lib().mx_pad_quantize(_ptr(x), _ptr(sizes), E, T, C, multiple, Tcap, _MODES[mode], dirs,
                               _LAYOUTS[layout], _ptr(out.get("q_row")), _ptr(out.get("s_row")),
                               _ptr(out.get("q_col")), _ptr(out.get("s_col")), _ptr(out["offs"]),
                               _ptr(out["src_row"]), _ptr(dev_err), _stream(dev))
    _check(st, "mx_pad_quantize")
    return out


def unpad_groups(y_pad, src_row, T, out=None):
    Tcap = y_pad.shape[0]
    row_bytes = y_pad[0].numel() * y_pad.element_size()
    if out is None:
        out = torch.empty((T,) + tuple(y_pad.shape[1:]), dtype=y_pad.dtype, device=y_pad.device)
    st = lib().mx_unpad_groups(_ptr(y_pad), _ptr(src_row), Tcap, T, row_bytes, _ptr(out),
                               _stream(y_pad.device))
    _check(st, "mx_unpad_groups")
    return out
