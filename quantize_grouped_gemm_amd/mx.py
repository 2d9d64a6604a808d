"""Thin Python binding of libmxfp8.so (C ABI in include/mxfp8.h).

Argument marshalling only: every function checks that the tensors it hands
over match the sizes it passes with them (the library sees bare pointers),
allocates its outputs with torch (device memory is torch's) and calls the
library on torch's current stream. All arithmetic happens in the HIP
kernels. If the library is missing or cannot run on the current device, the
call raises; there is no fallback.
"""

import ctypes
import math
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


# Buffer checks. The C ABI receives bare pointers and cannot tell a buffer's
# size, so the binding checks each tensor it passes (dtype, element count,
# layout, device) against the sizes it passes with it: a buffer too small for
# the sizes would otherwise be read or written past its end on the device.
# Structural checks come first, the device check last.

def _want(t, name, dtype, numel=None, shape=None, contiguous=True):
    if not isinstance(t, torch.Tensor):
        raise MXError(f"{name}: expected a tensor, got {type(t).__name__}")
    if t.dtype != dtype:
        raise MXError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise MXError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if numel is not None and t.numel() != numel:
        raise MXError(f"{name}: {t.numel()} elements, expected {numel}")
    if contiguous and not t.is_contiguous():
        raise MXError(f"{name} must be contiguous")
    return t


def _want_rows(t, name, dtype, shape):
    """A matrix whose rows are contiguous and may be spaced further apart
    (row stride >= columns)."""
    _want(t, name, dtype, shape=shape, contiguous=False)
    if t.dim() != 2 or t.stride(1) != 1 or t.stride(0) < t.shape[1]:
        raise MXError(f"{name} must have contiguous rows (strides {tuple(t.stride())})")
    return t


def _want_out(t, name, numel=None, shape=None, dtypes=(torch.bfloat16, torch.float32)):
    if not isinstance(t, torch.Tensor) or t.dtype not in dtypes:
        raise MXError(f"{name}: expected a tensor of {', '.join(str(d) for d in dtypes)}")
    return _want(t, name, t.dtype, numel, shape)


def _flag(dev_err):
    if dev_err is not None:
        _want(dev_err, "dev_err", torch.int32)
        if dev_err.numel() < 1:
            raise MXError("dev_err: needs one int32")
    return dev_err


def _device(*tensors):
    """The CUDA (HIP) device every given tensor is on; it must be the
    current device, on which the library launches."""
    dev = None
    for t in tensors:
        if t is None:
            continue
        if t.device.type != "cuda":
            raise MXError(f"tensor on {t.device}: libmxfp8 takes device (cuda) tensors")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise MXError(f"tensors on {dev} and {t.device}")
    if dev is not None and dev.index != torch.cuda.current_device():
        raise MXError(f"tensors on {dev} but the current device is cuda:{torch.cuda.current_device()}")
    return dev


def _check_q_outs(out, lead_n, R, C, rowwise, colwise):
    """Codes and scales of a [R, C] matrix (lead_n of them): row-wise codes
    [R, C], column-wise codes [C, R], scales one byte per 32 codes."""
    if rowwise:
        _want(out["q_row"], "q_row", torch.uint8, lead_n * R * C)
        _want(out["s_row"], "s_row", torch.uint8, lead_n * R * C // 32)
    if colwise:
        _want(out["q_col"], "q_col", torch.uint8, lead_n * R * C)
        _want(out["s_col"], "s_col", torch.uint8, lead_n * R * C // 32)


def _batched_input(x, name="x"):
    """bf16 x [..., R, C] with contiguous rows, matrices spaced R rows apart.
    Returns (lead, batch, R, C, ld)."""
    if not isinstance(x, torch.Tensor) or x.dtype != torch.bfloat16 or x.dim() < 2:
        raise MXError(f"{name}: expected a bf16 tensor of at least 2 dimensions")
    R, C = x.shape[-2], x.shape[-1]
    lead = tuple(x.shape[:-2])
    batch = 1
    for d in lead:
        batch *= d
    ld = x.stride(-2)
    if x.stride(-1) != 1 or (R > 1 and ld < C):
        raise MXError(f"{name} must have contiguous rows (strides {tuple(x.stride())})")
    if batch > 1 and not x.is_contiguous():
        dense_lead = all(x.stride(i) == x.stride(i + 1) * x.shape[i + 1] for i in range(len(lead) - 1))
        if not dense_lead or x.stride(-3) != R * ld:
            raise MXError(f"{name}: its matrices must follow each other R rows apart (strides {tuple(x.stride())})")
    return lead, batch, R, C, ld


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
    lead, batch, R, C, ld = _batched_input(x)
    out = dict(out or {})
    dev = x.device
    if rowwise:
        out.setdefault("q_row", _u8(lead + (R, C), dev))
        out.setdefault("s_row", _u8(lead + scale_shape(R, C, layout), dev))
    if colwise:
        out.setdefault("q_col", _u8(lead + (C, R), dev))
        out.setdefault("s_col", _u8(lead + scale_shape(C, R, layout), dev))
    _check_q_outs(out, batch, R, C, rowwise, colwise)
    _device(x, out.get("q_row"), out.get("s_row"), out.get("q_col"), out.get("s_col"))
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
    lead, batch, R, C, ld = _batched_input(x)
    out = dict(out or {})
    dev = x.device
    E = 0 if offs is None else offs.numel()
    if offs is not None:
        _want(offs, "offs", torch.int32)
    _flag(dev_err)
    if rowwise and colwise and fused:
        out.setdefault("q_row", _u8(lead + (R, C), dev))
        out.setdefault("s_row", _u8(lead + scale_shape(R, C), dev))
        out.setdefault("q_col", _u8(lead + (C, R), dev))
        out.setdefault("s_col", _u8(lead + scale_shape(C, R), dev))
        _check_q_outs(out, batch, R, C, True, True)
        _device(x, offs, dev_err, out["q_row"], out["s_row"], out["q_col"], out["s_col"])
        work = torch.empty((batch * ((E + 1) * C + R),), dtype=torch.int32, device=dev)
        st = lib().mx_quantize_fp8_dual(_ptr(x), batch, R, C, ld, _ptr(offs), E, _ptr(out["q_row"]),
                                        _ptr(out["s_row"]), _ptr(out["q_col"]), _ptr(out["s_col"]), _ptr(work),
                                        _ptr(dev_err), _stream(dev))
        _check(st, "mx_quantize_fp8_dual")
        return out
    if rowwise:
        out.setdefault("q_row", _u8(lead + (R, C), dev))
        out.setdefault("s_row", _u8(lead + scale_shape(R, C), dev))
        _check_q_outs(out, batch, R, C, True, False)
        _device(x, out["q_row"], out["s_row"])
        st = lib().mx_quantize_fp8_rowwise(_ptr(x), batch, R, C, ld, _ptr(out["q_row"]), _ptr(out["s_row"]),
                                           _stream(dev))
        _check(st, "mx_quantize_fp8_rowwise")
    if colwise:
        out.setdefault("q_col", _u8(lead + (C, R), dev))
        out.setdefault("s_col", _u8(lead + scale_shape(C, R), dev))
        _check_q_outs(out, batch, R, C, False, True)
        _device(x, offs, dev_err, out["q_col"], out["s_col"])
        work = torch.empty((batch * (E + 1) * C,), dtype=torch.int32, device=dev)
        st = lib().mx_quantize_fp8_colwise(_ptr(x), batch, R, C, ld, _ptr(offs), E, _ptr(out["q_col"]),
                                           _ptr(out["s_col"]), _ptr(work), _ptr(dev_err), _stream(dev))
        _check(st, "mx_quantize_fp8_colwise")
    return out


def quantize_fp8_dual_scratch(x, offs=None, out=None, dev_err=None):
    """quantize_fp8(x, True, True, offs) through the allocation-free entry
    point: the library's own device work area instead of a torch-allocated
    one (outputs are still allocated here unless given in `out`)."""
    lead, batch, R, C, ld = _batched_input(x)
    out = dict(out or {})
    dev = x.device
    E = 0 if offs is None else offs.numel()
    if offs is not None:
        _want(offs, "offs", torch.int32)
    _flag(dev_err)
    out.setdefault("q_row", _u8(lead + (R, C), dev))
    out.setdefault("s_row", _u8(lead + scale_shape(R, C), dev))
    out.setdefault("q_col", _u8(lead + (C, R), dev))
    out.setdefault("s_col", _u8(lead + scale_shape(C, R), dev))
    _check_q_outs(out, batch, R, C, True, True)
    _device(x, offs, dev_err, out["q_row"], out["s_row"], out["q_col"], out["s_col"])
    st = lib().mx_quantize_fp8_dual_scratch(_ptr(x), batch, R, C, ld, _ptr(offs), E, _ptr(out["q_row"]),
                                            _ptr(out["s_row"]), _ptr(out["q_col"]), _ptr(out["s_col"]),
                                            _ptr(dev_err), _stream(dev))
    _check(st, "mx_quantize_fp8_dual_scratch")
    return out


def dequantize(q, s, out_dtype=torch.float32, layout=None, out=None):
    """layout defaults to k128 for a 3-D scale tensor, plain for 2-D."""
    if not isinstance(q, torch.Tensor) or q.dim() != 2:
        raise MXError("q: expected a 2-D code matrix")
    R, C = q.shape
    _want(q, "q", torch.uint8)
    _want(s, "s", torch.uint8, R * C // 32)
    if layout is None:
        layout = "k128" if s.dim() == 3 else "plain"
    if out is None:
        out = torch.empty((R, C), dtype=out_dtype, device=q.device)
    _want_out(out, "out", shape=(R, C))
    _device(q, s, out)
    _check(lib().mx_dequantize(_ptr(q), _ptr(s), R, C, _LAYOUTS[layout], _DT[out.dtype], _ptr(out),
                               _stream(q.device)), "mx_dequantize")
    return out


def swiglu_quant_fwd(a, b, mode="rceil", want_h=False, layout="k128", out=None):
    """Fused SwiGLU + dual quantization. a, b: bf16 [T, H] views sharing a row
    stride (e.g. the two halves of the w13 output)."""
    if not isinstance(a, torch.Tensor) or a.dim() != 2:
        raise MXError("a: expected a 2-D bf16 tensor")
    T, H = a.shape
    _want_rows(a, "a", torch.bfloat16, (T, H))
    _want_rows(b, "b", torch.bfloat16, (T, H))
    if a.stride(0) != b.stride(0):
        raise MXError("a and b must share a row stride")
    dev = a.device
    out = dict(out or {})
    out.setdefault("q_row", _u8((T, H), dev))
    out.setdefault("s_row", _u8(scale_shape(T, H, layout), dev))
    out.setdefault("q_col", _u8((H, T), dev))
    out.setdefault("s_col", _u8(scale_shape(H, T, layout), dev))
    if want_h:
        out.setdefault("h", torch.empty((T, H), dtype=torch.bfloat16, device=dev))
    _check_q_outs(out, 1, T, H, True, True)
    if out.get("h") is not None:
        _want(out["h"], "h", torch.bfloat16, shape=(T, H))
    _device(a, b, out["q_row"], out["s_row"], out["q_col"], out["s_col"], out.get("h"))
    st = lib().mx_swiglu_quant_fwd(_ptr(a), _ptr(b), a.stride(0), T, H, _MODES[mode], _LAYOUTS[layout],
                                   _ptr(out["q_row"]), _ptr(out["s_row"]), _ptr(out["q_col"]),
                                   _ptr(out["s_col"]), _ptr(out.get("h")), _stream(dev))
    _check(st, "mx_swiglu_quant_fwd")
    return out


def swiglu_quant_bwd(dh, a, b, mode="rceil", want_dab=False, layout="k128", out=None):
    """Backward of swiglu_quant_fwd: dh bf16 [T, H] and the forward's a, b
    give dA|dB [T, 2H], dual-quantized (and kept in bf16 if asked)."""
    if not isinstance(a, torch.Tensor) or a.dim() != 2:
        raise MXError("a: expected a 2-D bf16 tensor")
    T, H = a.shape
    _want_rows(a, "a", torch.bfloat16, (T, H))
    _want_rows(b, "b", torch.bfloat16, (T, H))
    _want_rows(dh, "dh", torch.bfloat16, (T, H))
    if a.stride(0) != b.stride(0):
        raise MXError("a and b must share a row stride")
    dev = a.device
    out = dict(out or {})
    out.setdefault("q_row", _u8((T, 2 * H), dev))
    out.setdefault("s_row", _u8(scale_shape(T, 2 * H, layout), dev))
    out.setdefault("q_col", _u8((2 * H, T), dev))
    out.setdefault("s_col", _u8(scale_shape(2 * H, T, layout), dev))
    if want_dab:
        out.setdefault("dab", torch.empty((T, 2 * H), dtype=torch.bfloat16, device=dev))
    _check_q_outs(out, 1, T, 2 * H, True, True)
    if out.get("dab") is not None:
        _want(out["dab"], "dab", torch.bfloat16, shape=(T, 2 * H))
    _device(dh, a, b, out["q_row"], out["s_row"], out["q_col"], out["s_col"], out.get("dab"))
    st = lib().mx_swiglu_quant_bwd(_ptr(dh), dh.stride(0), _ptr(a), _ptr(b), a.stride(0), T, H,
                                   _MODES[mode], _LAYOUTS[layout], _ptr(out["q_row"]), _ptr(out["s_row"]),
                                   _ptr(out["q_col"]), _ptr(out["s_col"]), _ptr(out.get("dab")),
                                   _stream(dev))
    _check(st, "mx_swiglu_quant_bwd")
    return out


def scaled_mm(qa, sa, qb, sb, out_dtype=torch.bfloat16, out=None):
    """GEMM of two MX operands with k128 scales: qa [M, K] and qb [N, K]
    codes (both quantized along K) give out [M, N] = A B^T."""
    M, K = _codes2d(qa, "qa")
    N, Kb = _codes2d(qb, "qb")
    if Kb != K:
        raise MXError(f"qa has K={K}, qb has K={Kb}")
    _want(sa, "sa", torch.uint8, M * K // 32)
    _want(sb, "sb", torch.uint8, N * K // 32)
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=qa.device)
    if not isinstance(out, torch.Tensor) or out.dtype not in (torch.bfloat16, torch.float32):
        raise MXError("out: expected a tensor of torch.bfloat16, torch.float32")
    _want_rows(out, "out", out.dtype, (M, N))   # rows may be spaced wider (ld_out)
    _device(qa, sa, qb, sb, out)
    st = lib().mx_scaled_mm(_ptr(qa), _ptr(sa), _ptr(qb), _ptr(sb), M, N, K, _DT[out.dtype],
                            _ptr(out), out.stride(0), _stream(qa.device))
    _check(st, "mx_scaled_mm")
    return out


def _codes2d(q, name):
    if not isinstance(q, torch.Tensor) or q.dim() != 2:
        raise MXError(f"{name}: expected a 2-D code matrix")
    _want(q, name, torch.uint8)
    return q.shape


def _grouped_operands(qa, sa, qw, sw, offs):
    """qa [Tcap, K] token codes, qw [E, N, K] expert codes, offs int32 [E]."""
    Tcap, K = _codes2d(qa, "qa")
    if not isinstance(qw, torch.Tensor) or qw.dim() != 3:
        raise MXError("qw: expected [E, N, K] codes")
    E, N, Kw = qw.shape
    if Kw != K:
        raise MXError(f"qa has K={K}, qw has K={Kw}")
    _want(qw, "qw", torch.uint8)
    _want(sa, "sa", torch.uint8, Tcap * K // 32)
    _want(sw, "sw", torch.uint8, E * N * K // 32)
    _want(offs, "offs", torch.int32, E)
    return Tcap, K, E, N


def _grouped(name, qa, sa, qw, sw, offs, out_dtype, out, dev_err):
    Tcap, K, E, N = _grouped_operands(qa, sa, qw, sw, offs)
    if out is None:
        out = torch.empty((Tcap, N), dtype=out_dtype, device=qa.device)
    _want_out(out, "out", shape=(Tcap, N))
    _device(qa, sa, qw, sw, offs, out, _flag(dev_err))
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
    Tcap, K, E, H2 = _grouped_operands(qa, sa, qw13, sw13, offs)
    if H2 % 2:
        raise MXError(f"qw13 has {H2} rows per expert; expected 2H")
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
    _want(out["z"], "z", torch.bfloat16, shape=(Tcap, H2))
    _check_q_outs(out, 1, Tcap, H, True, True)
    if out.get("h") is not None:
        _want(out["h"], "h", torch.bfloat16, shape=(Tcap, H))
    _device(qa, sa, qw13, sw13, offs, out["z"], out["q_row"], out["s_row"], out["q_col"], out["s_col"],
            out.get("h"), _flag(dev_err))
    st = lib().mx_scaled_grouped_mm_swiglu_fwd(_ptr(qa), _ptr(sa), _ptr(qw13), _ptr(sw13), _ptr(offs), E, Tcap, H,
                                               K, _MODES[mode], _ptr(out["z"]), _ptr(out["q_row"]),
                                               _ptr(out["s_row"]), _ptr(out["q_col"]), _ptr(out["s_col"]),
                                               _ptr(out.get("h")), _ptr(dev_err), _stream(dev))
    _check(st, "mx_scaled_grouped_mm_swiglu_fwd")
    return out


def _grouped_unpad(name, qa, sa, qw, sw, offs, sizes, T, out_dtype, out, dev_err):
    Tcap, K, E, N = _grouped_operands(qa, sa, qw, sw, offs)
    _want(sizes, "sizes", torch.int32, E)
    if out is None:
        out = torch.empty((T, N), dtype=out_dtype, device=qa.device)
    _want_out(out, "out", shape=(T, N))
    _device(qa, sa, qw, sw, offs, sizes, out, _flag(dev_err))
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
    """dW [E, N, K] from qg [N, Tcap] and qx [K, Tcap], both quantized along
    the tokens; group g contracts its own token range of offs."""
    N, Tcap = _codes2d(qg, "qg")
    K, Tx = _codes2d(qx, "qx")
    if Tx != Tcap:
        raise MXError(f"qg has {Tcap} token columns, qx has {Tx}")
    _want(sg, "sg", torch.uint8, N * Tcap // 32)
    _want(sx, "sx", torch.uint8, K * Tcap // 32)
    if not isinstance(offs, torch.Tensor) or offs.dim() != 1:
        raise MXError("offs: expected int32 [E]")
    _want(offs, "offs", torch.int32)
    E = offs.shape[0]
    if out is None:
        out = torch.empty((E, N, K), dtype=out_dtype, device=qg.device)
    _want_out(out, "out", shape=(E, N, K))
    _device(qg, sg, qx, sx, offs, out, _flag(dev_err))
    st = lib().mx_scaled_grouped_mm_wgrad(_ptr(qg), _ptr(sg), _ptr(qx), _ptr(sx), _ptr(offs), E, Tcap,
                                          N, K, _DT[out.dtype], _ptr(out), _ptr(dev_err),
                                          _stream(qg.device))
    _check(st, "mx_scaled_grouped_mm_wgrad")
    return out


def grouped_mm_wgrad_hp(g, x, offs, out=None, dev_err=None):
    """bf16 dW [E, N, K] from bf16 g [Tcap, N] and x [Tcap, K]."""
    for t, nm in ((g, "g"), (x, "x")):
        if not isinstance(t, torch.Tensor) or t.dim() != 2:
            raise MXError(f"{nm}: expected a 2-D bf16 tensor")
        _want(t, nm, torch.bfloat16)
    Tcap, N = g.shape
    Tx, K = x.shape
    if Tx != Tcap:
        raise MXError(f"g has {Tcap} rows, x has {Tx}")
    if not isinstance(offs, torch.Tensor) or offs.dim() != 1:
        raise MXError("offs: expected int32 [E]")
    _want(offs, "offs", torch.int32)
    E = offs.shape[0]
    if out is None:
        out = torch.empty((E, N, K), dtype=torch.bfloat16, device=g.device)
    _want(out, "out", torch.bfloat16, shape=(E, N, K))
    _device(g, x, offs, out, _flag(dev_err))
    st = lib().mx_grouped_mm_wgrad_hp(_ptr(g), _ptr(x), _ptr(offs), E, Tcap, N, K, _ptr(out),
                                      _ptr(dev_err), _stream(g.device))
    _check(st, "mx_grouped_mm_wgrad_hp")
    return out


def pad_groups(x, sizes, Tcap, multiple=128, out=None, dev_err=None):
    """x [T, ...] rows grouped by expert; sizes int32 [E] on the device.
    Returns (x_pad [Tcap, ...], offs int32 [E], src_row int32 [Tcap])."""
    if not isinstance(x, torch.Tensor) or x.dim() < 1:
        raise MXError("x: expected a tensor of rows")
    _want(x, "x", x.dtype)
    T = x.shape[0]
    row_bytes = math.prod(x.shape[1:]) * x.element_size()
    if not isinstance(sizes, torch.Tensor) or sizes.dim() != 1:
        raise MXError("sizes: expected int32 [E]")
    _want(sizes, "sizes", torch.int32)
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
    _want(x_pad, "x_pad", x.dtype, shape=(Tcap,) + tuple(x.shape[1:]))
    _want(offs, "offs", torch.int32, E)
    _want(src, "src_row", torch.int32, Tcap)
    _device(x, sizes, x_pad, offs, src, _flag(dev_err))
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
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        raise MXError("x: expected a 2-D bf16 tensor")
    _want(x, "x", torch.bfloat16)
    T, C = x.shape
    if not isinstance(sizes, torch.Tensor) or sizes.dim() != 1:
        raise MXError("sizes: expected int32 [E]")
    _want(sizes, "sizes", torch.int32)
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
    _check_q_outs(out, 1, Tcap, C, rowwise, colwise)
    _want(out["offs"], "offs", torch.int32, E)
    _want(out["src_row"], "src_row", torch.int32, Tcap)
    _device(x, sizes, out.get("q_row"), out.get("s_row"), out.get("q_col"), out.get("s_col"), out["offs"],
            out["src_row"], _flag(dev_err))
    dirs = (ROWWISE if rowwise else 0) | (COLWISE if colwise else 0)
    st = lib().mx_pad_quantize(_ptr(x), _ptr(sizes), E, T, C, multiple, Tcap, _MODES[mode], dirs,
                               _LAYOUTS[layout], _ptr(out.get("q_row")), _ptr(out.get("s_row")),
                               _ptr(out.get("q_col")), _ptr(out.get("s_col")), _ptr(out["offs"]),
                               _ptr(out["src_row"]), _ptr(dev_err), _stream(dev))
    _check(st, "mx_pad_quantize")
    return out


def unpad_groups(y_pad, src_row, T, out=None):
    """Rows of y_pad [Tcap, ...] back to token order [T, ...] through the
    row map that pad_groups returned."""
    if not isinstance(y_pad, torch.Tensor) or y_pad.dim() < 1:
        raise MXError("y_pad: expected a tensor of rows")
    _want(y_pad, "y_pad", y_pad.dtype)
    Tcap = y_pad.shape[0]
    row_bytes = math.prod(y_pad.shape[1:]) * y_pad.element_size()
    _want(src_row, "src_row", torch.int32, Tcap)
    if out is None:
        out = torch.empty((T,) + tuple(y_pad.shape[1:]), dtype=y_pad.dtype, device=y_pad.device)
    _want(out, "out", y_pad.dtype, shape=(T,) + tuple(y_pad.shape[1:]))
    _device(y_pad, src_row, out)
    st = lib().mx_unpad_groups(_ptr(y_pad), _ptr(src_row), Tcap, T, row_bytes, _ptr(out),
                               _stream(y_pad.device))
    _check(st, "mx_unpad_groups")
    return out
