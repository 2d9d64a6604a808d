"""A second, independent CPU implementation of the MXFP8 MLP step, written
with torch primitives instead of the oracle's numpy bit arithmetic. It pins
the oracle's two MLP compositions (which chain the oracle's separately pinned
functions) stage by stage: every stage here starts from the oracle's own
inputs to that stage, so a disagreement points at one wiring mistake (a wrong
operand, axis, scale mode, gate half or a missing rounding) rather than at
noise carried down the chain.

Independence from the oracle: scale exponents come from float64 log2 and
ceil / floor (the oracle uses frexp and a bound comparison), elements are
encoded by torch's own float8_e4m3fn cast after clamping to +-448, scale
bytes by torch's float8_e8m0fnu cast, products by torch float64 matmuls,
SwiGLU by torch.nn.functional.silu and its gradient by autograd, bf16 by
torch's cast. The one known difference: torch rounds float64 to bf16 through
float32 (two roundings), so a bf16 result may differ from a single rounding
by one ulp on rare elements; comparisons allow exactly that.
"""

import numpy as np
import torch

F64 = torch.float64


def from_bits(b):
    """uint16 bf16 bit patterns -> float64 torch tensor (exact)."""
    t = torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16)
    return t.to(F64)


def to_bf16(x):
    """float64 -> bf16 values (as float64), torch's cast."""
    return x.to(torch.bfloat16).to(F64)


def block_exponent(amax, mode):
    """Scale exponent per block maximum: RCEIL = ceil(log2(amax / 448)),
    FLOOR = floor(log2(amax)) - 8, clamped to [-127, 127]; 0 for amax = 0
    maps to -127."""
    pos = amax > 0
    safe = torch.where(pos, amax, torch.ones_like(amax))
    if mode == "rceil":
        e = torch.ceil(torch.log2(safe / 448.0))
    else:
        e = torch.floor(torch.log2(safe)) - 8
    e = torch.where(pos, e, torch.full_like(e, -127.0))
    return e.clamp(-127, 127)


def mx_quant(x, mode):
    """Row-wise MX quantization of float64 x [..., C] along the last axis.
    Returns (dequantized values float64, codes uint8, scale bytes uint8)."""
    shp = x.shape
    blk = x.reshape(shp[:-1] + (shp[-1] // 32, 32))
    e = block_exponent(blk.abs().amax(-1), mode)
    scale = torch.pow(2.0, e).unsqueeze(-1)
    y = (blk / scale).clamp(-448.0, 448.0)
    f8 = y.to(torch.float8_e4m3fn)
    deq = (f8.to(F64) * scale).reshape(shp)
    sbytes = torch.pow(2.0, e).to(torch.float32).to(torch.float8_e8m0fnu).view(torch.uint8)
    return deq, f8.view(torch.uint8).reshape(shp), sbytes


def mx_rows(x, mode):
    return mx_quant(x, mode)[0]


def mx_cols(x, mode):
    """Column-wise: quantized along dim 0, returned in x's orientation."""
    return mx_quant(x.transpose(-1, -2).contiguous(), mode)[0].transpose(-1, -2)


def fp8_rows(x):
    """One power-of-two scale per row (RCEIL over the whole row)."""
    e = block_exponent(x.abs().amax(-1), "rceil").unsqueeze(-1)
    scale = torch.pow(2.0, e)
    return (x / scale).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).to(F64) * scale


def fp8_cols(x, segments=None):
    """One scale per column, or per (column, segment) of rows."""
    if segments is None:
        return fp8_rows(x.transpose(-1, -2).contiguous()).transpose(-1, -2)
    out = torch.zeros_like(x)
    start = 0
    for end in list(segments) + [x.shape[0]]:
        if end > start:
            out[start:end] = fp8_rows(x[start:end].transpose(0, 1).contiguous()).transpose(0, 1)
        start = end
    return out


def swiglu(a, b):
    return torch.nn.functional.silu(a) * b


def swiglu_grads(dh, a, b):
    a = a.clone().requires_grad_()
    b = b.clone().requires_grad_()
    swiglu(a, b).backward(dh)
    return a.grad, b.grad


def pad(x, sizes, multiple, Tcap):
    """Group g's rows to the start of a slot of ceil(n_g / multiple) * multiple
    rows; returns (padded, slot ends, row index of each real row)."""
    sizes = [int(s) for s in sizes]
    ends, idx, at = [], [], 0
    src = 0
    for n in sizes:
        idx += list(range(at, at + n))
        at += -(-n // multiple) * multiple
        ends.append(at)
        src += n
    out = torch.zeros((Tcap,) + tuple(x.shape[1:]), dtype=x.dtype)
    out[torch.tensor(idx, dtype=torch.long)] = x
    return out, ends, torch.tensor(idx, dtype=torch.long)


def groups(ends):
    start = 0
    for g, end in enumerate(ends):
        yield g, start, end
        start = end
