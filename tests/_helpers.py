"""Shared helpers of the GPU parity tests: device transfer, seeded synthetic
MX operands, and the tolerance checks.

Tolerances
  * quantized bytes (E4M3 codes, E8M0 scales), padding, integer work:
    bit-exact.
  * fused SwiGLU + quantization: compared as dequantized values; an element
    may differ by at most one E4M3 step at its magnitude under the larger of
    the two block scales, and at most 1e-5 of all elements may differ
    (``code_tolerance``).
  * float32 GEMM outputs: relative Frobenius error <= 1e-5 (``frob_rel``).
  * bf16 GEMM outputs: within 2 bf16 ulp elementwise, the ulp taken at
    max(|ref|, 2^-10 * rms(ref row)) so that outputs which cancel to far
    below their row's scale are judged against the float32 accumulation
    noise of that row (``bf16_ulp_check``).
"""

import numpy as np
import torch

from oracle import mx as O


def dev():
    return torch.device("cuda:0")


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def host(t):
    return t.detach().cpu().numpy()


def bf16_host(t):
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def rand_mx(shape, seed, scale_lo=118, scale_hi=132):
    """Seeded synthetic MX operand: codes uniform over the finite E4M3 codes
    (either sign), scale bytes uniform in [scale_lo, scale_hi)."""
    rng = np.random.default_rng(seed)
    q = rng.integers(0, 0x7F, shape) | (rng.integers(0, 2, shape) << 7)
    s = rng.integers(scale_lo, scale_hi, shape[:-1] + (shape[-1] // 32,))
    return q.astype(np.uint8), s.astype(np.uint8)


def frob_rel(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.sqrt(np.sum(ref * ref))
    return float(np.sqrt(np.sum((got - ref) ** 2)) / max(den, 1e-300))


def bf16_ulp_check(got_bits, ref, max_ulp=2.0):
    """Returns (worst ulp distance, count of strict-ulp failures)."""
    got = O.bf16_to_f64(got_bits)
    ref = np.asarray(ref, np.float64)
    rms = np.sqrt(np.mean(ref * ref, axis=-1, keepdims=True))
    mag = np.maximum(np.abs(ref), 2.0 ** -10 * rms)
    e = np.floor(np.log2(np.where(mag > 0, mag, 1.0)))
    ulp = np.exp2(np.maximum(e, -126) - 7)
    d = np.abs(got - ref) / ulp
    strict_e = np.floor(np.log2(np.where(np.abs(ref) > 0, np.abs(ref), 1.0)))
    strict = np.abs(got - ref) / np.exp2(np.maximum(strict_e, -126) - 7)
    return float(d.max(initial=0.0)), int(np.sum(strict > max_ulp))


def _step(v, scale_exp):
    """E4M3 grid spacing at |v| under block scale 2**scale_exp."""
    y = np.abs(v) * np.exp2(-scale_exp)
    e = np.floor(np.log2(np.where(y > 0, y, 1.0)))
    return np.exp2(np.maximum(e, -6) - 3 + scale_exp)


def code_tolerance(qg, sg, qr, sr, frac=1e-5):
    """Dequantized comparison of two MX tensors (same layout). Returns
    (n_differing, n_beyond_one_code, n_total, n_scale_bytes_differing)."""
    dg = O.dequantize(qg, sg)
    dr = O.dequantize(qr, sr)
    E = np.repeat(np.maximum(sg.astype(np.int64), sr.astype(np.int64)) - 127, 32, axis=-1)
    step = _step(np.maximum(np.abs(dg), np.abs(dr)), E.astype(np.float64))
    diff = dg != dr
    beyond = np.abs(dg - dr) > step * (1 + 1e-12)
    return int(diff.sum()), int(beyond.sum()), dg.size, int((sg != sr).sum())
