"""Every finite bf16 value under every block scale it can meet, through
mx_quantize, bit-exact against the oracle.

The element conversion on the GPU is a hardware instruction that scales by
2^-E and rounds to E4M3; this test pins it (and the scale choice around it)
over the whole reachable input space rather than on random samples. For each
mode and each scale exponent E the mode can produce for finite input, one
"partner" element sets the block's amax to the largest bf16 value that still
gives that E; the other 31 elements of the block run through every finite
bf16 pattern (either sign, zeros and subnormals included) whose magnitude
does not exceed the partner, so the block keeps exponent E. The partner sits
at a different position in successive blocks.

  RCEIL: E = ceil(log2(amax / 448)); the largest amax for E is 448 * 2^E =
         1.75 * 2^(E+8) while that is a bf16 value (E <= 119), and the
         largest finite bf16 for E = 120. E = -127 also holds every smaller
         amax (the clamp). Reachable: E = -127 .. 120.
  FLOOR: E = floor(log2(amax)) - 8; the largest amax for E is the largest
         bf16 below 2^(E+9), 1.9921875 * 2^(E+8). Reachable: -127 .. 119.

The blocks are laid out along rows (row-wise quantization; and dual, whose
column-wise half is checked too) and, transposed, down columns (column-wise
quantization of the crafted blocks)."""

import numpy as np
import pytest
import torch

from _helpers import host, plain, to_dev
from oracle import mx as O
from quantize_grouped_gemm_amd import mx

pytestmark = pytest.mark.gpu

_FINITE = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
_FINITE = _FINITE[(_FINITE & 0x7F80) != 0x7F80]
_MAG = _FINITE & np.uint16(0x7FFF)   # magnitude patterns order like magnitudes


def _partner(mode, E):
    """bf16 bits of the largest block maximum that gives scale exponent E."""
    if mode == "rceil":
        if E == 120:
            return 0x7F7F                        # largest finite bf16
        return ((E + 8 + 127) << 7) | 0x60        # 1.75 * 2^(E+8)
    return ((E + 8 + 127) << 7) | 0x7F            # 1.9921875 * 2^(E+8)


def _blocks(mode):
    """[n, 32] bf16 bit patterns: every (value, reachable E) pair once."""
    lo, hi = -127, (120 if mode == "rceil" else 119)
    out = []
    nblk = 0
    for E in range(lo, hi + 1):
        p = np.uint16(_partner(mode, E))
        vals = _FINITE[_MAG <= p]
        nb = -(-len(vals) // 31)
        fill = np.zeros(nb * 31, np.uint16)      # +0 fills the last block
        fill[:len(vals)] = vals
        body = fill.reshape(nb, 31)
        pos = (nblk + np.arange(nb)) % 32
        blk = np.empty((nb, 32), np.uint16)
        for j in range(32):
            sel = pos == j
            blk[sel, j] = p | np.uint16(0x8000 * (j & 1))   # partner, either sign
            blk[sel, :j] = body[sel, :j]
            blk[sel, j + 1:] = body[sel, j:]
        out.append(blk)
        nblk += nb
    b = np.concatenate(out)
    pad = (-len(b)) % 2048                        # whole 128 x 512 tiles both ways
    return np.concatenate([b, np.zeros((pad, 32), np.uint16)])


def _dev_bf16(bits):
    return to_dev(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)


def _expect_equal(got, ref, what):
    for k, r in ref.items():
        g = host(got[k])
        if k.startswith("s_"):
            g = plain(g)
        assert g.shape == r.shape, (what, k)
        bad = np.argwhere(g != r)
        assert len(bad) == 0, f"{what} {k}: {len(bad)} bytes differ, first at {bad[:4].tolist()}"


@pytest.mark.parametrize("mode", ["rceil", "floor"])
def test_every_value_under_every_scale(gpu, mode):
    blk = _blocks(mode)
    n = len(blk)
    # along rows: 4 blocks per 128-column row
    xr = blk.reshape(n // 4, 128)
    scales = O.quantize_bf16(xr, mode, True, False)["s_row"]
    want_E = np.arange(-127, (121 if mode == "rceil" else 120))
    assert set(np.unique(scales.astype(int) - 127)) == set(want_E)   # every reachable E appears
    xt = _dev_bf16(xr)
    _expect_equal(mx.quantize(xt, mode, True, False), O.quantize_bf16(xr, mode, True, False), f"{mode} row")
    _expect_equal(mx.quantize(xt, mode, True, True), O.quantize_bf16(xr, mode, True, True), f"{mode} dual")
    # down columns: block j of column c is rows 32 j .. 32 j + 31
    C = 512
    J = n // C
    xc = np.ascontiguousarray(blk.reshape(J, C, 32).transpose(0, 2, 1).reshape(J * 32, C))
    _expect_equal(mx.quantize(_dev_bf16(xc), mode, False, True), O.quantize_bf16(xc, mode, False, True),
                  f"{mode} col")
