"""GPU parity of the FP8 row-scaled quantizers (one power-of-two scale per
row; column-wise per column or per column and group) against the oracle,
bit-exact, and of the grouped GEMMs on those operands (the MXFP8 kernels
with equal block scales along each row) against the oracle's GEMM of the
dequantized operands."""

import numpy as np
import pytest
import torch

from _helpers import FROB_MFMA, dev, frob_rel, host, plain, to_dev
from oracle import mx as O
from quantize_grouped_gemm_amd import mx, synth

pytestmark = pytest.mark.gpu


def _bf16_dev(b):
    return to_dev(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16)


def _inputs(shape, seed):
    g = synth.generator(seed)
    b = synth.bits(synth.normal_bf16(shape, 1.0, g))
    flat = b.reshape(-1, shape[-1])
    flat[1] = 0                                            # an all-zero row
    flat[2, 5] = 0x7F80                                    # +inf
    flat[3, 7] = 0x7FC1                                    # NaN
    flat[4] = (flat[4] & 0x807F) | (0x20 << 7)             # tiny magnitudes
    flat[5, 9] = 0x4700                                    # 32768, an outlier
    return b


@pytest.mark.parametrize("shape", [(128, 128), (300, 256), (2, 96, 384)])
def test_fp8_rowwise(gpu, shape):
    b = _inputs(shape, sum(shape))
    got = mx.quantize_fp8(_bf16_dev(b), rowwise=True)
    ref = O.quantize_fp8_bf16(b, rowwise=True)
    np.testing.assert_array_equal(host(got["q_row"]), ref["q_row"])
    np.testing.assert_array_equal(plain(host(got["s_row"])), ref["s_row"])


@pytest.mark.parametrize("shape", [(128, 128), (512, 256), (2, 256, 384)])
def test_fp8_colwise(gpu, shape):
    b = _inputs(shape, 3 * sum(shape))
    got = mx.quantize_fp8(_bf16_dev(b), rowwise=False, colwise=True)
    ref = O.quantize_fp8_bf16(b, rowwise=False, colwise=True)
    np.testing.assert_array_equal(host(got["q_col"]), ref["q_col"])
    np.testing.assert_array_equal(plain(host(got["s_col"])), ref["s_col"])


@pytest.mark.parametrize("slots", [[256, 0, 640, 128], [128], [0, 384, 0]])
def test_fp8_colwise_per_group(gpu, slots):
    offs = np.cumsum(slots).astype(np.int32)
    R = int(offs[-1]) + 256                                # a tail of two tiles
    b = _inputs((R, 384), R)
    got = mx.quantize_fp8(_bf16_dev(b), rowwise=False, colwise=True, offs=to_dev(offs))
    ref = O.quantize_fp8_bf16(b, rowwise=False, colwise=True, segments=offs)
    np.testing.assert_array_equal(host(got["q_col"]), ref["q_col"])
    np.testing.assert_array_equal(plain(host(got["s_col"])), ref["s_col"])


@pytest.mark.parametrize("shape,slots", [((256, 384), None), ((640, 256), [256, 0, 128]),
                                         ((2, 256, 384), None), ((1024, 128), [0, 384, 0, 512])])
def test_fp8_dual(gpu, shape, slots):
    """Both directions from the fused entry point: the oracle's bytes, and
    bit for bit what the separate row-wise and column-wise calls write."""
    b = _inputs(shape, 7 * sum(shape))
    offs = None if slots is None else np.cumsum(slots).astype(np.int32)
    offs_d = None if offs is None else to_dev(offs)
    x = _bf16_dev(b)
    got = mx.quantize_fp8(x, rowwise=True, colwise=True, offs=offs_d)
    sep = mx.quantize_fp8(x, rowwise=True, colwise=True, offs=offs_d, fused=False)
    ref = O.quantize_fp8_bf16(b, rowwise=True, colwise=True, segments=offs)
    for k in ("q_row", "s_row", "q_col", "s_col"):
        assert torch.equal(got[k], sep[k]), k
    np.testing.assert_array_equal(host(got["q_row"]), ref["q_row"])
    np.testing.assert_array_equal(plain(host(got["s_row"])), ref["s_row"])
    np.testing.assert_array_equal(host(got["q_col"]), ref["q_col"])
    np.testing.assert_array_equal(plain(host(got["s_col"])), ref["s_col"])


@pytest.mark.parametrize("seed", range(6))
def test_fp8_random_shapes(gpu, seed):
    """Seeded random requests for the three FP8 entry points: batch of 1..2
    matrices, rows and columns multiples of 128 up to 1024 (row-wise rows:
    any count), a row stride wider than the columns, per-group column
    scales over random segments (empty ones included) or none."""
    rng = np.random.default_rng(9000 + seed)
    batch = 2 if seed % 3 == 0 else 1
    R = 128 * int(rng.integers(1, 9))
    C = 128 * int(rng.integers(1, 9))
    ld = C + 8 * int(rng.integers(0, 4))
    slots = None
    if batch == 1 and rng.random() < 0.6:
        n = int(rng.integers(1, 6))
        parts = np.sort(rng.integers(0, R // 128 + 1, n - 1))
        slots = np.diff(np.concatenate([[0], parts, [R // 128 - int(rng.integers(0, 2))]])) * 128
        slots = np.maximum(slots, 0)
    print(f"seed {seed}: batch={batch} R={R} C={C} ld={ld} slots={None if slots is None else list(slots)}",
          flush=True)
    full = _inputs((batch, R, ld), 9100 + seed)
    b = np.ascontiguousarray(full[..., :C])
    x = _bf16_dev(full)[..., :C]
    if batch == 1:
        b, x = b[0], x[0]
    offs = None if slots is None else np.cumsum(slots).astype(np.int32)
    offs_d = None if offs is None else to_dev(offs)
    err = torch.zeros(1, dtype=torch.int32, device=dev())
    got = mx.quantize_fp8(x, rowwise=True, colwise=True, offs=offs_d, dev_err=err)
    sep = mx.quantize_fp8(x, rowwise=True, colwise=True, offs=offs_d, fused=False, dev_err=err)
    ref = O.quantize_fp8_bf16(b, rowwise=True, colwise=True, segments=offs)
    for k in ("q_row", "s_row", "q_col", "s_col"):
        assert torch.equal(got[k], sep[k]), k
    np.testing.assert_array_equal(host(got["q_row"]), ref["q_row"])
    np.testing.assert_array_equal(plain(host(got["s_row"])), ref["s_row"])
    np.testing.assert_array_equal(host(got["q_col"]), ref["q_col"])
    np.testing.assert_array_equal(plain(host(got["s_col"])), ref["s_col"])
    assert int(err.item()) == 0


def test_fp8_grouped_gemms_through_the_mx_kernels(gpu):
    """Forward and weight gradient on FP8 row-scaled operands: the MXFP8
    grouped kernels against the oracle's float64 GEMM of the dequantized
    operands, within the MFMA accumulation model's Frobenius bound."""
    E, N, K = 3, 256, 384
    slots = np.array([256, 0, 384])
    offs = np.cumsum(slots).astype(np.int32)
    Tcap = int(offs[-1]) + 128
    g = synth.generator(9)
    xb = synth.bits(synth.normal_bf16((Tcap, K), 1.0, g))
    wb = synth.bits(synth.normal_bf16((E, N, K), 0.05, g))
    gb = synth.bits(synth.normal_bf16((Tcap, N), 1.0, g))
    x, w, gr = _bf16_dev(xb), _bf16_dev(wb), _bf16_dev(gb)
    qx = mx.quantize_fp8(x, rowwise=True, colwise=True, offs=to_dev(offs))
    qw = mx.quantize_fp8(w, rowwise=True)
    qg = mx.quantize_fp8(gr, rowwise=False, colwise=True, offs=to_dev(offs))
    fwd = mx.grouped_mm_fwd(qx["q_row"], qx["s_row"], qw["q_row"], qw["s_row"], to_dev(offs), torch.float32)
    rx = O.quantize_fp8_bf16(xb, rowwise=True, colwise=True, segments=offs)
    rw = O.quantize_fp8_bf16(wb, rowwise=True)
    ref = O.grouped_mm(rx["q_row"], rx["s_row"], rw["q_row"], rw["s_row"], offs)
    assert frob_rel(host(fwd)[:int(offs[-1])], ref[:int(offs[-1])]) <= FROB_MFMA
    dw = mx.grouped_mm_wgrad(qg["q_col"], qg["s_col"], qx["q_col"], qx["s_col"], to_dev(offs), torch.float32)
    rg = O.quantize_fp8_bf16(gb, rowwise=False, colwise=True, segments=offs)
    ref = O.grouped_mm_wgrad(rg["q_col"], rg["s_col"], rx["q_col"], rx["s_col"], offs)
    for e in (0, 2):
        assert frob_rel(host(dw[e]), ref[e]) <= FROB_MFMA, e
    assert torch.all(dw[1] == 0)


@pytest.mark.parametrize("fused", [True, False])
def test_fp8_bad_offsets_flag_dev_err(gpu, fused):
    """Segment offsets that are not non-decreasing multiples of 128 within the
    rows raise bit 0 of dev_err (both the column-wise and the dual entry
    point); valid ones leave it clear."""
    b = _inputs((512, 256), 11)
    x = _bf16_dev(b)
    for bad in ([128, 100, 512], [256, 128, 384], [128, 256, 640]):
        err = torch.zeros(1, dtype=torch.int32, device=dev())
        mx.quantize_fp8(x, rowwise=fused, colwise=True, offs=to_dev(np.array(bad, np.int32)), fused=fused,
                        dev_err=err)
        torch.cuda.synchronize()
        assert int(err.item()) & 1, bad
    err = torch.zeros(1, dtype=torch.int32, device=dev())
    mx.quantize_fp8(x, rowwise=fused, colwise=True, offs=to_dev(np.array([128, 128, 384], np.int32)), fused=fused,
                    dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
