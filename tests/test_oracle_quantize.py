"""Pins of the oracle's MX block quantization: hand-derived golden blocks
(tests/golden/mx_blocks.json) and invariants the OCP MX definitions fix."""

import json
import os

import numpy as np
import pytest

from oracle import mx
from quantize_grouped_gemm_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mx_blocks.json")


def _golden_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: f"{c['name']}-{c['mode']}")
def test_golden_blocks(case):
    if "values_bf16" in case:
        vals = mx.bf16_to_f64(np.array([int(v, 16) for v in case["values_bf16"]], np.uint16))
    else:
        vals = np.array(case["values"], np.float64)
    blk = np.zeros(32)
    blk[:len(vals)] = vals
    # the block must hold bf16 values (inputs are bf16)
    np.testing.assert_array_equal(mx.bf16_to_f64(mx.f64_to_bf16(blk)), blk)
    q, s = mx.quantize(blk[None, :], case["mode"])
    assert s[0, 0] == case["scale"]
    exp = [int(c, 16) for c in case["codes"]]
    assert list(q[0, :len(exp)]) == exp
    rest = q[0, len(exp):]
    np.testing.assert_array_equal(rest, np.where(np.signbit(blk[len(exp):]), 0x80, 0))


def _rand_bf16(shape, seed):
    g = synth.generator(seed)
    return synth.bits(synth.normal_bf16(shape, 1.0, g))


@pytest.mark.parametrize("mode", ["rceil", "floor"])
def test_sign_symmetry_and_power_of_two_shift(mode):
    xb = _rand_bf16((64, 256), 5)
    x = mx.bf16_to_f64(xb)
    q, s = mx.quantize(x, mode)
    qn, sn = mx.quantize(-x, mode)
    np.testing.assert_array_equal(qn, q ^ 0x80)
    np.testing.assert_array_equal(sn, s)
    for j in (-40, -3, 1, 17, 60):
        qj, sj = mx.quantize(x * 2.0 ** j, mode)
        np.testing.assert_array_equal(qj, q)
        np.testing.assert_array_equal(sj.astype(int), s.astype(int) + j)


@pytest.mark.parametrize("mode", ["rceil", "floor"])
def test_round_trip_error_bound_and_idempotence(mode):
    xb = synth.bits(synth.stress_tensor(256, 512, seed=7))
    x = mx.bf16_to_f64(xb)
    q, s = mx.quantize(x, mode)
    d = mx.dequantize(q, s)
    E = np.repeat(s.astype(np.int64) - 127, 32, axis=-1)
    y = np.abs(x) * np.exp2(-E.astype(np.float64))
    # half an E4M3 step at |y| (subnormal spacing below 2**-6), times the scale
    e = np.maximum(np.floor(np.log2(np.where(y > 0, y, 1.0))), -6)
    half_step = np.exp2(e - 4) * np.exp2(E.astype(np.float64))
    sat = y > 448.0
    err = np.abs(d - x)
    assert np.all(err[~sat] <= half_step[~sat])
    if mode == "rceil":
        assert not sat.any()                               # RCEIL never saturates
    else:
        assert np.all(np.abs(d[sat]) == 448.0 * np.exp2(E[sat].astype(np.float64)))
    # dequantized values are fixed points of quantize->dequantize in both modes
    q2, s2 = mx.quantize(d, mode)
    np.testing.assert_array_equal(mx.dequantize(q2, s2), d)
    if mode == "floor":                                    # FLOOR bytes are idempotent too
        np.testing.assert_array_equal(q2, q)
        np.testing.assert_array_equal(s2, s)


def test_rceil_bytes_not_idempotent_example():
    # scaled amax 230 (in (224, 232)) rounds to 224 and drops a binade on
    # requantization, so RCEIL scale bytes need not be idempotent.
    blk = np.zeros(32)
    blk[0] = 230.0 * 2.0 ** -8 * 2                          # amax 1.796875
    q, s = mx.quantize(blk[None], "rceil")
    q2, s2 = mx.quantize(mx.dequantize(q, s), "rceil")
    assert s2[0, 0] == s[0, 0] - 1


def test_colwise_is_rowwise_of_transpose_and_batches_are_independent():
    xb = _rand_bf16((3, 64, 96), 9)
    out = mx.quantize_bf16(xb, "rceil", rowwise=True, colwise=True)
    assert out["q_col"].shape == (3, 96, 64) and out["s_col"].shape == (3, 96, 2)
    for e in range(3):
        one = mx.quantize_bf16(xb[e], "rceil", rowwise=True, colwise=True)
        np.testing.assert_array_equal(out["q_row"][e], one["q_row"])
        np.testing.assert_array_equal(out["q_col"][e], one["q_col"])
        # a column block of 32 rows, quantized by hand as a vector
        c, b = 5, 1
        qv, sv = mx.quantize(mx.bf16_to_f64(xb[e, 32 * b:32 * b + 32, c])[None], "rceil")
        np.testing.assert_array_equal(out["q_col"][e, c, 32 * b:32 * b + 32], qv[0])
        assert out["s_col"][e, c, b] == sv[0, 0]


def test_nonfinite_blocks():
    blk = np.zeros((2, 32))
    blk[0, 3] = np.nan
    blk[0, 4] = -1.0
    blk[1, 7] = -np.inf
    q, s = mx.quantize(blk, "rceil")
    assert list(s[:, 0]) == [255, 255]
    assert q[0, 4] == 0xFF and q[0, 0] == 0x7F and q[1, 7] == 0xFF


def test_dequantize_is_exact_product():
    rng = np.random.default_rng(11)
    q = rng.integers(0, 256, (8, 64)).astype(np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x11
    s = rng.integers(0, 255, (8, 2)).astype(np.uint8)
    d = mx.dequantize(q, s)
    for r in range(8):
        for c in range(64):
            assert d[r, c] == mx.E4M3_VALUES[q[r, c]] * 2.0 ** (int(s[r, c // 32]) - 127)


# ---------------------------------------------------------------- FP8 row-scaled

def _fp8_rows_brute(x):
    """One scale per row by direct search: the smallest integer E in the E8M0
    range with every |x| <= 448 * 2**E; codes by torch's own float8 cast of
    x * 2**-E (exact in float32 for these inputs)."""
    import torch
    x = np.asarray(x, np.float64)
    R, C = x.shape
    q = np.zeros((R, C), np.uint8)
    sc = np.zeros((R, C // 32), np.uint8)
    for r in range(R):
        amax = np.max(np.abs(x[r]))
        E = -127
        while E < 127 and amax > 448.0 * 2.0 ** E:
            E += 1
        y = torch.from_numpy((x[r] * 2.0 ** -E).astype(np.float32))
        q[r] = y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        sc[r] = E + 127
    return q, sc


def test_fp8_rows_against_brute_force_and_torch_cast():
    rng = np.random.default_rng(11)
    bits = _rand_bf16((24, 96), 11)
    x = mx.bf16_to_f64(bits)
    x[3] *= 2.0 ** -120            # near the bottom of the scale range
    x[4] *= 2.0 ** 100             # near the top
    x[5] = 0.0                     # amax 0
    x[6, 7] = 448.0 * 2.0 ** 3     # amax exactly on a power-of-two bound
    x[7] = rng.choice([-1.0, 1.0], 96) * 2.0 ** rng.integers(-20, 20, 96)
    q, sc = mx.quantize_fp8_rows(x)
    bq, bsc = _fp8_rows_brute(x)
    np.testing.assert_array_equal(sc, bsc)
    np.testing.assert_array_equal(q, bq)


def test_fp8_rows_reduce_to_mx_when_every_block_holds_the_row_max():
    """With the row's largest magnitude present in every 32-block, the row
    scale and each MX block scale (RCEIL) coincide, so the bytes are the MX
    quantization's."""
    bits = _rand_bf16((16, 128), 12)
    x = mx.bf16_to_f64(bits)
    amax = np.max(np.abs(x), axis=1, keepdims=True)
    x[:, ::32] = amax          # plant the row max at the start of every block
    q, sc = mx.quantize_fp8_rows(x)
    mq, msc = mx.quantize(x, "rceil")
    np.testing.assert_array_equal(q, mq)
    np.testing.assert_array_equal(sc, msc)
    # and a row whose blocks differ gets one scale for all of them
    y = x.copy()
    y[0, 40] = amax[0, 0] * 64
    q2, sc2 = mx.quantize_fp8_rows(y)
    assert len(set(sc2[0].tolist())) == 1 and sc2[0, 0] == sc[0, 0] + 6


def test_fp8_columns_by_segment_and_nonfinite_rows():
    bits = _rand_bf16((384, 64), 13)
    seg = np.array([128, 128, 256])           # an empty segment, then a tail of 128
    out = mx.quantize_fp8_bf16(bits, rowwise=False, colwise=True, segments=seg)
    x = mx.bf16_to_f64(bits)
    for s, e in ((0, 128), (128, 256), (256, 384)):
        q, sc = mx.quantize_fp8_rows(x[s:e].T)
        np.testing.assert_array_equal(out["q_col"][:, s:e], q)
        np.testing.assert_array_equal(out["s_col"][:, s // 32:e // 32], sc)
    whole = mx.quantize_fp8_bf16(bits, rowwise=True, colwise=True)
    np.testing.assert_array_equal(whole["q_col"], mx.quantize_fp8_rows(x.T)[0])
    np.testing.assert_array_equal(whole["q_row"], mx.quantize_fp8_rows(x)[0])
    z = x[:2].copy()
    z[0, 5] = np.nan
    z[1, 9] = -np.inf
    q, sc = mx.quantize_fp8_rows(z)
    assert np.all(sc == 255)
    np.testing.assert_array_equal(q & 0x7F, 0x7F)
    np.testing.assert_array_equal(q >> 7, np.signbit(z).astype(np.uint8))
