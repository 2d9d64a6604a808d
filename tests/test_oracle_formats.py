"""Pins of the oracle's number-format functions against independent routines:
torch CPU casts, exhaustive nearest-value search over the formats' value sets,
and exact rational arithmetic (Fraction). No GPU."""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import mx

ALL_BF16 = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
FINITE_BF16 = ALL_BF16[(ALL_BF16 & 0x7F80) != 0x7F80]


def _torch_bf16_to_f64(bits):
    t = torch.from_numpy(bits.astype(np.uint16).view(np.int16)).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


def test_bf16_decode_all_patterns_match_torch():
    ours = mx.bf16_to_f64(ALL_BF16)
    ref = _torch_bf16_to_f64(ALL_BF16)
    np.testing.assert_array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(ours[ok], ref[ok])
    np.testing.assert_array_equal(np.signbit(ours[ok]), np.signbit(ref[ok]))


def test_e4m3_table_matches_torch_and_closed_forms():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = mx.E4M3_VALUES
    np.testing.assert_array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(ours[ok], ref[ok])
    # closed forms of the OCP E4M3FN format
    assert ours[0x7E] == 448.0 and ours[0xFE] == -448.0
    assert ours[0x08] == 2.0 ** -6 and ours[0x01] == 2.0 ** -9
    assert ours[0x38] == 1.0 and ours[0x00] == 0.0 and np.signbit(ours[0x80])
    assert np.isnan(ours[0x7F]) and np.isnan(ours[0xFF])
    assert np.sum(np.isnan(ours)) == 2
    pos = ours[:0x7F]
    assert np.all(np.diff(pos) > 0)            # codes order like values


def test_e8m0_matches_torch():
    b = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = b.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    ours = mx.e8m0_to_f64(np.arange(256))
    assert np.isnan(ours[255]) and np.isnan(ref[255])
    np.testing.assert_array_equal(ours[:255], ref[:255])
    assert ours[127] == 1.0 and ours[0] == 2.0 ** -127 and ours[254] == 2.0 ** 127


def _bf16_nearest_even(x):
    """Independent bf16 RNE: nearest neighbour search over every positive
    finite bf16 value, ties to the even bit pattern."""
    pats = np.arange(0, 0x7F80, dtype=np.uint16)     # +0 .. largest finite
    vals = mx.bf16_to_f64(pats)
    a = np.abs(x)
    i = np.clip(np.searchsorted(vals, a, side="right") - 1, 0, len(vals) - 1)
    lo = vals[i]
    hi_i = np.minimum(i + 1, len(vals) - 1)
    hi = np.where(i + 1 < len(vals), vals[hi_i], 2.0 ** 128)
    dlo = a - lo
    dhi = hi - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (pats[i] % 2 == 1))
    out = np.where(pick_hi, (i + 1), i).astype(np.uint32)
    out = np.where(out >= 0x7F80, 0x7F80, out)          # rounds to infinity
    return (out | np.where(np.signbit(x), 0x8000, 0)).astype(np.uint16)


def test_f64_to_bf16_float32_inputs_match_torch():
    rng = np.random.default_rng(1)
    u = rng.integers(0, 1 << 32, 400000, dtype=np.uint64).astype(np.uint32)
    f = u.view(np.float32)
    f = f[np.isfinite(f)]
    # add exact ties and the overflow boundary
    ties = (rng.integers(0, 0x7F7F, 20000).astype(np.uint32) << 16 | 0x8000).view(np.float32)
    f = np.concatenate([f, ties, np.float32([3.3961514e38, 3.4e38, -0.0, 0.0, 1e-45])])
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ours = mx.f64_to_bf16(f.astype(np.float64))
    np.testing.assert_array_equal(ours, ref)


def test_f64_to_bf16_float64_inputs_match_nearest_search():
    rng = np.random.default_rng(2)
    x = rng.standard_normal(200000) * np.exp2(rng.integers(-140, 128, 200000))
    # float64 values within one float32 ulp of a bf16 midpoint, where a float32
    # stop would double-round
    mid = mx.bf16_to_f64((rng.integers(0, 0x7F7F, 20000).astype(np.uint16))) * (1 + 2.0 ** -9)
    x = np.concatenate([x, mid, np.nextafter(mid, 0), np.nextafter(mid, np.inf), -mid])
    x = x[np.isfinite(x)]
    np.testing.assert_array_equal(mx.f64_to_bf16(x), _bf16_nearest_even(x))


def _e4m3_nearest_even(y):
    """Independent saturating RNE: nearest of the 127 finite non-negative E4M3
    values, ties to the even code; beyond 448 clamp."""
    vals = mx.E4M3_VALUES[:0x7F]
    a = np.minimum(np.abs(y), 448.0)
    i = np.clip(np.searchsorted(vals, a, side="right") - 1, 0, 0x7E)
    hi_i = np.minimum(i + 1, 0x7E)
    dlo = a - vals[i]
    dhi = vals[hi_i] - a
    pick_hi = (i < 0x7E) & ((dhi < dlo) | ((dhi == dlo) & (i % 2 == 1)))
    code = np.where(pick_hi, i + 1, i)
    return (code | np.where(np.signbit(y), 0x80, 0)).astype(np.uint8)


@pytest.mark.slow
def test_e4m3_encode_exhaustive_all_bf16_times_all_scales():
    """All 65280 finite bf16 values times every scale 2**j, j in [-127, 127]
    (16.6M cases): the oracle's encoder equals torch's float8_e4m3fn cast of
    the clamped value and the nearest-value search."""
    v = mx.bf16_to_f64(FINITE_BF16)
    for j0 in range(-127, 128, 32):
        js = np.arange(j0, min(j0 + 32, 128))
        y = (v[None, :] * np.exp2(js)[:, None]).ravel()
        ours = mx.e4m3_encode(y)
        clamped = np.clip(y, -448.0, 448.0).astype(np.float32)
        ref = torch.from_numpy(clamped).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        np.testing.assert_array_equal(ours, ref)
        np.testing.assert_array_equal(ours, _e4m3_nearest_even(y))


def test_e4m3_encode_midpoints_and_neighbours():
    vals = mx.E4M3_VALUES[:0x7F]
    mids = (vals[:-1] + vals[1:]) / 2
    below = np.nextafter(mids, 0)
    above = np.nextafter(mids, np.inf)
    lo_codes = np.arange(0x7E)
    np.testing.assert_array_equal(mx.e4m3_encode(below), lo_codes)
    np.testing.assert_array_equal(mx.e4m3_encode(above), lo_codes + 1)
    even = np.where(lo_codes % 2 == 0, lo_codes, lo_codes + 1)
    np.testing.assert_array_equal(mx.e4m3_encode(mids), even)
    np.testing.assert_array_equal(mx.e4m3_encode(-mids), even | 0x80)
    # saturation: everything beyond 448 maps to 0x7E, never NaN
    big = np.array([448.0, 449.0, 464.0, 480.0, 1e30, np.inf])
    np.testing.assert_array_equal(mx.e4m3_encode(big), 0x7E)
    np.testing.assert_array_equal(mx.e4m3_encode(-big), 0xFE)
    assert mx.e4m3_encode(np.array([-0.0]))[0] == 0x80
    assert mx.e4m3_encode(np.array([np.nan]))[0] == 0x7F


def _floor_log2(fr):
    lo, hi = -200, 200                      # 2**lo <= fr < 2**hi
    while hi - lo > 1:
        mid = (lo + hi) // 2
        if Fraction(2) ** mid <= fr:
            lo = mid
        else:
            hi = mid
    return lo


def _rceil_exact(fr):
    """Smallest integer E with fr <= 448 * 2**E, by bisection."""
    lo, hi = -200, 200                      # fr > 448*2**lo, fr <= 448*2**hi
    while hi - lo > 1:
        mid = (lo + hi) // 2
        if fr <= 448 * Fraction(2) ** mid:
            hi = mid
        else:
            lo = mid
    return hi


def test_scale_exponent_all_bf16_amax_exact_rationals():
    pats = np.arange(1, 0x7F80, dtype=np.uint16)      # every positive finite bf16
    amax = mx.bf16_to_f64(pats)
    got_f = mx.scale_exponent(amax, "floor")
    got_r = mx.scale_exponent(amax, "rceil")
    exp_f = np.empty(len(pats), np.int64)
    exp_r = np.empty(len(pats), np.int64)
    for i, a in enumerate(amax.tolist()):
        fr = Fraction(a)
        exp_f[i] = min(max(_floor_log2(fr) - 8, -127), 127)
        exp_r[i] = min(max(_rceil_exact(fr), -127), 127)
    np.testing.assert_array_equal(got_f, exp_f)
    np.testing.assert_array_equal(got_r, exp_r)
    assert set(np.unique(got_r - got_f)) <= {0, 1}
    assert got_f.max() <= 120 and got_r.max() <= 120      # 0xFF never produced


def test_scale_exponent_properties_float32_amax():
    rng = np.random.default_rng(3)
    amax = np.abs(rng.standard_normal(200000) * np.exp2(rng.integers(-100, 100, 200000)))
    amax = amax.astype(np.float32).astype(np.float64)
    Er = mx.scale_exponent(amax, "rceil")
    Ef = mx.scale_exponent(amax, "floor")
    yr = amax * np.exp2(-Er.astype(np.float64))
    yf = amax * np.exp2(-Ef.astype(np.float64))
    assert np.all(yr <= 448.0) and np.all(yr > 224.0)     # smallest such power
    assert np.all((yf >= 256.0) & (yf < 512.0))
    # exact boundary: 448 * 2**k stays at k, one float32 step above goes to k+1
    k = np.arange(-100, 100)
    edge = 448.0 * np.exp2(k)
    np.testing.assert_array_equal(mx.scale_exponent(edge, "rceil"), k)
    up = np.nextafter(edge.astype(np.float32), np.float32(np.inf)).astype(np.float64)
    np.testing.assert_array_equal(mx.scale_exponent(up, "rceil"), k + 1)
    assert mx.scale_exponent(np.array([0.0]), "rceil")[0] == -127
    assert mx.scale_exponent(np.array([0.0]), "floor")[0] == -127
