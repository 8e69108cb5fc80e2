"""Pins of the oracle's number formats against exact rational arithmetic and the OCP E4M3 definition."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import numerics as nm


def _all_finite_f16():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    v = bits.view(np.float16)
    return v[np.isfinite(v)]


def _nearest_even_f16(t: Fraction) -> float:
    """Exact nearest binary16 to rational t by bracketing, ties to even significand."""
    lo = np.float16(float(t))            # within one ulp of t
    cands = {lo, np.nextafter(lo, np.float16(np.inf)), np.nextafter(lo, np.float16(-np.inf))}
    cands = [c for c in cands if np.isfinite(c)]
    best = min(abs(Fraction(float(c)) - t) for c in cands)
    tied = [c for c in cands if abs(Fraction(float(c)) - t) == best]
    if len(tied) == 1:
        return float(tied[0])
    even = [c for c in tied if (np.array(c, np.float16).view(np.uint16) & 1) == 0]
    return float(even[0])


def test_f16_rounding_matches_exact_nearest_even():
    rng = np.random.default_rng(7)
    xs = list(rng.standard_normal(3000) * np.exp2(rng.integers(-26, 16, 3000)))
    # exact midpoints between neighbouring fp16 values, and values a hair away from them
    base = rng.choice(_all_finite_f16()[1000:30000], 1500)
    for b in base:
        a = Fraction(float(b))
        nb = Fraction(float(np.nextafter(b, np.float16(np.inf))))
        mid = (a + nb) / 2
        xs += [float(mid), float(mid + Fraction(1, 2 ** 60) * abs(mid)), float(mid - Fraction(1, 2 ** 60) * abs(mid))]
    for x in xs:
        t = Fraction(x)
        if abs(t) >= 65520:
            continue
        assert float(nm.f16(x)) == _nearest_even_f16(t), x


# --- OCP E4M3 (8-bit float, 4 exponent bits with bias 7, 3 mantissa bits, no inf, 0x7F NaN)
OCP_E4M3_POINTS = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0,
                   0x3C: 1.5, 0x40: 2.0, 0x7E: 448.0, 0x77: 240.0, 0x80: -0.0, 0xFE: -448.0}


def test_e4m3_decode_spec_points():
    for code, val in OCP_E4M3_POINTS.items():
        assert nm.e4m3_decode(code) == val
    assert np.isnan(nm.e4m3_decode(0x7F)) and np.isnan(nm.e4m3_decode(0xFF))
    vals = nm.e4m3_decode(np.arange(0, 0x7F))
    assert np.all(np.diff(vals) > 0)          # codes 0..0x7E are increasing


def test_e4m3_encode_exhaustive_over_fp16_amax():
    """For every positive finite fp16 amax, the scale byte of amax/6 is the exact nearest
    E4M3 value (ties to even mantissa), saturating at 448."""
    grid = [Fraction(float(v)) for v in nm.e4m3_decode(np.arange(0, 0x7F))]
    amax = _all_finite_f16()
    amax = amax[amax > 0]
    codes = nm.e4m3_encode(amax.astype(np.float64) / 6.0)
    ties = 0
    import bisect
    for a, c in zip(amax, codes):
        t = Fraction(float(a)) / 6
        if t >= 448:
            assert c == 0x7E
            continue
        k = bisect.bisect_left(grid, t)
        cands = [i for i in (k - 1, k, k + 1) if 0 <= i < len(grid)]
        best = min(abs(grid[i] - t) for i in cands)
        tied = [i for i in cands if abs(grid[i] - t) == best]
        if len(tied) > 1:
            ties += 1
            tied = [i for i in tied if i % 2 == 0]
        assert c == tied[0], (float(a), c, tied)
    assert ties > 0                        # the exhaustive sweep does contain exact ties


def test_e4m3_cast_exhaustive_over_fp16():
    """Every finite fp16 value cast to E4M3 (the FP8 cache format): the magnitude byte is the
    exact nearest E4M3 value (ties to the even code), saturating at 448; the sign bit is
    the sign bit of x, -0 included."""
    import bisect
    grid = [Fraction(float(v)) for v in nm.e4m3_decode(np.arange(0, 0x7F))]
    x = _all_finite_f16()
    codes = nm.e4m3_cast(x)
    ties = 0
    for xv, c in zip(x, codes):
        assert (c >> 7) == int(np.signbit(xv))
        t = abs(Fraction(float(xv)))
        mag = c & 0x7F
        if t >= 448:
            assert mag == 0x7E
            continue
        k = bisect.bisect_left(grid, t)
        cands = [i for i in (k - 1, k, k + 1) if 0 <= i < len(grid)]
        best = min(abs(grid[i] - t) for i in cands)
        tied = [i for i in cands if abs(grid[i] - t) == best]
        if len(tied) > 1:
            ties += 1
            tied = [i for i in tied if i % 2 == 0]
        assert mag == tied[0], (float(xv), hex(c), tied)
    assert ties > 0


def test_e4m3_cast_round_trips_every_e4m3_value():
    """Casting the fp16 form of each finite E4M3 value returns its code (0x80 = -0 included)."""
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = nm.e4m3_decode(codes).astype(np.float16)
    np.testing.assert_array_equal(nm.e4m3_cast(vals), codes)


def test_e2m1_encode_exhaustive_brute_force():
    """All finite fp16 x against all 126 positive finite E4M3 scales: the oracle's
    midpoint comparison equals a brute-force nearest-magnitude search (exact float64
    distances), ties to the even code, sign bit kept, |x|/s clipped at 6."""
    xs = _all_finite_f16()
    mags = np.asarray(nm.E2M1_MAGNITUDES)
    for sb in range(1, 0x7F):
        s = float(nm.e4m3_decode(sb))
        codes = nm.e2m1_encode(xs, s)
        a = np.abs(xs.astype(np.float64))
        dist = np.abs(a[:, None] - mags[None, :] * s)           # exact in float64
        best = dist.min(axis=1, keepdims=True)
        tied = dist == best
        # lowest even index among the tied ones, else the single nearest
        even_tied = tied & (np.arange(8)[None, :] % 2 == 0)
        idx = np.where(tied.sum(axis=1) > 1, np.argmax(even_tied, axis=1), np.argmax(tied, axis=1))
        expect = idx + 8 * np.signbit(xs).astype(np.int64)
        assert np.array_equal(codes.astype(np.int64), expect), sb


def test_e2m1_zero_scale_and_signed_zero():
    x = np.array([0.0, -0.0, 1.0, -3.0], np.float16)
    assert list(nm.e2m1_encode(x, 0.0)) == [0, 8, 0, 8]
    assert list(nm.e2m1_encode(np.array([-0.0, -0.1], np.float16), 1.0)) == [8, 8]


def test_e2m1_decode_exact_products_fit_fp16():
    """Every E2M1 magnitude times every positive E4M3 scale is exactly representable in fp16."""
    s = nm.e4m3_decode(np.arange(1, 0x7F))
    prod = np.asarray(nm.E2M1_MAGNITUDES)[None, :] * s[:, None]
    assert np.array_equal(prod.astype(np.float16).astype(np.float64), prod)
