"""Pins the once-rounding of exact sums to binary64 / binary32."""
import math
import random
from fractions import Fraction

import numpy as np
import pytest

from oracle import round_scaled_int, to_binary32, to_binary64


def _cases(seed=7, count=4000):
    rng = random.Random(seed)
    out = [0, 1, -1, 3, (1 << 24) + 1, (1 << 53) + 1, (1 << 53) + 3, -(1 << 60) - 12345]
    for _ in range(count):
        bits = rng.choice([8, 20, 30, 40, 54, 60, 70, 90])
        v = rng.getrandbits(bits)
        out.append(-v if rng.random() < 0.5 else v)
    return out


def test_binary64_matches_fraction_to_float():
    # Python's Fraction -> float conversion is correctly rounded (nearest-even)
    for q in _cases():
        assert to_binary64(q) == float(Fraction(q, 1 << 24)), q


def test_binary32_equals_numpy_single_rounding_when_double_is_exact():
    # when q * 2^-24 is exact in float64, numpy's float64 -> float32 cast is the
    # only rounding, so it must agree bit for bit
    for q in _cases():
        if abs(q) < (1 << 53):
            assert to_binary32(q).view(np.uint32) == np.float32(q * 2.0 ** -24).view(np.uint32), q


def test_binary32_is_nearest_with_ties_to_even():
    for q in _cases(seed=11):
        exact = Fraction(q, 1 << 24)
        r = to_binary32(q)
        assert np.isfinite(r)
        lo = np.nextafter(r, np.float32(-np.inf))
        hi = np.nextafter(r, np.float32(np.inf))
        d = abs(Fraction(float(r)) - exact)
        for nb in (lo, hi):
            dn = abs(Fraction(float(nb)) - exact)
            assert d <= dn, q
            if d == dn and d != 0:
                assert int(r.view(np.uint32)) % 2 == 0, ("tie must go to even", q)


@pytest.mark.parametrize("q,expect", [
    ((1 << 24) + 1, 1.0),                        # 1 + 2^-24: tie -> 1
    ((1 << 24) + 3, 1.0 + 2.0 ** -22),           # 1 + 3*2^-24: tie -> even 1 + 2^-22
    ((1 << 24) + 2, 1.0 + 2.0 ** -23),           # exact
    ((1 << 25) + 3, 2.0 + 2.0 ** -22),           # 2 + 3*2^-24 is 0.75 ulp: rounds up
    (-(1 << 24) - 1, -1.0),
])
def test_binary32_hand_cases(q, expect):
    assert to_binary32(q) == np.float32(expect)


def test_binary32_overflow_and_subnormal_formats():
    assert math.isinf(round_scaled_int(1, 128, 24, -126, 127))
    # largest finite binary32 stays finite; half an ulp above rounds to inf
    big = ((1 << 24) - 1) << 104
    assert round_scaled_int(big, 0, 24, -126, 127) == float(np.finfo(np.float32).max)
    assert math.isinf(round_scaled_int((big << 1) + (1 << 104), -1, 24, -126, 127))
    # subnormal range of binary32 rounds on the fixed 2^-149 grid
    assert round_scaled_int(3, -150, 24, -126, 127) == 2.0 ** -148   # 1.5 * 2^-149 ties to even
