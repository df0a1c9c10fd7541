"""Pins the exact-sum oracle: brute force with rationals, math.fsum, closed
forms and IEEE special values.  The operation is the arithmetic reduction of n
numbers of "GPU Tensor Cores for fast Arithmetic Reductions" (arXiv
2001.05585, Abstract)."""
import math
from fractions import Fraction

import numpy as np
import pytest

import synth_inputs as si
from oracle import exact_row_sums, exact_sum, exact_sum_of_parts


def _brute(x16):
    return sum((Fraction(float(v)) for v in x16.astype(np.float64)), Fraction(0))


@pytest.mark.parametrize("n", [1, 2, 3, 255, 256, 257, 511, 512, 513, 1000, 4096])
def test_exact_matches_rational_brute_force(n):
    x = si.generate("bits_finite", n, seed=100 + n)
    e = exact_sum(x)
    ref = _brute(x)
    assert Fraction(e.q, 1 << 24) == ref
    assert e.f64 == float(ref)                      # correctly rounded binary64
    assert Fraction(e.a, 1 << 24) == sum(abs(Fraction(float(v))) for v in x.astype(np.float64))


@pytest.mark.parametrize("dist,n,seed", [
    ("bits_finite", 1 << 16, 1), ("uniform11", 1 << 20, 2), ("normal", 300_001, 3),
    ("logu_signed", 1 << 18, 4),
])
def test_exact_f64_matches_fsum(dist, n, seed):
    x = si.generate(dist, n, seed)
    assert exact_sum(x).f64 == math.fsum(x.astype(np.float64).tolist())


def test_closed_form_ones_and_alternating():
    for n in (1, 7, 4096, (1 << 22) + 5):
        assert exact_sum(si.generate("ones", n)).q == n << 24
        assert exact_sum(si.generate("ones", n)).f32 == np.float32(n)
        alt = exact_sum(si.generate("alternating", n))
        assert alt.q == (n % 2) << 24
        assert alt.a == n << 24


def test_closed_form_ramp():
    # x_i = i mod 2048 (integers up to 2047 are exact in binary16); every full
    # period sums to 2047 * 2048 / 2 = 2,096,128
    n = 1 << 20
    assert exact_sum(si.generate("ramp2048", n)).q == (n // 2048) * 2_096_128 << 24
    assert exact_sum(si.generate("ramp2048", n)).f32 == np.float32(1_073_217_536)
    n2 = 5000   # two full periods and 904 more: 2*2096128 + 903*904/2
    assert exact_sum(si.generate("ramp2048", n2)).q == (2 * 2_096_128 + 903 * 904 // 2) << 24


def test_closed_form_all_binary16_values():
    pos = np.arange(0x0001, 0x7C00, dtype=np.uint16).view(np.float16)
    # subnormals: 2^-24 * (1 + ... + 1023) = 523776 * 2^-24
    # normals:   sum_{e=1..30} sum_{f} (1024 + f) 2^(e-25) = 1572352 * (64 - 2^-24)
    # total = 100630528 - 1048576 * 2^-24 = 100630527.9375
    e = exact_sum(pos)
    assert e.f64 == 100630527.9375
    assert Fraction(e.q, 1 << 24) == Fraction(1572352 * 64) - Fraction(1572352 - 523776, 1 << 24)
    neg = np.arange(0x8001, 0xFC00, dtype=np.uint16).view(np.float16)
    assert exact_sum(neg).f64 == -100630527.9375
    every_finite = np.concatenate([pos, neg, np.array([0, 0x8000], np.uint16).view(np.float16)])
    z = exact_sum(every_finite)
    assert z.q == 0 and z.f32 == 0 and not np.signbit(z.f32)


def test_specials_follow_ieee_addition():
    inf, nan = np.float16(np.inf), np.float16(np.nan)
    one = np.float16(1)
    assert math.isnan(exact_sum(np.array([one, nan, one], np.float16)).f64)
    assert exact_sum(np.array([one, inf, one], np.float16)).f32 == np.inf
    assert exact_sum(np.array([one, -inf], np.float16)).f32 == -np.inf
    assert np.isnan(exact_sum(np.array([inf, one, -inf], np.float16)).f32)
    assert exact_sum(np.array([], np.float16)).f32 == 0


@pytest.mark.parametrize("cuts", [[0, 1000, 1000, 5000, 65536], [0, 7, 65536], [0, 65536]])
def test_exact_sum_of_parts_equals_whole(cuts):
    x = si.generate("bits_finite", 65536, seed=len(cuts))
    parts = [exact_sum(x[a:b]) for a, b in zip(cuts[:-1], cuts[1:])]
    whole, joined = exact_sum(x), exact_sum_of_parts(parts)
    assert (joined.q, joined.a, joined.n, joined.special) == (whole.q, whole.a, whole.n, None)
    # non-finite parts combine by the IEEE rules of one sum
    inf, one = np.float16(np.inf), np.float16(1)
    p_inf = exact_sum(np.array([one, inf], np.float16))
    p_ninf = exact_sum(np.array([-inf], np.float16))
    p_nan = exact_sum(np.array([np.float16(np.nan)], np.float16))
    assert exact_sum_of_parts([parts[0], p_inf]).f32 == np.inf
    assert np.isnan(exact_sum_of_parts([p_inf, parts[0], p_ninf]).f32)
    assert np.isnan(exact_sum_of_parts([p_nan, parts[0]]).f32)
    assert exact_sum_of_parts([]).f32 == 0


def test_f32_worked_ties():
    # exact 1 + 3*2^-24 is a tie between 1 + 2^-23 and 1 + 2^-22 -> even
    x = np.array([1, 2.0 ** -24, 2.0 ** -24, 2.0 ** -24], np.float16)
    assert exact_sum(x).f32 == np.float32(1 + 2.0 ** -22)
    # 1024 copies of 65504 = (2^11 - 1) * 2^15 exactly, 11 significant bits
    assert exact_sum(np.full(1024, 65504, np.float16)).f32 == np.float32(67_076_096)
    # 4097 ones and one 2^-24 -> 4097: the 2^-24 is far below half an ulp
    x = np.concatenate([np.ones(4097, np.float16), np.array([2.0 ** -24], np.float16)])
    assert exact_sum(x).f32 == np.float32(4097)
    # 2^24 + 1 is a tie between 2^24 and 2^24 + 2 -> even 2^24; +3 rounds to 2^24 + 4
    y = np.full((1 << 24) + 1, 1, np.float16)
    assert exact_sum(y).f32 == np.float32(1 << 24)
    y3 = np.full((1 << 24) + 3, 1, np.float16)
    assert exact_sum(y3).f32 == np.float32((1 << 24) + 4)


def test_row_sums_match_brute_force_and_flat_sums():
    x = si.generate_rows("bits_finite", 37, 129, seed=9)
    rs = exact_row_sums(x)
    assert len(rs) == 37
    for r in range(37):
        assert Fraction(rs[r].q, 1 << 24) == _brute(x[r])
        assert rs[r].q == exact_sum(x[r]).q
    # rows of ramp values: row r covers flat indices r*cols .. r*cols+cols-1
    y = si.generate_rows("ramp2048", 4, 2048)
    assert all(e.q == 2_096_128 << 24 for e in exact_row_sums(y))


def test_row_sums_specials_per_row():
    x = np.ones((3, 5), np.float16)
    x[1, 2] = np.inf
    x[2, 0] = np.nan
    rs = exact_row_sums(x)
    assert rs[0].f32 == 5 and rs[1].f32 == np.inf and np.isnan(rs[2].f32)
