"""The digit identity behind reduce_sum_exact's integer-limb form, over every
finite binary16 pattern (host arithmetic only).

"AWE: Adaptive Weight Encoding for Exact Integer Matrix Products with Fewer
GEMMs on FP4 Tensor Cores", Abstract: an integer is carried as narrow limbs
with fixed weights and recovered exactly from them.  The kernel writes a
value's count q of 2^-24 (|q| < 2^40) as g = |q| xor (all ones if negative),
i.e. q or q - 1 in two's complement, and hands the eight bytes of g, each
with its top bit flipped, to an int8 MFMA as signed digits d_m = g_m - 128.
It recombines positions 0-4 with weights 2^(8m), adds 0x8080808080 per
value, and (1 - 2^40) per negative value, whose count it takes from the sum
of digit 7 (127 for a negative value, -128 otherwise).  The expected q comes
from numpy's own float16 decoding, not from these formulas.
"""
import numpy as np

C40 = 0x8080808080


def _digits(h):
    """The kernel's digit word for each 16-bit pattern in h, as eight int64
    digit arrays (position 0 first)."""
    h = h.astype(np.uint64)
    e = (h >> np.uint64(10)) & np.uint64(31)
    mn = np.minimum(e, np.uint64(1))
    m = (mn << np.uint64(10)) | (h & np.uint64(1023))
    mag = m << (e - mn)
    sign = np.where(h & np.uint64(0x8000), np.uint64(0xFFFFFFFF), np.uint64(0))
    k = sign ^ np.uint64(0x80808080)
    z = mag ^ ((k << np.uint64(32)) | k)
    return [((((z >> np.uint64(8 * i)) & np.uint64(0xFF)).astype(np.int64)) ^ 0x80) - 0x80
            for i in range(8)]


def _finite_patterns():
    h = np.arange(1 << 16, dtype=np.uint32)
    return h[((h >> 10) & 31) != 31]


def test_every_finite_value_from_its_digits():
    h = _finite_patterns()
    assert len(h) == 63488
    q = h.astype(np.uint16).view(np.float16).astype(np.float64) * 2.0 ** 24
    assert np.all(q == np.round(q)) and np.all(np.abs(q) < 2.0 ** 40)
    d = _digits(h)
    for m in range(8):
        assert d[m].min() >= -128 and d[m].max() <= 127
    neg = (h & 0x8000) != 0
    low = sum(d[m] * (1 << (8 * m)) for m in range(5))
    got = low + C40 + np.where(neg, 1 - (1 << 40), 0)
    assert np.array_equal(got.astype(np.float64), q)
    for m in (5, 6, 7):
        assert np.array_equal(d[m], np.where(neg, 127, -128))


def test_sums_and_negative_count_from_digit_planes():
    rng = np.random.default_rng(7)
    h = _finite_patterns()
    for size in (1, 8, 4096, 200000):
        pick = rng.choice(h, size=size)
        pick = np.concatenate([pick, np.zeros(size % 7, np.uint32)])   # padding zeros count too
        n = len(pick)
        d = _digits(pick)
        D = [int(x.sum()) for x in d]
        neg, rem = divmod(D[7] + 128 * n, 255)
        assert rem == 0 and neg == int(((pick & 0x8000) != 0).sum())
        total = sum(D[m] << (8 * m) for m in range(5)) + n * C40 + neg * (1 - (1 << 40))
        want = sum(int(v) for v in
                   (pick.astype(np.uint16).view(np.float16).astype(np.float64) * 2.0 ** 24))
        assert total == want
