"""Pins the oracle's binary16 decode against numpy's own float16 conversion."""
import numpy as np

from oracle import decode_table
from oracle.binary16 import CLASS_FINITE, CLASS_NAN, CLASS_NEG_INF, CLASS_POS_INF


def test_decode_matches_numpy_for_every_pattern():
    q, cls = decode_table()
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = pats.view(np.float16).astype(np.float64)   # library conversion, exact
    finite = np.isfinite(ref)
    assert np.array_equal(cls == CLASS_FINITE, finite)
    # q * 2^-24 is exact in float64 (|q| < 2^40)
    assert np.array_equal(q[finite].astype(np.float64) * 2.0 ** -24, ref[finite])
    # signed zeros both decode to 0
    assert q[0x0000] == 0 and q[0x8000] == 0


def test_decode_classes_of_specials():
    q, cls = decode_table()
    assert cls[0x7C00] == CLASS_POS_INF and cls[0xFC00] == CLASS_NEG_INF
    assert cls[0x7E00] == CLASS_NAN and cls[0xFE01] == CLASS_NAN
    assert int((cls == CLASS_NAN).sum()) == 2 * 1023
    assert q[0x7C00] == 0


def test_decode_extremes():
    q, _ = decode_table()
    assert q[0x0001] == 1                    # smallest subnormal 2^-24
    assert q[0x03FF] == 1023                 # largest subnormal
    assert q[0x0400] == 1024                 # smallest normal 2^-14
    assert q[0x3C00] == 1 << 24              # 1.0
    assert q[0x7BFF] == 65504 * (1 << 24)    # largest finite
    assert q[0xFBFF] == -65504 * (1 << 24)
