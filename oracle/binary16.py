"""binary16 decoding written out from the IEEE 754 definition (test oracle).

A binary16 pattern has sign s (bit 15), biased exponent e (bits 10..14) and
fraction f (bits 0..9).  Every finite value is an integer multiple of 2^-24:

* e == 0 (zero or subnormal):  value = f * 2^-24
* 1 <= e <= 30 (normal):       value = (1024 + f) * 2^(e - 25)
                                     = ((1024 + f) << (e - 1)) * 2^-24
* e == 31:                     infinity (f == 0) or NaN (f != 0)

so a finite value is exactly q * 2^-24 with |q| <= 65504 * 2^24 < 2^40.
"""
from __future__ import annotations

import numpy as np

BINARY16_QUANTUM_EXP = -24

CLASS_FINITE = 0
CLASS_POS_INF = 1
CLASS_NEG_INF = 2
CLASS_NAN = 3


def decode_bits(h: int) -> tuple[int, int]:
    """(q, class) for one 16-bit pattern; q counts 2^-24 and is 0 unless finite."""
    s = (h >> 15) & 1
    e = (h >> 10) & 0x1F
    f = h & 0x3FF
    if e == 31:
        if f != 0:
            return 0, CLASS_NAN
        return 0, (CLASS_NEG_INF if s else CLASS_POS_INF)
    q = f if e == 0 else (1024 + f) << (e - 1)
    return (-q if s else q), CLASS_FINITE


_TABLE: tuple[np.ndarray, np.ndarray] | None = None


def decode_table() -> tuple[np.ndarray, np.ndarray]:
    """(q, class) for all 65536 patterns, indexed by the pattern, as int64/int8."""
    global _TABLE
    if _TABLE is None:
        q = np.zeros(65536, dtype=np.int64)
        c = np.zeros(65536, dtype=np.int8)
        for h in range(65536):
            q[h], c[h] = decode_bits(h)
        q.setflags(write=False)
        c.setflags(write=False)
        _TABLE = (q, c)
    return _TABLE
