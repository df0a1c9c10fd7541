"""Round-to-nearest-even of an exact scaled integer (test oracle).

The exact sum of binary16 inputs is an integer Q times 2^-24.  Rounding it once
to a binary floating-point format follows the IEEE 754 definition directly:
keep the ``precision`` leading significant bits (fewer below the format's
smallest normal exponent), and if the dropped part is more than half a unit in
the last kept place round up, if exactly half round to the even neighbour.
"""
from __future__ import annotations

import math

import numpy as np


def round_scaled_int(q: int, scale_exp: int, precision: int, emin: int, emax: int) -> float:
    """Nearest-even value of ``q * 2**scale_exp`` in a binary format with
    ``precision`` significand bits and normal exponents ``emin..emax``.

    Returns an exactly representable Python float (+-inf on overflow).  An
    exact zero returns +0.0.
    """
    if q == 0:
        return 0.0
    negative = q < 0
    m = -q if negative else q
    e = scale_exp
    lead = e + m.bit_length() - 1          # exponent of the leading bit
    quantum = max(lead, emin) - (precision - 1)
    drop = quantum - e
    if drop > 0:
        kept = m >> drop
        rest = m - (kept << drop)
        half = 1 << (drop - 1)
        if rest > half or (rest == half and (kept & 1)):
            kept += 1
        m, e = kept, quantum
    if e + m.bit_length() - 1 > emax:
        return -math.inf if negative else math.inf
    v = math.ldexp(m, e)
    return -v if negative else v


def to_binary32(q: int, scale_exp: int = -24) -> np.float32:
    return np.float32(round_scaled_int(q, scale_exp, 24, -126, 127))


def to_binary64(q: int, scale_exp: int = -24) -> float:
    return round_scaled_int(q, scale_exp, 53, -1022, 1023)
