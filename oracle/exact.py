"""Exact sum of binary16 inputs (test oracle).

[TCR] (GPU Tensor Cores for fast Arithmetic Reductions, Abstract) defines the
operation as the arithmetic reduction of n numbers, with a 32-bit float final
result.  The plain definition of that result is the real sum S = sum_i x_i.
Each finite binary16 input is q_i * 2^-24 for an integer q_i, so S is held
exactly as the integer Q = sum_i q_i, accumulated in int64 over chunks small
enough that no chunk can overflow (2^22 terms of magnitude < 2^40) and then in
Python's unbounded int.  Integer addition is associative, so the order of this
loop is irrelevant.  S is rounded once to binary32 or binary64.

Non-finite inputs follow IEEE 754 addition: any NaN, or +Inf together with
-Inf, gives NaN; otherwise an infinity of either sign gives that infinity.
An exact zero is reported as +0.0.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

from .binary16 import CLASS_NAN, CLASS_NEG_INF, CLASS_POS_INF, decode_table
from .rounding import to_binary32, to_binary64

_CHUNK = 1 << 22


@dataclass(frozen=True)
class ExactSum:
    """Exact sum of n binary16 values: Q * 2^-24, plus sum |x_i| = A * 2^-24."""

    q: int
    a: int
    n: int
    special: str | None = None   # None, "nan", "+inf" or "-inf"

    @property
    def f32(self) -> np.float32:
        if self.special == "nan":
            return np.float32(np.nan)
        if self.special == "+inf":
            return np.float32(np.inf)
        if self.special == "-inf":
            return np.float32(-np.inf)
        return to_binary32(self.q)

    @property
    def f64(self) -> float:
        if self.special == "nan":
            return math.nan
        if self.special == "+inf":
            return math.inf
        if self.special == "-inf":
            return -math.inf
        return to_binary64(self.q)

    @property
    def abs_sum(self) -> float:
        """sum_i |x_i| over the finite inputs, rounded once to binary64."""
        return to_binary64(self.a)


def _special(n_nan: int, n_pinf: int, n_ninf: int) -> str | None:
    if n_nan or (n_pinf and n_ninf):
        return "nan"
    if n_pinf:
        return "+inf"
    if n_ninf:
        return "-inf"
    return None


def exact_sum(x: np.ndarray) -> ExactSum:
    """Exact sum of a 1-D binary16 array."""
    x = np.ascontiguousarray(x)
    if x.dtype != np.float16:
        raise TypeError("exact_sum expects a binary16 (float16) array")
    bits = x.reshape(-1).view(np.uint16)
    qtab, ctab = decode_table()
    total = 0
    total_abs = 0
    n_nan = n_pinf = n_ninf = 0
    for s in range(0, bits.size, _CHUNK):
        b = bits[s:s + _CHUNK]
        q = qtab[b]
        total += int(q.sum())
        total_abs += int(np.abs(q).sum())
        cls = ctab[b]
        if cls.any():
            n_nan += int((cls == CLASS_NAN).sum())
            n_pinf += int((cls == CLASS_POS_INF).sum())
            n_ninf += int((cls == CLASS_NEG_INF).sum())
    return ExactSum(total, total_abs, int(bits.size), _special(n_nan, n_pinf, n_ninf))


def exact_sum_of_parts(parts: list[ExactSum]) -> ExactSum:
    """The exact sum of a concatenation, from the exact sums of its parts:
    the integers add (integer addition is associative), and the non-finite
    cases follow the same IEEE rules as within one part."""
    parts = list(parts)
    specials = {p.special for p in parts}
    n_nan = int("nan" in specials)
    return ExactSum(sum(p.q for p in parts), sum(p.a for p in parts), sum(p.n for p in parts),
                    _special(n_nan, int("+inf" in specials), int("-inf" in specials)))


def exact_row_sums(x: np.ndarray) -> list[ExactSum]:
    """Exact sum of every row of a 2-D binary16 array (row r: sum_c x[r, c])."""
    if x.ndim != 2 or x.dtype != np.float16:
        raise TypeError("exact_row_sums expects a 2-D binary16 array")
    rows, cols = x.shape
    qtab, ctab = decode_table()
    out: list[ExactSum] = []
    # columns are split into pieces of at most 2^22 so one int64 row-piece sum
    # cannot overflow; the pieces are added as Python ints
    col_step = min(max(cols, 1), _CHUNK)
    row_step = max(1, _CHUNK // col_step)
    for r0 in range(0, rows, row_step):
        r1 = min(rows, r0 + row_step)
        qs = [0] * (r1 - r0)
        qa = [0] * (r1 - r0)
        nan = np.zeros(r1 - r0, dtype=np.int64)
        pinf = np.zeros(r1 - r0, dtype=np.int64)
        ninf = np.zeros(r1 - r0, dtype=np.int64)
        for c0 in range(0, cols, col_step):
            b = np.ascontiguousarray(x[r0:r1, c0:c0 + col_step]).view(np.uint16)
            q = qtab[b]
            piece = q.sum(axis=1)
            piece_abs = np.abs(q).sum(axis=1)
            for i in range(r1 - r0):
                qs[i] += int(piece[i])
                qa[i] += int(piece_abs[i])
            cls = ctab[b]
            if cls.any():
                nan += (cls == CLASS_NAN).sum(axis=1)
                pinf += (cls == CLASS_POS_INF).sum(axis=1)
                ninf += (cls == CLASS_NEG_INF).sum(axis=1)
        for i in range(r1 - r0):
            out.append(ExactSum(qs[i], qa[i], cols,
                                _special(int(nan[i]), int(pinf[i]), int(ninf[i]))))
    return out
