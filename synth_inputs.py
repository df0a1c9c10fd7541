"""Seeded synthetic fp16 inputs for the sum-reduction tests and benchmark.

This module only makes data.  It holds no summation, no rounding of sums and
no other arithmetic of the reduction method, so that the CPU oracle and the
GPU library can both be fed from it without sharing any of the method's code.

Counter-based generation
------------------------
Element ``i`` of a buffer made with seed ``s`` is a pure function of ``(s, i)``:
its 64 random bits are the ``i``-th output of the SplitMix64 generator started
at state ``s`` (Steele, Lea and Flood, "Fast splittable pseudorandom number
generators", OOPSLA 2014; the finaliser below is the mix64 variant with shifts
30/27/31 and the two published odd multipliers).  Because nothing depends on
the order of generation, a buffer is identical whether it is made in one piece
or in chunks on many threads.

The pages define no data set; every workload here is synthetic.  Each
distribution maps the 64 bits to a float64, then rounds once to binary16 with
round-to-nearest-even (numpy's ``astype(np.float16)``).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_MUL1 = np.uint64(0xBF58476D1CE4E5B9)
_MUL2 = np.uint64(0x94D049BB133111EB)
_CHUNK = 1 << 22

DISTRIBUTIONS = (
    "uniform01",     # uniform on [0, 1)
    "uniform11",     # uniform on [-1, 1)
    "normal",        # standard normal (Box-Muller)
    "logu_signed",   # random sign, magnitude log-uniform on [2^-14, 2^8]
    "ones",          # every element 1.0
    "alternating",   # +1, -1, +1, ...
    "ramp2048",      # element i is (i mod 2048), exact in binary16
    "bits_finite",   # uniformly random binary16 bit patterns, Inf/NaN excluded
)


def splitmix64(seed: int, start: int, count: int) -> np.ndarray:
    """Outputs ``start .. start+count-1`` of SplitMix64 seeded with ``seed``.

    Output ``i`` is mix64(seed + (i + 1) * gamma), computed mod 2**64.
    """
    z = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    z *= _GAMMA
    z += np.uint64(seed & 0xFFFFFFFFFFFFFFFF)
    z ^= z >> np.uint64(30)
    z *= _MUL1
    z ^= z >> np.uint64(27)
    z *= _MUL2
    z ^= z >> np.uint64(31)
    return z


def _unit53(bits: np.ndarray) -> np.ndarray:
    """Top 53 bits as a float64 in [0, 1)."""
    return (bits >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


def _to_half_below(v: np.ndarray, hi: float) -> np.ndarray:
    """Round to binary16; a value that rounds up to ``hi`` becomes the next
    binary16 below ``hi`` so the half-open interval stays half-open."""
    h = v.astype(np.float16)
    top = np.float16(hi)
    if np.isfinite(top):
        mask = h >= top
        if mask.any():
            h[mask] = np.nextafter(top, np.float16(-np.inf))
    return h


def _chunk(dist: str, seed: int, start: int, count: int) -> np.ndarray:
    if dist == "ones":
        return np.ones(count, dtype=np.float16)
    if dist == "alternating":
        idx = np.arange(start, start + count, dtype=np.int64)
        return np.where(idx % 2 == 0, 1.0, -1.0).astype(np.float16)
    if dist == "ramp2048":
        idx = np.arange(start, start + count, dtype=np.int64)
        return (idx % 2048).astype(np.float16)
    bits = splitmix64(seed, start, count)
    if dist == "uniform01":
        return _to_half_below(_unit53(bits), 1.0)
    if dist == "uniform11":
        return _to_half_below(-1.0 + 2.0 * _unit53(bits), 1.0)
    if dist == "normal":
        # Box-Muller with the two 32-bit halves of one draw:
        # u1 in (0, 1] from the high half, u2 in [0, 1) from the low half.
        u1 = ((bits >> np.uint64(32)).astype(np.float64) + 1.0) * (2.0 ** -32)
        u2 = (bits & np.uint64(0xFFFFFFFF)).astype(np.float64) * (2.0 ** -32)
        return (np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * np.pi * u2)).astype(np.float16)
    if dist == "logu_signed":
        # sign from bit 0, exponent uniform on [-14, 8) from bits 11..63
        mag = np.exp2(-14.0 + 22.0 * _unit53(bits))
        sign = np.where((bits & np.uint64(1)) == 1, -1.0, 1.0)
        return (sign * mag).astype(np.float16)
    if dist == "bits_finite":
        h = (bits >> np.uint64(24)).astype(np.uint16)
        # an all-ones exponent field (Inf/NaN) has bit 14 cleared, which
        # turns it into the finite exponent 15
        special = (h & np.uint16(0x7C00)) == np.uint16(0x7C00)
        h[special] &= np.uint16(0xBFFF)
        return h.view(np.float16)
    raise ValueError(f"unknown distribution {dist!r}; known: {DISTRIBUTIONS}")


def _threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n))


def generate(dist: str, n: int, seed: int = 0, *, threads: int | None = None) -> np.ndarray:
    """A binary16 array of ``n`` elements drawn from ``dist`` with ``seed``.

    The result does not depend on ``threads``; it only sets how many chunks
    are made at once.
    """
    if n < 0:
        raise ValueError("n must be non-negative")
    out = np.empty(n, dtype=np.float16)
    if n == 0:
        return out
    starts = list(range(0, n, _CHUNK))

    def fill(s: int) -> None:
        c = min(_CHUNK, n - s)
        out[s:s + c] = _chunk(dist, seed, s, c)

    workers = threads if threads is not None else _threads()
    if workers <= 1 or len(starts) == 1:
        for s in starts:
            fill(s)
    else:
        with ThreadPoolExecutor(max_workers=workers) as pool:
            list(pool.map(fill, starts))
    return out


def generate_rows(dist: str, rows: int, cols: int, seed: int = 0, **kw) -> np.ndarray:
    """Row-major ``rows x cols`` binary16 matrix; element (r, c) is element
    ``r * cols + c`` of the flat stream."""
    return generate(dist, rows * cols, seed, **kw).reshape(rows, cols)


# Workloads by name: (kind, shape, distribution, seed).  Seeds are fixed so
# every run and every machine sees the same bytes.
WORKLOADS = {
    "sum_2p20_u01": ("sum", (1 << 20,), "uniform01", 1),
    "sum_2p28_u11": ("sum", (1 << 28,), "uniform11", 2),
    "rows_4096x65536_normal": ("rows", (4096, 65536), "normal", 3),
    "sum_2p30_logu": ("sum", (1 << 30,), "logu_signed", 4),
    "fixed_2p26_u11": ("fixed", (1 << 26,), "uniform11", 5),
}


def workload(name: str, **kw) -> np.ndarray:
    kind, shape, dist, seed = WORKLOADS[name]
    if kind == "rows":
        return generate_rows(dist, shape[0], shape[1], seed, **kw)
    return generate(dist, shape[0], seed, **kw)
