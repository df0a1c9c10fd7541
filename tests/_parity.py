"""Shared helpers for the GPU parity tests."""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np
import pytest

REL = 1e-5   # free-order gate: relative error against the exact sum


def require_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device (run them on an MI355X)")


def to_dev(x: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda")


def bits32(v) -> int:
    return int(np.asarray(v, dtype=np.float32).reshape(()).view(np.uint32))


def free_order_scale(e) -> float:
    """max(|S|, sum|x| / sqrt(n)): the relative gate, falling back to a
    normwise one when the exact sum nearly cancels."""
    n = max(e.n, 1)
    return max(abs(e.f64), e.abs_sum / math.sqrt(n))


def check_free_order(got: float, e, what: str = "") -> float:
    """Asserts the free-order gate; returns the pure relative error (or 0)."""
    if e.special == "nan":
        assert math.isnan(got), (what, got)
        return 0.0
    if e.special in ("+inf", "-inf"):
        assert got == (math.inf if e.special == "+inf" else -math.inf), (what, got)
        return 0.0
    err = abs(Fraction(got) - Fraction(e.q, 1 << 24))
    assert float(err) <= REL * free_order_scale(e), (what, got, e.f64, float(err))
    return float(err) / abs(e.f64) if e.f64 else 0.0


NAN16 = np.uint16(0x7E00)
INF16 = np.uint16(0x7C00)


def strided(x, ld, junk=NAN16, tail=64):
    """Device view of x with row pitch ld, built in a flat buffer of exactly
    (rows - 1) * ld + cols values plus `tail` more; every value that is not
    part of a row (the padding of each pitch and the tail) holds `junk`."""
    import torch
    rows, cols = x.shape
    size = (rows - 1) * ld + cols if rows else 0
    flat = np.full(size + tail, junk, np.uint16)
    for r in range(rows):
        flat[r * ld:r * ld + cols] = x[r].view(np.uint16)
    buf = torch.from_numpy(flat.view(np.float16)).to("cuda")
    return torch.as_strided(buf, (rows, cols), (ld, 1))
