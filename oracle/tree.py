"""Fixed balanced-tree summation order (test oracle).

[TBB] (Taming Bitwise Behavior in GPU Kernels with Tensor Core, Abstract)
names reduction order as the main reason two deterministic kernels differ bit
for bit, with partial-sum precision, fused multiply-add and rounding placement
next, and makes results reproducible by enforcing a balanced-tree reduction.
[TCR] (GPU Tensor Cores for fast Arithmetic Reductions, Abstract) keeps
partial results as 32-bit floats.  The order prescribed here is:

* leaves: x_i widened to binary32 (exact for every binary16, subnormals too);
* the leaves are padded to N = 2^ceil(log2 n) with -0.0.  -0.0 is the exact
  identity of round-to-nearest-even addition (x + -0.0 == x for every x,
  including +0.0), so padding is the same as letting a node with no right
  child pass its left child up unchanged;
* the node over [a, a + 2s) is the binary32 round-to-nearest-even sum of the
  nodes over [a, a + s) and [a + s, a + 2s), level by level from the leaves;
* the result is the root; n == 0 gives +0.0.

Groups of 256 consecutive leaves are complete depth-8 subtrees of this tree,
which is what makes "256-element leaf tiles" a unit of work that does not
change the arithmetic.  Only additions occur, no multiply-add, and numpy
float32 addition is IEEE binary32 addition rounded to nearest even.
"""
from __future__ import annotations

import numpy as np


def _pad_pow2(level: np.ndarray, axis_len: int) -> np.ndarray:
    size = 1 << (axis_len - 1).bit_length()
    if size == axis_len:
        return level
    pad_shape = level.shape[:-1] + (size - axis_len,)
    return np.concatenate([level, np.full(pad_shape, -0.0, dtype=np.float32)], axis=-1)


def fixed_tree_sum(x: np.ndarray) -> np.float32:
    """Balanced-tree binary32 sum of a 1-D binary16 array."""
    if x.dtype != np.float16:
        raise TypeError("fixed_tree_sum expects a binary16 (float16) array")
    x = x.reshape(-1)
    n = x.size
    if n == 0:
        return np.float32(0.0)
    level = _pad_pow2(x.astype(np.float32), n)
    with np.errstate(invalid="ignore", over="ignore"):   # Inf - Inf -> NaN is intended
        while level.size > 1:
            level = level[0::2] + level[1::2]
    return level[0]


def fixed_tree_row_sums(x: np.ndarray) -> np.ndarray:
    """The same tree applied to every row of a 2-D binary16 array."""
    if x.ndim != 2 or x.dtype != np.float16:
        raise TypeError("fixed_tree_row_sums expects a 2-D binary16 array")
    rows, cols = x.shape
    if cols == 0:
        return np.zeros(rows, dtype=np.float32)
    level = _pad_pow2(x.astype(np.float32), cols)
    with np.errstate(invalid="ignore", over="ignore"):
        while level.shape[1] > 1:
            level = level[:, 0::2] + level[:, 1::2]
    return np.ascontiguousarray(level[:, 0])
