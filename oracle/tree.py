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

from .binary16 import CLASS_FINITE, CLASS_NAN, decode_table
from .mfma_model import columns_from_zero


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


def tree_over_nodes(nodes: np.ndarray) -> np.float32:
    """The same balanced tree over binary32 values that are themselves nodes:
    padded with -0.0 to a power of two, pairs added level by level.  The
    roots of consecutive aligned subtrees of 2^k leaves (the last one
    possibly short, since its -0.0 padding to 2^k changes nothing) are the
    nodes of level k, so this tree over them is the root of the whole tree.
    No values gives +0.0."""
    nodes = np.ascontiguousarray(nodes, dtype=np.float32).reshape(-1)
    if nodes.size == 0:
        return np.float32(0.0)
    return _tree_levels(_pad_pow2(nodes, nodes.size))


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


# ---- fixed order with MFMA leaves ------------------------------------------
#
# A second prescribed order, whose leaves are tensor-core operations: the
# values are cut into chunks of 512 (the last one padded with zeros), each
# chunk is one v_mfma_f32_16x16x32_f16 against an all-ones operand from a zero
# accumulator, and the chunk's node is the balanced tree over that MFMA's 16
# column sums in column order.  Above the chunks it is the balanced tree of
# fixed_tree_sum (padded with -0.0 nodes).  [TBB] (Abstract) names tensor-core
# arithmetic as a source of bit differences and reconstructs it from outputs;
# with that reconstruction (oracle.mfma_model) such an order is reproducible
# and checkable.  Column j of a chunk holds, in K order, the 8 values of each
# of the 16-byte slots j, j + 16, j + 32 and j + 48 (slot s = values 8s ..
# 8s + 7): the B operand each lane supplies from its own load.


def _tree_levels(level: np.ndarray) -> np.ndarray:
    """Balanced tree over the last axis (a power of two long)."""
    with np.errstate(invalid="ignore", over="ignore"):
        while level.shape[-1] > 1:
            level = level[..., 0::2] + level[..., 1::2]
    return level[..., 0]


def mma_leaf_columns(x: np.ndarray) -> np.ndarray:
    """(chunks, 16, 32): each chunk's 16 MFMA columns, K values in K order."""
    x = np.ascontiguousarray(x, dtype=np.float16).reshape(-1)
    chunks = -(-x.size // 512)
    xp = np.zeros(chunks * 512, np.float16)
    xp[:x.size] = x
    # (chunk, slot group q, column j, value e) -> (chunk, column j, K = 8 q + e)
    return xp.reshape(chunks, 4, 16, 8).transpose(0, 2, 1, 3).reshape(chunks, 16, 32)


def mma_column_sums(cols: np.ndarray) -> np.ndarray:
    """Each column's MFMA sum (binary32), non-finite values by IEEE rules:
    NaN if the column holds a NaN or both infinities, else the infinity."""
    flat = cols.reshape(-1, 32)
    bits = flat.view(np.uint16)
    _, cls = decode_table()
    c = cls[bits]
    finite = (c == CLASS_FINITE).all(axis=1)
    out = np.zeros(flat.shape[0], np.float32)
    if finite.any():
        out[finite] = columns_from_zero(flat[finite])
    for i in np.nonzero(~finite)[0]:
        v = flat[i].astype(np.float32)
        has_nan = (c[i] == CLASS_NAN).any()
        pos, neg = (v == np.inf).any(), (v == -np.inf).any()
        out[i] = np.nan if has_nan or (pos and neg) else (np.inf if pos else -np.inf)
    return out.reshape(cols.shape[:-1])


def mma_leaf_values(x: np.ndarray) -> np.ndarray:
    """The chunk nodes: the balanced tree over each chunk's 16 column sums."""
    return _tree_levels(mma_column_sums(mma_leaf_columns(x)))


def fixed_tree_sum_mma_leaves(x: np.ndarray) -> np.float32:
    """The MFMA-leaf fixed order over a 1-D binary16 array; n == 0 gives +0.0."""
    if x.dtype != np.float16:
        raise TypeError("fixed_tree_sum_mma_leaves expects a binary16 (float16) array")
    x = x.reshape(-1)
    if x.size == 0:
        return np.float32(0.0)
    leaves = mma_leaf_values(x)
    return _tree_levels(_pad_pow2(leaves, leaves.size))


def fixed_tree_row_sums_mma_leaves(x: np.ndarray) -> np.ndarray:
    """The MFMA-leaf order applied to every row of a 2-D binary16 array
    (each row on its own: its own chunks, its own tree); rows of no values
    give +0.0."""
    if x.ndim != 2 or x.dtype != np.float16:
        raise TypeError("fixed_tree_row_sums_mma_leaves expects a 2-D binary16 array")
    rows, cols = x.shape
    if cols == 0 or rows == 0:
        return np.zeros(rows, dtype=np.float32)
    chunks = -(-cols // 512)
    xp = np.zeros((rows, chunks * 512), np.float16)
    xp[:, :cols] = x
    # (row, chunk, slot group q, column j, value e) -> (row, chunk, column j, K)
    cols_k = xp.reshape(rows, chunks, 4, 16, 8).transpose(0, 1, 3, 2, 4).reshape(rows, chunks, 16, 32)
    leaves = _tree_levels(mma_column_sums(cols_k))            # (rows, chunks)
    return np.ascontiguousarray(_tree_levels(_pad_pow2(leaves, chunks)))
