"""Seeded random row shapes, pitches and configurations through both row
entry points, so that every planner mapping -- short rows, row streams, a
block per row, rows split over blocks, rows in two ranges -- meets shapes
nobody picked by hand (one case in forty is just past one round of the
fixed-order stream):
reduce_rows_fixed_order must equal the per-row balanced-tree
oracles bit for bit ("Taming Bitwise Behavior in GPU Kernels with Tensor
Core", arXiv 2609.11356, Abstract), reduce_rows must pass the free-order gate
against the exact per-row sums on sampled rows."""
import numpy as np
import pytest

import arithmetic_reduction_matrix_amd as armx
import synth_inputs as si
from oracle import exact_row_sums, fixed_tree_row_sums
from oracle.tree import fixed_tree_row_sums_mma_leaves

from _parity import NAN16, check_free_order, require_gpu, strided

pytestmark = pytest.mark.gpu

MAX_VALUES = 6_000_000   # per case, so the oracles stay quick


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def bits(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def draw_case(seed):
    rng = np.random.default_rng(seed)
    kind = rng.integers(0, 4) if seed % 40 != 39 else 4
    if kind == 4:     # just past one round of the fixed-order stream (rows in two ranges)
        rows = int(rng.integers(1025, 1300))
        cols = int(rng.integers(16_400, 20_000))
    elif kind == 0:   # short rows
        cols = int(rng.integers(1, 513))
        rows = int(rng.integers(1, MAX_VALUES // cols // 4 + 2))
    elif kind == 1:   # few long rows
        rows = int(rng.integers(1, 65))
        cols = int(rng.integers(513, MAX_VALUES // rows + 1))
    elif kind == 2:   # around the grid's wavefront count
        rows = int(rng.integers(200, 2400))
        cols = int(rng.integers(513, MAX_VALUES // rows + 1))
    else:             # anything
        cols = int(np.exp(rng.uniform(0, np.log(MAX_VALUES))))
        rows = int(rng.integers(1, MAX_VALUES // max(cols, 1) + 2))
    ld = (cols + 7) // 8 * 8 + 8 * int(rng.integers(0, 3))
    cfg = {}
    pick = rng.integers(0, 6)
    if pick == 1:
        cfg["block_threads"] = int(64 * 2 ** rng.integers(0, 5))
    elif pick == 2:
        cfg["chain_r"] = int(rng.integers(1, 9))
    elif pick == 3:
        cfg["grid_blocks"] = int(rng.integers(1, 600))
    elif pick == 4:
        cfg["cached_loads"] = True
    dist = ["uniform11", "normal", "logu_signed", "bits_finite"][int(rng.integers(0, 4))]
    return rows, cols, ld, cfg, dist


@pytest.mark.parametrize("seed", range(160))
def test_random_row_shapes(seed):
    rows, cols, ld, cfg, dist = draw_case(seed)
    x = si.generate_rows(dist, rows, cols, seed=seed)
    xd = strided(x, ld, junk=NAN16)
    what = (rows, cols, ld, cfg, dist)
    want = bits(fixed_tree_row_sums(x))
    got = armx.reduce_rows_fixed_order(xd, **cfg).cpu().numpy()
    assert np.array_equal(bits(got), want), what
    if seed % 4 == 0:
        got_mma = armx.reduce_rows_fixed_order(xd, mma_leaves=True, **cfg).cpu().numpy()
        idx = np.unique(np.linspace(0, rows - 1, 16).astype(int))
        assert np.array_equal(bits(got_mma[idx]), bits(fixed_tree_row_sums_mma_leaves(x[idx]))), what
    free = armx.reduce_rows(xd, **cfg).cpu().numpy()
    idx = np.unique(np.linspace(0, rows - 1, 24).astype(int))
    for r, e in zip(idx, exact_row_sums(x[idx])):
        check_free_order(float(free[r]), e, f"{what} row {r}")
