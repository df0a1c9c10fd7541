"""reduce_rows_fixed_order with ARMX_FLAG_MMA_LEAVES against the oracle's
MFMA-leaf order applied to every row (oracle.tree
fixed_tree_row_sums_mma_leaves, built on the reconstructed MFMA accumulation
of oracle.mfma_model), bit for bit: rows of at most 512 values packed several
to a load (one MFMA per load with a K-group selector, or one masked MFMA per
lane block where a load holds an Inf or a NaN), long rows streamed by one
wavefront or summed by a block, ragged rows and pitches, non-finite values,
and batch invariance -- the balanced-tree reproducibility of "Taming Bitwise
Behavior in GPU Kernels with Tensor Core" (arXiv 2609.11356, Abstract) with
tensor-core leaves."""
import os

import numpy as np
import pytest
import torch

import arithmetic_reduction_matrix_amd as armx
import synth_inputs as si
from oracle import exact_row_sums
from oracle.tree import fixed_tree_row_sums_mma_leaves, fixed_tree_sum_mma_leaves

from _parity import NAN16, INF16, check_free_order, require_gpu, strided

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def bits(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def mma_rows(xd, **cfg):
    return armx.reduce_rows_fixed_order(xd, mma_leaves=True, **cfg).cpu().numpy()


def check(x, xd, what="", **cfg):
    got = mma_rows(xd, **cfg)
    want = fixed_tree_row_sums_mma_leaves(x)
    bad = np.flatnonzero(bits(got) != bits(want))
    assert bad.size == 0, (what, cfg, bad[:5], got[bad[:5]], want[bad[:5]])
    return got


def pitch(cols):
    return max(8, (cols + 7) // 8 * 8)


# every lane-group size of the packed kernel (full, ragged, padded lanes) and
# rows of one chunk and more
COLS = [1, 2, 7, 8, 9, 16, 17, 31, 64, 65, 100, 128, 129, 200, 255, 256, 257, 300, 384, 505,
        512, 513, 1000, 1024, 1500, 4096, 5000]


@pytest.mark.parametrize("cols", COLS)
def test_every_row_length(cols):
    p = 1 << max(0, (cols + 7) // 8 - 1).bit_length() if cols <= 512 else 64
    rows = (64 // p) * 8 * 5 + 3 if cols <= 512 else 301
    x = si.generate_rows("logu_signed", rows, cols, seed=cols + 3)
    got = check(x, strided(x, pitch(cols)), f"{rows}x{cols}")
    idx = np.unique(np.linspace(0, rows - 1, 20).astype(int))
    for i, e in zip(idx, exact_row_sums(x[idx])):
        check_free_order(float(got[i]), e, f"row {i}")


@pytest.mark.parametrize("rows,cols", [(3, 4096), (2, 70000), (1, 513), (5, 200000)])
def test_few_long_rows_take_a_block_each(rows, cols):
    x = si.generate_rows("uniform11", rows, cols, seed=rows * 7 + cols)
    xd = strided(x, pitch(cols))
    check(x, xd, f"{rows}x{cols}")
    check(x, xd, f"{rows}x{cols}", block_threads=1024, chain_r=3)


@pytest.mark.parametrize("cfg", [dict(block_threads=64), dict(block_threads=256),
                                 dict(block_threads=1024), dict(grid_blocks=1),
                                 dict(grid_blocks=5, block_threads=128),
                                 dict(cached_loads=True), dict(chain_r=1), dict(chain_r=2),
                                 dict(chain_r=3), dict(chain_r=8)])
@pytest.mark.parametrize("cols", [45, 300, 512, 1000, 9000])
def test_configurations_give_the_same_bits(cfg, cols):
    x = si.generate_rows("bits_finite", 1201, cols, seed=cols)
    check(x, strided(x, pitch(cols)), f"1201x{cols}", **cfg)


@pytest.mark.parametrize("cols,ld", [(5, 16), (100, 104), (257, 264), (512, 520), (700, 712),
                                     (2049, 2056)])
@pytest.mark.parametrize("junk", [NAN16, INF16])
def test_pitch_padding_is_never_summed(cols, ld, junk):
    x = si.generate_rows("uniform11", 700, cols, seed=ld)
    check(x, strided(x, ld, junk=junk), f"ld={ld}")


@pytest.mark.parametrize("rows", [1, 2, 7, 65, 513])
@pytest.mark.parametrize("cols", [1, 13, 77, 509, 600, 1029])
def test_last_row_ends_at_the_allocation(rows, cols):
    x = si.generate_rows("logu_signed", rows, cols, seed=rows * 1000 + cols)
    check(x, strided(x, pitch(cols), tail=0), f"{rows}x{cols}")


@pytest.mark.parametrize("cols", [20, 64, 200, 512, 1500])
def test_non_finite_values_stay_in_their_row(cols):
    # rows packed next to a row holding Inf or NaN share MFMA columns with it
    # unless the kernel zeroes the other rows' lanes: every finite row must
    # stay finite and exact
    x = si.generate_rows("uniform11", 64, cols, seed=cols)
    x[3, cols // 2] = np.inf
    x[10, 0] = np.nan
    x[17, 0], x[17, cols - 1] = np.inf, -np.inf
    x[25, :] = np.float16(-0.0)
    x[33, cols - 1] = -np.inf
    got = mma_rows(strided(x, pitch(cols)))
    want = fixed_tree_row_sums_mma_leaves(x)
    assert got[3] == np.inf and np.isnan(got[10]) and np.isnan(got[17]) and got[33] == -np.inf
    assert bits(got[25:26])[0] == 0   # an MFMA from a zero accumulator gives +0.0
    fin = np.isfinite(want)
    assert fin.sum() == 60
    assert np.array_equal(bits(got[fin]), bits(want[fin]))


@pytest.mark.parametrize("cols", [8, 40, 64, 100, 200, 264])
def test_scattered_non_finite_rows(cols):
    # most loads take one MFMA with a K-group selector; the few that hold an
    # Inf or a NaN take one masked MFMA per lane block instead, in the same
    # launch -- both must give the oracle's bits
    rows = 20011
    x = si.generate_rows("logu_signed", rows, cols, seed=cols + 100)
    rng = np.random.default_rng(cols)
    bad = rng.choice(rows, 12, replace=False)
    for k, r in enumerate(bad):
        x[r, rng.integers(0, cols)] = (np.inf, -np.inf, np.nan)[k % 3]
    got = mma_rows(strided(x, pitch(cols)))
    want = fixed_tree_row_sums_mma_leaves(x)
    fin = np.isfinite(want)
    assert fin.sum() == rows - 12
    assert np.array_equal(bits(got[fin]), bits(want[fin]))
    assert np.array_equal(got[~fin], want[~fin], equal_nan=True)


@pytest.mark.parametrize("cols", [24, 130, 512, 3000])
def test_batch_invariance(cols):
    # a row's bits do not depend on the rows around it, its position or the
    # number of rows
    base = si.generate_rows("normal", 1, cols, seed=cols)[0]
    alone = mma_rows(strided(base[None, :], pitch(cols)))[0]
    assert bits(alone) == bits(fixed_tree_sum_mma_leaves(base))
    for rows, pos in ((2, 1), (97, 50), (4099, 4098), (4099, 0)):
        x = si.generate_rows("logu_signed", rows, cols, seed=rows + pos)
        x[pos] = base
        got = mma_rows(strided(x, pitch(cols)))
        assert bits(got[pos]) == bits(alone), (rows, pos)


def test_differs_from_the_valu_tree_but_stays_close():
    x = si.generate_rows("logu_signed", 4000, 300, seed=2)
    xd = strided(x, 304)
    a = mma_rows(xd)
    b = armx.reduce_rows_fixed_order(xd).cpu().numpy()
    assert (bits(a) != bits(b)).any()
    for i, e in zip(range(0, 4000, 400), exact_row_sums(x[::400])):
        check_free_order(float(a[i]), e, "mma leaves")
        check_free_order(float(b[i]), e, "valu tree")


@pytest.mark.parametrize("rows,cols", [(1 << 22, 64), (268435, 1000)])
def test_full_size_matrices_every_row(rows, cols):
    # the row workloads of the benchmark, in its launch configuration, every
    # row against the oracle; the oracle runs on batches of rows in threads
    # (rows are independent, and numpy releases the interpreter lock)
    from concurrent.futures import ThreadPoolExecutor
    x = si.generate_rows("uniform11", rows, cols, seed=cols)
    xd = torch.from_numpy(x).to("cuda")
    got = mma_rows(xd)
    del xd
    step = 32768
    threads = max(1, min(16, len(os.sched_getaffinity(0))))
    with ThreadPoolExecutor(threads) as pool:
        parts = list(pool.map(lambda r0: fixed_tree_row_sums_mma_leaves(x[r0:r0 + step]),
                              range(0, rows, step)))
    want = np.concatenate(parts)
    bad = np.flatnonzero(bits(got) != bits(want))
    assert bad.size == 0, (rows, cols, bad[:10])
