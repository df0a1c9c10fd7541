"""Rows longer than one chunk whose length is not a whole number of chains:
the cross-row pipelined paths of both row entry points read a row's last
chain with loads kept inside the row's pitch and mask what is not the row's.
reduce_rows_fixed_order must equal the per-row balanced-tree oracle bit for
bit ("Taming Bitwise Behavior in GPU Kernels with Tensor Core", arXiv
2609.11356, Abstract), reduce_rows must pass the free-order gate against the
exact per-row sums ("GPU Tensor Cores for fast Arithmetic Reductions", arXiv
2001.05585, Abstract).  Enough rows are used that the pipelined mapping (one
wavefront per row, rows streamed back to back) is the one that runs; the pitch
padding holds NaN or Inf and the last row ends at the end of its allocation."""
import numpy as np
import pytest

import arithmetic_reduction_matrix_amd as armx
import synth_inputs as si
from oracle import exact_row_sums, fixed_tree_row_sums

from _parity import INF16, NAN16, check_free_order, require_gpu, strided

pytestmark = pytest.mark.gpu

ROWS = 4099   # more rows than the persistent grid has wavefronts for any R


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def bits(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def check(x, xd, what="", sample=48, **cfg):
    got = armx.reduce_rows_fixed_order(xd, **cfg).cpu().numpy()
    assert np.array_equal(bits(got), bits(fixed_tree_row_sums(x))), ("fixed", what, cfg)
    got = armx.reduce_rows(xd, **cfg).cpu().numpy()
    idx = np.unique(np.concatenate([np.linspace(0, x.shape[0] - 1, sample).astype(int),
                                    [x.shape[0] - 1]]))
    for i, e in zip(idx, exact_row_sums(x[idx])):
        check_free_order(float(got[i]), e, f"{what} row {i} {cfg}")


@pytest.mark.parametrize("cols", [513, 520, 777, 1000, 1023, 1025, 1536, 2049, 2560, 4095,
                                  5000, 8193])
def test_partial_last_chain(cols):
    x = si.generate_rows("normal", ROWS, cols, seed=cols)
    ld = (cols + 7) // 8 * 8
    check(x, strided(x, ld, tail=0), f"{ROWS}x{cols}")


@pytest.mark.parametrize("cols,ld", [(1000, 1008), (1000, 1024), (3001, 3008), (600, 4096)])
@pytest.mark.parametrize("junk", [NAN16, INF16])
def test_pitch_padding_is_never_summed(cols, ld, junk):
    x = si.generate_rows("uniform11", ROWS, cols, seed=ld)
    check(x, strided(x, ld, junk=junk, tail=0), f"{ROWS}x{cols} ld={ld}")


@pytest.mark.parametrize("cfg", [dict(chain_r=1), dict(chain_r=2), dict(chain_r=3),
                                 dict(chain_r=4), dict(chain_r=8), dict(block_threads=256),
                                 dict(cached_loads=True), dict(grid_blocks=5)])
def test_configurations(cfg):
    x = si.generate_rows("bits_finite", ROWS, 1500, seed=7)
    check(x, strided(x, 1504, tail=0), "4099x1500", **cfg)


def test_long_ragged_rows():
    # rows of many chains ending in a partial one: the free-order stream; with
    # fewer rows than its wavefronts, fixed order takes the block-per-row path
    rows, cols = 600, 66048 + 5
    x = si.generate_rows("uniform11", rows, cols, seed=3)
    check(x, strided(x, (cols + 7) // 8 * 8, tail=0), f"{rows}x{cols}", sample=24)
