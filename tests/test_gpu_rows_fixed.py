"""reduce_rows_fixed_order against the per-row balanced-tree oracle, bit for
bit, and its batch invariance: a row's bits do not depend on the other rows,
the row's position or the configuration.  The order is the balanced tree of
"Taming Bitwise Behavior in GPU Kernels with Tensor Core" (arXiv 2609.11356,
Abstract), which also names batch invariance as what tile shapes break."""
import numpy as np
import pytest
import torch

import arithmetic_reduction_matrix_amd as armx
import synth_inputs as si
from oracle import fixed_tree_row_sums, fixed_tree_sum

from _parity import require_gpu, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def padded(x):
    """Device view of x whose row pitch is a multiple of 8 elements."""
    rows, cols = x.shape
    ld = max(8, (cols + 7) // 8 * 8)
    buf = np.zeros((rows, ld), np.float16)
    buf[:, :cols] = x
    return to_dev(buf)[:, :cols]


def bits(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def check(x, **cfg):
    got = armx.reduce_rows_fixed_order(padded(x), **cfg).cpu().numpy()
    want = fixed_tree_row_sums(x)
    assert np.array_equal(bits(got), bits(want)), (x.shape, cfg)


@pytest.mark.parametrize("rows,cols", [(1, 1), (3, 8), (5, 1000), (17, 513), (64, 4096),
                                       (33, 2048 * 5 + 7), (2, 300_000), (1000, 4096),
                                       (300, 8192 * 3), (9, 65536 * 8)])
def test_shapes(rows, cols):
    check(si.generate_rows("normal", rows, cols, seed=rows + cols))


@pytest.mark.parametrize("block", [64, 256, 1024])
@pytest.mark.parametrize("r", [1, 2, 4, 5, 8])
def test_block_chain_matrix(block, r):
    # 1024-value rows take the flat path for R <= 2 at 64 threads; 40000-value
    # rows (ragged) always take the general path
    check(si.generate_rows("uniform11", 700, 1024, seed=r), block_threads=block, chain_r=r)
    check(si.generate_rows("bits_finite", 24, 40_000, seed=r), block_threads=block, chain_r=r)


@pytest.mark.parametrize("cols", [4001, 6000, 9000])
@pytest.mark.parametrize("mma_leaves", [False, True])
def test_row_stream_last_group(cols, mma_leaves):
    # the flat row stream keeps the matrix's last row in it and reads only
    # that row's last group apart (4001: the row ends inside a lane's 8
    # values); a small grid puts every R on the stream
    x = si.generate_rows("normal", 1500, cols, seed=cols)
    extra = dict(mma_leaves=True) if mma_leaves else {}
    for cfg in [dict()] + [dict(chain_r=r, block_threads=64, grid_blocks=16) for r in (1, 2, 4, 8)]:
        if mma_leaves:
            from oracle import fixed_tree_row_sums_mma_leaves
            got = armx.reduce_rows_fixed_order(padded(x), **cfg, **extra).cpu().numpy()
            assert np.array_equal(bits(got), bits(fixed_tree_row_sums_mma_leaves(x))), (cols, cfg)
        else:
            check(x, **cfg)


def test_batch_invariance():
    x = si.generate_rows("logu_signed", 512, 8192, seed=17)
    want = bits(fixed_tree_row_sums(x))
    xd = to_dev(x)
    full = bits(armx.reduce_rows_fixed_order(xd).cpu().numpy())
    assert np.array_equal(full, want)
    # sub-batches at other offsets, other configurations, single rows
    sub = bits(armx.reduce_rows_fixed_order(xd[37:300], block_threads=256, chain_r=4)
               .cpu().numpy())
    assert np.array_equal(sub, want[37:300])
    for r in (0, 1, 255, 511):
        one = bits(armx.reduce_rows_fixed_order(xd[r:r + 1], chain_r=5).cpu().numpy())
        assert one[0] == want[r]
        # and the flat entry point on the same values
        flat = armx.reduce_sum_fixed_order(xd[r].contiguous()).cpu().numpy()
        assert bits(flat)[()] == want[r]


def test_specials_and_empty():
    out = armx.reduce_rows_fixed_order(torch.empty(4, 0, dtype=torch.float16, device="cuda"))
    assert bits(out.cpu().numpy()).tolist() == [0] * 4
    x = si.generate_rows("uniform11", 6, 4096, seed=2)
    x[0, :] = -0.0
    x[1, 10] = np.inf
    x[2, 10], x[2, 4000] = np.inf, -np.inf
    x[3, 99] = np.nan
    got = armx.reduce_rows_fixed_order(to_dev(x)).cpu().numpy()
    assert bits(got)[0] == bits(np.float32(-0.0))[()]
    assert got[1] == np.inf and np.isnan(got[2]) and np.isnan(got[3])
    assert np.array_equal(bits(got[4:]), bits(fixed_tree_row_sums(x[4:])))


def test_full_4096x65536_normal():
    x = si.workload("rows_4096x65536_normal")
    want = bits(fixed_tree_row_sums(x))
    xd = to_dev(x)
    for cfg in (dict(), dict(block_threads=256, chain_r=4), dict(chain_r=5)):
        got = bits(armx.reduce_rows_fixed_order(xd, **cfg).cpu().numpy())
        assert np.array_equal(got, want), cfg
    # batch invariance against the flat fixed order on sampled rows
    for r in (0, 1234, 4095):
        assert bits(armx.reduce_sum_fixed_order(xd[r].contiguous()).cpu().numpy())[()] == want[r]


@pytest.mark.parametrize("cols", [601, 1003, 2261, 4005])
def test_pitch_padding_never_summed(cols):
    # as in the free order: a NaN pitch past each row must not reach a root,
    # and the zeros of the range-checked loads past the row must act as -0.0
    rows = 2000
    ld = (cols + 7) // 8 * 8 + 8
    x = si.generate_rows("normal", rows, cols, seed=cols + 2)
    pad = np.full((rows, ld), np.nan, np.float16)
    pad[:, :cols] = x
    xd = to_dev(pad)[:, :cols]
    want = bits(fixed_tree_row_sums(x))
    for cfg in [dict(), dict(chain_r=1), dict(chain_r=4, block_threads=64, grid_blocks=32)]:
        got = armx.reduce_rows_fixed_order(xd, **cfg).cpu().numpy()
        assert np.array_equal(bits(got), want), (cols, cfg)
