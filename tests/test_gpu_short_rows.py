"""Rows of at most 512 values: both row entry points sum them with the
segmented kernel (each row on a power-of-two group of lanes, several rows per
wavefront load).  reduce_rows_fixed_order must equal the per-row balanced-tree
oracle bit for bit ("Taming Bitwise Behavior in GPU Kernels with Tensor Core",
arXiv 2609.11356, Abstract); reduce_rows must pass the free-order gate against
the exact per-row sums and, for these rows, returns the same tree sum.  Row
pitches larger than the row, padding that holds NaN and Inf, and a last row
that ends exactly at the end of its allocation are covered, since the kernel
reads whole 16-byte slots and masks what is not the row's."""
import numpy as np
import pytest
import torch

import arithmetic_reduction_matrix_amd as armx
import synth_inputs as si
from oracle import exact_row_sums, fixed_tree_row_sums, fixed_tree_row_sums_mma_leaves

from _parity import NAN16, INF16, check_free_order, require_gpu, strided

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def bits(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def check_both(x, xd, what="", **cfg):
    want = fixed_tree_row_sums(x)
    got_fixed = armx.reduce_rows_fixed_order(xd, **cfg).cpu().numpy()
    assert np.array_equal(bits(got_fixed), bits(want)), ("fixed", what, cfg)
    got_free = armx.reduce_rows(xd, **cfg).cpu().numpy()
    assert np.array_equal(bits(got_free), bits(want)), ("free", what, cfg)
    # the free-order gate too, on a sample of rows (the exact oracle is slow)
    idx = np.unique(np.linspace(0, x.shape[0] - 1, 40).astype(int))
    for i, e in zip(idx, exact_row_sums(x[idx])):
        check_free_order(float(got_free[i]), e, f"{what} row {i}")


# every lane-group size, each with a full, a ragged and a padded-lane case
COLS = [1, 2, 3, 7, 8, 9, 15, 16, 17, 24, 31, 32, 33, 63, 64, 65, 100, 127, 128, 129,
        200, 255, 256, 257, 300, 383, 384, 385, 504, 505, 511, 512]


@pytest.mark.parametrize("cols", COLS)
def test_every_lane_group_size(cols):
    # rows span several steps of every wavefront and a partial last step
    p = 1 << max(0, (cols + 7) // 8 - 1).bit_length()
    rows = (64 // p) * 8 * 5 + 3
    x = si.generate_rows("normal", rows, cols, seed=cols)
    ld = (cols + 7) // 8 * 8
    check_both(x, strided(x, ld), f"{rows}x{cols}")


@pytest.mark.parametrize("cols,ld", [(5, 16), (100, 104), (100, 512), (257, 264), (512, 520),
                                     (33, 40)])
@pytest.mark.parametrize("junk", [NAN16, INF16])
def test_pitch_padding_is_never_summed(cols, ld, junk):
    rows = 1000
    x = si.generate_rows("uniform11", rows, cols, seed=ld)
    check_both(x, strided(x, ld, junk=junk), f"{rows}x{cols} ld={ld}")


@pytest.mark.parametrize("rows", [1, 2, 7, 64, 65, 511, 513])
@pytest.mark.parametrize("cols", [1, 5, 13, 64, 77, 509])
def test_last_row_ends_at_the_allocation(rows, cols):
    # no values after the last row (tail=0): a read past it would fault or
    # pick up junk; the pitch padding in between is NaN
    x = si.generate_rows("logu_signed", rows, cols, seed=rows * 1000 + cols)
    ld = (cols + 7) // 8 * 8
    check_both(x, strided(x, ld, tail=0), f"{rows}x{cols}")


@pytest.mark.parametrize("cfg", [dict(block_threads=64), dict(block_threads=256),
                                 dict(block_threads=1024), dict(grid_blocks=1),
                                 dict(grid_blocks=3, block_threads=128),
                                 dict(cached_loads=True), dict(chain_r=3)])
def test_configurations_give_the_same_bits(cfg):
    x = si.generate_rows("bits_finite", 3001, 45, seed=11)
    check_both(x, strided(x, 48), str(cfg), **cfg)
    y = si.generate_rows("normal", 777, 512, seed=12)
    check_both(y, strided(y, 512), str(cfg), **cfg)


def test_plain_flag_is_accepted():
    x = si.generate_rows("normal", 500, 40, seed=5)
    xd = strided(x, 40)
    got = armx.reduce_rows(xd, plain=True).cpu().numpy()
    assert np.array_equal(bits(got), bits(fixed_tree_row_sums(x)))


def test_specials():
    x = np.ones((6, 20), np.float16)
    x[1, 3] = np.inf
    x[2, 19] = np.nan
    x[3, 0], x[3, 19] = np.inf, -np.inf
    x[4, :] = -0.0
    x[5, :] = 0.0
    xd = strided(x, 24)
    for fn in (armx.reduce_rows, armx.reduce_rows_fixed_order):
        got = fn(xd).cpu().numpy()
        assert got[0] == 20 and got[1] == np.inf and np.isnan(got[2]) and np.isnan(got[3])
        assert bits(got[4:5])[0] == 0x80000000 and bits(got[5:6])[0] == 0   # -0.0, +0.0


def test_every_binary16_value_as_a_one_value_row():
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = pats.view(np.float16).reshape(-1, 1)
    xd = strided(x, 8)
    want = fixed_tree_row_sums(x)
    for fn in (armx.reduce_rows, armx.reduce_rows_fixed_order):
        got = fn(xd).cpu().numpy()
        fin = np.isfinite(want)
        assert np.array_equal(bits(got[fin]), bits(want[fin]))
        assert np.array_equal(np.isnan(got), np.isnan(want))


@pytest.mark.parametrize("rows,cols", [((1 << 22) + 3, 64), ((1 << 20) + 1, 250),
                                       ((1 << 21) + 5, 100)])
def test_large_matrices(rows, cols):
    # at the 2^28-value scale: every row against the tree oracle (64 and 250
    # values: whole-line pitches, 4 groups per step; 100 values at a pitch of
    # 104: 8 groups per step and a ragged last row)
    x = si.generate_rows("uniform11", rows, cols, seed=cols)
    ld = (cols + 7) // 8 * 8
    if ld == cols:
        xd = torch.from_numpy(x).to("cuda")
    else:
        buf = np.zeros((rows, ld), np.float16)
        buf[:, :cols] = x
        xd = torch.from_numpy(buf).to("cuda")[:, :cols]
    want = fixed_tree_row_sums(x)
    for fn in (armx.reduce_rows, armx.reduce_rows_fixed_order):
        got = fn(xd).cpu().numpy()
        assert np.array_equal(bits(got), bits(want)), (fn.__name__, rows, cols)


@pytest.mark.parametrize("cols", [8, 33, 64, 100, 512])
@pytest.mark.parametrize("grid_blocks", [1, 3])
def test_many_steps_per_wavefront(cols, grid_blocks):
    # few wavefronts and many rows: every wavefront runs many steps of its
    # pipeline, and the last one a partial step
    rows = 60_007 if cols <= 64 else 30_001
    x = si.generate_rows("logu_signed", rows, cols, seed=cols + grid_blocks)
    ld = (cols + 7) // 8 * 8
    xd = strided(x, ld)
    want = fixed_tree_row_sums(x)
    for fn in (armx.reduce_rows_fixed_order, armx.reduce_rows):
        got = fn(xd, grid_blocks=grid_blocks).cpu().numpy()
        assert np.array_equal(bits(got), bits(want)), (fn.__name__, cols, grid_blocks)
    got = armx.reduce_rows_fixed_order(xd, grid_blocks=grid_blocks, mma_leaves=True)
    want = fixed_tree_row_sums_mma_leaves(x)
    assert np.array_equal(bits(got.cpu().numpy()), bits(want)), ("mma leaves", cols)


@pytest.mark.parametrize("cols", [8, 64, 257])
def test_output_not_16_byte_aligned(cols):
    # results written through an output view at an odd 4-byte offset, with
    # guard values around it left untouched
    rows = 20_011
    x = si.generate_rows("normal", rows, cols, seed=cols)
    xd = strided(x, (cols + 7) // 8 * 8)
    buf = torch.full((rows + 5,), 12345.0, dtype=torch.float32, device="cuda")
    out = buf[1:rows + 1]
    armx.reduce_rows_fixed_order(xd, out=out)
    host = buf.cpu().numpy()
    assert np.array_equal(bits(host[1:rows + 1]), bits(fixed_tree_row_sums(x)))
    assert host[0] == 12345.0 and (host[rows + 1:] == 12345.0).all()
