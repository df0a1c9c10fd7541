"""reduce_rows against the per-row exact-sum oracle (free order within each
row), a row-segmented form of the reduction of "GPU Tensor Cores for fast
Arithmetic Reductions" (arXiv 2001.05585, Abstract)."""
import math

import numpy as np
import pytest
import torch

import arithmetic_reduction_matrix_amd as armx
import synth_inputs as si
from oracle import decode_table, exact_row_sums

from _parity import check_free_order, require_gpu, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def check_rows(x, got, what=""):
    for r, e in enumerate(exact_row_sums(x)):
        check_free_order(float(got[r]), e, f"{what} row {r}")


@pytest.mark.parametrize("rows,cols", [(1, 1), (3, 8), (5, 1000), (17, 513), (64, 4096),
                                       (33, 2048 * 5 + 7), (2, 300_000)])
@pytest.mark.parametrize("design", [dict(), dict(plain=True), dict(all_ones=True)],
                         ids=["signed", "plain", "ones"])
def test_shapes(rows, cols, design):
    x = si.generate_rows("normal", rows, cols, seed=rows * 7 + cols)
    if cols % 8:
        # rows must start 16-byte aligned: pad the pitch, sum only `cols`
        ld = (cols + 7) // 8 * 8
        pad = np.zeros((rows, ld), np.float16)
        pad[:, :cols] = x
        xd = to_dev(pad)[:, :cols]
    else:
        xd = to_dev(x)
    got = armx.reduce_rows(xd, **design).cpu().numpy()
    check_rows(x, got, f"{rows}x{cols} {design}")


@pytest.mark.parametrize("block", [64, 256, 1024])
@pytest.mark.parametrize("r", [1, 2, 4, 5, 8])
def test_block_chain_matrix(block, r):
    x = si.generate_rows("uniform11", 40, 20000, seed=3)
    got = armx.reduce_rows(to_dev(x), block_threads=block, chain_r=r).cpu().numpy()
    check_rows(x, got, f"block={block} r={r}")


def test_strided_rows_and_small_grid():
    base = si.generate_rows("uniform01", 50, 4096, seed=8)
    xd = to_dev(base)[:, :1000]           # ld 4096, cols 1000
    got = armx.reduce_rows(xd, grid_blocks=7).cpu().numpy()
    check_rows(base[:, :1000], got, "strided")


def test_zero_cols_and_specials():
    out = armx.reduce_rows(torch.empty(5, 0, dtype=torch.float16, device="cuda"))
    assert out.cpu().numpy().tolist() == [0.0] * 5
    x = np.ones((4, 704), np.float16)
    x[1, 5] = np.inf
    x[2, 600] = np.nan
    x[3, 0], x[3, 1] = np.inf, -np.inf
    for plain in (False, True):
        got = armx.reduce_rows(to_dev(x), plain=plain).cpu().numpy()
        assert got[0] == 704 and got[1] == np.inf and math.isnan(got[2]) and math.isnan(got[3])
    # a pitch that is not a multiple of 8 elements is rejected, not misread
    with pytest.raises(armx.ArmxError) as ei:
        armx.reduce_rows(to_dev(np.ones((4, 700), np.float16)))
    assert ei.value.name == "ARMX_ERR_ALIGN"


@pytest.mark.parametrize("plain", [False, True])
def test_every_binary16_value_converts_exactly(plain):
    # one value per row: row r holds pattern r, so out[r] is its exact value
    # (subnormals included -- nothing may be flushed)
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = np.zeros((65536, 8), np.uint16)
    x[:, 0] = pats
    got = armx.reduce_rows(to_dev(x.view(np.float16))[:, :1], plain=plain).cpu().numpy()
    q, cls = decode_table()
    fin = cls == 0
    want = q[fin].astype(np.float64) * 2.0 ** -24
    assert np.array_equal(got[fin].astype(np.float64), want)
    assert np.isnan(got[cls == 3]).all()


@pytest.mark.parametrize("rows,cols", [(4096, 8192), (3000, 4096 * 3), (1000, 4096)])
def test_many_rows_flat_pipeline(rows, cols):
    # rows that are whole numbers of chains take the cross-row pipelined path
    x = si.generate_rows("uniform11", rows, cols, seed=rows)
    xd = to_dev(x)
    for cfg in (dict(), dict(plain=True), dict(all_ones=True), dict(chain_r=4, block_threads=64)):
        got = armx.reduce_rows(xd, **cfg).cpu().numpy()
        check_rows(x, got, str(cfg))


def test_full_4096x65536_normal():
    x = si.workload("rows_4096x65536_normal")
    xd = to_dev(x)
    for cfg in (dict(), dict(plain=True)):
        got = armx.reduce_rows(xd, **cfg).cpu().numpy()
        check_rows(x, got, str(cfg))


@pytest.mark.parametrize("cols", [33001, 36000, 40960])
def test_long_rows_stream(cols):
    # rows of at least 32768 values in a well-filled row stream take
    # rows_stream_kernel: the matrix's last row stays in the stream and only
    # its last chain is read apart (33001: the row ends inside a lane's 8
    # values; 36000: inside a chain; 40960: whole chains of 8)
    rows = 1000
    ld = (cols + 7) // 8 * 8
    x = si.generate_rows("normal", rows, cols, seed=cols)
    pad = np.zeros((rows, ld), np.float16)
    pad[:, :cols] = x
    xd = to_dev(pad)[:, :cols]
    # (a small grid keeps every chain length on the row stream)
    small = [dict(chain_r=r, block_threads=64, grid_blocks=16) for r in (1, 2, 4, 5, 8)]
    for cfg in [dict(), dict(plain=True), dict(all_ones=True),
                dict(chain_r=3, block_threads=256, grid_blocks=8)] + small:
        got = armx.reduce_rows(xd, **cfg).cpu().numpy()
        check_rows(x, got, f"{rows}x{cols} {cfg}")



@pytest.mark.parametrize("cols", [601, 1003, 2261, 4005])
def test_pitch_padding_never_summed(cols):
    # the row stream reads a row's last lane slot whole and masks the values
    # past the row; a pitch one slot wider than needed, full of NaN, shows
    # any value past the row that reaches a sum (601 and 1003: the row ends
    # inside a lane's 8 values; 2261, 4005 at the default and other chain
    # lengths: inside a chain, with whole chunks past the row)
    rows = 2000
    ld = (cols + 7) // 8 * 8 + 8
    x = si.generate_rows("normal", rows, cols, seed=cols + 1)
    pad = np.full((rows, ld), np.nan, np.float16)
    pad[:, :cols] = x
    xd = to_dev(pad)[:, :cols]
    for cfg in [dict(), dict(plain=True), dict(chain_r=4, block_threads=256),
                dict(chain_r=8, block_threads=64, grid_blocks=32)]:
        got = armx.reduce_rows(xd, **cfg).cpu().numpy()
        check_rows(x, got, f"{rows}x{cols} ld {ld} {cfg}")
