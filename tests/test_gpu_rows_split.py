"""Few long rows: with a workspace, both row entry points split every row over
several wavefronts in different blocks (plan mode 3) and the last block to
finish combines each row's parts.  reduce_rows must pass the free-order gate
against the exact per-row sums and give the same bits on every call;
reduce_rows_fixed_order must equal the per-row balanced-tree oracles bit for
bit (both orders: "Taming Bitwise Behavior in GPU Kernels with Tensor Core",
arXiv 2609.11356, Abstract), whatever the split, and also without a
workspace, where each row is summed by one block."""
import ctypes

import numpy as np
import pytest
import torch

import arithmetic_reduction_matrix_amd as armx
import synth_inputs as si
from oracle import exact_row_sums, fixed_tree_row_sums, fixed_tree_sum
from oracle.tree import fixed_tree_row_sums_mma_leaves

from _parity import NAN16, check_free_order, require_gpu, strided

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def bits(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def pitch(cols):
    return max(8, (cols + 7) // 8 * 8)


def no_workspace(fn, xd, **cfg):
    """The entry point called through the C ABI with ws NULL (no split)."""
    rows, cols = xd.shape
    out = torch.empty(rows, dtype=torch.float32, device=xd.device)
    ld = xd.stride(0) if rows > 1 else cols
    c = armx._config(**cfg)
    st = fn(xd.data_ptr(), rows, cols, ld, out.data_ptr(), None, 0, ctypes.byref(c),
            torch.cuda.current_stream().cuda_stream)
    assert st == 0, armx.lib.armx_status_string(st)
    return out.cpu().numpy()


# (1, 6_297_088): 12299 chunks, R = 5, 1024 wavefronts: 768 segments of 8192
# values, more parts than the last block's tree over a row holds unless the
# plan caps them
SHAPES = [(1, 1 << 20), (1, (1 << 20) + 777), (1, 6_297_088), (2, 300_001), (3, 1 << 18),
          (5, 200_000), (8, 131_072 + 4096 + 13), (31, 65_536 + 5), (64, 40_000),
          (100, 66_000)]


@pytest.mark.parametrize("rows,cols", SHAPES)
def test_free_order_split(rows, cols):
    assert armx.workspace_bytes(armx.OP_ROWS, rows, cols) > 0, "expected a split plan"
    x = si.generate_rows("logu_signed", rows, cols, seed=rows * 7 + cols)
    xd = strided(x, pitch(cols))
    got = armx.reduce_rows(xd).cpu().numpy()
    again = armx.reduce_rows(xd).cpu().numpy()
    assert np.array_equal(bits(got), bits(again))           # same bits every call
    plain = armx.reduce_rows(xd, plain=True).cpu().numpy()
    ones = armx.reduce_rows(xd, all_ones=True).cpu().numpy()
    unsplit = no_workspace(armx.lib.reduce_rows, xd)
    for r, e in enumerate(exact_row_sums(x)):
        check_free_order(float(got[r]), e, f"row {r}")
        check_free_order(float(plain[r]), e, f"plain row {r}")
        check_free_order(float(ones[r]), e, f"all-ones row {r}")
        check_free_order(float(unsplit[r]), e, f"unsplit row {r}")


@pytest.mark.parametrize("rows,cols", SHAPES)
def test_fixed_order_split(rows, cols):
    assert armx.workspace_bytes(armx.OP_ROWS_FIXED, rows, cols) > 0, "expected a split plan"
    x = si.generate_rows("uniform11", rows, cols, seed=rows * 11 + cols)
    xd = strided(x, pitch(cols))
    want = bits(fixed_tree_row_sums(x))
    assert np.array_equal(bits(armx.reduce_rows_fixed_order(xd).cpu().numpy()), want)
    assert np.array_equal(bits(no_workspace(armx.lib.reduce_rows_fixed_order, xd)), want)
    want_mma = bits(fixed_tree_row_sums_mma_leaves(x))
    got_mma = armx.reduce_rows_fixed_order(xd, mma_leaves=True).cpu().numpy()
    assert np.array_equal(bits(got_mma), want_mma)


@pytest.mark.parametrize("cfg", [dict(block_threads=64), dict(block_threads=256),
                                 dict(block_threads=1024), dict(chain_r=1), dict(chain_r=3),
                                 dict(chain_r=8), dict(grid_blocks=7), dict(grid_blocks=100),
                                 dict(cached_loads=True)])
def test_configurations(cfg):
    x = si.generate_rows("bits_finite", 6, 150_000, seed=5)
    xd = strided(x, pitch(150_000))
    want = bits(fixed_tree_row_sums(x))
    assert np.array_equal(bits(armx.reduce_rows_fixed_order(xd, **cfg).cpu().numpy()), want), cfg
    got = armx.reduce_rows(xd, **cfg).cpu().numpy()
    for r, e in enumerate(exact_row_sums(x)):
        check_free_order(float(got[r]), e, f"{cfg} row {r}")


def test_pitch_padding_is_never_summed():
    x = si.generate_rows("uniform11", 4, 100_003, seed=8)
    xd = strided(x, 100_008 + 64, junk=NAN16)
    assert np.array_equal(bits(armx.reduce_rows_fixed_order(xd).cpu().numpy()),
                          bits(fixed_tree_row_sums(x)))
    got = armx.reduce_rows(xd).cpu().numpy()
    for r, e in enumerate(exact_row_sums(x)):
        check_free_order(float(got[r]), e, f"row {r}")


def test_one_row_of_2p27_values():
    # beyond what one block's node logs hold: refused without a workspace,
    # exact to the oracle with the split
    n = 1 << 27
    x = si.generate("uniform11", n, seed=27)
    xd = torch.from_numpy(x).to("cuda").view(1, n)
    want = bits(np.float32(fixed_tree_sum(x)))
    assert bits(armx.reduce_rows_fixed_order(xd).cpu().numpy())[0] == want
    assert bits(armx.reduce_sum_fixed_order(xd.view(-1)).cpu().numpy()) == want
    c = armx._config()
    out = torch.empty(1, dtype=torch.float32, device="cuda")
    st = armx.lib.reduce_rows_fixed_order(xd.data_ptr(), 1, n, n, out.data_ptr(), None, 0,
                                          ctypes.byref(c), torch.cuda.current_stream().cuda_stream)
    assert st == -5   # ARMX_ERR_SHAPE: too long for one block


def test_workspace_shared_with_the_flat_sums():
    # one cached workspace per stream serves every entry point: a split row
    # call between flat calls must find its counter at zero and leave it so
    y = torch.from_numpy(si.generate("uniform11", 1 << 22, seed=3)).to("cuda")
    x = si.generate_rows("normal", 3, 500_000, seed=4)
    xd = strided(x, 500_000)
    want = bits(fixed_tree_row_sums(x))
    s0 = armx.reduce_sum(y).item()
    for _ in range(3):
        assert np.array_equal(bits(armx.reduce_rows_fixed_order(xd).cpu().numpy()), want)
        armx.reduce_rows(xd)
        assert armx.reduce_sum(y).item() == s0
        armx.reduce_sum_fixed_order(y)


def test_split_in_a_graph():
    x = si.generate_rows("uniform11", 4, 262_144 + 104, seed=9)
    pool = [si.generate_rows("uniform11", 4, 262_144 + 104, seed=90 + i) for i in range(4)]
    m = torch.from_numpy(x).to("cuda")
    o_free = torch.empty(4, dtype=torch.float32, device="cuda")
    o_fixed = torch.empty(4, dtype=torch.float32, device="cuda")
    ws = torch.zeros(armx.workspace_bytes(armx.OP_ROWS, 4, 262_144 + 104)
                     + armx.workspace_bytes(armx.OP_ROWS_FIXED, 4, 262_144 + 104),
                     dtype=torch.uint8, device="cuda")

    def calls():
        armx.reduce_rows(m, out=o_free, workspace=ws)
        armx.reduce_rows_fixed_order(m, out=o_fixed, workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    for rep in range(4):
        m.copy_(torch.from_numpy(pool[rep]).to("cuda"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(o_fixed.cpu().numpy()), bits(fixed_tree_row_sums(pool[rep])))
        eager = armx.reduce_rows(m, workspace=ws).cpu().numpy()
        assert np.array_equal(bits(o_free.cpu().numpy()), bits(eager)), rep


@pytest.mark.parametrize("rows,cols", [(900, 20_000), (1100, 16_400)])
def test_stream_with_a_poor_last_round_is_split(rows, cols):
    # more rows than the free-order stream's wavefronts, but a last round
    # under 90% full: each row is split in two (a workspace)
    assert armx.workspace_bytes(armx.OP_ROWS, rows, cols) > 0, "expected a split plan"
    x = si.generate_rows("normal", rows, cols, seed=rows + cols)
    xd = strided(x, pitch(cols))
    got = armx.reduce_rows(xd).cpu().numpy()
    assert np.array_equal(bits(got), bits(armx.reduce_rows(xd).cpu().numpy()))
    unsplit = no_workspace(armx.lib.reduce_rows, xd)
    idx = np.unique(np.linspace(0, rows - 1, 60).astype(int))
    for r, e in zip(idx, exact_row_sums(x[idx])):
        check_free_order(float(got[r]), e, f"row {r}")
        check_free_order(float(unsplit[r]), e, f"unsplit row {r}")


def test_fixed_order_tail_launch():
    # 2049 rows of 100 chunks: two full rounds of the fixed-order stream (100
    # MiB each, long enough to pay for a second launch), then the last round's
    # single row split over the device in that second launch
    rows, cols = 2049, 51_192
    assert armx.workspace_bytes(armx.OP_ROWS_FIXED, rows, cols) > 0, "expected a tail plan"
    x = si.generate_rows("uniform11", rows, cols, seed=2049)
    xd = strided(x, cols)
    idx = np.unique(np.r_[np.linspace(0, rows - 1, 61).astype(int), rows - 3, rows - 2, rows - 1])
    want = bits(fixed_tree_row_sums(x[idx]))
    assert np.array_equal(bits(armx.reduce_rows_fixed_order(xd).cpu().numpy()[idx]), want)
    assert np.array_equal(bits(no_workspace(armx.lib.reduce_rows_fixed_order, xd)[idx]), want)
    got = armx.reduce_rows_fixed_order(xd, mma_leaves=True).cpu().numpy()
    assert np.array_equal(bits(got[-3:]), bits(fixed_tree_row_sums_mma_leaves(x[-3:])))


def test_fixed_order_two_rounds_in_halves():
    # just past one round of the fixed-order stream, the second round poorly
    # filled: one split launch with every row in two aligned chunk ranges
    rows, cols = 1100, 18_000
    assert armx.workspace_bytes(armx.OP_ROWS_FIXED, rows, cols) > 0, "expected a split plan"
    x = si.generate_rows("uniform11", rows, cols, seed=1100)
    xd = strided(x, pitch(cols), junk=NAN16)
    want = bits(fixed_tree_row_sums(x))
    assert np.array_equal(bits(armx.reduce_rows_fixed_order(xd).cpu().numpy()), want)
    assert np.array_equal(bits(no_workspace(armx.lib.reduce_rows_fixed_order, xd)), want)
    got = armx.reduce_rows_fixed_order(xd, mma_leaves=True).cpu().numpy()
    idx = np.unique(np.linspace(0, rows - 1, 40).astype(int))
    assert np.array_equal(bits(got[idx]), bits(fixed_tree_row_sums_mma_leaves(x[idx])))
