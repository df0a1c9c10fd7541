"""Out-of-bounds writes: every output and workspace region is placed between
guard bands filled with a pattern; after each entry point runs (at sizes with
ragged tails, several blocks and both ticket levels), the guards must be
intact, the workspace's counter region must be back at zero, and the part of
the workspace past what armx_workspace_bytes asks for must be untouched (also
for few long rows, which the row entry points split over blocks with a
workspace, and for rows of at most 512 values, whose sums a block may stage
in LDS and write out a chunk at a time)."""
import numpy as np
import pytest
import torch

import arithmetic_reduction_matrix_amd as armx
import synth_inputs as si
from oracle import fixed_tree_row_sums, fixed_tree_row_sums_mma_leaves

from _parity import require_gpu, to_dev

pytestmark = pytest.mark.gpu

GUARD = 4096      # bytes on each side (a multiple of 256, so regions stay aligned)
PATTERN = 0xA5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


class Guarded:
    """`nbytes` usable bytes between two guard bands of PATTERN."""

    def __init__(self, nbytes: int, fill: int = PATTERN):
        self.n = nbytes
        self.buf = torch.full((GUARD + nbytes + GUARD,), fill, dtype=torch.uint8, device="cuda")
        self.buf[:GUARD] = PATTERN
        self.buf[GUARD + nbytes:] = PATTERN

    def body(self, dtype=torch.uint8):
        return self.buf[GUARD:GUARD + self.n].view(dtype)

    def guards_intact(self) -> bool:
        g = torch.cat([self.buf[:GUARD], self.buf[GUARD + self.n:]])
        return bool((g == PATTERN).all().item())


SIZES = [1, 513, (1 << 20) + 37, (1 << 23) + 4097]


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("name,op,cfg", [
    ("sum", armx.OP_SUM, dict()),
    ("sum-plain", armx.OP_SUM, dict(plain=True)),
    ("sum-one-chain", armx.OP_SUM, dict(one_chain=True, block_threads=64, chain_r=1)),
    ("sum-two-pass", armx.OP_SUM, dict(two_pass=True)),
    ("sum-levels", armx.OP_SUM, dict(mma_levels=True, chain_r=1)),
    ("fixed", armx.OP_FIXED, dict()),
    ("exact", armx.OP_EXACT, dict()),
])
def test_flat_entry_points_stay_in_bounds(n, name, op, cfg):
    x = to_dev(si.generate("uniform11", n, seed=n))
    need = armx.workspace_bytes(op, n, **cfg)
    spare = 1024
    ws = Guarded(need + spare, fill=0)            # zero-filled workspace body
    ws.body()[need:] = PATTERN                     # the unused tail keeps a pattern
    out = Guarded(4)
    fixed = Guarded(16)
    kw = dict(out=out.body(torch.float32).reshape(()), **cfg)
    if need:
        kw["workspace"] = ws.body()[:need]
    for _ in range(2):                             # the second call reuses the workspace
        if op == armx.OP_EXACT:
            armx.reduce_sum_exact(x, fixed=fixed.body(torch.int64), **kw)
        elif op == armx.OP_FIXED:
            armx.reduce_sum_fixed_order(x, **kw)
        else:
            armx.reduce_sum(x, **kw)
    torch.cuda.synchronize()
    assert out.guards_intact() and ws.guards_intact() and fixed.guards_intact(), (name, n)
    assert bool((ws.body()[need:] == PATTERN).all().item()), (name, n, "workspace tail")
    if need:   # the ticket paths restore their counters; the levels form never touches them
        assert int(ws.body()[:armx.COUNTER_BYTES].count_nonzero().item()) == 0, (name, n, "counter region")


# rows of at most 512 values: the direct kernel (8 values) and the staged one
# (45, 64, 100, 512 values: chunks of rows through LDS, a ragged last row for
# 45 and 100, one block looping over several chunks with grid_blocks=2)
_SHORT = [(1, 1, {}), (5000, 8, {}), (3001, 45, {}), (40_000, 64, {}), (20_001, 100, {}),
          (777, 512, {}), (40_000, 64, dict(grid_blocks=2)), (20_001, 100, dict(grid_blocks=2))]


@pytest.mark.parametrize("rows,cols,cfg", _SHORT)
@pytest.mark.parametrize("fixed_order,mma_leaves", [(False, False), (True, False), (True, True)])
def test_short_rows_stay_in_bounds(rows, cols, cfg, fixed_order, mma_leaves):
    ld = (cols + 7) // 8 * 8
    x = si.generate_rows("normal", rows, cols, seed=rows + cols)
    buf = np.zeros((rows, ld), np.float16)
    buf[:, :cols] = x
    m = to_dev(buf)[:, :cols]
    out = Guarded(4 * rows)
    fn = armx.reduce_rows_fixed_order if fixed_order else armx.reduce_rows
    extra = dict(mma_leaves=True) if mma_leaves else {}
    fn(m, out=out.body(torch.float32), **cfg, **extra)
    torch.cuda.synchronize()
    assert out.guards_intact(), (rows, cols, cfg, fixed_order, mma_leaves)
    got = out.body(torch.float32).cpu().numpy()
    want = fixed_tree_row_sums_mma_leaves(x) if mma_leaves else fixed_tree_row_sums(x)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), (rows, cols, cfg)


@pytest.mark.parametrize("rows,cols", [(1, 1), (3, 700), (300, 4096), (4097, 2048 + 8),
                                       (1000, 33001)])
@pytest.mark.parametrize("fixed_order", [False, True])
def test_row_entry_points_stay_in_bounds(rows, cols, fixed_order):
    ld = (cols + 7) // 8 * 8
    m = to_dev(si.generate_rows("normal", rows, ld, seed=rows))[:, :cols]
    out = Guarded(4 * rows)
    fn = armx.reduce_rows_fixed_order if fixed_order else armx.reduce_rows
    fn(m, out=out.body(torch.float32))
    torch.cuda.synchronize()
    assert out.guards_intact(), (rows, cols, fixed_order)


_FEW_ROWS = [(rows, cols, fo, mm) for rows, cols in
             [(1, (1 << 22) + 13), (5, 200_000), (100, 66_000)]
             for fo, mm in [(False, False), (True, False), (True, True)]]
# row streams whose last round would be poorly filled (on 256 compute units):
# the fixed-order stream plus a split second launch over the last rows
# (2049 x 51192), every row in two aligned ranges in one launch (1100 x
# 18000, both fixed orders), and the free-order stream split in two halves
# (900 x 20000)
_LAST_ROUND = [(2049, 51192, True, False), (2049, 51192, True, True),
               (1100, 18000, True, False), (1100, 18000, True, True),
               (900, 20000, False, False)]


@pytest.mark.parametrize("rows,cols,fixed_order,mma_leaves", _FEW_ROWS + _LAST_ROUND)
def test_split_rows_stay_in_bounds(rows, cols, fixed_order, mma_leaves):
    # few long rows split over blocks (a workspace): guards intact, counter
    # region back at zero, the workspace tail untouched, over two calls
    op = armx.OP_ROWS_FIXED if fixed_order else armx.OP_ROWS
    cfg = dict(mma_leaves=True) if mma_leaves else {}
    need = armx.workspace_bytes(op, rows, cols, **cfg)
    assert need > 0
    ld = (cols + 7) // 8 * 8
    m = to_dev(si.generate_rows("normal", rows, ld, seed=rows))[:, :cols]
    ws = Guarded(need + 1024, fill=0)
    ws.body()[need:] = PATTERN
    out = Guarded(4 * rows)
    fn = armx.reduce_rows_fixed_order if fixed_order else armx.reduce_rows
    first = fn(m, out=out.body(torch.float32), workspace=ws.body()[:need], **cfg).clone()
    second = fn(m, out=out.body(torch.float32), workspace=ws.body()[:need], **cfg)
    torch.cuda.synchronize()
    assert torch.equal(first, second)
    assert out.guards_intact() and ws.guards_intact(), (rows, cols)
    assert bool((ws.body()[need:] == PATTERN).all().item()), (rows, cols, "workspace tail")
    assert int(ws.body()[:armx.COUNTER_BYTES].count_nonzero().item()) == 0, (rows, cols, "counter region")
