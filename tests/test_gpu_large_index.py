"""Inputs past 2^32 elements (64-bit indexing).  n = 2^32 + 4099 binary16
values, ones except the last 4099, which are twos: a kernel that wrapped an
index at 2^32 would read ones where the twos are, or miss the tail.  Expected
values are closed forms:
  exact sum    Q = (2^32 + 2 * 4099) * 2^24 (the 128-bit output), rounded once;
  fixed order  the padded tree's left half [0, 2^32) is all ones, so exactly
               2^32; the right half holds the 4099 twos (8198, exact); the root
               is the binary32 nearest to 2^32 + 8198 -> 2^32 + 8192;
  free order   within the free-order gate of 2^32 + 8198;
  rows         65537 rows of 65536 (2^32 + 65536 values): every row of ones
               sums to 65536 exactly, the last row (twos) to 131072;
  short rows   2^26 + 1 rows of 60 values at pitch 64 (the pitch padding also
               ones): 60 per row, 120 for the last row (twos);
  ragged rows  4294968 rows of 1000 values (past 2^32 values): 1000 per row,
               2000 for the last row (twos);
  one row      the whole input as one row, split over many blocks: the flat
               sums' closed forms."""
import numpy as np
import pytest
import torch

import arithmetic_reduction_matrix_amd as armx
from oracle.exact import ExactSum

from _parity import check_free_order, require_gpu

pytestmark = pytest.mark.gpu

TAIL = 4099
N = (1 << 32) + TAIL


@pytest.fixture(scope="module")
def big():
    require_gpu()
    x = torch.ones(N, dtype=torch.float16, device="cuda")
    x[-TAIL:] = 2.0
    yield x
    del x
    torch.cuda.empty_cache()


def test_exact_and_fixed_order_past_2p32(big):
    q = torch.zeros(2, dtype=torch.int64, device="cuda")
    e = armx.reduce_sum_exact(big, fixed=q)
    want = (1 << 32) + 2 * TAIL
    assert armx.fixed_to_int(q.cpu()) == want << 24
    assert e.item() == float(np.float32(want))
    f = armx.reduce_sum_fixed_order(big)
    assert f.item() == float((1 << 32) + 8192)


def test_free_order_and_levels_past_2p32(big):
    want = (1 << 32) + 2 * TAIL
    exact = ExactSum(want << 24, want << 24, N)
    for cfg in (dict(), dict(plain=True), dict(mma_levels=True), dict(chain_r=3, block_threads=1024)):
        check_free_order(armx.reduce_sum(big, **cfg).item(), exact, str(cfg))


def test_one_row_past_2p32_split(big):
    # the whole input as one row: split over wavefronts of many blocks (the
    # same closed forms as the flat sums)
    row = big.view(1, N)
    assert armx.workspace_bytes(armx.OP_ROWS, 1, N) > 0
    assert armx.workspace_bytes(armx.OP_ROWS_FIXED, 1, N) > 0
    assert armx.reduce_rows_fixed_order(row).item() == float((1 << 32) + 8192)
    assert armx.reduce_rows_fixed_order(row, mma_leaves=True).item() == float((1 << 32) + 8192)
    want = (1 << 32) + 2 * TAIL
    exact = ExactSum(want << 24, want << 24, N)
    for cfg in (dict(), dict(plain=True)):
        check_free_order(armx.reduce_rows(row, **cfg).item(), exact, str(cfg))


def test_rows_past_2p32():
    require_gpu()
    rows, cols = 65537, 65536
    m = torch.ones((rows, cols), dtype=torch.float16, device="cuda")
    m[-1] = 2.0
    want = torch.full((rows,), 65536.0, device="cuda")
    want[-1] = 131072.0
    for fn, cfg in ((armx.reduce_rows, {}), (armx.reduce_rows, dict(plain=True)),
                    (armx.reduce_rows_fixed_order, {})):
        got = fn(m, **cfg)
        assert torch.equal(got, want), (fn.__name__, cfg)
    del m
    torch.cuda.empty_cache()


@pytest.mark.parametrize("rows,cols,ld", [((1 << 26) + 1, 60, 64), (4294968, 1000, 1000)])
def test_short_and_ragged_rows_past_2p32(rows, cols, ld):
    require_gpu()
    buf = torch.ones((rows, ld), dtype=torch.float16, device="cuda")
    buf[-1] = 2.0
    m = buf[:, :cols]
    want = torch.full((rows,), float(cols), device="cuda")
    want[-1] = 2.0 * cols
    for fn in (armx.reduce_rows, armx.reduce_rows_fixed_order):
        got = fn(m)
        assert torch.equal(got, want), (fn.__name__, rows, cols, ld)
    del buf, m
    torch.cuda.empty_cache()
