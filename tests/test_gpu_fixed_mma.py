"""reduce_sum_fixed_order with ARMX_FLAG_MMA_LEAVES against the oracle's
MFMA-leaf order (oracle.tree fixed_tree_sum_mma_leaves, built on the
reconstructed MFMA accumulation of oracle.mfma_model), bit for bit, for every
block size, chain length and grid: the balanced-tree reproducibility of
"Taming Bitwise Behavior in GPU Kernels with Tensor Core" (arXiv 2609.11356,
Abstract) with tensor-core leaves."""
import numpy as np
import pytest
import torch

import arithmetic_reduction_matrix_amd as armx
import synth_inputs as si
from oracle import exact_sum
from oracle.tree import fixed_tree_sum_mma_leaves

from _parity import bits32, check_free_order, require_gpu, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def mma(xd, **cfg):
    return bits32(armx.reduce_sum_fixed_order(xd, mma_leaves=True, **cfg).cpu().numpy())


@pytest.mark.parametrize("n", [1, 2, 7, 8, 9, 255, 256, 511, 512, 513, 1023, 1025, 4097,
                               65536 + 3, (1 << 20) - 1, (1 << 20) + 37, 3 * (1 << 20) + 1234])
@pytest.mark.parametrize("dist", ["uniform11", "logu_signed"])
def test_sizes(n, dist):
    x = si.generate(dist, n, seed=n + 7)
    want = bits32(fixed_tree_sum_mma_leaves(x))
    xd = to_dev(x)
    assert mma(xd) == want
    assert mma(xd, block_threads=1024, chain_r=5) == want


@pytest.mark.parametrize("dist", ["bits_finite", "logu_signed", "normal", "uniform01"])
def test_block_chain_matrix(dist):
    n = (1 << 21) + 4099
    x = si.generate(dist, n, seed=31)
    want = bits32(fixed_tree_sum_mma_leaves(x))
    xd = to_dev(x)
    for block in (64, 256, 1024):
        for r in (1, 2, 3, 4, 5, 8):
            assert mma(xd, block_threads=block, chain_r=r) == want, (block, r)
    for extra in (dict(grid_blocks=1), dict(grid_blocks=7), dict(two_pass=True),
                  dict(cached_loads=True), dict(block_threads=128, grid_blocks=300)):
        assert mma(xd, **extra) == want, extra


def test_differs_from_the_valu_order_but_stays_close():
    # the two prescribed orders are different orders; both are within the
    # free-order gate of the exact sum
    x = si.generate("logu_signed", (1 << 22) + 5, seed=41)
    xd = to_dev(x)
    a = armx.reduce_sum_fixed_order(xd, mma_leaves=True).item()
    b = armx.reduce_sum_fixed_order(xd).item()
    e = exact_sum(x)
    check_free_order(a, e, "mma leaves")
    check_free_order(b, e, "valu tree")


def test_special_values():
    base = si.generate("uniform11", 5000, seed=3)
    cases = []
    x = base.copy(); x[17] = np.inf; cases.append(x)
    x = base.copy(); x[17] = np.inf; x[4000] = -np.inf; cases.append(x)   # different chunks
    x = base.copy(); x[0] = np.inf; x[128] = -np.inf; cases.append(x)     # same column
    x = base.copy(); x[3333] = np.nan; cases.append(x)
    x = base.copy(); x[:] = np.float16(-0.0); cases.append(x)
    x = np.full(3000, 65504.0, np.float16); cases.append(x)               # largest binary16
    for i, x in enumerate(cases):
        got = armx.reduce_sum_fixed_order(to_dev(x), mma_leaves=True).cpu().numpy()
        want = fixed_tree_sum_mma_leaves(x)
        if np.isnan(want):
            assert np.isnan(got), i
        else:
            assert bits32(got) == bits32(want), i


def test_full_2p26_workload():
    x = si.workload("fixed_2p26_u11")
    want = bits32(fixed_tree_sum_mma_leaves(x))
    xd = to_dev(x)
    assert mma(xd) == want
    assert mma(xd, block_threads=256, chain_r=4) == want
