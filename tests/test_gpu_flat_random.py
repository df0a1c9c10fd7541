"""Seeded random sizes and configurations through the flat entry points, so
that every grid the planner builds (small-input caps, persistent grids, one
chain per wavefront, one- and two-level tickets, two passes) meets sizes
nobody picked by hand: reduce_sum_fixed_order equals the balanced-tree oracle
bit for bit (both orders), reduce_sum_exact the correctly rounded exact sum,
and reduce_sum (MFMA, MFMA-free and the recursive MMA form) passes the
free-order gate ("GPU Tensor Cores for fast Arithmetic Reductions", arXiv
2001.05585, Abstract: 32-bit chain sub-results)."""
import numpy as np
import pytest

import arithmetic_reduction_matrix_amd as armx
import synth_inputs as si
from oracle import exact_sum, fixed_tree_sum
from oracle.tree import fixed_tree_sum_mma_leaves

from _parity import bits32, check_free_order, require_gpu, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def draw_case(seed):
    rng = np.random.default_rng(seed)
    n = int(np.exp(rng.uniform(0, np.log(12_000_000))))
    cfg = {}
    if rng.integers(0, 2):
        cfg["block_threads"] = int(64 * 2 ** rng.integers(0, 5))
    if rng.integers(0, 2):
        cfg["chain_r"] = int(rng.integers(1, 9))
    if rng.integers(0, 3) == 0:
        cfg["grid_blocks"] = int(rng.integers(1, 5000))
    if rng.integers(0, 4) == 0:
        cfg["cached_loads"] = True
    dist = ["uniform11", "normal", "logu_signed", "bits_finite"][int(rng.integers(0, 4))]
    return n, cfg, dist


@pytest.mark.parametrize("seed", range(120))
def test_random_flat_sizes(seed):
    n, cfg, dist = draw_case(seed)
    x = si.generate(dist, n, seed=seed)
    xd = to_dev(x)
    what = (n, cfg, dist)
    e = exact_sum(x)
    # the fixed order takes power-of-two blocks only; the others any block size
    assert bits32(armx.reduce_sum_fixed_order(xd, **cfg).item()) == bits32(fixed_tree_sum(x)), what
    if seed % 3 == 0:
        got = armx.reduce_sum_fixed_order(xd, mma_leaves=True, **cfg).item()
        assert bits32(got) == bits32(fixed_tree_sum_mma_leaves(x)), what
    assert bits32(armx.reduce_sum_exact(xd, **cfg).item()) == bits32(e.f32), what
    for extra in ({}, dict(plain=True), dict(two_pass=True)):
        check_free_order(armx.reduce_sum(xd, **cfg, **extra).item(), e, f"{what} {extra}")
    if "grid_blocks" not in cfg:
        check_free_order(armx.reduce_sum(xd, mma_levels=True, **cfg).item(), e, f"{what} levels")
        if n >= 512:
            one = dict(cfg, one_chain=True)
            check_free_order(armx.reduce_sum(xd, **one).item(), e, f"{what} one chain")
