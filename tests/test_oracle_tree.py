"""Pins the fixed balanced-tree oracle: hand-derived worked examples,
invariants, closed forms, the pairwise-summation error bound and rational
brute force on tiny inputs.  The order is the balanced-tree reduction of
"Taming Bitwise Behavior in GPU Kernels with Tensor Core" (arXiv 2609.11356,
Abstract) with the 32-bit partials of "GPU Tensor Cores for fast Arithmetic
Reductions" (arXiv 2001.05585, Abstract)."""
import math
import random
from fractions import Fraction

import numpy as np
import pytest

import synth_inputs as si
from oracle import exact_sum, fixed_tree_row_sums, fixed_tree_sum, to_binary32, tree_over_nodes

from _golden import bits32, tree_examples

EXAMPLES = tree_examples()


@pytest.mark.parametrize("name,x,tree,seq,exact,note", EXAMPLES, ids=[e[0] for e in EXAMPLES])
def test_worked_examples(name, x, tree, seq, exact, note):
    assert bits32(fixed_tree_sum(x)) == bits32(tree), note
    assert bits32(exact_sum(x).f32) == bits32(exact), note
    # the sequential column is checked too, so every fixture row is consistent
    acc = np.float32(x[0])
    for v in x[1:]:
        acc = np.float32(acc + np.float32(v))
    assert bits32(acc) == bits32(seq), note


def test_examples_discriminate_orders():
    # the fixtures must tell the prescribed order apart from the obvious
    # alternatives, or they would not pin it
    assert any(bits32(t) != bits32(s) for _, _, t, s, _, _ in EXAMPLES)
    assert any(bits32(t) != bits32(e) for _, _, t, _, e, _ in EXAMPLES)


def test_empty_is_positive_zero():
    r = fixed_tree_sum(np.array([], np.float16))
    assert r == 0 and not np.signbit(r)


@pytest.mark.parametrize("n", [1, 2, 3, 5, 255, 256, 257, 1000, 4096, 65537])
def test_negation_is_exact_mirror(n):
    x = si.generate("uniform11", n, seed=n)
    assert bits32(fixed_tree_sum(-x)) == bits32(-fixed_tree_sum(x))


@pytest.mark.parametrize("k", [-8, -3, 1, 4])
def test_power_of_two_scaling(k):
    # values with few significant bits, scaled so everything stays normal and
    # finite in binary16 and far from binary32 limits
    rng = np.random.default_rng(5)
    x = (rng.integers(-512, 512, 3001) * 2.0 ** -4).astype(np.float16)
    y = (x.astype(np.float64) * 2.0 ** k).astype(np.float16)
    assert np.array_equal(y.astype(np.float64), x.astype(np.float64) * 2.0 ** k)
    assert fixed_tree_sum(y) == np.float32(fixed_tree_sum(x) * np.float32(2.0 ** k))


@pytest.mark.parametrize("n", [1, 2, 3, 17, 256, 257, 4095, 1 << 20, (1 << 20) + 3])
def test_ones_and_ramp_are_exact(n):
    # every partial is an integer below 2^24, so the tree is exact and any
    # dropped or doubled term shows
    assert fixed_tree_sum(si.generate("ones", n)) == np.float32(n)
    r = si.generate("ramp2048", n)
    assert fixed_tree_sum(r) == exact_sum(r).f32


def _pairwise_bound(e):
    # |tree - S| <= gamma_h * sum|x_i|, gamma_h = h u / (1 - h u), h = ceil(log2 n)
    h = max(1, math.ceil(math.log2(max(e.n, 2))))
    u = 2.0 ** -24
    return (h * u / (1 - h * u)) * e.abs_sum


@pytest.mark.parametrize("dist,n,seed", [
    ("uniform11", 1 << 18, 1), ("normal", 100_000, 2), ("logu_signed", 1 << 16, 3),
    ("bits_finite", 1 << 12, 4), ("uniform01", 77_777, 5),
])
def test_error_within_pairwise_bound(dist, n, seed):
    x = si.generate(dist, n, seed)
    e = exact_sum(x)
    err = abs(Fraction(float(fixed_tree_sum(x))) - Fraction(e.q, 1 << 24))
    assert err <= Fraction(_pairwise_bound(e))


def _tree_brute(vals):
    """Recursive halving with exact rational sums, each node rounded to binary32
    by the oracle's once-rounding routine (independent of numpy's addition)."""
    n = len(vals)
    size = 1 << (n - 1).bit_length()
    leaves = [Fraction(float(v)) for v in vals] + [None] * (size - n)

    def node(lo, hi):
        if hi - lo == 1:
            return leaves[lo]
        a, b = node(lo, (lo + hi) // 2), node((lo + hi) // 2, hi)
        if b is None:
            return a
        if a is None:
            return b
        s = a + b
        return Fraction(float(to_binary32(int(s * (1 << 24)))))   # s is a multiple of 2^-24

    return node(0, size)


@pytest.mark.parametrize("seed", range(12))
def test_tiny_inputs_against_rational_recursion(seed):
    rng = random.Random(seed)
    n = rng.randint(1, 70)
    x = si.generate("bits_finite", n, seed=1000 + seed)
    # keep magnitudes moderate so no node can overflow binary32 (it cannot
    # anyway: |x| <= 65504 and n <= 70)
    got = Fraction(float(fixed_tree_sum(x)))
    assert got == _tree_brute(x)


def test_rows_equal_flat_tree_per_row():
    x = si.generate_rows("uniform11", 9, 1000, seed=3)
    rows = fixed_tree_row_sums(x)
    for r in range(9):
        assert bits32(rows[r]) == bits32(fixed_tree_sum(x[r]))


def test_tile_subtrees_compose():
    # a 256-leaf tile is a complete subtree: summing tiles first, then the
    # tile results in the same balanced tree, is the same computation
    x = si.generate("normal", 256 * 64, seed=8)
    tiles = fixed_tree_row_sums(x.reshape(64, 256))
    level = tiles.astype(np.float32)
    while level.size > 1:
        level = level[0::2] + level[1::2]
    assert bits32(level[0]) == bits32(fixed_tree_sum(x))


@pytest.mark.parametrize("n,log2_part", [(1000, 6), (100_003, 12), (1 << 16, 16), (5, 2),
                                         (70_000, 17)])
def test_tree_over_nodes_continues_the_tree(n, log2_part):
    # the roots of consecutive aligned subtrees of 2^k leaves (the last one
    # short) are level-k nodes: the tree over them is the whole tree's root
    x = si.generate("logu_signed", n, seed=n)
    step = 1 << log2_part
    roots = [fixed_tree_sum(x[i:i + step]) for i in range(0, n, step)]
    assert bits32(tree_over_nodes(np.array(roots, np.float32))) == bits32(fixed_tree_sum(x))


def test_tree_over_nodes_worked_example():
    # the nodes 1, 2^-24, 2^-24, 2^-24: (1 + 2^-24) is a tie -> 1, (2^-24 +
    # 2^-24) = 2^-23, 1 + 2^-23 exact; left to right would give 1.0
    got = tree_over_nodes(np.array([1, 2.0 ** -24, 2.0 ** -24, 2.0 ** -24], np.float32))
    assert got == np.float32(1 + 2.0 ** -23)
    # three nodes: the fourth is -0.0 padding, so +0.0 + +0.0 stays +0.0
    assert bits32(tree_over_nodes(np.array([0.0, 0.0, 0.0], np.float32))) == 0
    assert bits32(tree_over_nodes(np.array([-0.0, -0.0, -0.0], np.float32))) == 0x80000000
    assert bits32(tree_over_nodes(np.array([], np.float32))) == 0


def test_specials():
    x = np.ones(300, np.float16)
    x[17] = np.inf
    assert fixed_tree_sum(x) == np.inf
    x[200] = -np.inf
    assert np.isnan(fixed_tree_sum(x))
