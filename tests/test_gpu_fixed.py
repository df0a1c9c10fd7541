"""reduce_sum_fixed_order against the balanced-tree oracle: bit for bit, for
every block size and chain length.  The order is the balanced-tree reduction
of "Taming Bitwise Behavior in GPU Kernels with Tensor Core" (arXiv
2609.11356, Abstract), with fp32 partials ("GPU Tensor Cores for fast
Arithmetic Reductions", arXiv 2001.05585, Abstract)."""
import numpy as np
import pytest
import torch

import arithmetic_reduction_matrix_amd as armx
import synth_inputs as si
from oracle import fixed_tree_sum

from _golden import tree_examples
from _parity import bits32, require_gpu, to_dev

pytestmark = pytest.mark.gpu

BLOCKS = [64, 256, 1024]
CHAINS = [1, 2, 4, 5]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def fixed(xd, **cfg):
    return bits32(armx.reduce_sum_fixed_order(xd, **cfg).cpu().numpy())


@pytest.mark.parametrize("name,x,tree,seq,exact,note", tree_examples(),
                         ids=[e[0] for e in tree_examples()])
def test_worked_examples(name, x, tree, seq, exact, note):
    assert fixed(to_dev(x)) == bits32(tree), note


@pytest.mark.parametrize("n", [1, 2, 3, 7, 8, 9, 255, 256, 257, 511, 512, 513, 1023, 1024, 1025,
                               4097, 65536 + 3, (1 << 20) - 1, (1 << 20) + 37,
                               3 * (1 << 20) + 1234])
def test_sizes(n):
    x = si.generate("uniform11", n, seed=n)
    want = bits32(fixed_tree_sum(x))
    xd = to_dev(x)
    assert fixed(xd) == want
    assert fixed(xd, block_threads=1024, chain_r=5) == want


@pytest.mark.parametrize("dist", ["bits_finite", "logu_signed", "normal", "uniform01"])
def test_block_chain_matrix(dist):
    n = (1 << 21) + 4099
    x = si.generate(dist, n, seed=21)
    want = bits32(fixed_tree_sum(x))
    xd = to_dev(x)
    for block in BLOCKS:
        for r in CHAINS:
            assert fixed(xd, block_threads=block, chain_r=r) == want, (block, r)


@pytest.mark.parametrize("extra", [dict(chain_r=3), dict(chain_r=6), dict(chain_r=7),
                                   dict(chain_r=8), dict(block_threads=128),
                                   dict(block_threads=512), dict(cached_loads=True),
                                   dict(two_pass=True), dict(grid_blocks=1),
                                   dict(grid_blocks=3), dict(grid_blocks=4096),
                                   dict(two_pass=True, grid_blocks=3000)])
def test_other_configs(extra):
    n = (1 << 20) + 777
    x = si.generate("normal", n, seed=5)
    assert fixed(to_dev(x), **extra) == bits32(fixed_tree_sum(x)), extra


def test_signed_zeros_and_specials():
    z = armx.reduce_sum_fixed_order(torch.empty(0, dtype=torch.float16, device="cuda"))
    assert bits32(z.cpu().numpy()) == 0
    negz = np.full(1000, -0.0, np.float16)
    assert fixed(to_dev(negz)) == bits32(np.float32(-0.0))
    x = si.generate("uniform11", 5000, seed=1)
    x[123] = np.inf
    assert fixed(to_dev(x)) == bits32(np.float32(np.inf))
    x[4000] = -np.inf
    assert np.isnan(armx.reduce_sum_fixed_order(to_dev(x)).item())


def test_every_binary16_value_first_level():
    # n = 2 inputs [h, +0]: the root is level 1, fl32(h + 0), which is h
    # exactly (a -0 input gives +0); every pattern, subnormals included
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = np.zeros((65536, 8), np.uint16)
    x[:, 0] = pats
    xd = to_dev(x.view(np.float16).reshape(-1))
    out = torch.empty(65536, dtype=torch.float32, device="cuda")
    for i in range(65536):
        armx.reduce_sum_fixed_order(xd[8 * i: 8 * i + 2], out=out[i:i + 1])
    got = out.cpu().numpy()
    want = np.array([fixed_tree_sum(np.array([p, 0], np.uint16).view(np.float16))
                     for p in range(0, 65536, 1)], np.float32)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))


def test_random_pairs_and_quads():
    # level 1 and 2 rounding on random patterns (wide exponent range)
    for n in (2, 4, 8):
        x = si.generate("bits_finite", 4096 * n, seed=n).reshape(4096, n)
        buf = np.zeros((4096, 8), np.float16)
        buf[:, :n] = x
        xd = to_dev(buf.reshape(-1))
        out = torch.empty(4096, dtype=torch.float32, device="cuda")
        for i in range(4096):
            armx.reduce_sum_fixed_order(xd[8 * i: 8 * i + n], out=out[i:i + 1])
        got = out.cpu().numpy()
        want = np.array([fixed_tree_sum(x[i]) for i in range(4096)], np.float32)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), n


def test_full_2p26_bit_identity_matrix():
    x = si.workload("fixed_2p26_u11")
    want = bits32(fixed_tree_sum(x))
    xd = to_dev(x)
    seen = {}
    for block in BLOCKS:
        for r in CHAINS:
            seen[(block, r)] = fixed(xd, block_threads=block, chain_r=r)
    assert set(seen.values()) == {want}, seen
    assert fixed(xd, cached_loads=True) == want
    assert fixed(xd, two_pass=True) == want


def test_large_n_node_logs():
    # 2^30 values: long per-wavefront node logs (per chunk for R = 5, per
    # group of 8 for R = 8) and several rows of 64 in the wavefront tree
    x = si.generate("uniform11", 1 << 30, seed=31)
    want = bits32(fixed_tree_sum(x))
    xd = to_dev(x)
    del x
    for cfg in (dict(), dict(chain_r=5), dict(block_threads=1024, chain_r=1),
                dict(block_threads=64, chain_r=2)):
        assert fixed(xd, **cfg) == want, cfg
