"""The gfx950 MFMA accumulation against its reconstructed model
(oracle.mfma_model): black-box probing of the tile step the sum kernels use,
as "Taming Bitwise Behavior in GPU Kernels with Tensor Core" (arXiv
2609.11356, Abstract) does for closed libraries.

A row of reduce_rows with the all-ones operand (ARMX_FLAG_ALL_ONES) and R x
512 values (then a chain of zeros) whose only non-zero values sit in MFMA
column 0 returns exactly that column's chain of R MFMAs: the other 15 column sums are zero and the combines only add zeros.  Column 0's
K position k is element (k // 8) * 128 + k % 8 of each 512-value tile (lane
16 (k // 8) holds K values 8 (k // 8) .. + 7 of column 0)."""
import numpy as np
import pytest
import torch

import arithmetic_reduction_matrix_amd as armx
from oracle import exact_sum
from oracle.mfma_model import chain_column

from _parity import require_gpu, to_dev

pytestmark = pytest.mark.gpu

U = 2.0 ** -24
KPOS = np.array([(k // 8) * 128 + k % 8 for k in range(32)])


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def gpu_chains(tiles: np.ndarray) -> np.ndarray:
    """tiles: (n, R, 32) binary16 K values of column 0 -> (n,) binary32.
    Each row is the chain's R tiles and then one more chain of zeros: rows of
    at most 512 values would take the MFMA-free short-row kernel, and adding
    the zero chain's +0.0 to the chain value is exact."""
    n, R, _ = tiles.shape
    x = np.zeros((n, 512 * (R + 1)), np.float16)
    for r in range(R):
        x[:, r * 512 + KPOS] = tiles[:, r, :]
    return armx.reduce_rows(to_dev(x), chain_r=R, block_threads=64,
                            all_ones=True).cpu().numpy()


def col(*pairs):
    v = np.zeros(32, np.float16)
    for k, x in pairs:
        v[k] = x
    return v


TARGETED = [
    ([col((0, 1024.0), *[(k, 2.0 ** -15) for k in range(1, 8)])], 1024.0),
    ([col((0, 1024.0), *[(k, -2.0 ** -15) for k in range(1, 8)])], 1024.0),
    ([col((0, 2.0), (1, 3 * U))], 2.0),
    ([col((0, 1024.0), (1, -1024.0), (2, 2.0 ** -20))], 0.0),
    ([col((0, 1.0), (1, U), (7, U))], 1.0 + 2 * U),
    ([col((0, 1.0), (1, U), (8, U))], 1.0),
    ([col((8, U), (16, U), (24, 1.0))], 1.0 + 2 * U),
    ([col((0, 1024.0)), col((0, 2.0 ** -14), (1, 2.0 ** -20))], 1024.0 + 2.0 ** -13),
    ([col((0, 1024.0)), col((0, 2.0 ** -14), (1, 2.0 ** -24))], 1024.0),
    ([col((0, 1024.0)), col((0, 2.0 ** -14), (1, 2.0 ** -23), (2, -2.0 ** -24))], 1024.0),
    ([col((0, 1024.0)), col(*[(k, -2.0 ** -17) for k in range(32)])], 1024.0 - 4 * 2.0 ** -14),
    ([col((0, 1024.0)), col(*[(k, 2.0 ** -17) for k in range(32)])], 1024.0),
    # the products' sum floored once (per-product floors would round up)
    ([col((0, 1024.0)), col((0, 2.0 ** -14 + 2.0 ** -21), (1, -2.0 ** -24))], 1024.0),
    ([col((0, -1024.0)), col((0, 2.0 ** -14 + 2.0 ** -21), (1, -2.0 ** -24))],
     -1024.0 + 2.0 ** -14),
    ([col((0, 2.0 ** -14 + 2.0 ** -21), (1, -2.0 ** -24))], 2.0 ** -14 + 7 * U),
]


def test_targeted_cases_match_the_model_bit_for_bit():
    by_r = {}
    for tiles, want in TARGETED:
        by_r.setdefault(len(tiles), []).append((np.stack(tiles), want))
    for R, cases in by_r.items():
        got = gpu_chains(np.stack([t for t, _ in cases]))
        for (t, want), g in zip(cases, got):
            assert float(chain_column(t)) == want          # the model, as derived
            assert float(g) == want, (R, t[np.nonzero(t)], float(g), want)


def random_tiles(rng, n, R):
    """Column values with wide dynamic range: full-range patterns, narrow
    exponent bands, and single-sign columns."""
    bits = rng.integers(0, 0x7C00, (n, R, 32)).astype(np.uint16)
    sign = (rng.integers(0, 2, (n, R, 32)) << 15).astype(np.uint16)
    fam = rng.integers(0, 3, n)[:, None, None]
    band_e = np.clip(rng.integers(0, 31, n)[:, None, None] + rng.integers(-3, 4, (n, R, 32)), 0, 30)
    band = ((band_e << 10) | rng.integers(0, 1024, (n, R, 32))).astype(np.uint16)
    v = np.where(fam == 1, band | sign, bits | sign)
    v = np.where(fam == 2, v & 0x7FFF, v)
    return v.astype(np.uint16).view(np.float16)


@pytest.mark.parametrize("R,n", [(1, 20000), (2, 10000), (4, 5000), (8, 3000)])
def test_random_columns_follow_the_model(R, n):
    # fresh seeds (not those the model was fitted on): every chain must match
    # the model bit for bit
    rng = np.random.default_rng(1000 + R)
    tiles = random_tiles(rng, n, R)
    got = gpu_chains(tiles)
    model = np.array([chain_column(t) for t in tiles], dtype=np.float32)
    same = got.view(np.uint32) == model.view(np.uint32)
    off = np.abs(got.view(np.int32).astype(np.int64) - model.view(np.int32).astype(np.int64))
    print(f"R={R}: {int(same.sum())} of {n} bit-identical to the model; "
          f"differences (ulps): {sorted(set(off[~same].tolist()))}")
    assert same.all(), [(i, float(got[i]), float(model[i])) for i in np.nonzero(~same)[0][:5]]


@pytest.mark.parametrize("R", [2, 4])
def test_accumulator_dominated_chains_follow_the_model(R):
    # a large first tile, then tiles 6 to 29 binades smaller with mixed signs:
    # the accumulator bound binds in every later group
    rng = np.random.default_rng(2000 + R)
    n = 6000
    hi_e = rng.integers(24, 31, (n, 1, 32))
    lo_e = np.clip(hi_e - rng.integers(6, 30, (n, R - 1, 32)), 0, 30)
    e = np.concatenate([hi_e, lo_e], axis=1)
    bits = (e << 10) | rng.integers(0, 1024, (n, R, 32))
    bits |= rng.integers(0, 2, (n, R, 32)) << 15
    tiles = bits.astype(np.uint16).view(np.float16)
    got = gpu_chains(tiles)
    model = np.array([chain_column(t) for t in tiles], dtype=np.float32)
    same = got.view(np.uint32) == model.view(np.uint32)
    assert same.all(), [(i, float(got[i]), float(model[i])) for i in np.nonzero(~same)[0][:5]]


def test_mfma_is_not_correctly_rounded_and_leans_negative():
    # one MFMA per column: compare with the correctly rounded exact sum
    rng = np.random.default_rng(7)
    tiles = random_tiles(rng, 2000, 1)
    got = gpu_chains(tiles)
    exact = [exact_sum(t[0]) for t in tiles]
    cr = np.array([e.f32 for e in exact], dtype=np.float32)
    differs = got.view(np.uint32) != cr.view(np.uint32)
    err = np.array([float(g) - e.f64 for g, e in zip(got, exact)])
    print(f"not correctly rounded: {int(differs.sum())} of {len(got)}; "
          f"mean signed error {err.mean():.3e}, negative {int((err < 0).sum())}, "
          f"positive {int((err > 0).sum())}")
    assert differs.mean() > 0.2
    assert (err < 0).sum() > (err > 0).sum()
