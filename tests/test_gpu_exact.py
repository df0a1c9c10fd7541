"""reduce_sum_exact against the exact-sum oracle, bit for bit: the binary32
result must be the oracle's correctly rounded S (round to nearest, ties to
even) and the 128-bit output must equal the oracle's integer Q = S 2^24.
The operation is the arithmetic reduction of "GPU Tensor Cores for fast
Arithmetic Reductions" (arXiv 2001.05585, Abstract) kept free of rounding
error up to the final 32-bit result; the sum is carried as integer limbs with
fixed weights, the representation of "AWE: Adaptive Weight Encoding ..."
(arXiv 2609.24519, Abstract).  Both forms are checked: binary64 chain sums
into two 32-bit limbs (the default), and eight signed 8-bit limbs per value
summed by integer MFMAs (ARMX_FLAG_INT_LIMBS)."""
import math

import numpy as np
import pytest
import torch

import arithmetic_reduction_matrix_amd as armx
import synth_inputs as si
from oracle import exact_sum

from _parity import bits32, require_gpu, to_dev

pytestmark = pytest.mark.gpu


FORMS = {"binary64": {}, "int_limbs": dict(int_limbs=True)}
form_param = pytest.mark.parametrize("form", list(FORMS))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def run(xd, **cfg):
    fixed = torch.full((2,), 77, dtype=torch.int64, device=xd.device)
    out = armx.reduce_sum_exact(xd, fixed=fixed, **cfg)
    return out.cpu().numpy(), armx.fixed_to_int(fixed.cpu())


def check(x, what="", **cfg):
    e = exact_sum(x)
    got, q = run(to_dev(x), **cfg)
    assert bits32(got) == bits32(e.f32), (what, cfg, float(got), float(e.f32))
    assert q == (e.q if e.special is None else 0), (what, cfg, q, e.q)
    return got, q


SIZES = [1, 2, 7, 8, 9, 255, 256, 257, 511, 512, 513, 4095, 4096, 4097, 65536 + 3,
         (1 << 20) + 37, 3 * (1 << 20) + 1234]


@pytest.mark.parametrize("n", SIZES)
@form_param
def test_sizes(n, form):
    check(si.generate("uniform11", n, seed=n), f"n={n}", **FORMS[form])


@pytest.mark.parametrize("block", [64, 128, 256, 1024])
@pytest.mark.parametrize("r", [1, 2, 3, 4, 5, 8])
@form_param
def test_every_configuration_gives_the_oracle_bits(block, r, form):
    n = (1 << 20) + 4099
    x = si.generate("logu_signed", n, seed=3)
    for extra in (dict(), dict(grid_blocks=5), dict(cached_loads=True)):
        check(x, f"block={block} r={r}", block_threads=block, chain_r=r, **extra,
              **FORMS[form])


@pytest.mark.parametrize("dist", ["uniform01", "uniform11", "normal", "logu_signed",
                                  "bits_finite", "alternating", "ones", "ramp2048"])
@form_param
def test_distributions(dist, form):
    check(si.generate(dist, (1 << 21) + 5, seed=91), dist, **FORMS[form])


@form_param
def test_every_binary16_value(form):
    # every finite pattern: all together, in blocks of 4096, and each one
    # beside its negation's neighbour (so every digit position carries)
    pats = np.arange(1 << 16, dtype=np.uint32)
    vals = pats[((pats >> 10) & 31) != 31].astype(np.uint16).view(np.float16)
    check(vals, "all finite patterns", **FORMS[form])
    for k in range(0, vals.size, 4096):
        check(vals[k:k + 4096], f"patterns {k}..", **FORMS[form])
    pair = np.stack([vals, np.roll(vals, 1)], axis=1).reshape(-1)
    check(pair[::3].copy(), "pairs", **FORMS[form])


@form_param
def test_rounding_ties_and_near_ties(form):
    # ties go to the even neighbour; one unit past a tie goes up
    cases = [
        ([1.0, 2.0 ** -24], 1.0),                                  # tie, 1 is even
        ([1.0, 2.0 ** -23, 2.0 ** -24], 1.0 + 2.0 ** -22),        # tie, odd below
        ([1.0, 2.0 ** -24, 2.0 ** -24, 2.0 ** -24], 1.0 + 2.0 ** -22),
        ([1.0, 2.0 ** -24, 2.0 ** -24], 1.0 + 2.0 ** -23),        # exact
        ([2048.0, 2.0 ** -13], 2048.0),                            # tie (ulp 2^-12)
        ([2048.0, 2.0 ** -13, 2.0 ** -24], 2048.0 + 2.0 ** -12),  # just past the tie
        ([2048.0, 2.0 ** -12, 2.0 ** -13], 2048.0 + 2.0 ** -11),  # tie, odd below
        ([-1.0, -(2.0 ** -24)], -1.0),
        ([32768.0, 2.0 ** -24, -32768.0, 2.0 ** -24], 2.0 ** -23),
    ]
    for vals, want in cases:
        x = np.array(vals, np.float16)
        assert [float(v) for v in x] == vals      # every value is binary16-exact
        got, q = run(to_dev(x), **FORMS[form])
        assert float(got) == want, (vals, float(got), want)
        assert bits32(got) == bits32(exact_sum(x).f32)
        # the same values spread over many chains and blocks, with zeros between
        y = np.zeros(3 * (1 << 20) + 11, np.float16)
        y[np.linspace(0, y.size - 1, len(vals)).astype(np.int64)] = x
        got, _ = run(to_dev(y), **FORMS[form])
        assert float(got) == want, ("spread", vals, float(got))


@form_param
def test_zero_results_are_positive(form):
    kw = FORMS[form]
    z, q = run(torch.empty(0, dtype=torch.float16, device="cuda"), **kw)
    assert bits32(z) == 0 and q == 0
    x = np.full(5000, -0.0, np.float16)
    z, q = run(to_dev(x), **kw)
    assert bits32(z) == 0 and q == 0
    y = si.generate("uniform11", 100_001, seed=2)
    z, q = run(to_dev(np.concatenate([y, -y])), **kw)
    assert bits32(z) == 0 and q == 0


@form_param
def test_non_finite(form):
    x = si.generate("uniform11", 300_000, seed=3)
    for pos, vals in [((17,), (np.inf,)), ((299_999,), (-np.inf,)),
                      ((5, 200_000), (np.inf, -np.inf)), ((6, 7), (np.inf, -np.inf)),
                      ((150_000,), (np.nan,)), ((1, 2), (np.inf, np.inf))]:
        y = x.copy()
        for p, v in zip(pos, vals):
            y[p] = v
        e = exact_sum(y)
        got, q = run(to_dev(y), **FORMS[form])
        if e.special == "nan":
            assert math.isnan(float(got)), pos
        else:
            assert float(got) == float(e.f32), (pos, float(got))
        assert q == 0


@form_param
def test_limb_carries_and_128_bit_totals(form):
    kw = FORMS[form]
    # |sum| 2^24 beyond 2^64: the high word of the 128-bit count is in use
    n = 1 << 26
    for v in (65504.0, -65504.0):
        xd = torch.full((n,), v, dtype=torch.float16, device="cuda")
        got, q = run(xd, **kw)
        want_q = int(v) * n * (1 << 24)
        assert q == want_q and abs(q) >= 1 << 64
        assert float(got) == v * n
    # one large value and many tiny ones: the low limb carries into the high one
    y = np.full((1 << 22) + 3, 2.0 ** -24, np.float16)
    y[123] = 65504.0
    y[4_000_000] = -65504.0
    check(y, "carries", **kw)


def test_concurrent_streams_and_workspace_reuse():
    xs = [si.generate("normal", (1 << 20) + k, seed=k) for k in range(4)]
    streams = [torch.cuda.Stream() for _ in xs]
    outs = []
    for s, x in zip(streams, xs):
        with torch.cuda.stream(s):
            xd = to_dev(x)
            for _ in range(3):
                fixed = torch.zeros(2, dtype=torch.int64, device="cuda")
                out = armx.reduce_sum_exact(xd, fixed=fixed)
            outs.append((out, fixed))
    torch.cuda.synchronize()
    for (out, fixed), x in zip(outs, xs):
        e = exact_sum(x)
        assert bits32(out.cpu().numpy()) == bits32(e.f32)
        assert armx.fixed_to_int(fixed.cpu()) == e.q


def test_full_2p28_uniform11():
    x = si.workload("sum_2p28_u11")
    xd = to_dev(x)
    e = exact_sum(x)
    for cfg in (dict(), dict(chain_r=4, block_threads=256), dict(cached_loads=True),
                dict(int_limbs=True), dict(int_limbs=True, chain_r=2, block_threads=1024)):
        got, q = run(xd, **cfg)
        assert bits32(got) == bits32(e.f32) and q == e.q, cfg
    print(f"2^28 exact: {float(got)!r} (Q = {q})")


def test_full_2p30_logu():
    x = si.workload("sum_2p30_logu")
    e = exact_sum(x)
    xd = to_dev(x)
    del x
    for cfg in (dict(), dict(int_limbs=True)):
        got, q = run(xd, **cfg)
        assert bits32(got) == bits32(e.f32) and q == e.q, cfg
    print(f"2^30 logu exact: {float(got)!r} (oracle {float(e.f32)!r})")
