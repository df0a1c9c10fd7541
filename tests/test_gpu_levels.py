"""reduce_sum with ARMX_FLAG_MMA_LEVELS: the recursive all-MMA form of "GPU
Tensor Cores for fast Arithmetic Reductions" (arXiv 2001.05585, Abstract) --
level 1 reduces chains of R x 512 binary16 values to one fp32 each with MFMAs
only, further levels reduce chains of R x 256 fp32 values the same way, one
launch per level.  Checked against the exact-sum oracle (free-order gate);
its order depends on n and R only, so block size and grid must not change a
bit."""
import math

import numpy as np
import pytest
import torch

import arithmetic_reduction_matrix_amd as armx
import synth_inputs as si
from oracle import exact_sum

from _parity import bits32, check_free_order, require_gpu, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def levels(n: int, r: int) -> int:
    """Launches the MMA-levels form makes for n values and chain length r."""
    c = -(-n // (512 * r))
    k = 1
    while c > 1:
        c = -(-c // (256 * r))
        k += 1
    return k


SIZES = [1, 2, 7, 8, 9, 511, 512, 513, 4095, 4096, 4097, 65536 + 3, (1 << 20) + 37,
         3 * (1 << 20) + 1234]


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("r", [1, 2, 4, 8])
def test_sizes_and_chains(n, r):
    x = si.generate("uniform11", n, seed=n + r)
    got = float(armx.reduce_sum(to_dev(x), mma_levels=True, chain_r=r).item())
    check_free_order(got, exact_sum(x), f"n={n} r={r} levels={levels(n, r)}")


# n at and just past the boundaries where a level is added (R = 1: one value
# per 512 inputs at level 1, per 256 above)
@pytest.mark.parametrize("n,expect", [(512, 1), (513, 2), (512 * 256, 2), (512 * 256 + 1, 3),
                                      (512 * 256 * 256, 3), (512 * 256 * 256 + 1, 4)])
def test_level_boundaries(n, expect):
    assert levels(n, 1) == expect
    x = si.generate("uniform01", n, seed=5)
    e = exact_sum(x)
    for block in (64, 256):
        got = float(armx.reduce_sum(to_dev(x), mma_levels=True, chain_r=1,
                                    block_threads=block).item())
        check_free_order(got, e, f"n={n} block={block}")


@pytest.mark.parametrize("r", [1, 3, 4, 5, 8])
def test_block_and_grid_do_not_change_bits(r):
    n = (1 << 21) + 4099
    x = si.generate("normal", n, seed=r)
    xd = to_dev(x)
    e = exact_sum(x)
    ref = None
    for cfg in (dict(), dict(block_threads=64), dict(block_threads=1024),
                dict(block_threads=320), dict(grid_blocks=3), dict(grid_blocks=1000),
                dict(one_chain=True), dict(cached_loads=True)):
        got = armx.reduce_sum(xd, mma_levels=True, chain_r=r, **cfg).item()
        check_free_order(got, e, f"r={r} {cfg}")
        b = bits32(got)
        ref = b if ref is None else ref
        assert b == ref, (r, cfg)


def test_closed_forms_are_exact():
    # all partial sums are integers below 2^24, exactly representable
    for n in (1 << 20, (1 << 24) + 17):
        for dist in ("ones", "ramp2048"):
            x = si.generate(dist, n)
            e = exact_sum(x)
            for r in (1, 8):
                got = armx.reduce_sum(to_dev(x), mma_levels=True, chain_r=r).item()
                assert got == float(e.f32), (dist, n, r, got, e.f32)


@pytest.mark.parametrize("dist", ["bits_finite", "logu_signed", "alternating"])
def test_distributions(dist):
    x = si.generate(dist, (1 << 21) + 5, seed=78)
    e = exact_sum(x)
    for r in (2, 8):
        check_free_order(armx.reduce_sum(to_dev(x), mma_levels=True, chain_r=r).item(), e,
                         f"{dist} r={r}")


def test_non_finite():
    x = si.generate("uniform11", 300_000, seed=3)
    for pos, vals, expect in [((17,), (np.inf,), math.inf), ((299_999,), (-np.inf,), -math.inf),
                              ((5, 200_000), (np.inf, -np.inf), math.nan),
                              ((150_000,), (np.nan,), math.nan)]:
        y = x.copy()
        for p, v in zip(pos, vals):
            y[p] = v
        for r in (1, 8):
            got = armx.reduce_sum(to_dev(y), mma_levels=True, chain_r=r).item()
            if math.isnan(expect):
                assert math.isnan(got), (pos, r)
            else:
                assert got == expect, (pos, r, got)


def test_empty_and_single():
    z = armx.reduce_sum(torch.empty(0, dtype=torch.float16, device="cuda"), mma_levels=True)
    assert z.item() == 0.0 and math.copysign(1.0, z.item()) > 0
    for v in (0.5, -3.0, 65504.0, 2.0 ** -24):
        x = np.array([v], np.float16)
        assert armx.reduce_sum(to_dev(x), mma_levels=True).item() == float(np.float32(x[0]))


def test_workspace_counter_region_untouched():
    # the level buffers start after the counter region, so a workspace shared
    # with the ticket-completed reduce_sum stays usable
    x = si.generate("uniform11", (1 << 22) + 9, seed=21)
    xd = to_dev(x)
    e = exact_sum(x)
    need = armx.workspace_bytes(armx.OP_SUM, x.size, mma_levels=True)
    need = max(need, armx.workspace_bytes(armx.OP_SUM, x.size))
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    for _ in range(2):
        check_free_order(armx.reduce_sum(xd, mma_levels=True, workspace=ws).item(), e)
        assert int(ws[:256].count_nonzero().item()) == 0
        check_free_order(armx.reduce_sum(xd, workspace=ws).item(), e)
    with pytest.raises(armx.ArmxError) as ei:
        armx.reduce_sum(xd, mma_levels=True, workspace=ws[:512])
    assert ei.value.name == "ARMX_ERR_WORKSPACE"


def test_rejected_combinations():
    xd = to_dev(si.generate("uniform01", 4096, seed=1))
    for cfg in (dict(plain=True), dict(two_pass=True)):
        with pytest.raises(armx.ArmxError) as ei:
            armx.reduce_sum(xd, mma_levels=True, **cfg)
        assert ei.value.name == "ARMX_ERR_CONFIG"
    with pytest.raises(armx.ArmxError):
        armx.reduce_sum_fixed_order(xd, mma_levels=True)


def test_events_span_all_levels():
    n = 1 << 24                       # three launches at R = 8
    x = si.generate("uniform11", n, seed=12)
    xd = to_dev(x)
    s, t = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(3):
        out = armx.reduce_sum(xd, mma_levels=True, start_event=s, stop_event=t)
    torch.cuda.synchronize()
    assert 0.0 < s.elapsed_time(t) < 50.0
    check_free_order(out.item(), exact_sum(x))


def test_full_2p28_uniform11():
    x = si.workload("sum_2p28_u11")
    e = exact_sum(x)
    xd = to_dev(x)
    for r in (1, 4, 8):
        got = armx.reduce_sum(xd, mma_levels=True, chain_r=r).item()
        rel = check_free_order(got, e, f"r={r}")
        print(f"2^28 mma levels r={r} ({levels(x.size, r)} launches): got {got!r} "
              f"exact {e.f64!r} rel {rel:.3e}")


def test_full_2p30_precision_stress():
    x = si.workload("sum_2p30_logu")
    e = exact_sum(x)
    xd = to_dev(x)
    del x
    got = armx.reduce_sum(xd, mma_levels=True).item()
    rel = check_free_order(got, e)
    print(f"2^30 logu mma levels: got {got!r} exact {e.f64!r} rel {rel:.3e}")
