"""reduce_sum_noalloc, the entry point for callers that cannot allocate
device memory: through the C ABI, on two calls in a row (the second on a
smaller input, so the shared scratch array holds the first call's contents),
its result must be bit-identical to reduce_sum's with the same input and
configuration, and within the free-order gate of the exact sum."""
import ctypes

import numpy as np
import pytest
import torch

import arithmetic_reduction_matrix_amd as armx
import synth_inputs as si
from oracle import exact_sum

from _parity import bits32, check_free_order, require_gpu, to_dev

pytestmark = pytest.mark.gpu

CONFIGS = [dict(), dict(plain=True), dict(mma_levels=True), dict(two_pass=True),
           dict(one_chain=True, block_threads=256, chain_r=4), dict(grid_blocks=7),
           dict(block_threads=1024, chain_r=1), dict(cached_loads=True, chain_r=5)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _noalloc(xd, out, **cfg):
    c = armx._config(**cfg)
    stream = torch.cuda.current_stream().cuda_stream
    return armx.lib.reduce_sum_noalloc(xd.data_ptr() if xd.numel() else None, xd.numel(),
                                       out.data_ptr(), ctypes.byref(c), stream)


@pytest.mark.parametrize("cfg", CONFIGS, ids=[str(c) for c in CONFIGS])
def test_noalloc_matches_reduce_sum_on_two_calls(cfg):
    sizes = [3 * (1 << 20) + 1234, 100_003]      # the second call is smaller
    inputs = [si.generate("uniform11", m, seed=900 + m) for m in sizes]
    outs = [torch.full((1,), 7.0, device="cuda") for _ in sizes]
    for x, out in zip(inputs, outs):
        st = _noalloc(to_dev(x), out, **cfg)
        assert st == 0, (cfg, armx.lib.armx_status_string(st))
    torch.cuda.synchronize()
    for x, out in zip(inputs, outs):
        want = armx.reduce_sum(to_dev(x), **cfg).cpu().numpy()
        got = out.cpu().numpy()[0]
        assert bits32(got) == bits32(want), (cfg, x.size, got, want)
        check_free_order(float(got), exact_sum(x), f"noalloc {cfg} n={x.size}")


def test_noalloc_large_and_empty():
    x = si.generate("uniform11", (1 << 26) + 3, seed=17)
    xd = to_dev(x)
    out = torch.empty(1, device="cuda")
    assert _noalloc(xd, out) == 0
    assert bits32(out.cpu().numpy()[0]) == bits32(armx.reduce_sum(xd).cpu().numpy())
    check_free_order(float(out.item()), exact_sum(x))
    empty = torch.empty(0, dtype=torch.float16, device="cuda")
    assert _noalloc(empty, out) == 0
    assert bits32(out.cpu().numpy()[0]) == 0
    # the Python wrapper, and the refusal of a plan larger than the array
    y = to_dev(si.generate("normal", 5000, seed=3))
    assert bits32(armx.reduce_sum_noalloc(y, out=out).cpu().numpy()[0]) == bits32(
        armx.reduce_sum(y).cpu().numpy())
    big = torch.empty(1 << 28, dtype=torch.float16, device="cuda")
    assert _noalloc(big, out, one_chain=True, block_threads=64, chain_r=1) == -4


def test_noalloc_inside_a_captured_graph():
    # the callers it is for: code under HIP graph capture.  The call is
    # captured (its counter clear is a kernel, not a memset), replayed on
    # new data with eager work and synchronisations between the replays, and
    # every replay is checked against an eager reduce_sum of the same data.
    n = (1 << 22) + 5
    pool = [to_dev(si.generate("uniform11", n, seed=300 + i)) for i in range(4)]
    x = torch.empty_like(pool[0])
    out = torch.empty(1, dtype=torch.float32, device="cuda")
    x.copy_(pool[0])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        assert _noalloc(x, out) == 0          # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st = _noalloc(x, out)
    assert st == 0
    for i in range(1, 4):
        x.copy_(pool[i])
        g.replay()
        torch.cuda.synchronize()
        want = armx.reduce_sum(pool[i]).cpu().numpy()
        assert bits32(out.cpu().numpy()[0]) == bits32(want), i
        # eager calls of both entry points between replays
        assert _noalloc(pool[i - 1], torch.empty(1, device="cuda")) == 0
        torch.cuda.synchronize()
