"""Benchmark of the fp16 sum-reduction hot path on one MI355X.

One step = one reduce_sum call (chained MFMAs against ones, fp32 chain sub-results,
block combine, completion-ticket final reduce) over n = 2^28 binary16 values
drawn uniformly from [-1, 1) with seed 2, the input already resident in HBM.
Two copies of the input are used in turn so that no step reads data the
previous step left in the 256 MB Infinity Cache.

Prints ONE JSON line.  `value` is elements/s over the timed steps (wall clock
between two synchronisations; each step one call through the C ABI, nothing
else in the loop); `roofline.achieved` is the algorithmic bytes of one launch
(2 bytes per element) divided by the average kernel time: the elapsed time of
HIP events recorded on the kernel's stream around the timed steps (the
kernels run back to back), over the step count.  As a cross-check, a pass of
its own after the timed steps times single launches with HIP events that the
kernel's own dispatch stamps (hipExtLaunchKernel).  `cpu_baseline`
is the CPU oracle timed on this host: the exact integer sum and the
balanced-tree emulator, each on one thread and on all the host threads it may
use; its results also give `check`, the errors of the headline, of every
block size x R point of the 2^28 matrix and of the 2^30 precision-stress sums.
`variants` times the other rows of the hot path (MFMA-free design, exact sum,
MMA-levels form, fixed balanced-tree order beside the free order on the same
data, row sums, fixed-order row sums, the block size x R matrix in both grids)
on their own workloads.

`--levels-sweep` times the recursive all-MMA form (one launch per level)
against the single-launch form over n = 2^9 .. 2^28, for the running-time
model T(n) = 5 log_{m^2}(n) of "GPU Tensor Cores for fast Arithmetic
Reductions" (arXiv 2001.05585, Abstract), which counts levels.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-variants]
                    [--no-cpu-baseline] [--levels-sweep] [--copy-calibration]
"""
from __future__ import annotations

import argparse
import functools
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
METRIC = "elements/s and achieved HBM GB/s (% of peak), fp16 sum n=2^28"
KERNEL_SOURCES = ["arithmetic_reduction_matrix_amd/csrc/sum_kernels.hip",
                  "arithmetic_reduction_matrix_amd/csrc/device_common.hpp"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "sum_kernel_n2p28_traffic.txt")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded_traffic(n_launch_bytes: int):
    """HBM bytes per launch from the committed counter summary, or None if it
    is missing or was taken on a different kernel source."""
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    m_hash = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != kernel_source_hash():
        return None
    return float(m_bytes.group(1))


def event_timed(torch, fn, iters: int, warmup: int = 5):
    """Average ms per call of fn(i) over `iters` back-to-back eager calls: one
    pair of events on the current stream around all of them (as for the
    headline's timed steps), so no marker packets sit between the calls; for
    calls shorter than their host overhead this is the eager call rate."""
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for i in range(iters):
        fn(i)
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / iters


def graph_timed(torch, call, calls: int, reps: int = 5):
    """Average ms per call of call(i) with `calls` calls captured back to back
    in one HIP graph and replayed: no host work between the calls, so short
    kernels are timed with the queue kept full (events around each eager call
    would time the host's call overhead instead).  Best of `reps` replays."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(3):
            call(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(calls):
            call(i)
    g.replay()
    torch.cuda.synchronize()
    per_call = []
    for _ in range(reps):
        s_ev, e_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s_ev.record()
        g.replay()
        e_ev.record()
        torch.cuda.synchronize()
        per_call.append(s_ev.elapsed_time(e_ev) / calls)
    del g
    return min(per_call)


def stamped_timed(torch, call, iters: int = 50):
    """Average ms of one kernel: call(i, start, stop) passes HIP events that the
    library's dispatch packet stamps around its main kernel."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(iters)]
    for i, (s_ev, e_ev) in enumerate(evs):
        call(i, s_ev, e_ev)
    torch.cuda.synchronize()
    return sum(s_ev.elapsed_time(e_ev) for s_ev, e_ev in evs) / iters


def read_ceiling(torch, bufs, n: int, cus: int, iters: int = 20):
    """Best HBM read rate of the plain load stream of libarmx_probe.so over a
    sweep of launch shapes (dispatch-stamped events, inputs rotated), in GB/s,
    and the shape that reached it."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "arithmetic_reduction_matrix_amd", "libarmx_probe.so"))
    vp, sz, ci = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    lib.armx_probe_read.argtypes = [vp, sz, vp, sz, ci, ci, ci, ci, ci, vp, vp, vp]
    lib.armx_probe_read.restype = ci
    words = 16 * 1024 * cus
    out = torch.empty(words, dtype=torch.int32, device=bufs[0].device)
    stream = torch.cuda.current_stream().cuda_stream
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(iters)]
    for s_ev, e_ev in evs:
        s_ev.record()
        e_ev.record()
    shapes = [(64, k) for k in (1, 2, 4, 8, 16)] + [(256, k) for k in (1, 2, 4)] + [(1024, 1)]
    results = []
    kinds = [(loads, nt, 0) for loads in (4, 8, 16) for nt in (1, 0)]
    kinds += [(loads, 1, pause) for loads in (4, 8, 16) for pause in (2, 4, 8)]
    for block, per_cu in shapes:
        for loads, nt, pause in kinds:
            def call(i, ev=(None, None)):
                st = lib.armx_probe_read(bufs[i & 1].data_ptr(), n, out.data_ptr(), words,
                                         cus * per_cu, block, loads, nt, pause,
                                         ev[0].cuda_event if ev[0] else None,
                                         ev[1].cuda_event if ev[1] else None, stream)
                if st != 0:
                    raise RuntimeError(f"armx_probe_read returned {st}")
            for i in range(3):
                call(i)
            for i, ev in enumerate(evs):
                call(i, ev)
            torch.cuda.synchronize()
            ms = sum(a.elapsed_time(b) for a, b in evs) / iters
            results.append((2 * n / (ms * 1e-3) / 1e9, dict(
                block_threads=block, blocks=cus * per_cu, waves_per_cu=per_cu * block // 64,
                loads=loads, nontemporal=bool(nt), pause=pause, launch_ms_avg=ms)))
    results.sort(key=lambda r: -r[0])
    return results[0]


def mma_levels_count(n: int, r: int) -> int:
    """Launches of the MMA-levels form: one value per R x 512 inputs at level
    1, per R x 256 values above, until one value is left."""
    c, k = -(-n // (512 * r)), 1
    while c > 1:
        c, k = -(-c // (256 * r)), k + 1
    return k


def host_threads() -> int:
    """Threads the CPU baseline may use: the CPUs this process may run on,
    at most 16 (a one-GPU share of the host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(x_np, xf_np, budget_s: float = 4.0, stress_np=None):
    """The CPU oracle on this host, as it stands: oracle.exact_sum (exact
    integer sum) over the n = 2^28 headline input and oracle.fixed_tree_sum
    (balanced-tree emulator) over the n = 2^26 fixed-order input, each on one
    thread and on `host_threads()` threads.  With T threads the input is cut
    into T aligned power-of-two parts, each part run through the same oracle
    function in a thread (numpy releases the interpreter lock in its array
    loops), and the parts joined by the oracle (exact_sum_of_parts: integer
    addition; tree_over_nodes: the tree continued above the parts' roots, so
    the bits equal the one-thread result).  Each of the four legs makes whole
    passes until `budget_s` seconds have passed (at least one).  Then one
    pass of the exact sum over the 2^30 precision-stress input, on T threads.
    Returns the record and the oracle's results."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle

    T = host_threads()

    def parts(x, k):
        step = 1 << max(0, (x.size - 1).bit_length() - (k - 1).bit_length())
        return [x[i:i + step] for i in range(0, x.size, step)]

    def exact_mt(x, pool):
        return oracle.exact_sum_of_parts(list(pool.map(oracle.exact_sum, parts(x, T))))

    def tree_mt(x, pool):
        return oracle.tree_over_nodes(list(pool.map(oracle.fixed_tree_sum, parts(x, T))))

    legs = {}
    results = {}
    with ThreadPoolExecutor(T) as pool:
        for name, fn, x, threads in (
                ("exact_sum_1t", oracle.exact_sum, x_np, 1),
                (f"exact_sum_{T}t", lambda v: exact_mt(v, pool), x_np, T),
                ("fixed_tree_sum_1t", oracle.fixed_tree_sum, xf_np, 1),
                (f"fixed_tree_sum_{T}t", lambda v: tree_mt(v, pool), xf_np, T)):
            t0 = time.perf_counter()
            passes = 0
            while True:
                r = fn(x)
                passes += 1
                el = time.perf_counter() - t0
                if el >= budget_s:
                    break
            results[name] = r
            legs[name] = {"elements_per_s": passes * x.size / el, "threads": threads,
                          "passes": passes, "n": int(x.size), "seconds": el}
        e_stress = exact_mt(stress_np, pool) if stress_np is not None else None
    e = results["exact_sum_1t"]
    same = (results[f"exact_sum_{T}t"].q == e.q and
            np.float32(results[f"fixed_tree_sum_{T}t"]).view(np.uint32)
            == np.float32(results["fixed_tree_sum_1t"]).view(np.uint32))
    head = legs[f"exact_sum_{T}t"]
    record = {"value": head["elements_per_s"], "unit": "elements/s", "cores": T, "kind": "oracle",
              "sample": (f"oracle.exact_sum on {T} threads, {head['passes']} whole pass(es) over "
                         f"the n=2^28 input ({head['seconds']:.1f} s); legs: exact_sum and "
                         "fixed_tree_sum (n=2^26 fixed-order input), 1 thread and all threads"),
              "cpu_model": cpu_model(), "nproc": os.cpu_count(), "legs": legs,
              "threads_agree_bitwise": bool(same)}
    return record, e, e_stress, results["fixed_tree_sum_1t"]


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-variants", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--levels-sweep", action="store_true",
                    help="also time the MMA-levels form against the single-launch form "
                         "over n = 2^lo .. 2^hi (level count vs time)")
    ap.add_argument("--levels-log2", default="9-28",
                    help="lo-hi: the sizes of --levels-sweep (default 9-28)")
    ap.add_argument("--no-read-ceiling", action="store_true",
                    help="skip the sweep of the plain read-stream probe")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 512 MiB device copy (torch) five times, the "
                         "known-size reference for HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        return 2

    import torch

    import arithmetic_reduction_matrix_amd as armx
    import synth_inputs as si

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(dev)

    # ---- headline workload -------------------------------------------------
    x_np = si.workload("sum_2p28_u11")
    n = x_np.size
    bufs = [torch.from_numpy(x_np).to(dev)]
    bufs.append(bufs[0].clone())
    out = torch.empty((), dtype=torch.float32, device=dev)
    ws = torch.zeros(armx.workspace_bytes(armx.OP_SUM, n), dtype=torch.uint8, device=dev)
    head_plan = armx.launch_plan(armx.OP_SUM, n)

    # The timed steps: one call through the C ABI each, its arguments
    # marshalled once beforehand, nothing else in the loop (no events).
    import ctypes
    cfg_plain = armx.Config(0, 0, 0, 0, None, None)
    stream = torch.cuda.current_stream().cuda_stream
    call_args = [(bufs[k].data_ptr(), n, out.data_ptr(), ws.data_ptr(), ws.numel(),
                  ctypes.byref(cfg_plain), stream) for k in range(2)]
    reduce_sum_c = armx.lib.reduce_sum

    def step(i):
        st = reduce_sum_c(*call_args[i & 1])
        if st != 0:
            raise RuntimeError(f"reduce_sum returned {st}")

    # HIP events recorded on the stream the kernel runs on (torch's current
    # stream) bracket the timed region: one marker just before the first
    # step and one after the last; the kernels run back to back between
    # them, so the elapsed time over the step count is the average launch
    # duration (each launch's own time plus the few nanoseconds between
    # dispatches, and the first launch's host latency spread over the
    # steps).  Measured on MI355X at 20 steps, markers cost the wall clock
    # about 1 us per step less than stamping the first and last steps'
    # dispatches (hipExtLaunchKernel), for the same event average.
    region = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    region[0].record()
    for i in range(args.steps):
        step(i)
    region[1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    region_ms = region[0].elapsed_time(region[1])
    result = float(out.item())

    # Per-launch timing, in a pass of its own after the timed steps: HIP
    # events stamped by the kernel's own dispatch packet (hipExtLaunchKernel)
    # on the stream it runs on, on every 4th of 64 back-to-back calls (a
    # stamp adds dispatch time, so unstamped calls keep the queue full).
    stamped = list(range(0, 64, 4))
    evs = {i: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for i in stamped}
    for s_ev, e_ev in evs.values():
        s_ev.record()
        e_ev.record()
    torch.cuda.synchronize()
    for i in range(64):
        ev = evs.get(i, (None, None))
        armx.reduce_sum(bufs[i & 1], out=out, workspace=ws, start_event=ev[0], stop_event=ev[1])
    torch.cuda.synchronize()
    launch_ms = sorted(s_ev.elapsed_time(e_ev) for s_ev, e_ev in evs.values())
    stamped_avg_ms = sum(launch_ms) / len(launch_ms)
    avg_ms = region_ms / args.steps

    bytes_per_launch = 2 * n
    achieved = bytes_per_launch / (avg_ms * 1e-3) / 1e9
    traffic = recorded_traffic(bytes_per_launch)
    record = {
        "metric": METRIC,
        "value": n * args.steps / wall,
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16->f32",
        "data": "synthetic",
        "config": {
            "workload": "sum of n=2^28 fp16 uniform[-1,1) seed 2 (512 MiB), fp32 result",
            "n": n, "block_threads": head_plan["block_threads"], "chain_r": head_plan["chain_r"],
            "loads": "non-temporal", "grid_blocks": head_plan["grid_blocks"],
            "grid": f"persistent, {head_plan['waves_per_cu']:g} wavefronts per CU",
            "final": "last-block ticket",
            "input_copies_rotated": 2, "device": props.name, "cus": props.multi_processor_count,
            "workspace_bytes": ws.numel(),
        },
        "hbm_gbs": bytes_per_launch * args.steps / wall / 1e9,
        "pct_hbm_peak": 100.0 * bytes_per_launch * args.steps / wall / 1e9 / HBM_PEAK_GBS,
        "roofline": {
            "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": traffic,
            "kernel": f"sum_kernel<R={head_plan['chain_r']}, non-temporal, MFMA>",
            "launch_ms_avg": avg_ms,
            "launch_timing": "HIP events recorded on the kernel's stream just before the "
                             "first timed step and after the last, elapsed time / steps",
            "launches_timed": args.steps,
            "stamped_launch_ms_avg": stamped_avg_ms,
            "stamped_launch_ms_median": launch_ms[len(launch_ms) // 2],
            "stamped_launch_ms_p10": launch_ms[len(launch_ms) // 10],
            "stamped_launch_ms_p90": launch_ms[(9 * len(launch_ms)) // 10],
            "stamped_launches": len(launch_ms),
            "algorithmic_bytes_per_launch": bytes_per_launch,
            "kernel_source_sha256_16": kernel_source_hash(),
        },
        "result": result,
    }

    print(f"bench: headline done, {avg_ms * 1e3:.2f} us per launch", file=sys.stderr, flush=True)
    # ---- the achievable read rate on this device -------------------------------
    if not args.no_read_ceiling:
        ceil_gbs, ceil_cfg = read_ceiling(torch, bufs, n, props.multi_processor_count)
        record["read_ceiling"] = {
            "gbs": ceil_gbs, "frac_of_peak": ceil_gbs / HBM_PEAK_GBS,
            "headline_frac_of_ceiling": achieved / ceil_gbs,
            "kernel": "read_probe_kernel (libarmx_probe.so): 16-byte loads, one XOR per word",
            "best_shape": ceil_cfg,
        }

    print("bench: read ceiling done", file=sys.stderr, flush=True)
    # ---- the other rows of the hot path ---------------------------------------
    stress_np = None   # the 2^30 precision-stress input, drawn with the variants
    if not args.no_variants:
        var = {}
        ms = event_timed(torch, lambda i: armx.reduce_sum(bufs[i & 1], plain=True), 200)
        var["plain_shuffle_2p28"] = {"ms": ms, "gbs": 2 * n / ms / 1e6,
                                     "vs_mfma": avg_ms / ms}
        ms = event_timed(torch, lambda i: armx.reduce_sum(bufs[i & 1], all_ones=True), 200)
        var["mfma_all_ones_2p28"] = {"ms": ms, "gbs": 2 * n / ms / 1e6, "vs_signed": avg_ms / ms}
        ms = event_timed(torch, lambda i: armx.reduce_sum(
            bufs[i & 1], one_chain=True, block_threads=256, chain_r=4), 50)
        var["one_chain_b256_r4_2p28"] = {"ms": ms, "gbs": 2 * n / ms / 1e6}
        ms = event_timed(torch, lambda i: bufs[i & 1].sum(dtype=torch.float32), 100)
        var["torch_sum_2p28"] = {"ms": ms, "gbs": 2 * n / ms / 1e6}
        ms = event_timed(torch, lambda i: armx.reduce_sum_exact(bufs[i & 1]), 200)
        exact_val = armx.reduce_sum_exact(bufs[0]).cpu().numpy()
        var["exact_2p28"] = {"ms": ms, "gbs": 2 * n / ms / 1e6, "vs_free_order": avg_ms / ms,
                             "result_bits": int(exact_val.view(np.uint32))}
        # the exact sum with integer MFMAs over 8-bit limbs (ARMX_FLAG_INT_LIMBS)
        ms = event_timed(torch, lambda i: armx.reduce_sum_exact(bufs[i & 1], int_limbs=True),
                              200)
        k_ms = stamped_timed(torch, lambda i, s_ev, e_ev: armx.reduce_sum_exact(
            bufs[i & 1], int_limbs=True, start_event=s_ev, stop_event=e_ev))
        limb_val = armx.reduce_sum_exact(bufs[0], int_limbs=True).cpu().numpy()
        var["exact_int_limbs_2p28"] = {"ms": ms, "gbs": 2 * n / ms / 1e6, "kernel_ms": k_ms,
                                       "vs_binary64_form": var["exact_2p28"]["ms"] / ms,
                                       "result_bits": int(limb_val.view(np.uint32))}
        for r in (8, 4):
            ms = event_timed(torch, lambda i: armx.reduce_sum(
                bufs[i & 1], mma_levels=True, chain_r=r), 200)
            var[f"mma_levels_r{r}_2p28"] = {"ms": ms, "gbs": 2 * n / ms / 1e6,
                                            "launches": mma_levels_count(n, r),
                                            "vs_single_launch": avg_ms / ms}

        # the small and the large single sums: 2^20 (2 MiB, cache-resident,
        # latency-bound) and 2^30 (2 GiB; timing only, so its values are drawn
        # on the device rather than by the seeded generator)
        # At 2^20 a call's host overhead (about 10 us) exceeds the kernel, so
        # the small sums are timed in a captured graph (the rate with the queue
        # full) and by their own dispatch stamps; the graph's result is checked
        # against the eager call's bits.
        xs = [torch.from_numpy(si.workload("sum_2p20_u01")).to(dev)]
        xs.append(xs[0].clone())
        small = {
            "sum_2p20": (armx.reduce_sum, armx.OP_SUM, {}),
            "fixed_order_2p20": (armx.reduce_sum_fixed_order, armx.OP_FIXED, {}),
            "exact_2p20": (armx.reduce_sum_exact, armx.OP_EXACT, {}),
        }
        for key, (fn, op, kw) in small.items():
            sws = torch.zeros(max(1, armx.workspace_bytes(op, 1 << 20)), dtype=torch.uint8,
                              device=dev)
            sout = torch.empty((), dtype=torch.float32, device=dev)
            eager = fn(xs[1], workspace=sws, **kw).cpu().numpy()
            g_ms = graph_timed(torch, lambda i: fn(xs[i & 1], out=sout, workspace=sws, **kw), 200)
            assert sout.cpu().numpy().view(np.uint32) == eager.view(np.uint32), key
            k_ms = stamped_timed(torch, lambda i, s_ev, e_ev: fn(
                xs[i & 1], out=sout, workspace=sws, start_event=s_ev, stop_event=e_ev, **kw))
            e_ms = event_timed(torch, lambda i: fn(xs[i & 1], out=sout, workspace=sws, **kw),
                                  200)
            var[key] = {"ms": g_ms, "gbs": 2 * (1 << 20) / g_ms / 1e6,
                        "timing": "graph of 200 back-to-back calls",
                        "kernel_ms": k_ms, "eager_call_ms": e_ms}
        del xs
        xl = torch.empty(1 << 30, dtype=torch.float16, device=dev).uniform_(-1, 1)
        ms = event_timed(torch, lambda i: armx.reduce_sum(xl), 50)
        var["sum_2p30"] = {"ms": ms, "gbs": 2 * (1 << 30) / ms / 1e6}
        ms = event_timed(torch, lambda i: armx.reduce_sum_exact(xl), 50)
        var["exact_2p30"] = {"ms": ms, "gbs": 2 * (1 << 30) / ms / 1e6}
        del xl

        # the precision-stress input (2^30 values, random signs, magnitudes
        # log-uniform over 2^-14 .. 2^8): results here, their errors against
        # the exact sum in `check` (computed in the CPU-baseline leg)
        stress_np = si.workload("sum_2p30_logu")
        xs30 = torch.from_numpy(stress_np).to(dev)
        var["precision_2p30_logu"] = {
            "mfma": float(armx.reduce_sum(xs30).item()),
            "mfma_all_ones": float(armx.reduce_sum(xs30, all_ones=True).item()),
            "plain": float(armx.reduce_sum(xs30, plain=True).item()),
            "exact_result_bits": int(armx.reduce_sum_exact(xs30).cpu().numpy().view(np.uint32)),
        }
        del xs30

        xf_np = si.workload("fixed_2p26_u11")
        fbufs = [torch.from_numpy(xf_np).to(dev)]
        fbufs += [fbufs[0].clone() for _ in range(3)]
        # four 128 MiB copies in turn, so the reads come from HBM rather than
        # the 256 MB Infinity Cache; at about 25 us a kernel is short enough
        # for eager calls to leave the queue empty now and then, so the rate
        # is taken with the calls captured back to back in a graph (and each
        # kernel by its own dispatch stamps), the eager figure beside it
        fws = torch.zeros(max(armx.workspace_bytes(armx.OP_FIXED, xf_np.size),
                              armx.workspace_bytes(armx.OP_FIXED, xf_np.size, mma_leaves=True)),
                          dtype=torch.uint8, device=dev)
        fout = torch.empty((), dtype=torch.float32, device=dev)
        # the free-order sum on the same four copies, for the fixed/free ratio
        fws = torch.zeros(max(fws.numel(), armx.workspace_bytes(armx.OP_SUM, xf_np.size)),
                          dtype=torch.uint8, device=dev)
        for key, fn, kw in (("free_order_2p26", armx.reduce_sum, {}),
                            ("fixed_order_2p26", armx.reduce_sum_fixed_order, {}),
                            ("fixed_order_mma_leaves_2p26", armx.reduce_sum_fixed_order,
                             dict(mma_leaves=True))):
            val = fn(fbufs[0], workspace=fws, **kw).cpu().numpy()
            g_ms = graph_timed(torch, lambda i: fn(fbufs[i & 3], out=fout, workspace=fws, **kw),
                               200)
            k_ms = stamped_timed(torch, lambda i, s_ev, e_ev: fn(
                fbufs[i & 3], out=fout, workspace=fws, start_event=s_ev, stop_event=e_ev, **kw))
            e_ms = event_timed(torch, lambda i: fn(fbufs[i & 3], out=fout, workspace=fws, **kw),
                                  200)
            var[key] = {"ms": g_ms, "gbs": 2 * xf_np.size / g_ms / 1e6,
                        "timing": "graph of 200 back-to-back calls", "kernel_ms": k_ms,
                        "eager_call_ms": e_ms, "result_bits": int(val.view(np.uint32))}
        for key in ("fixed_order_2p26", "fixed_order_mma_leaves_2p26"):
            var[key]["vs_free_order"] = var[key]["ms"] / var["free_order_2p26"]["ms"]
            var[key]["kernel_vs_free_order"] = (var[key]["kernel_ms"]
                                                / var["free_order_2p26"]["kernel_ms"])
        del fbufs

        xr_np = si.workload("rows_4096x65536_normal")
        rbufs = [torch.from_numpy(xr_np).to(dev)]
        rbufs.append(rbufs[0].clone())
        rout = torch.empty(4096, dtype=torch.float32, device=dev)
        ms = event_timed(torch, lambda i: armx.reduce_rows(rbufs[i & 1], out=rout), 200)
        var["rows_4096x65536"] = {"ms": ms, "gbs": 2 * xr_np.size / ms / 1e6}
        ms = event_timed(torch, lambda i: armx.reduce_rows(rbufs[i & 1], out=rout,
                                                                 plain=True), 100)
        var["rows_4096x65536_plain"] = {"ms": ms, "gbs": 2 * xr_np.size / ms / 1e6}
        ms = event_timed(torch, lambda i: armx.reduce_rows_fixed_order(rbufs[i & 1],
                                                                             out=rout), 200)
        var["rows_fixed_order_4096x65536"] = {"ms": ms, "gbs": 2 * xr_np.size / ms / 1e6}
        ms = event_timed(torch, lambda i: armx.reduce_rows_fixed_order(
            rbufs[i & 1], out=rout, mma_leaves=True), 200)
        var["rows_fixed_order_mma_leaves_4096x65536"] = {"ms": ms,
                                                         "gbs": 2 * xr_np.size / ms / 1e6}
        del rbufs
        # short and ragged rows: the headline buffers viewed as matrices;
        # bytes counted are the reads plus the fp32 results
        for cols in (64, 1000):
            nrows = n // cols
            views = [b[: nrows * cols].view(nrows, cols) for b in bufs]
            vout = torch.empty(nrows, dtype=torch.float32, device=dev)
            moved = 2 * nrows * cols + 4 * nrows
            mma_rows = functools.partial(armx.reduce_rows_fixed_order, mma_leaves=True)
            for tag, fn in (("rows", armx.reduce_rows),
                            ("rows_fixed_order", armx.reduce_rows_fixed_order),
                            ("rows_fixed_order_mma_leaves", mma_rows)):
                ms = event_timed(torch, lambda i: fn(views[i & 1], out=vout), 100)
                var[f"{tag}_{nrows}x{cols}"] = {"ms": ms, "gbs": moved / ms / 1e6}
            del views, vout
        # few long rows, each split over wavefronts of several blocks
        for nrows in (1, 8):
            cols = n // nrows
            views = [b.view(nrows, cols) for b in bufs]
            vout = torch.empty(nrows, dtype=torch.float32, device=dev)
            moved = 2 * n + 4 * nrows
            for tag, fn in (("rows", armx.reduce_rows),
                            ("rows_fixed_order", armx.reduce_rows_fixed_order)):
                ms = event_timed(torch, lambda i: fn(views[i & 1], out=vout), 100)
                var[f"{tag}_{nrows}x{cols}"] = {"ms": ms, "gbs": moved / ms / 1e6}
            del views, vout

        # The block size x R matrix at n = 2^28 (the pages' configuration
        # study, "GPU Tensor Cores for fast Arithmetic Reductions", Abstract):
        # blocks of 64, 256 and 1024 threads x R in {1, 2, 4, 5}, in the
        # pages' grid (every wavefront one chain) and the persistent grid.
        # Kernel time by dispatch stamps (a one-chain grid at small R runs for
        # milliseconds); each point's launch shape from the library's own plan.
        matrix = {}
        for grid_kind in ("one_chain", "persistent"):
            for block in (64, 256, 1024):
                for r in (1, 2, 4, 5):
                    kw = dict(one_chain=grid_kind == "one_chain", block_threads=block, chain_r=r)
                    plan = armx.launch_plan(armx.OP_SUM, n, **kw)
                    mws = torch.zeros(max(1, plan["workspace_bytes"]), dtype=torch.uint8,
                                      device=dev)
                    mout = torch.empty((), dtype=torch.float32, device=dev)
                    for i in range(2):
                        armx.reduce_sum(bufs[i & 1], out=mout, workspace=mws, **kw)
                    iters = 6 if plan["grid_blocks"] > 8192 else 16
                    k_ms = stamped_timed(torch, lambda i, s_ev, e_ev: armx.reduce_sum(
                        bufs[i & 1], out=mout, workspace=mws, start_event=s_ev, stop_event=e_ev,
                        **kw), iters)
                    chains = -(-n // (512 * r))
                    waves = plan["grid_blocks"] * block // 64
                    in_flight = r if chains <= waves else 2 * r   # the pipeline's depth
                    matrix[f"{grid_kind}_b{block}_r{r}"] = {
                        "kernel_ms": k_ms, "gbs": 2 * n / k_ms / 1e6,
                        "frac": 2 * n / k_ms / 1e6 / HBM_PEAK_GBS,
                        "grid_blocks": plan["grid_blocks"], "waves_per_cu": plan["waves_per_cu"],
                        "loads_in_flight_per_cu": plan["waves_per_cu"] * in_flight,
                        "result": float(mout.item())}
                    print(f"{grid_kind}_b{block}_r{r}", f"{k_ms * 1e3:.1f} us",
                          f"{2 * n / k_ms / 1e6:.0f} GB/s", f"grid {plan['grid_blocks']}",
                          f"waves/CU {plan['waves_per_cu']:.2f}", file=sys.stderr, flush=True)
                    del mws
        var["block_r_matrix_2p28"] = matrix
        record["variants"] = var

    if args.copy_calibration:
        dst = torch.empty_like(bufs[0])
        for _ in range(5):
            dst.copy_(bufs[1])
        torch.cuda.synchronize()
        record["copy_calibration"] = {"bytes_read": 2 * n, "bytes_written": 2 * n,
                                      "launches": 5, "kernel": "torch copy_ (fp16, 512 MiB)"}
        del dst

    if args.levels_sweep:
        # GPU time per call with the queue kept full: a sleep kernel holds the
        # GPU while the host enqueues the whole batch, so the calls then run
        # back to back and the host's submission rate does not enter.  Inputs
        # are prefixes of the headline buffer (contiguous, aligned); rotation
        # only matters once a prefix outgrows the Infinity Cache.
        probe_s, probe_e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        probe_s.record()
        torch.cuda._sleep(1 << 22)
        probe_e.record()
        torch.cuda.synchronize()
        cycles_per_ms = (1 << 22) / probe_s.elapsed_time(probe_e)

        def queued_us(fn, calls):
            fn(0)
            torch.cuda.synchronize()
            s_ev, e_ev = (torch.cuda.Event(enable_timing=True),
                          torch.cuda.Event(enable_timing=True))
            torch.cuda._sleep(int(cycles_per_ms * max(4.0, calls * 0.05)))
            s_ev.record()
            h0 = time.perf_counter()
            for i in range(calls):
                fn(i)
            host_ms = (time.perf_counter() - h0) * 1e3
            e_ev.record()
            torch.cuda.synchronize()
            gpu_ms = s_ev.elapsed_time(e_ev)
            return gpu_ms * 1e3 / calls, host_ms < max(4.0, calls * 0.05)

        lv = {}
        lo, hi = (int(v) for v in args.levels_log2.split("-"))
        if not 0 <= lo <= hi <= 28:
            print("--levels-log2 must lie within 0-28", file=sys.stderr)
            return 2
        for k in range(lo, hi + 1):
            m = 1 << k
            views = [bufs[0][:m], bufs[1][:m]]
            calls = 100 if k < 26 else 40
            row = {"n": m}
            for r in (1, 8):      # block size: the levels form's default
                us, ok = queued_us(lambda i: armx.reduce_sum(
                    views[i & 1], out=out, mma_levels=True, chain_r=r), calls)
                row[f"launches_r{r}"] = mma_levels_count(m, r)
                row[f"mma_levels_r{r}_us"] = us
                row[f"queue_full_r{r}"] = ok
            us, ok = queued_us(lambda i: armx.reduce_sum(views[i & 1], out=out), calls)
            row["single_launch_us"] = us
            row["queue_full_single"] = ok
            lv[f"2^{k}"] = row
            print(f"n=2^{k}", json.dumps(row), file=sys.stderr, flush=True)
        record["levels_sweep"] = lv

    print("bench: variants done", file=sys.stderr, flush=True)
    if not args.no_cpu_baseline:
        xf_cpu = si.workload("fixed_2p26_u11")
        record["cpu_baseline"], e, e30, tree26 = cpu_baseline(x_np, xf_cpu, stress_np=stress_np)
        del xf_cpu
        record["check"] = {"exact_sum": e.f64, "abs_err": abs(result - e.f64),
                           "rel_err": abs(result - e.f64) / abs(e.f64)}
        if "variants" in record:
            v = record["variants"]
            want = int(np.float32(e.f32).view(np.uint32))
            record["check"]["exact_variant_matches_oracle"] = v["exact_2p28"]["result_bits"] == want
            record["check"]["exact_int_limbs_matches_oracle"] = (
                v["exact_int_limbs_2p28"]["result_bits"] == want)
            # every point of the block x R matrix against the exact sum
            # (the 1e-5 relative gate), and fixed order against the emulator
            errs = {k: abs(p["result"] - e.f64) / abs(e.f64)
                    for k, p in v["block_r_matrix_2p28"].items()}
            record["check"]["block_r_matrix_max_rel_err"] = max(errs.values())
            record["check"]["block_r_matrix_all_within_1e-5"] = all(
                err <= 1e-5 for err in errs.values())
            record["check"]["fixed_order_2p26_matches_oracle"] = (
                v["fixed_order_2p26"]["result_bits"] == int(np.float32(tree26).view(np.uint32)))
        if e30 is not None:
            p30 = record["variants"]["precision_2p30_logu"]
            record["check"]["precision_2p30_logu"] = {
                "exact_sum": e30.f64, "abs_sum": e30.abs_sum,
                "rel_err_mfma": abs(p30["mfma"] - e30.f64) / abs(e30.f64),
                "rel_err_mfma_all_ones": abs(p30["mfma_all_ones"] - e30.f64) / abs(e30.f64),
                "rel_err_plain": abs(p30["plain"] - e30.f64) / abs(e30.f64),
                "exact_variant_matches_oracle":
                    p30["exact_result_bits"] == int(np.float32(e30.f32).view(np.uint32)),
            }

    print(json.dumps(record), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
