"""Every entry point inside a captured HIP graph (replayed several times with
eager work and synchronisations between replays, each replay checked against
an eager call on the same data), and concurrent calls on several streams."""
import numpy as np
import pytest
import torch

import arithmetic_reduction_matrix_amd as armx
import synth_inputs as si
from oracle import exact_sum, fixed_tree_sum

from _parity import bits32, check_free_order, require_gpu, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _bits(t):
    return np.ascontiguousarray(t.cpu().numpy(), dtype=np.float32).view(np.uint32)


def test_graph_capture_and_replay():
    n = (1 << 22) + 5
    pool = [to_dev(si.generate("uniform11", n, seed=100 + i)) for i in range(5)]
    rpool = [to_dev(si.generate_rows("normal", 256, 4096, seed=200 + i)) for i in range(5)]
    # short rows (100 values, pitch 104) and ragged rows (1000 values)
    spool = [to_dev(si.generate_rows("uniform11", 3000, 104, seed=400 + i)) for i in range(5)]
    gpool = [to_dev(si.generate_rows("uniform11", 5000, 1000, seed=500 + i)) for i in range(5)]
    sm = torch.empty_like(spool[0])
    gm = torch.empty_like(gpool[0])
    sv = sm[:, :100]
    o_srows = torch.empty(3000, dtype=torch.float32, device="cuda")
    o_sfix = torch.empty(3000, dtype=torch.float32, device="cuda")
    o_grows = torch.empty(5000, dtype=torch.float32, device="cuda")
    o_gfix = torch.empty(5000, dtype=torch.float32, device="cuda")
    x = torch.empty_like(pool[0])
    m = torch.empty_like(rpool[0])
    x.copy_(pool[0])
    m.copy_(rpool[0])
    o_sum = torch.empty((), dtype=torch.float32, device="cuda")
    o_fix = torch.empty((), dtype=torch.float32, device="cuda")
    o_rows = torch.empty(256, dtype=torch.float32, device="cuda")
    o_rfix = torch.empty(256, dtype=torch.float32, device="cuda")
    ws_sum = torch.zeros(armx.workspace_bytes(armx.OP_SUM, n), dtype=torch.uint8, device="cuda")
    ws_fix = torch.zeros(armx.workspace_bytes(armx.OP_FIXED, n), dtype=torch.uint8, device="cuda")
    o_ex = torch.empty((), dtype=torch.float32, device="cuda")
    o_exq = torch.zeros(2, dtype=torch.int64, device="cuda")
    ws_ex = torch.zeros(armx.workspace_bytes(armx.OP_EXACT, n), dtype=torch.uint8, device="cuda")
    o_lv = torch.empty((), dtype=torch.float32, device="cuda")
    ws_lv = torch.zeros(armx.workspace_bytes(armx.OP_SUM, n, mma_levels=True), dtype=torch.uint8,
                        device="cuda")

    def calls():
        armx.reduce_sum(x, out=o_sum, workspace=ws_sum)
        armx.reduce_sum_fixed_order(x, out=o_fix, workspace=ws_fix)
        armx.reduce_rows(m, out=o_rows)
        armx.reduce_rows_fixed_order(m, out=o_rfix)
        armx.reduce_sum_exact(x, out=o_ex, fixed=o_exq, workspace=ws_ex)
        armx.reduce_sum(x, out=o_lv, workspace=ws_lv, mma_levels=True)
        armx.reduce_rows(sv, out=o_srows)
        armx.reduce_rows_fixed_order(sv, out=o_sfix)
        armx.reduce_rows(gm, out=o_grows)
        armx.reduce_rows_fixed_order(gm, out=o_gfix)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()

    for rep in range(5):
        x.copy_(pool[rep])           # eager work between replays
        m.copy_(rpool[rep])
        sm.copy_(spool[rep])
        gm.copy_(gpool[rep])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [_bits(o_sum), _bits(o_fix), _bits(o_rows), _bits(o_rfix), _bits(o_ex),
               _bits(o_lv)]
        got_q = armx.fixed_to_int(o_exq.cpu())
        # eager calls on the same data (own outputs and workspaces)
        e_sum = armx.reduce_sum(x)
        e_fix = armx.reduce_sum_fixed_order(x)
        e_rows = armx.reduce_rows(m)
        e_rfix = armx.reduce_rows_fixed_order(m)
        e_ex = armx.reduce_sum_exact(x)
        e_lv = armx.reduce_sum(x, mma_levels=True)
        torch.cuda.synchronize()
        assert np.array_equal(got[0], _bits(e_sum)), rep
        assert np.array_equal(got[1], _bits(e_fix)), rep
        assert np.array_equal(got[2], _bits(e_rows)), rep
        assert np.array_equal(got[3], _bits(e_rfix)), rep
        assert np.array_equal(got[4], _bits(e_ex)), rep
        assert np.array_equal(got[5], _bits(e_lv)), rep
        for o, fn, mat in ((o_srows, armx.reduce_rows, sv), (o_sfix, armx.reduce_rows_fixed_order, sv),
                           (o_grows, armx.reduce_rows, gm), (o_gfix, armx.reduce_rows_fixed_order, gm)):
            assert np.array_equal(_bits(o), _bits(fn(mat))), (rep, fn.__name__, tuple(mat.shape))
        if rep in (0, 4):
            xh = pool[rep].cpu().numpy()
            e = exact_sum(xh)
            assert got[1][()] == bits32(fixed_tree_sum(xh))
            assert got[4][()] == bits32(e.f32) and got_q == e.q
            check_free_order(float(o_sum.item()), e, f"replay {rep}")
            check_free_order(float(o_lv.item()), e, f"levels replay {rep}")


def test_concurrent_streams():
    n = (1 << 21) + 333
    data = [si.generate("uniform11", n, seed=300 + i) for i in range(4)]
    xs = [to_dev(d) for d in data]
    streams = [torch.cuda.Stream() for _ in range(4)]
    outs, fixed = [None] * 4, [None] * 4
    for i, s in enumerate(streams):
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for _ in range(3):
                outs[i] = armx.reduce_sum(xs[i])
                fixed[i] = armx.reduce_sum_fixed_order(xs[i])
    torch.cuda.synchronize()
    for i in range(4):
        check_free_order(float(outs[i].item()), exact_sum(data[i]), f"stream {i}")
        assert _bits(fixed[i])[()] == bits32(fixed_tree_sum(data[i]))
