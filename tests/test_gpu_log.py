"""ARMX_LOG: with the variable set, each accepted call writes its launch plan
to stderr; without it the library prints nothing.  Run in child processes so
the variable is read fresh."""
import os
import subprocess
import sys

import pytest

from _parity import require_gpu

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SCRIPT = """
import torch
import arithmetic_reduction_matrix_amd as armx
x = torch.ones(1 << 20, dtype=torch.float16, device="cuda")
assert armx.reduce_sum(x).item() == float(1 << 20)
assert armx.reduce_sum_exact(x).item() == float(1 << 20)
assert armx.reduce_rows(x.view(256, 4096))[0].item() == 4096.0
torch.cuda.synchronize()
"""


def _run(env_extra):
    env = dict(os.environ)
    env.pop("ARMX_LOG", None)
    env.update(env_extra)
    return subprocess.run([sys.executable, "-c", SCRIPT], cwd=ROOT, env=env,
                          capture_output=True, text=True, timeout=120)


def test_plan_lines_only_when_asked():
    require_gpu()
    on = _run({"ARMX_LOG": "1"})
    assert on.returncode == 0, on.stderr[-2000:]
    lines = [l for l in on.stderr.splitlines() if l.startswith("armx: ")]
    assert any(l.startswith("armx: reduce_sum n=1048576 ") for l in lines), lines
    assert any(l.startswith("armx: reduce_sum_exact ") for l in lines), lines
    assert any(l.startswith("armx: reduce_rows ") and "rows=256" in l for l in lines), lines
    off = _run({})
    assert off.returncode == 0, off.stderr[-2000:]
    assert not [l for l in off.stderr.splitlines() if l.startswith("armx: ")]
