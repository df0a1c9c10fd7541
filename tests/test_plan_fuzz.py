"""The launch planner (plain C++, no HIP) fuzzed on the host under
AddressSanitizer and UBSan: every accepted plan satisfies the invariants the
kernels rely on (all chunks covered, power-of-two ranges, LDS and workspace
sizes), and nothing reads out of bounds or overflows."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "arithmetic_reduction_matrix_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_plan_fuzz_under_sanitizers(tmp_path):
    exe = tmp_path / "plan_fuzz"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(ROOT, "tests", "native", "plan_fuzz.cpp"), os.path.join(CSRC, "plan.cpp"),
           "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe), "200000"], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "violations 0" in r.stdout
