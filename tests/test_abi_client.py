"""The C ABI from plain C: tests/native/abi_client.c, compiled with gcc
against include/armx.h and linked to libarmx.so, checks argument errors and
workspace sizes on the CPU and, on a GPU, runs three entry points on
hipMalloc'd buffers."""
import os
import shutil
import subprocess

import pytest

import arithmetic_reduction_matrix_amd as armx

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.dirname(armx.LIB_PATH)


def _build(tmp_path):
    exe = tmp_path / "abi_client"
    cmd = ["gcc", "-std=c99", "-O1", "-Wall", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "native", "abi_client.c"), "-o", str(exe),
           "-L", LIBDIR, "-larmx", "-L/opt/rocm/lib", "-lamdhip64",
           f"-Wl,-rpath,{LIBDIR}", "-Wl,-rpath,/opt/rocm/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_c_client_cpu(tmp_path):
    exe = _build(tmp_path)
    r = subprocess.run([str(exe), "cpu"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr


@pytest.mark.gpu
@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_c_client_gpu(tmp_path):
    exe = _build(tmp_path)
    r = subprocess.run([str(exe), "gpu"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "cpu+gpu checks: ok" in r.stdout
