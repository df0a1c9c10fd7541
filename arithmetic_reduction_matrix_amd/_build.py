"""Builds libarmx.so (the HIP kernels and the C entry points) for gfx950, and
libarmx_probe.so (a plain read stream, for measurement only).

Run ``python arithmetic_reduction_matrix_amd/_build.py`` or call ``build()`` (it needs
only the standard library, so it runs whether or not a library is built).
Every source is compiled each time; objects go to ``_build/`` next to this
file and the library is written to ``libarmx.so`` in this package.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libarmx.so")
# measurement only: the plain read stream the reductions are compared with
PROBE_LIB = os.path.join(PKG, "libarmx_probe.so")
PROBE_SOURCES = ["read_probe.hip"]

ARCH = "gfx950"
HIP_SOURCES = ["sum_kernels.hip", "fixed_kernels.hip", "rows_kernels.hip", "exact_kernels.hip",
               "rows_fixed_kernels.hip", "levels_kernels.hip", "short_rows_kernels.hip"]
HOST_SOURCES = ["api.cpp", "plan.cpp"]

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          f"-I{INCLUDE}", f"-I{CSRC}"]
# packed fp32 instructions are kept out of the device code
DEVICE = [f"--offload-arch={ARCH}", "-fno-gpu-rdc", "-ffp-contract=off",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def _run(cmd: list[str], verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    p = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature and says so; that
    # warning is expected and not shown
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in p.stderr.splitlines() if noise not in l)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compiles every source and links libarmx.so; returns its path."""
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(8, os.cpu_count() or 1)
    objs = []
    cmds = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        objs.append(obj)
        cmds.append([hipcc, *COMMON, *DEVICE, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj])
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        objs.append(obj)
        cmds.append([hipcc, *COMMON, "-c", os.path.join(CSRC, src), "-o", obj])
    probe_objs = []
    for src in PROBE_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        probe_objs.append(obj)
        cmds.append([hipcc, *COMMON, *DEVICE, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=jobs) as pool:
        list(pool.map(lambda c: _run(c, verbose), cmds))
    for out, parts in ((LIB, objs), (PROBE_LIB, probe_objs)):
        tmp = out + ".tmp"
        _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *parts, "-o", tmp], verbose)
        os.replace(tmp, out)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
