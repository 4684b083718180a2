"""In-tree builds of the package's native libraries.

- ``libsmla.so``: the HIP library behind the C ABI of ``include/smla.h`` (gfx950 only).
- ``workload/libsmla_workload.so``: the host-only input generator and result comparisons.

Built objects stay in the source tree so they travel with it; nothing is installed.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
INCLUDE = os.path.join(ROOT, "include")
CSRC = os.path.join(PKG, "csrc")
HIP_LIB = os.path.join(PKG, "libsmla.so")
WORKLOAD_LIB = os.path.join(PKG, "workload", "libsmla_workload.so")
ARCH = "gfx950"

# Packed FP32 instructions are kept out of the generated code (the code is written for scalar
# fp32; see the build notes of the library).
HIP_FLAGS = [
    "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-munsafe-fp-atomics", "-Wall", "-Wno-unused-function",
]
# Per-source additions (none at present).
FILE_FLAGS: dict = {}


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def build_workload(verbose: bool = False) -> str:
    src = os.path.join(PKG, "workload", "smla_workload.c")
    tmp = WORKLOAD_LIB + ".tmp"
    _run(["gcc", "-O3", "-std=c11", "-D_GNU_SOURCE", "-fPIC", "-shared", "-pthread", "-Wall",
          "-Wextra", f"-I{INCLUDE}", "-o", tmp, src, "-lm"], verbose)
    os.replace(tmp, WORKLOAD_LIB)
    return WORKLOAD_LIB


def hip_sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + sorted(
        glob.glob(os.path.join(CSRC, "*.cpp")))


def build_hip(verbose: bool = False, extra=()) -> str:
    """Compiles every source to an object (with its per-file flags), then links the library."""
    srcs = hip_sources()
    if not srcs:
        raise RuntimeError("no HIP sources found")
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    compile_flags = [f for f in HIP_FLAGS if f != "-shared"]
    objs = []
    for src in srcs:
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        _run([hipcc, *compile_flags, *FILE_FLAGS.get(os.path.basename(src), []), *extra,
              f"-I{INCLUDE}", f"-I{CSRC}", "-c", "-o", obj, src], verbose)
        objs.append(obj)
    tmp = HIP_LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-fPIC", "-shared", "-o", tmp, *objs], verbose)
    os.replace(tmp, HIP_LIB)
    return HIP_LIB


def build_all(verbose: bool = False):
    return [build_workload(verbose), build_hip(verbose)]


if __name__ == "__main__":
    build_all(verbose="-v" in sys.argv)
