"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU: the oracle, the
workload generator and the library's host side (argument validation, batch planning) built with
clang's sanitizers (the device code objects are the regular ones), then the oracle pins and the
C-ABI checks run against those builds in a child process with the sanitizer runtime preloaded.
Any report fails the test."""
import glob
import os
import subprocess
import sys

import pytest

from sparse_mla_attention_indexer_amd import _build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
       "-fno-omit-frame-pointer", "-shared-libasan"]


def _runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, (cmd, r.stdout[-2000:], r.stderr[-2000:])
    return r


@pytest.mark.skipif(not (os.path.exists(CLANG) and os.path.exists(HIPCC) and _runtime()),
                    reason="clang sanitizer runtime not installed")
def test_host_code_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    c_flags = ["-O1", "-g", "-std=c11", "-D_GNU_SOURCE", "-fPIC", "-shared", "-pthread", *SAN]
    oracle_so = str(tmp_path / "libsmla_oracle_san.so")
    workload_so = str(tmp_path / "libsmla_workload_san.so")
    _run([CLANG, *c_flags, "-o", oracle_so, os.path.join(ROOT, "oracle", "smla_oracle.c"), "-lm"])
    _run([CLANG, *c_flags, "-I", os.path.join(ROOT, "include"), "-o", workload_so,
          os.path.join(ROOT, "sparse_mla_attention_indexer_amd", "workload", "smla_workload.c"), "-lm"])
    # the library: host translation units sanitized (each flag for the host pass only), device
    # objects as the regular build makes them
    host = [a for f in SAN for a in ("-Xarch_host", f)]
    csrc = os.path.join(ROOT, "sparse_mla_attention_indexer_amd", "csrc")
    api_o = str(tmp_path / "api_san.o")
    _run([HIPCC, "-O1", "-g", "-std=c++17", f"--offload-arch={_build.ARCH}", "-fPIC",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *host,
          "-I", os.path.join(ROOT, "include"), "-I", csrc, "-c", os.path.join(csrc, "api.cpp"),
          "-o", api_o])
    objs = [o for o in sorted(glob.glob(os.path.join(os.path.join(_build.PKG, "_build"), "*.hip.o")))]
    if len(objs) != len(_build.hip_sources()) - 1:
        _build.build_hip()
        objs = sorted(glob.glob(os.path.join(os.path.join(_build.PKG, "_build"), "*.hip.o")))
    lib_so = str(tmp_path / "libsmla_san.so")
    _run([HIPCC, f"--offload-arch={_build.ARCH}", "-fPIC", "-shared", *host, "-o", lib_so, api_o, *objs])

    env = dict(os.environ,
               LD_PRELOAD=_runtime(),
               ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               SMLA_ORACLE_LIB=oracle_so, SMLA_WORKLOAD_LIB=workload_so, SMLA_LIB=lib_so)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
                        "tests/test_oracle_pins.py", "tests/test_abi.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=1200)
    out = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in r.stdout
