"""The library's host code under AddressSanitizer, on the CPU.

Builds the library with the host side instrumented (the device side only
compiled, unoptimised: nothing here launches a kernel) and runs a C program
that drives every entry point's argument checks and error-message paths
(tests/asan/abi_host.c).  Any heap or stack misuse, or a leak, in those paths
fails the run.  The build is cached under _build/asan and redone when a
source changes."""
import glob
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "asan")
SRC = os.path.join(ROOT, "step_flow_map_amd", "csrc", "flashmap.hip")
DRIVER = os.path.join(ROOT, "tests", "asan", "abi_host.c")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"


def _newest(paths):
    return max(os.path.getmtime(p) for p in paths)


def _stale(target, sources):
    return not os.path.exists(target) or os.path.getmtime(target) < _newest(sources)


def test_host_abi_under_asan():
    if not (os.path.exists(HIPCC) and os.path.exists(CLANG)):
        pytest.skip("ROCm toolchain not available")
    os.makedirs(OUT, exist_ok=True)
    lib = os.path.join(OUT, "libflashmap_asan.so")
    exe = os.path.join(OUT, "abi_host")
    sources = glob.glob(os.path.join(ROOT, "step_flow_map_amd", "csrc", "*")) + [
        os.path.join(ROOT, "include", "flashmap.h")]
    if _stale(lib, sources):
        cmd = [HIPCC, "--offload-arch=gfx950", "-g", "-std=c++17", "-fPIC", "-shared",
               "-Xarch_device", "-O0", "-Xarch_host", "-O1",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
               "-I", os.path.join(ROOT, "include"), "-o", lib + ".tmp", SRC]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-4000:]
        os.replace(lib + ".tmp", lib)
    if _stale(exe, [lib, DRIVER]):
        cmd = [CLANG, "-std=c11", "-g", "-fsanitize=address", "-fno-omit-frame-pointer",
               "-I", os.path.join(ROOT, "include"), "-o", exe, DRIVER,
               "-L", OUT, "-lflashmap_asan", "-Wl,-rpath," + OUT]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert "AddressSanitizer" not in r.stderr and "LeakSanitizer" not in r.stderr, r.stderr[-4000:]
    assert r.returncode == 0, r.stdout + r.stderr[-4000:]
    assert "all checks passed" in r.stdout
