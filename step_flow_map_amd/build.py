"""Build libflashmap.so (the HIP library behind include/flashmap.h) in-tree.

    python -m step_flow_map_amd.build

compiles step_flow_map_amd/csrc/flashmap.hip for gfx950 with hipcc.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "flashmap.hip")
OUT = os.path.join(PKG, "libflashmap.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # keep the compiler from forming packed fp32 instructions on its own
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPRs: no AGPR copies around loop joins (this
    # compiler under-counts the wait before reading an AGPR an MFMA wrote there)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I", os.path.join(ROOT, "include"),
]


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = OUT + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, "-o", tmp, SRC]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{' '.join(cmd)}\n{msg}")
    if verbose and msg.strip():
        print(msg)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
