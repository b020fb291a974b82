"""Build libvgemm.so in-tree with hipcc for gfx950.

``python -m verify_gemm_amd.build`` (or ``__graft_entry__.build()``)
compiles every HIP source under ``csrc/`` into ``verify_gemm_amd/libvgemm.so``.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libvgemm.so")
SOURCES = ["api.cpp", "stream.hip", "step_gemv.hip", "bwprobe.hip"]
ARCH = "gfx950"

# Packed-fp32 VALU forms are disabled for all device code: hipcc may form
# them from ordinary float code, and they are not needed on this path.
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result", "-Wno-inline-asm", "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libvgemm.so)")


def build(verbose: bool = False) -> str:
    """Compile libvgemm.so (always rebuilds).  Returns its path."""
    out_tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *[os.path.join(CSRC, s) for s in SOURCES], "-o", out_tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    os.replace(out_tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
