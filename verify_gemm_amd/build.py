"""Build libvgemm.so in-tree with hipcc for gfx950.

``python -m verify_gemm_amd.build`` (or ``__graft_entry__.build()``)
compiles every HIP source under ``csrc/`` into ``verify_gemm_amd/libvgemm.so``:
each source to an object file (in parallel: the stream kernel's variants
sit in one translation unit per M-tile class and weight format), then one
link.  It also links ``libvgemm_stamps.so``, the same library with the M = 1
step kernel built with VG_STAGE_STAMPS (per-stage timestamps, read by
``verify_gemm_amd.stage_stamps``); nothing else loads it.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libvgemm.so")
LIB_STAMPS = os.path.join(PKG, "libvgemm_stamps.so")
SOURCES = (["api.cpp", "stream.hip", "step_gemv.hip", "bwprobe.hip", "noalloc.hip"]
           + [f"stream_mt{mt}_f{fmt}.hip" for mt in range(6) for fmt in range(2)])
ARCH = "gfx950"

# Packed-fp32 VALU forms are disabled for all device code: hipcc may form
# them from ordinary float code, and they are not needed on this path.
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result", "-Wno-inline-asm", "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libvgemm.so)")


def _jobs() -> int:
    env = os.environ.get("MAX_JOBS")
    if env and env.isdigit() and int(env) > 0:
        return int(env)
    return max(1, min(16, len(os.sched_getaffinity(0))))


def build(verbose: bool = False) -> str:
    """Compile libvgemm.so (always rebuilds).  Returns its path."""
    cc = hipcc()
    with tempfile.TemporaryDirectory(prefix="vgemm_build_") as tmp:
        def compile_one(task):
            src, defs = task
            obj = os.path.join(tmp, src + ("".join(defs) if defs else "") + ".o")
            cmd = [cc, *HIPCC_FLAGS, *defs, "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            res = subprocess.run(cmd, capture_output=True, text=True)
            return src, obj, res

        # the slowest translation units first
        order = sorted(SOURCES, key=lambda f: (not f.startswith("stream_mt"), f))
        tasks = [(src, []) for src in order] + [("step_gemv.hip", ["-DVG_STAGE_STAMPS"])]
        with concurrent.futures.ThreadPoolExecutor(_jobs()) as ex:
            results = list(ex.map(compile_one, tasks))
        for src, _, res in results:
            if res.returncode != 0:
                sys.stderr.write(res.stdout + res.stderr)
                raise RuntimeError(f"hipcc failed on {src} with exit code {res.returncode}")
        plain = [obj for _, obj, _ in results[:len(order)]]
        stamped = [results[-1][1] if src == "step_gemv.hip" else obj for (src, obj, _) in results[:len(order)]]
        for lib, objs in ((LIB, plain), (LIB_STAMPS, stamped)):
            cmd = [cc, f"--offload-arch={ARCH}", "-fPIC", "-shared", *objs, "-o", lib + ".tmp"]
            if verbose:
                print(" ".join(cmd), flush=True)
            res = subprocess.run(cmd, capture_output=True, text=True)
            if res.returncode != 0:
                sys.stderr.write(res.stdout + res.stderr)
                raise RuntimeError(f"hipcc link of {os.path.basename(lib)} failed with exit code {res.returncode}")
    os.replace(LIB_STAMPS + ".tmp", LIB_STAMPS)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
