"""Where each dependency stage of the M = 1 step spends its time.

``python -m verify_gemm_amd.stage_stamps [--fused] [--out FILE]`` runs the
64-layer synthetic pass at M = 1 with ``libvgemm_stamps.so`` (the library
with the step kernel built with VG_STAGE_STAMPS; ``verify_gemm_amd.build``
links it beside ``libvgemm.so``) and reads, for every stage and workgroup,
the s_memrealtime stamps the kernel took:

  detect   the I/O wave saw the previous stage complete;
  ready    the stage's first activation row and scales were in LDS;
  done     the compute waves had finished the stage's last chunk;
  signal   its result stores had completed, just before the signal.

Per stage s it forms the parts of the span from the previous stage's last
signal to its own: detection (detect - last signal of s - 1), the
activation and scale copy (ready - detect), compute (done - ready), the
stores (signal - done), and the straggler (last signal - median signal);
medians over workgroups, then the mean over the layers of each stage kind
(q|k|v, o, gate|up, down), leaving out the first and last layer.  It writes
a markdown summary with the command that made it.  A diagnostic: each stamp
is an extra store, so the stamped pass runs a little slower than the
product library (the summary gives both pass times).
"""
from __future__ import annotations

import argparse
import ctypes
import os
import sys

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB_STAMPS = os.path.join(PKG, "libvgemm_stamps.so")
KINDS, STAGES, WGS = 4, 1024, 256   # the kernel's stamp array: [kind][stage][workgroup]
DETECT, READY, DONE, SIGNAL = range(4)
STAGE_NAMES = ("q|k|v", "o", "gate|up", "down")
TICK_US = 0.01                      # s_memrealtime counts at 100 MHz


def stage_parts(st: np.ndarray, nstages: int, grid: int) -> dict:
    """Per stage kind, the mean over layers of the per-stage medians (µs)."""
    st = st[:, :, :grid].astype(np.int64)
    rows = {k: [] for k in range(4)}
    for s in range(5, nstages - 5):       # layers 1 .. 62
        prev_last = st[SIGNAL, s - 1].max()
        det, rdy, done, sig = st[DETECT, s], st[READY, s], st[DONE, s], st[SIGNAL, s]
        rows[s % 4].append([np.median(det - prev_last), np.median(rdy - det), np.median(done - rdy),
                            np.median(sig - done), sig.max() - np.median(sig), sig.max() - prev_last])
    return {k: (np.mean(np.array(v), axis=0) * TICK_US).tolist() for k, v in rows.items()}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--fused", action="store_true", help="the 257-job step (q|k|v and gate|up stacked)")
    ap.add_argument("--out", default=None, help="write the markdown summary here (default: stdout)")
    args = ap.parse_args(argv)

    import torch
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    from verify_gemm_amd import binding, weightpass

    lib = binding.load(LIB_STAMPS)
    lib.vg_stage_stamps.restype = ctypes.c_int
    lib.vg_stage_stamps.argtypes = [ctypes.c_void_p]
    w = weightpass.PassWeights("cuda")
    run = weightpass.PassRun(w, 1, fused=args.fused)
    info = run.step.info()
    grid, nstages = info["grid"], info["stages"]
    if grid > WGS or nstages > STAGES:
        raise SystemExit(f"grid {grid} / {nstages} stages exceed the stamp array ({WGS} / {STAGES})")
    for _ in range(6):
        run.run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        run.run()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / 10 * 1000
    if run.step.check() != 0:
        raise SystemExit("a stage wait timed out: the stamps are not a normal run")
    st = np.zeros((KINDS, STAGES, WGS), dtype=np.uint64)
    if lib.vg_stage_stamps(st.ctypes.data_as(ctypes.c_void_p)) != 0:
        raise SystemExit("vg_stage_stamps failed")
    parts = stage_parts(st, nstages, grid)
    run.close()

    jobs = 257 if args.fused else 449
    cmd = "python -m verify_gemm_amd.stage_stamps" + (" --fused" if args.fused else "") + \
        (f" --out {os.path.relpath(args.out, ROOT)}" if args.out else "")
    lines = [f"# Each stage of the M = 1 step, part by part ({jobs} jobs)", "",
             "Command (from the repository root, `libvgemm_stamps.so` built by `verify_gemm_amd.build`):", "",
             "```", cmd, "```", "",
             f"The stamped library ran the {jobs}-job pass in {us:.1f} us (mean of 10 passes; each stamp is an "
             f"extra store, so the product library is a little faster). Grid {grid} workgroups, {nstages} stages. "
             "Medians over workgroups, mean over layers 1-62, us:", "",
             "| stage | detect | activations + scales | compute | stores | straggler | last signal to last signal |",
             "|---|---:|---:|---:|---:|---:|---:|"]
    for k in range(4):
        v = parts[k]
        lines.append(f"| {STAGE_NAMES[k]} | " + " | ".join(f"{x:.2f}" for x in v) + " |")
    per_layer = sum(parts[k][5] for k in range(4))
    boundary = sum(parts[k][0] + parts[k][1] + parts[k][3] + parts[k][4] for k in range(4))
    lines += ["", f"Per layer: {per_layer:.1f} us from one down-projection signal to the next, of which "
              f"{boundary:.1f} us are detection, copies, stores and the straggler (the median workgroup's "
              "parts plus the last signal's lag; compute of the median workgroup fills the rest)."]
    text = "\n".join(lines) + "\n"
    if args.out:
        with open(args.out, "w") as f:
            f.write(text)
    print(text, flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
