"""Benchmark: the full NVFP4 weight pass of a decode / verify step on one MI355X.

One step = one pass over the whole hot path: 64 layers x {q, k, v, o, gate,
up, down} NVFP4 GEMMs + the lm_head with fused argmax and greedy accept
(449 matrices, 14,115,962,880 weight bytes), captured once into a HIP graph
and replayed.  Reported at M = 1 (plain decode), 4, 17 (16 drafts + 1) and
68 (4 sequences x 17): microseconds per pass and effective weight GB/s
against the 8 TB/s HBM peak.  ``value`` is the M = 1 figure; the other
batch sizes are in ``per_m``.

Also measured in the same run:
  * the read ceiling of a pure streaming-read kernel (vg_bwprobe);
  * the dominant kernel (the 17408x5120 decode GEMV, rotating through the
    128 gate/up matrices so no launch is served from the 256 MB Infinity
    Cache) timed with events on its own stream -> ``roofline``;
  * the CPU oracle on a bounded sample (layer 0's seven matrices at M = 1)
    on this host's cores -> ``cpu_baseline``.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--ms 1,4,17,68]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

HBM_PEAK_GBPS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--ms", default="1,4,17,68")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-stream-ordered", action="store_true")
    ap.add_argument("--kernel-reps", type=int, default=256)
    return ap.parse_args()


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def time_replays(run, steps, warmup):
    import torch
    for _ in range(warmup):
        run.replay()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(steps):
        run.replay()
    e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def time_stream_ordered(run, steps):
    import torch
    run.launch()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(steps):
        run.launch()
    e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def dominant_kernel(weights, M, reps):
    """Average duration of the 17408x5120 GEMV at batch M, each launch on a
    different gate/up matrix (6.4 GB rotation: cold in the Infinity Cache),
    timed with events recorded on the stream the kernels run on."""
    import ctypes

    import torch

    from verify_gemm_amd import binding, synth
    lib = binding.load()
    mats = [m for m in weights.mats if m["name"] in ("gate", "up")]
    n, k = synth.MLP, synth.HIDDEN
    x = synth.gen_x_device(M, k, 4242, weights.device)
    y = torch.empty((M, n), dtype=torch.float32, device=weights.device)
    wsb = lib.vg_gemm_workspace_bytes(M, n, k)
    wsp = torch.zeros(max(wsb, 1), dtype=torch.uint8, device=weights.device)
    stream = torch.cuda.Stream()
    sp = int(stream.cuda_stream)

    def go(count):
        for i in range(count):
            m = mats[i % len(mats)]
            st = lib.nvfp4_gemm_ex(x.data_ptr(), m["wq"].data_ptr(), m["ws"].data_ptr(),
                                   ctypes.c_float(m["g"]), M, n, k, y.data_ptr(),
                                   wsp.data_ptr() if wsb else None, wsb, sp)
            if st:
                raise binding.VgemmError(st, "nvfp4_gemm_ex")
    with torch.cuda.stream(stream):
        go(len(mats))
        stream.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        go(reps)
        e1.record(stream)
        stream.synchronize()
    us = e0.elapsed_time(e1) * 1000.0 / reps
    bytes_per_launch = n * k // 2 + n * k // 16
    return us, bytes_per_launch


def bwprobe(device, gib=8, reps=10):
    import torch

    from verify_gemm_amd import binding
    nbytes = gib << 30
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device=device)
    sink = torch.empty(binding.bwprobe_sink_floats(), dtype=torch.float32, device=device)
    binding.bwprobe(buf, sink)
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(reps):
        binding.bwprobe(buf, sink)
    e1.record(s)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del buf
    return nbytes / (ms * 1e-3) / 1e9


def cpu_baseline(weights):
    """The CPU oracle, untuned, on layer 0's seven matrices at M = 1."""
    import numpy as np

    import oracle
    from verify_gemm_amd import synth
    cores = len(os.sched_getaffinity(0))
    mats = [m for m in weights.mats if m["layer"] == 0]
    host = []
    nbytes = 0
    for m in mats:
        host.append((m["wq"].cpu().numpy(), m["ws"].cpu().numpy(), m["g"], m["k"]))
        nbytes += m["wq"].numel() + m["ws"].numel()
    rng = np.random.default_rng(5)
    xs = {k: synth.gen_x(rng, 1, k, 0.1) for k in (synth.HIDDEN, synth.MLP)}
    t0 = time.perf_counter()
    for wq, ws, g, k in host:
        oracle.nvfp4_gemm_ref(xs[k], wq, ws, g, with_bound=False)
    dt = time.perf_counter() - t0
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"layer 0 (q,k,v,o,gate,up,down; {nbytes} weight bytes) at M=1, fp64 numpy "
                      f"oracle without bounds, {dt:.2f} s; x{14115962880 / nbytes:.1f} of this is one full pass "
                      f"(~{dt * 14115962880 / nbytes:.0f} s)"}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(sharding is design-only); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch

    from verify_gemm_amd import binding, weightpass
    binding.load()
    dev = torch.device("cuda:0")
    t_start = time.time()
    log("[bench] generating the 449 NVFP4 matrices on the device")
    weights = weightpass.PassWeights(dev)
    wbytes = weights.weight_bytes()
    torch.cuda.synchronize()
    log(f"[bench] weights: {wbytes} bytes in {time.time() - t_start:.1f}s")
    probe = bwprobe(dev)
    log(f"[bench] bwprobe read ceiling {probe:.0f} GB/s")
    ms_list = [int(v) for v in args.ms.split(",")]
    per_m = {}
    for M in ms_list:
        run = weightpass.PassRun(weights, M)
        run.capture()
        ms = time_replays(run, args.steps, args.warmup)
        entry = {"us_per_pass": round(ms * 1000, 2), "weight_gbps": round(wbytes / (ms * 1e-3) / 1e9, 1),
                 "pct_hbm_peak": round(100 * wbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
                 "pct_of_probe": round(100 * wbytes / (ms * 1e-3) / 1e9 / probe, 2)}
        if not args.no_stream_ordered:
            so = time_stream_ordered(run, 3)
            entry["stream_ordered_us_per_pass"] = round(so * 1000, 1)
        per_m[str(M)] = entry
        log(f"[bench] M={M}: {entry}")
        del run
        torch.cuda.empty_cache()
    dom_m = ms_list[0]
    kus, kbytes = dominant_kernel(weights, dom_m, args.kernel_reps)
    achieved = kbytes / (kus * 1e-6) / 1e9
    log(f"[bench] dominant kernel 17408x5120 at M={dom_m}: {kus:.2f} us, {achieved:.0f} GB/s")
    head = per_m[str(ms_list[0])]
    out = {
        "metric": "µs per full weight pass + effective weight GB/s (% HBM peak) at M=1/17/68",
        "value": head["weight_gbps"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["us_per_pass"] / 1000, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e2m1/e4m3 weights x bf16 activations, fp32 accumulation",
        "data": "synthetic (seeded device RNG, codes uniform, scales 2^u)",
        "config": {"workload": "full synthetic weight pass: 64 layers x {q,k,v,o 5120x5120; gate,up "
                               "17408x5120; down 5120x17408} + lm_head 248320x5120 with argmax/accept "
                               f"(449 NVFP4 matrices, {wbytes} weight bytes), one HIP graph per pass",
                   "M": ms_list[0], "M_reported": ms_list, "graph": True},
        "per_m": per_m,
        "bwprobe_read_gbps": round(probe, 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None,
                     "kernel": f"nvfp4_gemm 17408x5120 at M={dom_m}", "avg_us": round(kus, 3),
                     "bytes_per_launch": kbytes},
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on layer 0 (bounded sample)")
        out["cpu_baseline"] = cpu_baseline(weights)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
