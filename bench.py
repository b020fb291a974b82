"""Benchmark: the full NVFP4 weight pass of a decode / verify step on one MI355X.

One step = one pass over the whole hot path: 64 layers x {q, k, v, o, gate,
up, down} NVFP4 GEMMs + the lm_head with fused argmax and greedy accept
(449 matrices, 14,115,962,880 weight bytes), run by the native step
executor (vg_pass_run) in its faster schedule: ONE persistent kernel launch
at M = 1, one launch per job at M >= 2 (there the hardware dispatcher
balances each matrix's blocks; the persistent launch is timed beside it as
``persistent_us_per_pass``).  Each layer's q, k, v (and
gate, up) are stored back to back and read as one stacked matrix -- 257 jobs
-- with each member's own tensor scale kept as per-row scales, so every
output has the same bits as with 449 separate jobs (the fused projections
of dgx-spark-qwen38 README, opening section).  Reported at M = 1 (plain
decode), 4, 17 (16 drafts + 1) and 68 (4 sequences x 17): microseconds per
pass and effective weight GB/s against the 8 TB/s HBM peak.  ``value`` is
the M = 1 figure; every batch size is in ``per_m``.

Also measured in the same run:
  * the read ceiling of a pure streaming-read kernel (vg_bwprobe);
  * the same step as one launch per job, captured in a HIP graph
    (``unfused_graph_us_per_pass``), and as 449 separate jobs, one launch
    and one launch per job (``separate_jobs``): the schedules the single
    launch replaces;
  * ``roofline``: the dominant kernel is the step kernel itself (the whole
    pass is one launch): 14,115,962,880 weight bytes per launch over its
    event-timed average duration at the first M;
  * ``roofline.traffic``: HBM bytes per launch of that kernel from the
    committed rocprofv3 counter summary (profiles/), null once the kernel
    sources differ from the ones the counters were taken with;
  * the CPU oracle on a bounded sample (whole layers at M = 1, about 12 s
    of oracle time) on this host's cores -> ``cpu_baseline``.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--ms 1,4,17,68]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

HBM_PEAK_GBPS = 8000.0
PASS_WEIGHT_BYTES = 14115962880


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--ms", default="1,4,17,68")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-unfused", action="store_true")
    return ap.parse_args()


def step_kernel_name(M: int) -> str:
    """The kernel one persistent step launch runs: the M = 1 step kernel,
    else the static-schedule stream kernel <MT, MODE 2, NVFP4, every K a
    multiple of 128> (every job of the pass has K % 64 == 0 and K <= 18432,
    so M = 1 always takes the step kernel)."""
    return "step_gemv_kernel" if M == 1 else f"stream_kernel<{(M + 15) // 16}, 2, 0, 0>"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def time_launches(fn, steps, warmup, per_step=None):
    """Average ms of `fn` (work enqueued on the current stream), timed with
    events recorded on that stream.  With a list `per_step`, an event
    between consecutive steps also gives each step's ms (appended to it)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1 if per_step is not None else 2)]
    ev[0].record(s)
    for i in range(steps):
        fn()
        if per_step is not None:
            ev[i + 1].record(s)
    ev[-1].record(s)
    torch.cuda.synchronize()
    if per_step is not None:
        per_step.extend(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    return ev[0].elapsed_time(ev[-1]) / steps


def pass_io_bytes(M: int) -> int:
    """Algorithmic activation and output bytes of one pass of the timed
    step (257 jobs): 2*M*K of X in and 4*M*N of Y out per GEMM job, and for
    the lm_head 2*M*K in and 4*(M + S) out (argmax per row, accept length per
    sequence; S = M/17 sequences of 17 rows for M >= 17, else M)."""
    from verify_gemm_amd import synth
    h, f = synth.HIDDEN, synth.MLP
    jobs = [(3 * h, h), (h, h), (2 * f, h), (h, f)]  # q|k|v, o, gate|up, down: (N, K)
    layer = sum(2 * M * k + 4 * M * n for n, k in jobs)
    seqs = M // 17 if M >= 17 else M
    return synth.LAYERS * layer + 2 * M * h + 4 * (M + seqs)


def bwprobe(device, gib=8, reps=10):
    import torch

    from verify_gemm_amd import binding
    nbytes = gib << 30
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device=device)
    sink = torch.empty(binding.bwprobe_sink_floats(), dtype=torch.float32, device=device)
    ms = time_launches(lambda: binding.bwprobe(buf, sink), reps, 1)
    del buf
    return nbytes / (ms * 1e-3) / 1e9


def blas_threads() -> int:
    """Threads the oracle's BLAS calls run on (what numpy's library reports)."""
    try:
        from threadpoolctl import threadpool_info
        n = [p["num_threads"] for p in threadpool_info() if p.get("user_api") == "blas"]
        if n:
            return max(n)
    except Exception:  # noqa: BLE001 - the count is informational
        pass
    return len(os.sched_getaffinity(0))


def cpu_baseline(weights, budget_s: float = 12.0, max_layers: int = 16):
    """The CPU oracle, untuned, at M = 1 on whole layers (q, k, v, o, gate,
    up, down) in order, until about `budget_s` seconds of CPU work."""
    import numpy as np

    import oracle
    from verify_gemm_amd import synth
    rng = np.random.default_rng(5)
    xs = {k: synth.gen_x(rng, 1, k, 0.1) for k in (synth.HIDDEN, synth.MLP)}
    nbytes, dt, layers = 0, 0.0, 0
    while layers < max_layers and dt < budget_s:
        for m in (m for m in weights.mats if m["layer"] == layers):
            wq, ws = m["wq"].cpu().numpy(), m["ws"].cpu().numpy()
            t0 = time.perf_counter()
            oracle.nvfp4_gemm_ref(xs[m["k"]], wq, ws, m["g"], with_bound=False)
            dt += time.perf_counter() - t0
            nbytes += wq.size + ws.size
        layers += 1
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": blas_threads(), "kind": "oracle",
            "sample": f"layers 0-{layers - 1} (q,k,v,o,gate,up,down; {nbytes} weight bytes) at M=1 through the "
                      f"fp64 numpy oracle (no error bounds) in {dt:.1f} s of oracle time; a full pass is "
                      f"{PASS_WEIGHT_BYTES / nbytes:.1f}x this sample (~{dt * PASS_WEIGHT_BYTES / nbytes:.0f} s)"}


def recorded_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed counter summary,
    or None when it is missing or the kernel sources changed since."""
    from verify_gemm_amd import profile_summary
    rec = profile_summary.recorded_traffic(
        os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", "step_kernels_full_pass_hbm_traffic.md"))
    if rec is None:
        return None
    return rec["traffic_bytes"].get(kernel)


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(how the step would shard is described, not implemented); use --gpus 1", file=sys.stderr)
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
        # The timed step: every layer's {q,k,v} and {gate,up} read as one
        # stacked matrix each (257 jobs), each member keeping its own tensor
        # scale as per-row scales -- the same bytes and the same output bits
        # as 449 separate jobs -- in vg_pass_run's schedule for this M.
        run = weightpass.PassRun(weights, M, fused=True)
        run.run()
        torch.cuda.synchronize()
        if run.check():
            raise RuntimeError(f"M={M}: a stage wait timed out; the step is invalid")
        steps_ms = []
        ms = time_launches(run.run, args.steps, args.warmup, steps_ms)
        if run.check():
            raise RuntimeError(f"M={M}: a stage wait timed out during timing")
        gbps = wbytes / (ms * 1e-3) / 1e9
        q = sorted(steps_ms)
        pct = lambda f: round(q[min(len(q) - 1, int(f * (len(q) - 1) + 0.5))] * 1000, 2)  # noqa: E731
        entry = {"us_per_pass": round(ms * 1000, 2), "weight_gbps": round(gbps, 1),
                 "pct_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 2),
                 "pct_of_probe": round(100 * gbps / probe, 2),
                 "us_p10_p50_p90": [pct(0.1), pct(0.5), pct(0.9)],
                 "total_algorithmic_gbps": round((wbytes + pass_io_bytes(M)) / (ms * 1e-3) / 1e9, 1),
                 "jobs": run.step.info()["jobs"],
                 "schedule": "one persistent launch" if M == 1 else "one launch per job"}
        if M != 1:
            entry["persistent_us_per_pass"] = round(time_launches(run.run_persistent, args.steps, args.warmup) * 1000, 2)
            if run.check():
                raise RuntimeError(f"M={M}: a stage wait timed out in the persistent launch")
        if not args.no_unfused:
            reps = max(2, min(args.steps, 5))
            g = run.capture_unfused()
            entry["unfused_graph_us_per_pass"] = round(time_launches(g.replay, reps, 1) * 1000, 1)
            del g
            # the same step as 449 separate jobs, as one launch and as one
            # launch per job
            sr = weightpass.PassRun(weights, M)
            sr.run()
            torch.cuda.synchronize()
            if sr.check():
                raise RuntimeError(f"M={M}: a stage wait timed out in the 449-job step")
            sep = time_launches(sr.run, reps, 1)
            gs = sr.capture_unfused()
            entry["separate_jobs"] = {"jobs": sr.step.info()["jobs"], "us_per_pass": round(sep * 1000, 2),
                                      "unfused_graph_us_per_pass": round(time_launches(gs.replay, reps, 1) * 1000, 1)}
            del gs
            sr.close()
            del sr
        per_m[str(M)] = entry
        log(f"[bench] M={M}: {entry}")
        run.close()
        del run
        torch.cuda.empty_cache()
    head = per_m[str(ms_list[0])]
    kus = head["us_per_pass"]
    # the roofline is that of one launch of the whole step: at M >= 2 the
    # persistent launch timed beside the per-job schedule
    lus = head.get("persistent_us_per_pass", kus)
    achieved = wbytes / (lus * 1e-6) / 1e9
    out = {
        "metric": "µs per full weight pass + effective weight GB/s (% HBM peak) at M=1/17/68",
        "value": head["weight_gbps"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(kus / 1000, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e2m1/e4m3 weights x bf16 activations, fp32 accumulation",
        "data": "synthetic (seeded device RNG, codes uniform, scales 2^u)",
        "config": {"workload": "full synthetic weight pass: 64 layers x {q,k,v,o 5120x5120; gate,up "
                               "17408x5120; down 5120x17408} + lm_head 248320x5120 with argmax/accept "
                               f"(449 NVFP4 matrices, {wbytes} weight bytes), one persistent launch per pass at "
                               "M=1 (one launch per job at M>=2); "
                               "each layer's q|k|v and gate|up read as one stacked matrix (257 jobs, per-matrix "
                               "tensor scales kept as per-row scales, outputs bit-identical to 449 jobs)",
                   "M": ms_list[0], "M_reported": ms_list},
        "per_m": per_m,
        "bwprobe_read_gbps": round(probe, 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": recorded_traffic(step_kernel_name(ms_list[0])),
                     "kernel": (f"{step_kernel_name(ms_list[0])} (the whole step is one launch of it) "
                                f"at M={ms_list[0]}"),
                     "avg_us": lus, "bytes_per_launch": wbytes},
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on layer 0 (bounded sample)")
        out["cpu_baseline"] = cpu_baseline(weights)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
