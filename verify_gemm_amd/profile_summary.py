"""Short text summaries of rocprofv3 output for the profiles/ folder.

Three summaries, each written as Markdown with the exact commands that
produced its input:

  * ``trace``: the ``--kernel-trace --stats`` kernel statistics of a bench
    run, restricted to this library's kernels and the reference kernels of
    known size (the read probe, torch's fill);
  * ``pmc``: per-dispatch ``FETCH_SIZE`` and ``WRITE_SIZE`` (two separate
    counter runs) for the same kernels, the scale factors derived from the
    kernels of known size (the probe reads exactly its buffer, torch's fill
    writes exactly its buffer), and the resulting HBM traffic per launch of
    each step kernel.  It also records a hash of the kernel sources the
    counters were taken with: bench.py reports the traffic only while the
    sources still hash the same.

  * ``busy``: MFMA-busy and VALU-active cycles of the M >= 2 stream
    kernels from one counter run.

    python -m verify_gemm_amd.profile_summary trace STATS_CSV CMD OUT
    python -m verify_gemm_amd.profile_summary pmc FETCH_CSV WRITE_CSV CMD_F CMD_W PROBE_BYTES FILL_BYTES OUT
    python -m verify_gemm_amd.profile_summary busy COUNTER_CSV CMD OUT
    python -m verify_gemm_amd.profile_summary counters TITLE OUT CMD1 CSV1 [CMD2 CSV2 ...]

  * ``counters``: per-dispatch averages of every counter of one or more
    counter runs (one run per group of counters the hardware can collect
    together), per kernel, each shown also per SQ_BUSY_CYCLES x 32 SIMDs
    where the run has SQ_BUSY_CYCLES.
"""
from __future__ import annotations

import collections
import csv
import hashlib
import json
import os
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
# Sources whose change invalidates recorded counter values.
KERNEL_SOURCES = ["csrc/step_gemv.hip", "csrc/stream_kernel.h", "csrc/nvfp4_device.h", "csrc/launch.h"]
PASS_WEIGHT_BYTES = 14115962880


def code_only(text: str) -> str:
    """C/C++ source without comments, blank lines or indentation: what the
    compiler sees, so that editing a comment does not invalidate counters
    taken with the same code."""
    out, i, n = [], 0, len(text)
    while i < n:
        ch = text[i]
        if ch in "\"'":  # a string or character literal, escapes kept
            j = i + 1
            while j < n and text[j] != ch:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(ch)
            i += 1
    lines = (ln.strip() for ln in "".join(out).splitlines())
    return "\n".join(ln for ln in lines if ln)


def sources_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(PKG, rel), encoding="utf-8") as f:
            h.update(rel.encode() + b"\0" + code_only(f.read()).encode())
    return h.hexdigest()


def stream_args(name: str):
    """(MT, MODE, ...) of a stream_kernel<...> short name, or None."""
    if not name.startswith("stream_kernel<"):
        return None
    return tuple(int(v) for v in name[len("stream_kernel<"):-1].split(","))


def short_name(name: str) -> str | None:
    if "step_gemv_kernel" in name:
        return "step_gemv_kernel"
    if "stream_kernel<" in name:
        return "stream_kernel<" + name.split("stream_kernel<", 1)[1].split(">", 1)[0] + ">"
    if "bwprobe_kernel" in name:
        return "bwprobe_kernel (read probe)"
    if "FillFunctor" in name:
        return "torch fill (write reference)"
    return None


def trace(stats_csv: str, cmd: str, out: str) -> None:
    rows = list(csv.DictReader(open(stats_csv)))
    lines = ["# Kernel trace: full-pass step kernels", "", "Command (run from /tmp, `TMPDIR=/tmp`):", "",
             "```", cmd, "```", "",
             "| kernel | calls | avg us | min us | max us | share of GPU time |",
             "|---|---:|---:|---:|---:|---:|"]
    for r in rows:
        n = short_name(r["Name"])
        if n is None:
            continue
        lines.append(f"| {n} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | {float(r['MinNs']) / 1e3:.1f} | "
                     f"{float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.2f}% |")
    lines += ["", "stream_kernel<MT, MODE, FMT, ANYK, XH>: MT 16-row M-tiles (1 at M = 4, 2 at M = 17, 5 at M = 68), "
              "MODE 0 the GEMM jobs of one stage, 1 the lm_head, 2 the whole pass as one persistent launch; FMT 0 "
              "NVFP4; ANYK 0 when every K is a multiple of 128; XH 1 when the last M-tile is at most half used "
              "(M <= 16 MT - 8: eight activation rows fewer per window; the one-tile lm_head keeps XH 0).  A launch of "
              "step_gemv_kernel (M = 1) or of a "
              "MODE 2 kernel is one whole pass; vg_pass_run takes MODE 0 / 1 launches at M >= 2, one per stage "
              f"({GEMM_JOBS_PER_PASS} GEMM launches and one lm_head launch per pass, for the 449-job and the "
              "257-job step alike).", ""]
    with open(out, "w") as f:
        f.write("\n".join(lines))


# GEMM launches of a pass at M >= 2, one per stage: 64 layers x {q, k, v /
# q|k|v; o; gate, up / gate|up; down}, then the lm_head.
GEMM_JOBS_PER_PASS = 256


# The fill kernel of known size is one of many torch fills in a run (small
# buffers are filled too): only its dispatches, the large ones, calibrate.
CALIBRATION_FILL = "torch fill (write reference)"


def _per_dispatch(path: str, counter: str):
    agg = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        n = short_name(r["Kernel_Name"])
        if n is not None and r["Counter_Name"] == counter:
            agg[n].append(float(r["Counter_Value"]))
    if CALIBRATION_FILL in agg:
        top = max(agg[CALIBRATION_FILL])
        agg[CALIBRATION_FILL] = [v for v in agg[CALIBRATION_FILL] if v >= 0.5 * top]
    return {k: sum(v) / len(v) for k, v in agg.items()}, {k: len(v) for k, v in agg.items()}


def pmc(fetch_csv: str, write_csv: str, cmd_f: str, cmd_w: str, probe_bytes: int, fill_bytes: int,
        out: str) -> None:
    fetch, nf = _per_dispatch(fetch_csv, "FETCH_SIZE")
    write, nw = _per_dispatch(write_csv, "WRITE_SIZE")
    f_scale = probe_bytes / (fetch["bwprobe_kernel (read probe)"] * 1024)
    w_scale = fill_bytes / (write[CALIBRATION_FILL] * 1024)
    traffic = {}
    for k in sorted(set(fetch) | set(write)):
        if k.startswith("step_gemv") or k.startswith("stream_kernel"):
            traffic[k] = round(fetch.get(k, 0) * 1024 * f_scale + write.get(k, 0) * 1024 * w_scale)
    lines = ["# HBM traffic of the step kernels (rocprofv3 counters)", "",
             "Two counter runs (run from /tmp, `TMPDIR=/tmp`):", "", "```", cmd_f, cmd_w, "```", "",
             "| kernel | dispatches | FETCH_SIZE KiB/dispatch | WRITE_SIZE KiB/dispatch |",
             "|---|---:|---:|---:|"]
    for k in sorted(set(fetch) | set(write)):
        lines.append(f"| {k} | {nf.get(k, 0)} | {fetch.get(k, 0):.6g} | {write.get(k, 0):.6g} |")
    lines += ["", f"Scale factors from the kernels of known size: reads x{f_scale:.4f} "
              f"(the probe reads {probe_bytes} bytes per dispatch), writes x{w_scale:.4f} "
              f"(torch's fill of the probe buffer writes {fill_bytes} bytes per dispatch; the "
              "smaller fills of the same run are left out).", "",
              "Traffic per launch (scaled fetch + scaled write) against the pass's algorithmic "
              f"{PASS_WEIGHT_BYTES} weight bytes:", ""]
    # stream_kernel<MT, MODE, FMT, ANYK, XH>: MODE 2 is one persistent launch
    # of the whole pass; MODE 0 the per-stage GEMM launches, MODE 1 the lm_head
    for k, v in traffic.items():
        a = stream_args(k)
        if k.startswith("step_gemv") or (a is not None and a[1] == 2):
            lines.append(f"* {k} (one launch per pass): {v} bytes ({v / PASS_WEIGHT_BYTES:.3f}x)")
    # one launch per stage: the GEMM launches of a pass (same mix every pass)
    # plus its lm_head launch
    for k, v in traffic.items():
        a = stream_args(k)
        if a is not None and a[1] == 0:
            # the one-tile lm_head keeps the full activation loads (XH 0)
            lm_args = (a[0], 1) + a[2:4] + ((a[4] if a[0] >= 2 else 0),) + a[5:] if len(a) > 4 else (a[0], 1) + a[2:]
            lm = "stream_kernel<" + ", ".join(str(x) for x in lm_args) + ">"
            per_pass = v * GEMM_JOBS_PER_PASS + traffic.get(lm, 0)
            lines.append(f"* {k} x {GEMM_JOBS_PER_PASS} + {lm} (one launch per stage): {per_pass} bytes per pass "
                         f"({per_pass / PASS_WEIGHT_BYTES:.3f}x)")
    record = {"sources_sha256": sources_hash(), "traffic_bytes": traffic,
              "fetch_scale": f_scale, "write_scale": w_scale}
    lines += ["", "Machine-readable record (bench.py reads it):", "", "```json", json.dumps(record, indent=1),
              "```", ""]
    with open(out, "w") as f:
        f.write("\n".join(lines))


# SIMDs per shader engine on MI355X (8 CUs x 4 SIMDs): SQ_BUSY_CYCLES
# counts an SE's busy cycles, summed over the SEs, while the MFMA-busy and
# VALU counters sum over every SIMD.
SIMDS_PER_SE = 32
BUSY_COUNTERS = ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_ACTIVE_INST_VALU", "SQ_BUSY_CYCLES", "GRBM_GUI_ACTIVE"]


def busy(csv_path: str, cmd: str, out: str) -> None:
    """MFMA and VALU activity per stream kernel from one counter run."""
    vals = {c: _per_dispatch(csv_path, c)[0] for c in BUSY_COUNTERS}
    counts = _per_dispatch(csv_path, "SQ_BUSY_CYCLES")[1]
    lines = ["# MFMA and VALU activity of the M >= 2 stream kernels (rocprofv3 counters)", "",
             "Command (run from /tmp, `TMPDIR=/tmp`):", "", "```", cmd, "```", "",
             "| kernel | dispatches | SQ_VALU_MFMA_BUSY_CYCLES | SQ_ACTIVE_INST_VALU | SQ_BUSY_CYCLES | "
             "MFMA busy | VALU active |", "|---|---:|---:|---:|---:|---:|---:|"]
    for k in sorted(vals["SQ_BUSY_CYCLES"]):
        if not k.startswith("stream_kernel"):
            continue
        mf, va, sq = (vals[c].get(k, 0.0) for c in BUSY_COUNTERS[:3])
        den = sq * SIMDS_PER_SE
        lines.append(f"| {k} | {counts.get(k, 0)} | {mf:.4g} | {va:.4g} | {sq:.4g} | "
                     f"{100 * mf / den if den else 0:.1f} % | {100 * va / den if den else 0:.1f} % |")
    lines += ["", "Per dispatch, averaged.  MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (SQ_BUSY_CYCLES x "
              f"{SIMDS_PER_SE}); VALU active the same with SQ_ACTIVE_INST_VALU.  This reads the SQ "
              "counters as summed over shader engines (busy cycles) and over SIMDs (MFMA, VALU): a share "
              "of the SIMD cycles while the kernel runs, not an exact utilisation.  MODE 0 kernels are the "
              "per-stage GEMMs of the default schedule, MODE 1 the lm_head, MODE 2 the persistent launch.", ""]
    with open(out, "w") as f:
        f.write("\n".join(lines))


def counters(title: str, out: str, runs) -> None:
    """Per-kernel, per-dispatch averages of the counters of several runs."""
    lines = [f"# {title}", "", "Counter runs (run from /tmp, `TMPDIR=/tmp`), one per group of counters the "
             "hardware collects together:", "", "```"] + [cmd for cmd, _ in runs] + ["```", ""]
    for cmd, path in runs:
        names = []
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] not in names:
                names.append(r["Counter_Name"])
        vals = {c: _per_dispatch(path, c) for c in names}
        kernels = sorted({k for c in names for k in vals[c][0] if k.startswith(("stream_kernel", "step_gemv"))})
        busy = vals.get("SQ_BUSY_CYCLES", ({}, {}))[0]
        lines += ["| kernel | dispatches | " + " | ".join(names) + " |",
                  "|---|---:|" + "---:|" * len(names)]
        for k in kernels:
            cells = []
            for c in names:
                v = vals[c][0].get(k, 0.0)
                den = busy.get(k, 0.0) * SIMDS_PER_SE
                rel = f" ({100 * v / den:.1f} %)" if den and c.startswith("SQ_") and c != "SQ_BUSY_CYCLES" else ""
                cells.append(f"{v:.4g}{rel}")
            lines.append(f"| {k} | {vals[names[0]][1].get(k, 0)} | " + " | ".join(cells) + " |")
        lines.append("")
    lines += ["Per dispatch, averaged.  A percentage is the counter over SQ_BUSY_CYCLES x "
              f"{SIMDS_PER_SE} (the SQ counters sum over SIMDs, SQ_BUSY_CYCLES over shader engines): a "
              "share of the SIMD cycles while the kernel runs.  TA and TCP counters are sums over their "
              "units (the _sum forms).", ""]
    with open(out, "w") as f:
        f.write("\n".join(lines))


def recorded_traffic(path: str):
    """The traffic record of a pmc summary, or None if the summary is
    missing or the kernel sources changed since it was taken."""
    try:
        text = open(path).read()
    except OSError:
        return None
    try:
        block = text.split("```json", 1)[1].split("```", 1)[0]
        rec = json.loads(block)
    except (IndexError, ValueError):
        return None
    if rec.get("sources_sha256") != sources_hash():
        return None
    return rec


def main(argv):
    if argv[1] == "trace":
        trace(argv[2], argv[3], argv[4])
    elif argv[1] == "pmc":
        pmc(argv[2], argv[3], argv[4], argv[5], int(argv[6]), int(argv[7]), argv[8])
    elif argv[1] == "busy":
        busy(argv[2], argv[3], argv[4])
    elif argv[1] == "counters":
        counters(argv[2], argv[3], list(zip(argv[4::2], argv[5::2])))
    else:
        raise SystemExit(__doc__)


if __name__ == "__main__":
    main(sys.argv)
