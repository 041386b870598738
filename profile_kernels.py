#!/usr/bin/env python3
"""rocprofv3 passes behind the benchmark's roofline figures.

    python3 profile_kernels.py run [--out DIR]
    python3 profile_kernels.py summarize [--out DIR]
    python3 profile_kernels.py counters [--workload NAME] [--out DIR]

(DIR: where rocprofv3 writes its raw output, default prof_out/.)

`run` starts three rocprofv3 child processes over bench.py (each with its own
time limit, from /tmp with TMPDIR=/tmp):

  1. --kernel-trace --stats          per-kernel launch durations;
  2. --pmc FETCH_SIZE                 HBM read KiB per dispatch;
  3. --pmc WRITE_SIZE                 HBM write KiB per dispatch;

the two counter passes also run bench.py's plain 1 GiB copy first, whose
counter readings give the scale factors (bytes the copy really moves divided by
what the counter reports).  `summarize` (also done at the end of `run`) writes
one short text summary per measured kernel into profiles/, with the commands,
the average launch duration, the scaled per-launch HBM traffic and the sha256
of the kernel's source at the time.  bench.py reports `traffic` from these
summaries only while that source is unchanged.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import subprocess
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.abspath(__file__))
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "transformer_attention_diffattn_amd", "csrc")

# the trace pass runs the default benchmark command itself, so that its
# average launch durations are those of the reported figures
BENCH_ARGS: list = []
# the counter passes need only the headline prefill and the decode launches
PMC_BENCH_ARGS = ["--steps", "3", "--warmup", "1", "--no-cpu", "--no-backward", "--no-diag",
                  "--no-proj", "--no-fp8", "--copy-calibration"]
COPY_BYTES = 1 << 30
COPY_GRID = COPY_BYTES // 16  # threads of the vectorised copy (4 floats per thread)

# kernel -> (workload it runs on in bench.py, its source files joined by "+")
KERNELS = {
    "prefill_bf16_kernel": ("causal_prefill_bf16", "prefill_core.h+prefill_bf16.hip"),
    "decode_partial_kernel": ("decode_bf16", "decode.hip"),
}


def source_sha(fnames: str) -> str:
    """sha256 of the named source files, concatenated in order."""
    h = hashlib.sha256()
    for fname in fnames.split("+"):
        with open(os.path.join(CSRC, fname), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _commands(out: str):
    py = sys.executable or "python3"
    bench = os.path.join(ROOT, "bench.py")
    return {
        "trace": ["rocprofv3", "--kernel-trace", "--stats", "-T", "-d", os.path.join(out, "trace"),
                  "-o", "run", "-f", "csv", "--", py, bench, *BENCH_ARGS],
        "fetch": ["rocprofv3", "--pmc", "FETCH_SIZE", "-d", os.path.join(out, "fetch"), "-o",
                  "run", "-f", "csv", "--", py, bench, *PMC_BENCH_ARGS],
        "write": ["rocprofv3", "--pmc", "WRITE_SIZE", "-d", os.path.join(out, "write"), "-o",
                  "run", "-f", "csv", "--", py, bench, *PMC_BENCH_ARGS],
    }


def run(out: str) -> None:
    out = os.path.abspath(out)
    os.makedirs(out, exist_ok=True)
    env = dict(os.environ, TMPDIR="/tmp")
    for name, cmd in _commands(out).items():
        print(f"[profile] pass {name}: {' '.join(cmd)}", flush=True)
        with open(os.path.join(out, f"{name}.log"), "w") as log:
            # SIGKILL at the limit: a counter pass that cannot be collected hangs
            subprocess.run(cmd, cwd="/tmp", env=env, stdout=log, stderr=subprocess.STDOUT,
                           timeout=240, check=True)
        print(f"[profile] pass {name} done", flush=True)
    summarize(out)


def _find(out: str, sub: str, suffix: str) -> str:
    hits = glob.glob(os.path.join(out, sub, "**", f"*{suffix}"), recursive=True)
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {os.path.join(out, sub)}")
    return sorted(hits)[0]


def _bench_ms_in_trace(out: str, kernel: str):
    """The per-launch time bench.py measured with events inside the traced run."""
    try:
        with open(os.path.join(out, "trace.log")) as f:
            lines = [l for l in f if l.startswith("{")]
        rec = json.loads(lines[-1])
    except (OSError, IndexError, ValueError):
        return None
    if kernel == "prefill_bf16_kernel":
        return rec["roofline"]["launch_ms"]
    if kernel == "decode_partial_kernel" and "decode" in rec:
        return rec["decode"]["ms_per_call"]
    return None


def _kernel_stats(out: str):
    rows = {}
    with open(_find(out, "trace", "kernel_stats.csv")) as f:
        for r in csv.DictReader(f):
            rows[r["Name"]] = r
    return rows


def _counter(out: str, sub: str):
    """Per full kernel name: list of (grid size, counter KiB) in dispatch order."""
    per = defaultdict(list)
    with open(_find(out, sub, "counter_collection.csv")) as f:
        for r in csv.DictReader(f):
            per[r["Kernel_Name"]].append((int(r["Grid_Size"]), float(r["Counter_Value"])))
    return per


def _calibration(per) -> float:
    """Average counter KiB of the 1 GiB copy (elementwise multiply by one)."""
    vals = [v for name, xs in per.items() if "elementwise" in name and "Mul" in name
            for g, v in xs if g == COPY_GRID]
    if not vals:
        raise RuntimeError("copy calibration dispatches not found")
    return sum(vals) / len(vals)


def _short(name: str) -> str:
    """The library kernel a demangled dispatch name belongs to, else the name."""
    for k in KERNELS:
        if f"{k}<" in name or name == k or f"::{k}" in name:
            return k
    return name


def summarize(out: str) -> None:
    out = os.path.abspath(out)
    stats = _kernel_stats(out)
    fetch, write = _counter(out, "fetch"), _counter(out, "write")
    copy_kib = COPY_BYTES / 1024
    f_cal, w_cal = _calibration(fetch), _calibration(write)
    f_factor, w_factor = copy_kib / f_cal, copy_kib / w_cal
    cmds = _commands(os.path.relpath(out, ROOT))
    os.makedirs(PROFILES, exist_ok=True)
    sys.path.insert(0, ROOT)
    import workloads

    for kern, (wname, src) in KERNELS.items():
        st = stats.get(kern)
        fv = [v for n, xs in fetch.items() if _short(n) == kern for _, v in xs]
        wv = [v for n, xs in write.items() if _short(n) == kern for _, v in xs]
        if st is None or not fv or not wv:
            print(f"[profile] {kern}: not found, skipped", flush=True)
            continue
        w = workloads.get(wname)
        fk, wk = sum(fv) / len(fv), sum(wv) / len(wv)
        bench_ms = _bench_ms_in_trace(out, kern)
        traffic = int(round((fk * f_factor + wk * w_factor) * 1024))
        rec = {
            "kernel": kern, "workload": wname, "calls": int(st["Calls"]),
            "avg_ns": float(st["AverageNs"]), "min_ns": float(st["MinNs"]),
            "max_ns": float(st["MaxNs"]),
            "fetch_kib_per_dispatch": fk, "write_kib_per_dispatch": wk,
            "copy_fetch_kib": f_cal, "copy_write_kib": w_cal,
            "fetch_factor": f_factor, "write_factor": w_factor,
            "traffic_bytes_per_launch": traffic,
            "algorithmic_bytes_per_launch": w.algorithmic_bytes(),
            "source": src, "source_sha256": source_sha(src),
            "bench_event_ms_in_traced_run": bench_ms,
        }
        lines = [
            f"# {kern} on {wname}",
            "",
            f"Workload: {w.description}.",
            "",
            "Commands (from /tmp, TMPDIR=/tmp; written by `python3 profile_kernels.py run`):",
            "",
        ]
        for name, cmd in cmds.items():
            shown = ["python3" if c == (sys.executable or "python3") else
                     (os.path.relpath(c, ROOT) if c.startswith(ROOT) else c) for c in cmd]
            lines.append(f"- {name}: `{' '.join(shown)}`")
        lines += [
            "",
            "| quantity | value |",
            "|---|---|",
            f"| launches traced | {rec['calls']} |",
            f"| bench.py event-timed launch in the same traced run | "
            f"{'n/a' if bench_ms is None else f'{bench_ms * 1e3:.1f} us'} |",
            f"| average duration | {rec['avg_ns'] / 1e3:.1f} us (min {rec['min_ns'] / 1e3:.1f}, "
            f"max {rec['max_ns'] / 1e3:.1f}) |",
            f"| FETCH_SIZE per dispatch | {fk:,.1f} KiB |",
            f"| WRITE_SIZE per dispatch | {wk:,.1f} KiB |",
            f"| 1 GiB copy reads as | FETCH {f_cal:,.1f} KiB, WRITE {w_cal:,.1f} KiB |",
            f"| scale factors | fetch x{f_factor:.4f}, write x{w_factor:.4f} |",
            f"| HBM traffic per launch (scaled) | {traffic:,} B |",
            f"| algorithmic bytes per launch | {rec['algorithmic_bytes_per_launch']:,} B |",
            f"| traffic / algorithmic | {traffic / rec['algorithmic_bytes_per_launch']:.3f} |",
            "",
            "All kernels in the traced run:",
            "",
            "| kernel | calls | average (us) |",
            "|---|---|---|",
        ]
        for name, r in stats.items():
            lines.append(f"| {name} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} |")
        lines += ["", "```json", json.dumps(rec, indent=1), "```", ""]
        path = os.path.join(PROFILES, f"{kern}__{wname}.md")
        with open(path, "w") as f:
            f.write("\n".join(lines))
        print(f"[profile] wrote {os.path.relpath(path, ROOT)}", flush=True)


# counter groups for the prefill kernel (each fits one pass: <= 8 SQ, <= 2 GRBM)
COUNTER_PASSES = [
    ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES", "SQ_WAVE_CYCLES", "SQ_INSTS_VALU",
     "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT", "SQ_VALU_MFMA_COEXEC_CYCLES",
     "GRBM_GUI_ACTIVE"],
    ["SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS", "SQ_WAIT_INST_LDS", "SQ_WAIT_INST_ANY",
     "SQ_INSTS_VALU_TRANS_F32", "SQ_LDS_IDX_ACTIVE", "SQ_INSTS_SALU", "SQ_WAVES",
     "GRBM_GUI_ACTIVE"],
]
SIMDS = 256 * 4
XCDS = 8


def _counter_cmd(out: str, i: int, workload: str):
    py = sys.executable or "python3"
    return ["rocprofv3", "--pmc", *COUNTER_PASSES[i], "-d", os.path.join(out, f"counters{i}"),
            "-o", "run", "-f", "csv", "--", py, os.path.join(ROOT, "bench.py"), "--steps", "3",
            "--warmup", "1", "--no-cpu", "--no-decode", "--no-backward", "--no-diag", "--no-fp8",
            "--no-proj", "--workload", workload]


def prefill_kernel_of(workload: str) -> str:
    """The prefill kernel bench.py runs on `workload` (head_dim 128: the wide one)."""
    sys.path.insert(0, ROOT)
    import workloads
    return "prefill_bf16_wide_kernel" if workloads.get(workload).d == 128 else "prefill_bf16_kernel"


def counters(out: str, workload: str = "causal_prefill_bf16") -> None:
    """Runs the counter passes of COUNTER_PASSES over bench.py on one workload."""
    out = os.path.abspath(out)
    os.makedirs(out, exist_ok=True)
    env = dict(os.environ, TMPDIR="/tmp")
    for i in range(len(COUNTER_PASSES)):
        cmd = _counter_cmd(out, i, workload)
        print(f"[profile] counters pass {i}: {' '.join(cmd)}", flush=True)
        with open(os.path.join(out, f"counters{i}.log"), "w") as log:
            subprocess.run(cmd, cwd="/tmp", env=env, stdout=log, stderr=subprocess.STDOUT,
                           timeout=240, check=True)
    counters_summarize(out, workload, prefill_kernel_of(workload))


def counters_summarize(out: str, workload: str = "causal_prefill_bf16",
                       kernel: str = "prefill_bf16_kernel") -> None:
    """Per-dispatch SQ counters of one kernel, written to
    <profiles>/<kernel>__<workload>__counters.md."""
    out = os.path.abspath(out)
    vals = {}
    for i in range(len(COUNTER_PASSES)):
        per = defaultdict(lambda: defaultdict(float))
        with open(_find(out, f"counters{i}", "counter_collection.csv")) as f:
            for r in csv.DictReader(f):
                n = r["Kernel_Name"]
                if f"{kernel}<" in n or n == kernel or f"::{kernel}" in n:
                    per[r["Counter_Name"]][r["Dispatch_Id"]] += float(r["Counter_Value"])
        for name, disp in per.items():
            vals[name] = sum(disp.values()) / len(disp)
    # GRBM_GUI_ACTIVE reads as the sum over the 8 XCDs (8x the kernel's
    # duration in cycles), so one XCD's count is the kernel's cycle count
    gui = vals.get("GRBM_GUI_ACTIVE", 0.0) / XCDS
    derived = {}
    if gui and "SQ_VALU_MFMA_BUSY_CYCLES" in vals:
        derived["MFMA busy (% of SIMD cycles)"] = (
            100 * vals["SQ_VALU_MFMA_BUSY_CYCLES"] / (gui * SIMDS))
        derived["MFMA/VALU co-issue cycles (% of MFMA busy)"] = (
            100 * vals["SQ_VALU_MFMA_COEXEC_CYCLES"] / max(vals["SQ_VALU_MFMA_BUSY_CYCLES"], 1))
    if vals.get("SQ_WAVE_CYCLES") and "SQ_WAIT_INST_ANY" in vals:
        derived["waves stalled before issue, any cause (% of wave cycles)"] = (
            100 * vals["SQ_WAIT_INST_ANY"] / vals["SQ_WAVE_CYCLES"])
        derived["waiting on LDS (% of wave cycles)"] = (
            100 * vals["SQ_WAIT_INST_LDS"] / vals["SQ_WAVE_CYCLES"])
    if vals.get("SQ_LDS_IDX_ACTIVE"):
        derived["LDS bank-conflict cycles / LDS active cycles"] = (
            vals["SQ_LDS_BANK_CONFLICT"] / vals["SQ_LDS_IDX_ACTIVE"])
    if vals.get("SQ_INSTS_MFMA"):
        derived["VALU instructions per MFMA"] = vals["SQ_INSTS_VALU"] / vals["SQ_INSTS_MFMA"]
        derived["exp (TRANS) instructions per MFMA"] = (
            vals.get("SQ_INSTS_VALU_TRANS_F32", 0) / vals["SQ_INSTS_MFMA"])
        derived["LDS instructions per MFMA"] = vals["SQ_INSTS_LDS"] / vals["SQ_INSTS_MFMA"]
    src = {"prefill_bf16_wide_kernel": "prefill_bf16_wide.hip"}.get(
        kernel, KERNELS.get(kernel, (None, "prefill_core.h+prefill_bf16.hip"))[1])
    lines = [f"# {kernel} on {workload}: SQ counters per dispatch", "",
             "Commands (from /tmp, TMPDIR=/tmp; written by "
             f"`python3 profile_kernels.py counters --workload {workload}`):", ""]
    py = sys.executable or "python3"
    for i in range(len(COUNTER_PASSES)):
        shown = ["python3" if c == py else (os.path.relpath(c, ROOT) if c.startswith(ROOT) else c)
                 for c in _counter_cmd(os.path.relpath(out, ROOT), i, workload)]
        lines.append(f"- `{' '.join(shown)}`")
    lines += ["", "Kernel cycles = GRBM_GUI_ACTIVE / 8 (the counter sums the 8 XCDs); "
              "SIMD cycles = kernel cycles x 1024 SIMDs (256 CUs x 4).", "",
              "| counter | per dispatch |", "|---|---|"]
    lines += [f"| {k} | {v:,.0f} |" for k, v in sorted(vals.items())]
    lines += ["", "| derived | value |", "|---|---|"]
    lines += [f"| {k} | {v:.3f} |" for k, v in derived.items()]
    lines += ["", f"Kernel source sha256 ({src}): {source_sha(src)}", ""]
    os.makedirs(PROFILES, exist_ok=True)
    path = os.path.join(PROFILES, f"{kernel}__{workload}__counters.md")
    with open(path, "w") as f:
        f.write("\n".join(lines))
    print(f"[profile] wrote {path}", flush=True)


def load(kernel: str):
    """The stored summary of `kernel`, or None if absent or its source changed."""
    if kernel not in KERNELS:
        return None
    wname, src = KERNELS[kernel]
    path = os.path.join(PROFILES, f"{kernel}__{wname}.md")
    try:
        with open(path) as f:
            text = f.read()
        rec = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
    except (OSError, IndexError, ValueError):
        return None
    if rec.get("source_sha256") != source_sha(src):
        return None
    return rec


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("action", choices=["run", "summarize", "counters", "counters-summarize"])
    ap.add_argument("--out", default=os.path.join(ROOT, "prof_out"))
    ap.add_argument("--workload", default="causal_prefill_bf16")
    ap.add_argument("--profiles-dir", default=PROFILES,
                    help="where summaries go (on a remote GPU box: a folder that is copied back)")
    a = ap.parse_args()
    PROFILES = os.path.abspath(a.profiles_dir)
    if a.action == "run":
        run(a.out)
    elif a.action == "summarize":
        summarize(a.out)
    elif a.action == "counters":
        counters(a.out, a.workload)
    else:
        counters_summarize(a.out, a.workload, prefill_kernel_of(a.workload))
