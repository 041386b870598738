#!/usr/bin/env python3
"""rocprofv3 passes behind the benchmark's roofline figures.

    python3 profile_kernels.py run [--out DIR]
    python3 profile_kernels.py summarize [--out DIR]
    python3 profile_kernels.py counters [--workload NAME] [--out DIR]
    python3 profile_kernels.py counters --backward [--out DIR]

(DIR: where rocprofv3 writes its raw output, default prof_out/.)

`run` starts rocprofv3 child processes over bench.py (each with its own time
limit, from /tmp with TMPDIR=/tmp):

  trace          --kernel-trace --stats over the default bench.py command:
                 per-dispatch launch durations;
  fetch_*, write_*
                 --pmc FETCH_SIZE, then --pmc WRITE_SIZE (HBM read and write
                 KiB per dispatch), each over two short bench.py commands that
                 between them run every measured kernel on its workload, one
                 workload per kernel name in each command.

The counter passes also run bench.py's plain 1 GiB copy first, whose counter
readings give the scale factors (bytes the copy really moves divided by what
the counter reports).  `summarize` (also done at the end of `run`) writes one
short text summary per (kernel, workload) into profiles/, with the commands,
the average launch duration, the scaled per-launch HBM traffic and the sha256
of the kernel's source at the time.  bench.py reports `traffic` from these
summaries only while that source is unchanged.

Where one kernel runs on two workloads in the traced command (the head_dim-64
prefill on the 32K and the 2K workloads), each dispatch is attributed to the
workload whose event-timed launch in the same run is nearest in log time (the
two differ by a factor of ~50).
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import math
import os
import subprocess
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.abspath(__file__))
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "transformer_attention_diffattn_amd", "csrc")
sys.path.insert(0, ROOT)

# the trace pass runs the default benchmark command itself, so that its
# average launch durations are those of the reported figures
BENCH_ARGS: list = []
# counter passes: two short commands; in each, a kernel name runs on one workload
_PMC_COMMON = ["--steps", "3", "--warmup", "1", "--copy-calibration"]
PMC_BENCHES = {
    "a": ["--workload", "long_needles_bf16", "--legs", "decode", *_PMC_COMMON],
    "b": ["--workload", "causal_prefill_bf16", "--legs", "large_head_bf16,fp8,proj,backward",
          *_PMC_COMMON],
}
COPY_BYTES = 1 << 30
COPY_GRID = COPY_BYTES // 16  # threads of the vectorised copy (4 floats per thread)
_PREFILL = "prefill_core.h+prefill_bf16.hip"


def _wide() -> str:
    import transformer_attention_diffattn_amd as da
    return da.prefill_kernel_name(128, 256)


def entries():
    """(kernel, workload, source files joined by '+', counter pass, how bench.py
    reports its event-timed launch: a path into the JSON line)."""
    return [
        ("prefill_bf16_kernel", "long_needles_bf16", _PREFILL, "a", ("roofline", "launch_ms")),
        ("prefill_bf16_kernel", "causal_prefill_bf16", _PREFILL, "b",
         ("prefill_legs", "causal_prefill_bf16", "ms_per_launch")),
        (_wide(), "large_head_bf16", "prefill_twopass.hip", "b",
         ("prefill_legs", "large_head_bf16", "ms_per_launch")),
        ("decode_partial_kernel", "decode_bf16", "decode.hip", "a", ("decode", "ms_per_call")),
        ("prefill_fp8qk_kernel", "causal_prefill_bf16", _PREFILL, "b", ("fp8_qk", "ms_per_call")),
        ("prefill_fp8qk_twopass_kernel", "large_head_bf16", "prefill_twopass.hip", "b",
         ("fp8_qk_large_head", "ms_per_call")),
        ("qkv_proj_kernel", "causal_prefill_bf16", "proj.hip", "b", ("qkv_proj", "ms_per_call")),
        ("bwd_dq_kernel", "causal_prefill_bf16", "backward.hip+tile_ops.h", "b", None),
        ("bwd_dkdv16_kernel", "causal_prefill_bf16", "backward.hip+tile_ops.h", "b", None),
        ("bwd_dq_pair_kernel", "large_head_bf16", "backward_ring.hip+tile_ops.h", "b", None),
        ("bwd_dkdv_ring_kernel", "large_head_bf16", "backward_ring.hip+tile_ops.h", "b", None),
    ]


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
    cmds = {"trace": ["rocprofv3", "--kernel-trace", "--stats", "-T", "-d",
                      os.path.join(out, "trace"), "-o", "run", "-f", "csv", "--", py, bench,
                      *BENCH_ARGS]}
    for key, bargs in PMC_BENCHES.items():
        for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
            sub = f"{ctr.split('_')[0].lower()}_{key}"
            cmds[sub] = ["rocprofv3", "--pmc", ctr, "-d", os.path.join(out, sub), "-o", "run",
                         "-f", "csv", "--", py, bench, *bargs]
    return cmds


def run(out: str) -> None:
    out = os.path.abspath(out)
    os.makedirs(out, exist_ok=True)
    env = dict(os.environ, TMPDIR="/tmp")
    for name, cmd in _commands(out).items():
        print(f"[profile] pass {name}: {' '.join(cmd)}", flush=True)
        with open(os.path.join(out, f"{name}.log"), "w") as log:
            # SIGKILL at the limit: a counter pass that cannot be collected hangs
            subprocess.run(cmd, cwd="/tmp", env=env, stdout=log, stderr=subprocess.STDOUT,
                           timeout=300, check=True)
        print(f"[profile] pass {name} done", flush=True)
    summarize(out)


def _find(out: str, sub: str, suffix: str) -> str:
    hits = glob.glob(os.path.join(out, sub, "**", f"*{suffix}"), recursive=True)
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {os.path.join(out, sub)}")
    return sorted(hits)[0]


def _bench_record(out: str):
    """The JSON line bench.py printed inside the traced run."""
    try:
        with open(os.path.join(out, "trace.log")) as f:
            lines = [l for l in f if l.startswith("{")]
        return json.loads(lines[-1])
    except (OSError, IndexError, ValueError):
        return None


def _dig(rec, path):
    for k in path or ():
        if not isinstance(rec, dict) or k not in rec:
            return None
        rec = rec[k]
    return rec


def _short(name: str, kernels) -> str:
    """The library kernel a demangled dispatch name belongs to, else the name."""
    for k in kernels:
        if f"{k}<" in name or name == k or f"::{k}" in name or name.startswith(k + "("):
            return k
    return name


def _trace_durations(out: str, kernels):
    """Per library kernel: the durations (ns) of its dispatches, in order."""
    per = defaultdict(list)
    with open(_find(out, "trace", "kernel_trace.csv")) as f:
        for r in csv.DictReader(f):
            k = _short(r["Kernel_Name"], kernels)
            per[k].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    return per


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


def _attribute(durs, centers):
    """Split durations among workloads by nearest centre in log time.
    centers: {workload: ms}.  Returns {workload: [ns, ...]}."""
    got = defaultdict(list)
    named = {w: c for w, c in centers.items() if c}
    for d in durs:
        if not named:
            break
        w = min(named, key=lambda k: abs(math.log(d / 1e6) - math.log(named[k])))
        got[w].append(d)
    return got


def summarize(out: str) -> None:
    import workloads

    out = os.path.abspath(out)
    ents = entries()
    kernels = sorted({e[0] for e in ents}, key=len, reverse=True)
    durs = _trace_durations(out, kernels)
    stats = _kernel_stats(out)
    bench = _bench_record(out)
    copy_kib = COPY_BYTES / 1024
    fetch = {k: _counter(out, f"fetch_{k}") for k in PMC_BENCHES}
    write = {k: _counter(out, f"write_{k}") for k in PMC_BENCHES}
    cal = {k: (copy_kib / _calibration(fetch[k]), copy_kib / _calibration(write[k]))
           for k in PMC_BENCHES}
    cmds = _commands(os.path.relpath(out, ROOT))
    os.makedirs(PROFILES, exist_ok=True)
    centers = defaultdict(dict)
    for kern, wname, _, _, path in ents:
        centers[kern][wname] = _dig(bench, path) if path else None

    for kern, wname, src, pmc, path in ents:
        same = [w for w, c in centers[kern].items()]
        mine = (_attribute(durs.get(kern, []), centers[kern]).get(wname, [])
                if len(same) > 1 else durs.get(kern, []))
        fv = [v for n, xs in fetch[pmc].items() if _short(n, kernels) == kern for _, v in xs]
        wv = [v for n, xs in write[pmc].items() if _short(n, kernels) == kern for _, v in xs]
        if not mine or not fv or not wv:
            print(f"[profile] {kern} on {wname}: not found, skipped", flush=True)
            continue
        w = workloads.get(wname)
        f_factor, w_factor = cal[pmc]
        fk, wk = sum(fv) / len(fv), sum(wv) / len(wv)
        bench_ms = _dig(bench, path) if path else None
        traffic = int(round((fk * f_factor + wk * w_factor) * 1024))
        rec = {
            "kernel": kern, "workload": wname, "calls": len(mine),
            "avg_ns": sum(mine) / len(mine), "min_ns": float(min(mine)),
            "max_ns": float(max(mine)),
            "fetch_kib_per_dispatch": fk, "write_kib_per_dispatch": wk,
            "fetch_factor": f_factor, "write_factor": w_factor,
            "traffic_bytes_per_launch": traffic,
            "source": src, "source_sha256": source_sha(src),
            "bench_event_ms_in_traced_run": bench_ms,
        }
        if kern.startswith("prefill") or kern.startswith("decode"):
            rec["algorithmic_bytes_per_launch"] = w.algorithmic_bytes()
        lines = [
            f"# {kern} on {wname}",
            "",
            f"Workload: {w.description}.",
            "",
            "Commands (from /tmp, TMPDIR=/tmp; written by `python3 profile_kernels.py run`):",
            "",
        ]
        for name, cmd in cmds.items():
            if name != "trace" and not name.endswith("_" + pmc):
                continue
            shown = ["python3" if c == (sys.executable or "python3") else
                     (os.path.relpath(c, ROOT) if c.startswith(ROOT) else c) for c in cmd]
            lines.append(f"- {name}: `{' '.join(shown)}`")
        lines += [
            "",
            "| quantity | value |",
            "|---|---|",
            f"| launches traced (this workload) | {rec['calls']} |",
            f"| bench.py event-timed launch in the same traced run | "
            f"{'n/a' if bench_ms is None else f'{bench_ms * 1e3:.1f} us'} |",
            f"| average duration | {rec['avg_ns'] / 1e3:.1f} us (min {rec['min_ns'] / 1e3:.1f}, "
            f"max {rec['max_ns'] / 1e3:.1f}) |",
            f"| FETCH_SIZE per dispatch | {fk:,.1f} KiB |",
            f"| WRITE_SIZE per dispatch | {wk:,.1f} KiB |",
            f"| scale factors (1 GiB copy) | fetch x{f_factor:.4f}, write x{w_factor:.4f} |",
            f"| HBM traffic per launch (scaled) | {traffic:,} B |",
        ]
        if "algorithmic_bytes_per_launch" in rec:
            ab = rec["algorithmic_bytes_per_launch"]
            lines += [f"| algorithmic bytes per launch | {ab:,} B |",
                      f"| traffic / algorithmic | {traffic / ab:.3f} |"]
        lines += ["", "All kernels in the traced run (every workload):", "",
                  "| kernel | calls | average (us) |", "|---|---|---|"]
        for name, r in stats.items():
            lines.append(f"| {name} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} |")
        lines += ["", "```json", json.dumps(rec, indent=1), "```", ""]
        path_md = os.path.join(PROFILES, f"{kern}__{wname}.md")
        with open(path_md, "w") as f:
            f.write("\n".join(lines))
        print(f"[profile] wrote {os.path.relpath(path_md, ROOT)}", flush=True)


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


# the backward kernels, each on the one workload it runs on in bench.py's
# backward legs (the head_dim-64 pair on the 2K workload, the head_dim-128
# pair on the large-head one)
BACKWARD_KERNELS = [
    ("bwd_dq_kernel", "causal_prefill_bf16"),
    ("bwd_dkdv16_kernel", "causal_prefill_bf16"),
    ("bwd_dq_pair_kernel", "large_head_bf16"),
    ("bwd_dkdv_ring_kernel", "large_head_bf16"),
]


def _counter_cmd(out: str, i: int, workload: str, legs: str = "none"):
    py = sys.executable or "python3"
    return ["rocprofv3", "--pmc", *COUNTER_PASSES[i], "-d", os.path.join(out, f"counters{i}"),
            "-o", "run", "-f", "csv", "--", py, os.path.join(ROOT, "bench.py"), "--steps", "3",
            "--warmup", "1", "--legs", legs, "--workload", workload]


def prefill_kernel_of(workload: str) -> str:
    """The prefill kernel bench.py runs on `workload`."""
    import transformer_attention_diffattn_amd as da
    import workloads
    w = workloads.get(workload)
    return da.prefill_kernel_name(w.d, w.dv, w.dtype)


def counters(out: str, workload: str = "long_needles_bf16", backward: bool = False) -> None:
    """Runs the counter passes of COUNTER_PASSES over bench.py: on one
    workload's prefill, or (backward) over the two backward legs, whose
    kernels run only there (the headline prefill runs too, on the 2K
    workload, and is not summarised)."""
    out = os.path.abspath(out)
    os.makedirs(out, exist_ok=True)
    env = dict(os.environ, TMPDIR="/tmp")
    if backward:
        workload = "causal_prefill_bf16"
    for i in range(len(COUNTER_PASSES)):
        cmd = _counter_cmd(out, i, workload, "backward" if backward else "none")
        print(f"[profile] counters pass {i}: {' '.join(cmd)}", flush=True)
        with open(os.path.join(out, f"counters{i}.log"), "w") as log:
            subprocess.run(cmd, cwd="/tmp", env=env, stdout=log, stderr=subprocess.STDOUT,
                           timeout=240, check=True)
    if backward:
        for kern, wname in BACKWARD_KERNELS:
            counters_summarize(out, wname, kern, bench_workload=workload, legs="backward")
    else:
        counters_summarize(out, workload, prefill_kernel_of(workload))


def counters_summarize(out: str, workload: str = "causal_prefill_bf16",
                       kernel: str = "prefill_bf16_kernel", bench_workload: str = None,
                       legs: str = "none") -> None:
    """Per-dispatch SQ counters of one kernel, written to
    <profiles>/<kernel>__<workload>__counters.md.  bench_workload and legs:
    the bench.py command the passes ran (default: workload, no legs)."""
    out = os.path.abspath(out)
    bench_workload = bench_workload or workload
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
    src = ([e[2] for e in entries() if e[0] == kernel] or [_PREFILL])[0]
    if not vals:
        print(f"[profile] {kernel}: no dispatches in the counter passes, skipped", flush=True)
        return
    how = "--backward" if legs == "backward" else f"--workload {workload}"
    lines = [f"# {kernel} on {workload}: SQ counters per dispatch", "",
             "Commands (from /tmp, TMPDIR=/tmp; written by "
             f"`python3 profile_kernels.py counters {how}`):", ""]
    py = sys.executable or "python3"
    for i in range(len(COUNTER_PASSES)):
        shown = ["python3" if c == py else (os.path.relpath(c, ROOT) if c.startswith(ROOT) else c)
                 for c in _counter_cmd(os.path.relpath(out, ROOT), i, bench_workload, legs)]
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


def load(kernel: str, workload: str):
    """The stored summary of `kernel` on `workload`, or None if absent or the
    kernel's source changed since it was taken."""
    ent = [e for e in entries() if e[0] == kernel and e[1] == workload]
    if not ent:
        return None
    path = os.path.join(PROFILES, f"{kernel}__{workload}.md")
    try:
        with open(path) as f:
            text = f.read()
        rec = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
    except (OSError, IndexError, ValueError):
        return None
    if rec.get("source_sha256") != source_sha(ent[0][2]):
        return None
    return rec


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("action", choices=["run", "summarize", "counters", "counters-summarize"])
    ap.add_argument("--out", default=os.path.join(ROOT, "prof_out"))
    ap.add_argument("--workload", default="long_needles_bf16")
    ap.add_argument("--backward", action="store_true",
                    help="counters: the backward legs' kernels instead of a prefill")
    ap.add_argument("--profiles-dir", default=PROFILES,
                    help="where the summaries go (default: profiles/)")
    a = ap.parse_args()
    PROFILES = os.path.abspath(a.profiles_dir)
    if a.action == "run":
        run(a.out)
    elif a.action == "summarize":
        summarize(a.out)
    elif a.action == "counters":
        counters(a.out, a.workload, a.backward)
    elif a.backward:
        for kern, wname in BACKWARD_KERNELS:
            counters_summarize(a.out, wname, kern, bench_workload="causal_prefill_bf16",
                               legs="backward")
    else:
        counters_summarize(a.out, a.workload, prefill_kernel_of(a.workload))
