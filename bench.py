#!/usr/bin/env python3
"""Benchmark of the Differential Attention forward operator on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is one fused prefill launch over the whole batch of the headline
workload (causal_prefill_bf16: B4 H16 N2048, d64, dv128, bf16, causal), i.e.
operand staging, both score contractions, both online softmaxes, both P.V
contractions and the subtraction + GroupNorm epilogue.  Inputs are synthetic,
seeded, and resident in HBM before timing starts.  The throughput counts
4 (d + dv) flops per unmasked (query, key) pair (two Q.K^T and two P.V).

The same run also times the decode kernels (split-K partials + merge) on the
decode workload (B64 H32, one query against an 8192-entry KV cache) and
reports them in "decode" as GB/s of algorithmic cache traffic, times the
backward (diffattn_bwd after the training forward) on the headline workload
("backward", TFLOP/s at 12 d + 4 dv flops per unmasked pair: both score maps
recomputed, one shared dP, dV, dK1, dK2, dQ1, dQ2), runs the map
diagnostics on the 32K needle workload ("diagnostics": the row-max sweep at
4 d flops per unmasked pair, the needle weights, and the values they give on
those synthetic inputs), times the prefill with Q and K quantised to E4M3
("fp8_qk"), times the fused Q/K/V projection that produces the headline's
inputs from d_model = H dv hidden states ("qkv_proj"), and times the fp64 CPU
oracle on a bounded sample of
the headline workload ("cpu_baseline").

Prints one JSON line on stdout.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# MI355X published peaks: dense bf16 MFMA and HBM3E bandwidth
PEAK_BF16_TFLOPS = 2500.0
PEAK_F32_VALU_TFLOPS = 157.3  # the fp32 kernel runs on the vector ALUs
PEAK_HBM_GBS = 8000.0
METRIC = "DiffAttn fwd TFLOP/s (prefill) and KV GB/s (decode), % of roofline"


def _events_time(fn, steps: int):
    """Runs fn() `steps` times between two events on the current stream; returns ms per call."""
    import torch

    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        fn()
    stop.record()
    stop.synchronize()
    return start.elapsed_time(stop) / steps


def bench_prefill(w, steps: int, warmup: int):
    import torch

    import transformer_attention_diffattn_amd as da
    import workloads

    x = workloads.make_prefill(w, device="cuda")
    out = torch.empty((w.B, w.H, w.nq, w.dv), dtype=w.torch_dtype, device="cuda")

    def step():
        da.fwd(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], x["lam"], lambda_init=w.lambda_init,
               causal=w.causal, eps=w.eps, out=out)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # wall clock over exactly `steps` steps, bracketed by synchronisations
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    # per-launch device time from events on the launch stream
    kern_ms = _events_time(step, steps)
    del x, out
    return wall_ms, kern_ms


def bench_decode(w, steps: int, warmup: int):
    import torch

    import transformer_attention_diffattn_amd as da
    import workloads

    x = workloads.make_decode(w, device="cuda")
    out = torch.empty((w.B, w.H, w.dv), dtype=w.torch_dtype, device="cuda")
    splits = da.decode_default_splits(w.B, w.H, w.nk, w.d, w.dv)
    ws_bytes = da.decode_workspace_size(w.B, w.H, w.nk, w.d, w.dv, splits)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")

    def step():
        da.decode(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], x["lam"],
                  lambda_init=w.lambda_init, eps=w.eps, out=out, workspace=ws,
                  num_splits=splits)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    kern_ms = _events_time(step, steps)
    del x, out, ws
    torch.cuda.empty_cache()
    return kern_ms, splits, ws_bytes


def bench_backward(w, steps: int, warmup: int):
    """ms per diffattn_bwd call and per training-forward call on workload w."""
    import torch

    import transformer_attention_diffattn_amd as da
    import workloads

    x = workloads.make_prefill(w, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(1)
    dout = torch.randn((w.B, w.H, w.nq, w.dv), generator=g, device="cuda").to(w.torch_dtype)
    args = (x["q1"], x["q2"], x["k1"], x["k2"], x["v"], x["lam"])
    _, d_save, lse = da.fwd_train(*args, lambda_init=w.lambda_init, causal=w.causal, eps=w.eps)
    ws = torch.empty((max(da.bwd_workspace_size(w.B, w.H, w.nq, w.nk, w.d, w.dv), 16),),
                     dtype=torch.uint8, device="cuda")

    def bwd_step():
        da.bwd(*args, dout, d_save, lse, lambda_init=w.lambda_init, causal=w.causal, eps=w.eps,
               workspace=ws)

    def fwd_step():
        da.fwd_train(*args, lambda_init=w.lambda_init, causal=w.causal, eps=w.eps)

    for _ in range(warmup):
        bwd_step()
    torch.cuda.synchronize()
    bwd_ms = _events_time(bwd_step, steps)
    for _ in range(max(2, warmup // 4)):
        fwd_step()
    torch.cuda.synchronize()
    fwd_ms = _events_time(fwd_step, steps)
    del x, dout, d_save, lse, ws
    torch.cuda.empty_cache()
    return bwd_ms, fwd_ms


def bench_diag(steps: int):
    """Map diagnostics on the 32K needle workload: kernel times and values."""
    import numpy as np
    import torch

    import transformer_attention_diffattn_amd as da
    import workloads

    w = workloads.get("long_needles_bf16")
    x = workloads.make_prefill(w, device="cuda")
    args = (x["q1"], x["q2"], x["k1"], x["k2"], x["v"])
    _, _, lse = da.fwd_train(*args, x["lam"], lambda_init=w.lambda_init, causal=True, eps=w.eps)
    plans = workloads.needle_plan(w)
    nq = torch.tensor(np.stack([p[1] for p in plans]).reshape(w.B, w.H, -1), dtype=torch.int32)
    nk = torch.tensor(np.stack([p[0] for p in plans]).reshape(w.B, w.H, -1), dtype=torch.int32)
    nq, nk = nq.cuda(), nk.cuda()
    da.diag(*args, causal=True)  # warm-up
    rm_ms = _events_time(lambda: da.diag(*args, causal=True), steps)
    nd_ms = _events_time(lambda: da.diag(*args, causal=True, lse=lse, needle_q=nq, needle_k=nk,
                                          row_max=False), steps)
    rm, nd = da.diag(*args, causal=True, lse=lse, needle_q=nq, needle_k=nk)
    torch.cuda.synchronize()
    lam = x["lam"].view(1, w.H, 1)
    a1, a2 = nd[..., 0], nd[..., 1]
    m1, m2 = nd[..., 2], nd[..., 3]
    flops = w.pairs() * 4 * w.d
    out = {
        "workload": w.name,
        "row_max_ms": round(rm_ms, 4),
        "row_max_tflops": round(flops / (rm_ms * 1e-3) / 1e12, 2),
        "needles_ms": round(nd_ms, 4),
        "values": {
            "needle_weight_map1_mean": round(float(a1.mean()), 5),
            "needle_weight_map2_mean": round(float(a2.mean()), 6),
            "needle_weight_differential_mean": round(float((a1 - lam * a2).mean()), 5),
            "needle_row_mass_map1_mean": round(float(m1.mean()), 5),
            "needle_row_mass_differential_mean": round(float((m1 - lam * m2).mean()), 5),
            "top_logit_map1": round(float(rm[0].max()), 3),
            "top_logit_map2": round(float(rm[1].max()), 3),
        },
    }
    del x, lse, rm, nd
    torch.cuda.empty_cache()
    return out


def cpu_baseline(w, budget_s: float = 30.0):
    """Times the fp64 oracle (as it is) head by head over the workload, stopping
    after about budget_s seconds of compute or when every head is done; reports
    the rate in the headline's unit (4 (d + dv) flops per unmasked pair)."""
    import oracle
    import workloads

    x = workloads.make_prefill(w, device="cpu")
    lam = x["lam"].numpy()
    oracle.num_threads()  # load outside the timed region
    heads, pairs, elapsed = 0, 0, 0.0
    per_head = w.nq * (w.nq + 1) // 2 if w.causal else w.nq * w.nk
    for b in range(w.B):
        for h in range(w.H):
            args = [x[k][b, h].double().numpy() for k in ("q1", "q2", "k1", "k2", "v")]
            t0 = time.perf_counter()
            oracle.head_rows(*args, None, causal=w.causal, lam=float(lam[h]),
                             lambda_init=w.lambda_init, eps=w.eps)
            elapsed += time.perf_counter() - t0
            heads += 1
            pairs += per_head
            if elapsed >= budget_s:
                break
        if elapsed >= budget_s:
            break
    flops = 4 * (w.d + w.dv) * pairs
    return {
        "value": round(flops / elapsed / 1e12, 5),
        "unit": "TFLOP/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": f"{heads} of {w.B * w.H} heads, all {w.nq} query rows each "
                  f"({elapsed:.2f} s of fp64 compute, input upcast excluded)",
        "tokens_per_s": round(heads * w.nq / elapsed, 1),
    }


COPY_BYTES = 1 << 30


def _traffic(kernel: str):
    """Scaled HBM bytes per launch from the committed rocprofv3 counter summary
    of this kernel, or None when there is none or the kernel source changed."""
    import profile_kernels

    rec = profile_kernels.load(kernel)
    return None if rec is None else rec["traffic_bytes_per_launch"]


def copy_calibration():
    """A plain elementwise copy (dst = src * 1) reading and writing COPY_BYTES."""
    import torch

    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def bench_fp8(w, steps: int, warmup: int):
    """ms per diffattn_fwd_fp8 launch on workload w with Q1, Q2, K1, K2
    quantised per tensor to E4M3 (V stays bf16), and ms per bf16 launch on
    the unquantised inputs timed alternately with it (same clocks)."""
    import torch

    import transformer_attention_diffattn_amd as da
    import workloads

    x = workloads.make_prefill(w, device="cuda")
    x8 = workloads.make_prefill_fp8(w, device="cuda")
    out = torch.empty((w.B, w.H, w.nq, w.dv), dtype=torch.bfloat16, device="cuda")

    def step8():
        da.fwd_fp8(x8["q1"], x8["q2"], x8["k1"], x8["k2"], x8["v"], x8["scales"], x8["lam"],
                   lambda_init=w.lambda_init, causal=w.causal, eps=w.eps, out=out)

    def step16():
        da.fwd(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], x["lam"], lambda_init=w.lambda_init,
               causal=w.causal, eps=w.eps, out=out)

    for _ in range(warmup):
        step8()
        step16()
    torch.cuda.synchronize()
    t8, t16 = [], []
    for _ in range(3):
        t8.append(_events_time(step8, steps))
        t16.append(_events_time(step16, steps))
    del x, x8, out
    torch.cuda.empty_cache()
    return min(t8), min(t16)


def bench_proj(w, steps: int, warmup: int):
    """ms per diffattn_qkv_proj launch for workload w's attention shapes
    (d_model = H dv), and ms per library GEMM (torch.matmul) of the same
    operands without the head split, for context."""
    import torch

    import transformer_attention_diffattn_amd as da
    import workloads

    p = workloads.make_proj(w, device="cuda")
    x, wt = p["x"], p["w"]
    outs = [torch.empty(s, dtype=torch.bfloat16, device="cuda")
            for s in [(w.B, w.H, w.nq, w.d)] * 4 + [(w.B, w.H, w.nq, w.dv)]]
    y = torch.empty((w.B * w.nq, wt.shape[0]), dtype=torch.bfloat16, device="cuda")
    x2 = x.reshape(w.B * w.nq, p["d_model"])

    def step():
        da.qkv_proj(x, wt, w.H, w.d, w.dv, out=outs)

    def lib_step():
        torch.matmul(x2, wt.t(), out=y)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ms = _events_time(step, steps)
    for _ in range(max(2, warmup // 4)):
        lib_step()
    torch.cuda.synchronize()
    lib_ms = _events_time(lib_step, steps)
    flops = 2 * w.B * w.nq * p["d_model"] * wt.shape[0]
    del p, x, wt, outs, y
    torch.cuda.empty_cache()
    return ms, lib_ms, flops


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # a few hundred launches let the GPU reach its steady clocks before timing
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--workload", default="causal_prefill_bf16")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode leg")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward leg")
    ap.add_argument("--no-diag", action="store_true", help="skip the diagnostics leg")
    ap.add_argument("--no-fp8", action="store_true", help="skip the FP8 query/key leg")
    ap.add_argument("--no-proj", action="store_true", help="skip the Q/K/V projection leg")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a plain fp32 copy of 1 GiB (3 times), the reference the "
                         "HBM byte counters are scaled by")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this operator is built and timed on a single "
              "MI355X (multi-GPU sharding is a design note only); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import transformer_attention_diffattn_amd as da
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    da.lib()  # fail loudly if the HIP library is missing
    torch.cuda.set_device(0)

    if args.copy_calibration:
        copy_calibration()

    w = workloads.get(args.workload)
    if w.kind != "prefill":
        print("--workload must name a prefill workload", file=sys.stderr)
        sys.exit(2)
    wall_ms, kern_ms = bench_prefill(w, args.steps, args.warmup)
    flops = w.exec_flops()
    value = flops / (wall_ms * 1e-3) / 1e12
    achieved = flops / (kern_ms * 1e-3) / 1e12
    # the fp32 workload runs on the vector ALUs, the bf16 ones on the MFMA
    peak = PEAK_F32_VALU_TFLOPS if w.dtype == "f32" else PEAK_BF16_TFLOPS
    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded)",
        "config": {"workload": w.name, "batch": w.B, "heads": w.H, "seq_len": w.nq,
                   "head_dim": w.d, "v_dim": w.dv, "causal": w.causal,
                   "global_batch": w.B, "parallelism": "single GPU"},
        "tokens_per_s": round(w.B * w.nq / (wall_ms * 1e-3), 1),
        "formula_tflops": round(w.formula_flops() / (wall_ms * 1e-3) / 1e12, 2),
        "roofline": {
            "bound": "alu" if w.dtype == "f32" else "mfma",
            "kernel": ("prefill_f32_kernel" if w.dtype == "f32" else
                       "prefill_bf16_wide_kernel" if w.d == 128 else "prefill_bf16_kernel"),
            "achieved": round(achieved, 2),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": _traffic("prefill_bf16_kernel") if w.name == "causal_prefill_bf16" else None,
            "launch_ms": round(kern_ms, 4),
            "flops_per_launch": flops,
        },
    }

    if not args.no_decode:
        wd = workloads.get("decode_bf16")
        dec_steps = max(5, args.steps // 5)
        dms, splits, ws_bytes = bench_decode(wd, dec_steps, max(2, args.warmup // 30))
        nbytes = wd.algorithmic_bytes()
        gbs = nbytes / (dms * 1e-3) / 1e9
        rec["decode"] = {
            "workload": wd.name,
            "value": round(gbs, 1),
            "unit": "GB/s",
            "ms_per_call": round(dms, 4),
            "tokens_per_s": round(wd.B / (dms * 1e-3), 1),
            "splits": splits,
            "workspace_bytes": ws_bytes,
            "roofline": {"bound": "hbm", "kernel": "decode_partial_kernel (+ merge)",
                         "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "traffic": _traffic("decode_partial_kernel"),
                         "bytes_per_call": nbytes},
        }

    if not args.no_backward and w.dtype == "bf16" and (w.d, w.dv) in ((32, 64), (64, 128)):
        bms, tfms = bench_backward(w, max(5, args.steps // 5), max(3, args.warmup // 20))
        pairs = flops / (4 * (w.d + w.dv))
        bflops = pairs * (12 * w.d + 4 * w.dv)
        btf = bflops / (bms * 1e-3) / 1e12
        rec["backward"] = {
            "workload": w.name,
            "value": round(btf, 2),
            "unit": "TFLOP/s",
            "ms_per_call": round(bms, 4),
            "flops_per_call": int(bflops),
            "fwd_train_ms": round(tfms, 4),
            "roofline": {"bound": "mfma", "kernel": "bwd_prep + bwd_dq + bwd_dkdv + bwd_dlam",
                         "achieved": round(btf, 2), "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(btf / PEAK_BF16_TFLOPS, 4),
                         "traffic": None},
        }

    if not args.no_fp8 and w.dtype == "bf16" and (w.d, w.dv) == (64, 128):
        fms, bms16 = bench_fp8(w, max(10, args.steps // 3), max(20, args.warmup // 5))
        pairs = flops / (4 * (w.d + w.dv))
        # scores on the e4m3 MFMA (peak 2x bf16), P.V on the bf16 one: the
        # peak of this mix is the flops over their time at the two peaks
        mix_peak = flops / (pairs * (4 * w.d / (2 * PEAK_BF16_TFLOPS) + 4 * w.dv / PEAK_BF16_TFLOPS))
        ftf = flops / (fms * 1e-3) / 1e12
        rec["fp8_qk"] = {
            "workload": w.name + " (Q, K as e4m3, per-tensor scales)",
            "value": round(ftf, 2),
            "unit": "TFLOP/s",
            "ms_per_call": round(fms, 4),
            "bf16_ms_per_call_same_run": round(bms16, 4),
            "speedup_vs_bf16": round(bms16 / fms, 3),
            "roofline": {"bound": "mfma", "kernel": "prefill_fp8qk_kernel",
                         "achieved": round(ftf, 2), "peak": round(mix_peak, 1),
                         "unit": "TFLOP/s", "frac": round(ftf / mix_peak, 4),
                         "traffic": None},
        }

    if not args.no_proj and w.dtype == "bf16":
        pms, lms, pflops = bench_proj(w, max(10, args.steps // 3), max(20, args.warmup // 3))
        ptf = pflops / (pms * 1e-3) / 1e12
        rec["qkv_proj"] = {
            "workload": f"{w.name} projections (d_model {w.H * w.dv})",
            "value": round(ptf, 2),
            "unit": "TFLOP/s",
            "ms_per_call": round(pms, 4),
            "flops_per_call": pflops,
            "library_gemm_ms_no_head_split": round(lms, 4),
            "roofline": {"bound": "mfma", "kernel": "qkv_proj_kernel", "achieved": round(ptf, 2),
                         "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(ptf / PEAK_BF16_TFLOPS, 4), "traffic": None},
        }

    if not args.no_diag:
        rec["diagnostics"] = bench_diag(max(3, args.steps // 20))

    if not args.no_cpu:
        cb = cpu_baseline(w)
        cb["cpu"] = _cpu_model()
        rec["cpu_baseline"] = cb

    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
