#!/usr/bin/env python3
"""Benchmark of the Differential Attention forward operator on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--legs LIST]

One step is one fused prefill launch over the whole batch of the headline
workload (long_needles_bf16: B1 H16 N32768, d64, dv128, bf16, causal, 8
planted needles per head -- the largest prefill workload), i.e. operand
staging, both score contractions, both online softmaxes, both P.V
contractions and the subtraction + GroupNorm epilogue.  Inputs are synthetic,
seeded, and resident in HBM before timing starts.  The throughput counts
4 (d + dv) flops per unmasked (query, key) pair (two Q.K^T and two P.V).

Legs (--legs, comma-separated; default all), each timed with events on the
launch stream and reported with its own roofline block:

  peaks               microbenchmarks: dense bf16 MFMA rate, streaming HBM
                      read rate, v_exp_f32 and v_fma_f32 rates; every
                      roofline block also reports its fraction of these
                      measured peaks, beside the published ones;
  causal_prefill_bf16, large_head_bf16
                      the other two bf16 prefill workloads (B4 H16 N2048
                      d64; B2 H32 N8192 d128 dv256 Student-t, lambda 0.95);
  decode              the decode kernel on the decode workload (B64 H32, one
                      query against an 8192-entry KV cache, one split per
                      (batch, head)), GB/s of algorithmic cache traffic;
  decode_split        the same with 4 splits per (batch, head): partials
                      plus the merge kernel;
  backward            diffattn_bwd after the training forward on
                      causal_prefill_bf16 and on large_head_bf16 (12 d + 4 dv
                      flops per pair);
  fp8                 the prefill with Q and K as E4M3 on causal_prefill_bf16
                      and on large_head_bf16;
  proj                the fused Q/K/V projection for causal_prefill_bf16;
  diag                the map diagnostics on the 32K needle workload;
  cpu                 the fp64 CPU oracle on a bounded sample of the headline
                      workload ("cpu_baseline").

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
HEADLINE = "long_needles_bf16"
ALL_LEGS = ["peaks", "large_head_bf16", "causal_prefill_bf16", "decode", "decode_split",
            "backward", "fp8", "proj", "diag", "cpu"]
DECODE_SPLITS = 4  # the decode_split leg


def _events_time(fn, steps: int):
    """Runs fn() `steps` times between two events on the current stream (the
    stream the library launches on); returns ms per call."""
    import torch

    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        fn()
    stop.record()
    stop.synchronize()
    return start.elapsed_time(stop) / steps


def prefill_kernel_name(w) -> str:
    import transformer_attention_diffattn_amd as da

    return da.prefill_kernel_name(w.d, w.dv, w.dtype)


def bench_prefill(w, steps: int, warmup: int, wall: bool = True):
    """(wall-clock ms per step over exactly `steps` steps between
    synchronisations, or None; event-timed ms per launch)."""
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
    wall_ms = None
    if wall:
        t0 = time.perf_counter()
        for _ in range(steps):
            step()
        torch.cuda.synchronize()
        wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    kern_ms = _events_time(step, steps)
    del x, out
    torch.cuda.empty_cache()
    return wall_ms, kern_ms


def roofline(bound, kernel, achieved, peak, unit, measured_peak=None, traffic=None, **extra):
    """One roofline block: achieved against the published peak, and against
    the rate the microbenchmarks measured on this GPU when known."""
    r = {"bound": bound, "kernel": kernel, "achieved": round(achieved, 2), "peak": peak,
         "unit": unit, "frac": round(achieved / peak, 4), "traffic": traffic}
    if measured_peak:
        r["measured_peak"] = round(measured_peak, 1)
        r["frac_of_measured"] = round(achieved / measured_peak, 4)
    r.update(extra)
    return r


def _peaks_lib():
    import ctypes

    import transformer_attention_diffattn_amd as da

    path = os.path.join(os.path.dirname(da.library_path()), "libdiffattn_peaks.so")
    lib = ctypes.CDLL(path)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    lib.peaks_mfma_bf16.argtypes = [vp, i32, i32, vp]
    lib.peaks_read_bw.argtypes = [vp, i64, vp, i32, vp]
    lib.peaks_vector_rate.argtypes = [vp, i32, i32, i32, vp]
    lib.peaks_lds_read.argtypes = [vp, i32, i32, vp]
    for f in (lib.peaks_mfma_bf16, lib.peaks_read_bw, lib.peaks_vector_rate, lib.peaks_lds_read,
              lib.peaks_mfma_chains, lib.peaks_vector_chains):
        f.restype = ctypes.c_int
    return lib


def measure_peaks():
    """Rates of the roofline microbenchmarks (csrc/peaks.hip) on this GPU."""
    import torch

    lib = _peaks_lib()
    stream = torch.cuda.current_stream().cuda_stream
    cus = torch.cuda.get_device_properties(0).multi_processor_count

    def timed(launch, reps=5):
        for _ in range(2):
            if launch() != 0:
                raise RuntimeError("microbenchmark launch failed")
        torch.cuda.synchronize()
        return min(_events_time(launch, 3) for _ in range(reps))

    out = {"compute_units": cus}
    # bf16 MFMA: 8 blocks of 4 waves per CU (two waves per SIMD)
    blocks, iters = cus * 8, 4096
    sink = torch.empty(blocks * 512, dtype=torch.float32, device="cuda")
    ms = timed(lambda: lib.peaks_mfma_bf16(sink.data_ptr(), blocks, iters, stream))
    flops = blocks * 4 * iters * lib.peaks_mfma_chains() * 32768
    out["mfma_bf16_tflops"] = round(flops / (ms * 1e-3) / 1e12, 1)
    # the shader clock the matrix cores ran at: 4096 bf16 flops per CU and cycle
    out["mfma_clock_ghz"] = round(flops / (ms * 1e-3) / (cus * 4096) / 1e9, 3)
    # streaming reads of 4 GiB, each byte once: 16 blocks per CU, each one
    # contiguous 1 MiB piece
    nbytes = 4 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    rblocks = cus * 16
    rsink = torch.empty(rblocks * 256, dtype=torch.int32, device="cuda")
    ms = timed(lambda: lib.peaks_read_bw(src.data_ptr(), nbytes // 16, rsink.data_ptr(), rblocks,
                                         stream), reps=3)
    out["hbm_read_gbs"] = round(nbytes / (ms * 1e-3) / 1e9, 1)
    del src, rsink
    # vector rates: 8 blocks of 4 waves per CU, 8 independent chains per lane
    vblocks, viters = cus * 8, 2048
    per = vblocks * 256 * viters * lib.peaks_vector_chains()
    for name, use_fma in (("exp", 0), ("fma", 1)):
        ms = timed(lambda: lib.peaks_vector_rate(sink.data_ptr(), vblocks, viters, use_fma, stream))
        rate = per / (ms * 1e-3)
        out[f"v_{name}_f32_per_cu_clk"] = round(rate / cus / (out["mfma_clock_ghz"] * 1e9), 2)
    # LDS reads: two workgroups of 16 waves per CU, 64 KB each
    lblocks, liters = cus * 2, 2048
    lsink = torch.empty(lblocks * 1024, dtype=torch.int32, device="cuda")
    ms = timed(lambda: lib.peaks_lds_read(lsink.data_ptr(), lblocks, liters, stream))
    lbytes = lblocks * 1024 * liters * 8 * 16
    out["lds_read_gbs_per_cu"] = round(lbytes / (ms * 1e-3) / 1e9 / cus, 1)
    out["lds_read_bytes_per_cu_clk"] = round(lbytes / (ms * 1e-3) / cus / (out["mfma_clock_ghz"] * 1e9), 1)
    del lsink
    out["note"] = ("lanes (LDS: bytes) per CU and shader cycle, at the clock the MFMA test ran "
                   "at; v_fma_f32 counts one instruction per lane")
    del sink
    torch.cuda.empty_cache()
    return out


def device_info():
    """CU count and the shader clock range as the runtime reports them."""
    import subprocess

    import torch

    p = torch.cuda.get_device_properties(0)
    info = {"name": p.name, "arch": getattr(p, "gcnArchName", None),
            "compute_units": p.multi_processor_count}
    try:
        txt = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=30).stdout
        agent = [blk for blk in txt.split("Agent ") if "gfx950" in blk]
        if agent:
            for line in agent[0].splitlines():
                if "Max Clock Freq." in line:
                    info["max_clock_mhz"] = int(line.split(":")[1].split("(")[0])
                    break
    except (OSError, subprocess.SubprocessError, ValueError):
        pass
    return info


def bench_decode(w, steps: int, warmup: int, splits: int = 0):
    """ms per decode call on workload w (splits = 0: the library's default)."""
    import torch

    import transformer_attention_diffattn_amd as da
    import workloads

    x = workloads.make_decode(w, device="cuda")
    out = torch.empty((w.B, w.H, w.dv), dtype=w.torch_dtype, device="cuda")
    if splits <= 0:
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


def _traffic(kernel: str, workload: str):
    """Scaled HBM bytes per launch from the committed rocprofv3 counter summary
    of this kernel on this workload, or None when there is none or the
    kernel source changed since it was taken."""
    import profile_kernels

    rec = profile_kernels.load(kernel, workload)
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


def backward_record(w, args, mpk: dict) -> dict:
    """The backward leg on workload w: diffattn_bwd after the training
    forward, TFLOP/s at 12 d + 4 dv flops per unmasked (query, key) pair (the
    two score products again, dP, dV, dK_k and dQ_k)."""
    bms, tfms = bench_backward(w, max(20, args.steps // 5), max(5, args.warmup // 20))
    pairs = w.exec_flops() / (4 * (w.d + w.dv))
    bflops = pairs * (12 * w.d + 4 * w.dv)
    btf = bflops / (bms * 1e-3) / 1e12
    kern = ("bwd_prep + bwd_dq_ring + bwd_dkdv_ring + bwd_dlam" if w.d == 128
            else "bwd_prep + bwd_dq + bwd_dkdv16 + bwd_dlam" if w.d == 64
            else "bwd_prep + bwd_dq + bwd_dkdv + bwd_dlam")
    return {
        "workload": w.name,
        "value": round(btf, 2),
        "unit": "TFLOP/s",
        "ms_per_call": round(bms, 4),
        "flops_per_call": int(bflops),
        "fwd_train_ms": round(tfms, 4),
        "roofline": roofline("mfma", kern, btf, PEAK_BF16_TFLOPS, "TFLOP/s",
                             mpk.get("mfma_bf16_tflops")),
    }


def fp8_record(w, args, mpk: dict) -> dict:
    """The fp8 leg on workload w: TFLOP/s of diffattn_fwd_fp8 against the
    peak of its mix of products.  The scores run on the e4m3 MFMA (dense
    peak 2x bf16), P.V on the bf16 one, so the mix's peak is the flops over
    their time at the two peaks.  Per unmasked (query, key) pair the
    head_dim-128 kernel computes the scores twice (8 d flops: both maps, both
    sweeps) and one P.V of 2 dv; the head_dim-64 kernel 4 d and 4 dv."""
    fms, bms16 = bench_fp8(w, max(30, args.steps // 3), max(20, args.warmup // 5))
    f = w.exec_flops()
    pairs = f / (4 * (w.d + w.dv))
    sf, pf = (8 * w.d, 2 * w.dv) if w.d == 128 else (4 * w.d, 4 * w.dv)

    def mix(p):
        return f / (pairs * (sf / (2 * p) + pf / p))

    kern = "prefill_fp8qk_twopass_kernel" if w.d == 128 else "prefill_fp8qk_kernel"
    ftf = f / (fms * 1e-3) / 1e12
    mm = mpk.get("mfma_bf16_tflops")
    return {
        "workload": w.name + " (Q, K as e4m3, per-tensor scales)",
        "value": round(ftf, 2),
        "unit": "TFLOP/s",
        "ms_per_call": round(fms, 4),
        "bf16_ms_per_call_same_run": round(bms16, 4),
        "speedup_vs_bf16": round(bms16 / fms, 3),
        "roofline": roofline("mfma", kern, ftf, round(mix(PEAK_BF16_TFLOPS), 1), "TFLOP/s",
                             mix(mm) if mm else None, _traffic(kern, w.name)),
    }


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


def prefill_record(w, wall_ms, kern_ms, mpk):
    """Throughput of one prefill workload and its roofline block."""
    flops = w.exec_flops()
    achieved = flops / (kern_ms * 1e-3) / 1e12
    f32 = w.dtype == "f32"
    kernel = prefill_kernel_name(w)
    rec = {
        "workload": w.name,
        "ms_per_launch": round(kern_ms, 4),
        "tflops": round(achieved, 2),
        "tokens_per_s": round(w.B * w.nq / (kern_ms * 1e-3), 1),
        "formula_tflops": round(w.formula_flops() / (kern_ms * 1e-3) / 1e12, 2),
        "roofline": roofline(
            "alu" if f32 else "mfma", kernel, achieved,
            PEAK_F32_VALU_TFLOPS if f32 else PEAK_BF16_TFLOPS, "TFLOP/s",
            None if f32 else mpk.get("mfma_bf16_tflops"), _traffic(kernel, w.name),
            launch_ms=round(kern_ms, 4), flops_per_launch=flops),
    }
    if wall_ms is not None:
        rec["wall_ms_per_step"] = round(wall_ms, 4)
    return rec


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # a few hundred launches let the GPU reach its steady clocks before timing
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--legs", default=",".join(ALL_LEGS),
                    help="comma-separated legs to run besides the headline (or 'none'): "
                         + ", ".join(ALL_LEGS))
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a plain fp32 copy of 1 GiB (3 times), the reference the "
                         "HBM byte counters are scaled by")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this operator is built and timed on a single "
              "MI355X (multi-GPU sharding is a design note only); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    legs = [] if args.legs == "none" else [x for x in args.legs.split(",") if x]
    unknown = [x for x in legs if x not in ALL_LEGS]
    if unknown:
        print(f"unknown legs {unknown}; known: {ALL_LEGS}", file=sys.stderr)
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

    mpk = measure_peaks() if "peaks" in legs else {}

    # the other prefill workloads first, then the headline.  A leg times at
    # least 100 launches after at least 20 warm-up ones whatever --steps and
    # --warmup say: 20 launches of the 2K workload span 2.4 ms, short enough
    # for clock transitions to show in the figure (only the headline is tied
    # to exactly --steps steps)
    prefill_legs = {}
    for name in ("large_head_bf16", "causal_prefill_bf16"):
        if name in legs and name != w.name:
            wl = workloads.get(name)
            _, lms = bench_prefill(wl, max(args.steps, 100), max(args.warmup, 20), wall=False)
            prefill_legs[name] = prefill_record(wl, None, lms, mpk)

    wall_ms, kern_ms = bench_prefill(w, args.steps, args.warmup)
    flops = w.exec_flops()
    value = flops / (wall_ms * 1e-3) / 1e12
    head = prefill_record(w, wall_ms, kern_ms, mpk)
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
        "roofline": head["roofline"],
        "device": device_info(),
    }
    if mpk:
        rec["peaks"] = mpk
    if prefill_legs:
        rec["prefill_legs"] = prefill_legs

    wd = workloads.get("decode_bf16")
    nbytes = wd.algorithmic_bytes()
    for leg, want in (("decode", 0), ("decode_split", DECODE_SPLITS)):
        if leg not in legs:
            continue
        dms, splits, ws_bytes = bench_decode(wd, max(20, args.steps // 5), max(5, args.warmup // 10),
                                             splits=want)
        gbs = nbytes / (dms * 1e-3) / 1e9
        kern = "decode_partial_kernel" + (" + decode_merge_kernel" if splits > 1 else "")
        rec[leg] = {
            "workload": wd.name,
            "value": round(gbs, 1),
            "unit": "GB/s",
            "ms_per_call": round(dms, 4),
            "tokens_per_s": round(wd.B / (dms * 1e-3), 1),
            "splits": splits,
            "workspace_bytes": ws_bytes,
            "roofline": roofline("hbm", kern, gbs, PEAK_HBM_GBS, "GB/s",
                                 mpk.get("hbm_read_gbs"),
                                 _traffic("decode_partial_kernel", wd.name) if splits == 1 else None,
                                 bytes_per_call=nbytes),
        }

    w2 = workloads.get("causal_prefill_bf16")
    f2 = w2.exec_flops()
    pairs2 = f2 / (4 * (w2.d + w2.dv))
    if "backward" in legs:
        for key, wb in (("backward", w2), ("backward_large_head", workloads.get("large_head_bf16"))):
            rec[key] = backward_record(wb, args, mpk)

    if "fp8" in legs:
        for key, wf in (("fp8_qk", w2), ("fp8_qk_large_head", workloads.get("large_head_bf16"))):
            rec[key] = fp8_record(wf, args, mpk)

    if "proj" in legs:
        pms, lms, pflops = bench_proj(w2, max(30, args.steps // 3), max(20, args.warmup // 3))
        ptf = pflops / (pms * 1e-3) / 1e12
        rec["qkv_proj"] = {
            "workload": f"{w2.name} projections (d_model {w2.H * w2.dv})",
            "value": round(ptf, 2),
            "unit": "TFLOP/s",
            "ms_per_call": round(pms, 4),
            "flops_per_call": pflops,
            "library_gemm_ms_no_head_split": round(lms, 4),
            "roofline": roofline("mfma", "qkv_proj_kernel", ptf, PEAK_BF16_TFLOPS, "TFLOP/s",
                                 mpk.get("mfma_bf16_tflops"),
                                 _traffic("qkv_proj_kernel", w2.name)),
        }

    if "diag" in legs:
        rec["diagnostics"] = bench_diag(max(3, args.steps // 20))

    if "cpu" in legs:
        cb = cpu_baseline(w)
        cb["cpu"] = _cpu_model()
        rec["cpu_baseline"] = cb

    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
