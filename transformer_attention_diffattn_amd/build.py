"""Builds libdiffattn.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Usage: python -m transformer_attention_diffattn_amd.build [--jobs N]

Each source compiles to an object in ``_build/`` (in parallel), then the objects
link into ``transformer_attention_diffattn_amd/_lib/libdiffattn.so``.  The
library is always rebuilt when this runs.
"""
from __future__ import annotations

import argparse
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIBDIR = os.path.join(HERE, "_lib")
LIB = os.path.join(LIBDIR, "libdiffattn.so")
SOURCES = ["api.hip", "prefill_bf16.hip", "prefill_bf16_wide.hip", "prefill_f32.hip", "decode.hip", "backward.hip", "diag.hip", "proj.hip"]
# Per-source extra flags.  The narrow-head prefill kernel keeps its score
# accumulators in ordinary VGPRs, where the softmax reads them without a copy
# out of the accumulation registers; the compiler's default heuristic would
# put every matrix accumulator in AGPRs.
EXTRA_FLAGS = {"prefill_bf16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC",
    "-Wall", "-Wno-unused-function",
    # packed fp32 VALU instructions stay off in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def build(jobs: int = 4, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    objs, procs = [], []
    for src in SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmd = [HIPCC, *FLAGS, *EXTRA_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        if len(procs) >= jobs:
            _wait(procs.pop(0))
    for p in procs:
        _wait(p)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def _wait(item):
    src, proc = item
    out, _ = proc.communicate()
    text = out.decode(errors="replace")
    # the host pass does not know the device-only target feature; that note is harmless
    lines = [l for l in text.splitlines() if "packed-fp32-ops" not in l]
    if proc.returncode != 0:
        sys.stderr.write("\n".join(lines) + "\n")
        raise RuntimeError(f"hipcc failed on {src}")
    if lines:
        sys.stderr.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=4)
    ap.add_argument("-v", "--verbose", action="store_true")
    args = ap.parse_args()
    print(build(args.jobs, args.verbose))
