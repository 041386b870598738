"""Builds libdiffattn.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Usage: python -m transformer_attention_diffattn_amd.build [--jobs N] [--sanitize]

Each source compiles to an object in ``_build/`` (in parallel), then the objects
link into ``transformer_attention_diffattn_amd/_lib/libdiffattn.so``.  The
library is always rebuilt when this runs.

--sanitize builds ``_lib/libdiffattn_san.so`` instead (objects in
``_build/san/``): the host code (the C ABI's argument checks, split planning
and launch set-up) compiled with AddressSanitizer and
UndefinedBehaviorSanitizer; device code is unchanged.  A process loading it
needs the sanitizer runtime preloaded (``sanitizer_runtime()``).
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
SAN_LIB = os.path.join(LIBDIR, "libdiffattn_san.so")
# host-side sanitizers only: each flag goes to the host compilation
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host",
             "-fno-omit-frame-pointer"]
# the roofline microbenchmarks: a library of their own, not part of the operator
PEAKS_SRC = "peaks.hip"
PEAKS_LIB = os.path.join(LIBDIR, "libdiffattn_peaks.so")
SOURCES = ["api.hip", "prefill_bf16.hip", "prefill_twopass.hip", "prefill_f32.hip", "decode.hip", "backward.hip", "backward_ring.hip", "diag.hip", "proj.hip"]
# Per-source extra flags.  The narrow-head prefill kernel keeps its score
# accumulators in ordinary VGPRs, where the softmax reads them without a copy
# out of the accumulation registers; the compiler's default heuristic would
# put every matrix accumulator in AGPRs.
EXTRA_FLAGS = {"prefill_bf16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
               "prefill_twopass.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
               # builtin products in VGPRs; the accumulators are pinned to
               # AGPRs by the kernels' own asm
               "backward_ring.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
               # head_dim 32/64 backward: fewer copies between the register
               # files (2K workload backward 0.534 -> 0.516 ms, back to back)
               "backward.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC",
    "-Wall", "-Wno-unused-function",
    # packed fp32 VALU instructions stay off in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def sanitizer_runtime() -> str:
    """The clang ASan runtime (it carries the UBSan handlers too) that a
    process must preload to load the sanitized library."""
    import glob
    hits = sorted(glob.glob(os.path.join(os.path.dirname(os.path.dirname(HIPCC)), "llvm", "lib",
                                         "clang", "*", "lib", "linux",
                                         "libclang_rt.asan-x86_64.so")))
    if not hits:
        raise FileNotFoundError("clang ASan runtime not found under the ROCm LLVM")
    return hits[-1]


def build(jobs: int = 4, verbose: bool = False, sanitize: bool = False) -> str:
    bdir = os.path.join(BUILD, "san") if sanitize else BUILD
    os.makedirs(bdir, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    extra_all = SAN_FLAGS if sanitize else []
    objs, procs = [], []
    for src in SOURCES:
        obj = os.path.join(bdir, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmd = [HIPCC, *FLAGS, *extra_all, *EXTRA_FLAGS.get(src, []), "-c",
               os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        if len(procs) >= jobs:
            _wait(procs.pop(0))
    libs = [(SAN_LIB, objs)] if sanitize else [(LIB, objs)]
    if not sanitize:
        peaks_obj = os.path.join(bdir, os.path.splitext(PEAKS_SRC)[0] + ".o")
        procs.append((PEAKS_SRC, subprocess.Popen(
            [HIPCC, *FLAGS, "-c", os.path.join(CSRC, PEAKS_SRC), "-o", peaks_obj],
            stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        libs.append((PEAKS_LIB, [peaks_obj]))
    for p in procs:
        _wait(p)
    for lib, lib_objs in libs:
        tmp = lib + ".tmp"
        cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *extra_all, "-o", tmp,
               *lib_objs]
        if sanitize:
            # the runtime comes from the preloaded library, not the link
            cmd += ["-Xarch_host", "-shared-libsan"]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(tmp, lib)
    return libs[0][0]


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
    ap.add_argument("--sanitize", action="store_true",
                    help="host code with ASan + UBSan, into _lib/libdiffattn_san.so")
    args = ap.parse_args()
    print(build(args.jobs, args.verbose, args.sanitize))
