"""fp64 CPU oracle for the Differential Attention forward operator.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package; the GPU library never does, and this
package never imports the GPU library.

The arithmetic lives in ``diffattn_oracle.c`` (plain C, double precision,
OpenMP over query rows); this module builds it with gcc and wraps it.  What it
computes, with the passages it follows:

* the two scaled dot-product softmax maps and their lambda-weighted difference
  applied to V -- the DiffAttn formula on iloveeagents.com ("Mathematical
  Formula") and steps 2-3 on llmbytes.dev ("How Differential Attention Cancels
  Common-Mode Noise");
* the per-head GroupNorm over each head's value channels followed by the
  (1 - lambda_init) scale -- step 4 on the same llmbytes.dev page.

Readings taken where the pages are silent (causal mask on both maps, population
variance, eps inside the square root, no affine parameters) are listed in the C
file's header.  Decode is the same definition with one query that sees every
cached key.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import sys
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "diffattn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_SAN_LIB = os.path.join(_HERE, "liboracle_san.so")
_lib = None


def build(force: bool = True, src: str = _SRC, lib: str = _LIB, sanitize: bool = False) -> str:
    """Compile the oracle with gcc (-O2, IEEE semantics kept: no fast-math).

    sanitize: build liboracle_san.so with clang's AddressSanitizer and
    UndefinedBehaviorSanitizer instead (the ROCm LLVM's clang, whose ASan
    runtime a process must preload to load it)."""
    if sanitize and lib == _LIB:
        lib = _SAN_LIB
    if force or not os.path.exists(lib) or os.path.getmtime(lib) < os.path.getmtime(src):
        tmp = lib + ".tmp"
        if sanitize:
            cmd = ["/opt/rocm/llvm/bin/clang", "-O1", "-g", "-fno-omit-frame-pointer",
                   "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                   "-shared-libsan", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall",
                   "-Wextra", "-o", tmp, src, "-lm"]
        else:
            cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                   "-Wall", "-Wextra", "-o", tmp, src, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, lib)
    return lib


class Oracle:
    """ctypes handle on one compiled copy of diffattn_oracle.c."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        lib.oracle_diffattn_rows.restype = ctypes.c_int
        P = ctypes.c_void_p
        lib.oracle_diffattn_rows.argtypes = [
            P, P, P, P, P,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
            P, ctypes.c_int64,
            ctypes.c_int, ctypes.c_double, ctypes.c_double, ctypes.c_double,
            ctypes.c_int, P, P]
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_num_threads.argtypes = []
        self.lib = lib

    def num_threads(self) -> int:
        return int(self.lib.oracle_num_threads())

    def head_rows(self, q1, q2, k1, k2, v, rows: Optional[Sequence[int]], *, causal: bool,
                  lam: float, lambda_init: float = 0.8, eps: float = 1e-5,
                  pre_norm: bool = False, want_rowsum: bool = False):
        """Oracle rows of one head.

        q1, q2: [n_q, d]; k1, k2: [n_k, d]; v: [n_k, dv] (any float dtype; upcast
        exactly to fp64).  rows: query indices to compute (None = all).  Returns
        an fp64 array [len(rows), dv] (and the row sums of A1 - lam*A2 if asked).
        """
        q1, q2, k1, k2, v = (_f64(t) for t in (q1, q2, k1, k2, v))
        n_q, d = q1.shape
        n_k, dv = v.shape
        if q2.shape != (n_q, d) or k1.shape != (n_k, d) or k2.shape != (n_k, d):
            raise ValueError("inconsistent shapes")
        if rows is None:
            rows = np.arange(n_q, dtype=np.int64)
        rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        out = np.empty((len(rows), dv), dtype=np.float64)
        rs = np.empty(len(rows), dtype=np.float64) if want_rowsum else None
        rc = self.lib.oracle_diffattn_rows(
            _ptr(q1), _ptr(q2), _ptr(k1), _ptr(k2), _ptr(v),
            n_q, n_k, d, dv, _ptr(rows), len(rows),
            int(bool(causal)), float(lam), float(lambda_init), float(eps),
            int(bool(pre_norm)), _ptr(out), _ptr(rs) if rs is not None else None)
        if rc != 0:
            raise ValueError("oracle_diffattn_rows rejected its arguments")
        return (out, rs) if want_rowsum else out


def _load() -> Oracle:
    global _lib
    if _lib is None:
        # DIFFATTN_ORACLE_LIB: another build of the same source (the sanitized one)
        path = os.environ.get("DIFFATTN_ORACLE_LIB")
        if not path:
            build(force=False)
            path = _LIB
        _lib = Oracle(path)
    return _lib


def num_threads() -> int:
    return _load().num_threads()


def _f64(x) -> np.ndarray:
    """Exact upcast of a torch tensor or array (bf16/fp32/fp64) to C-contiguous fp64."""
    if hasattr(x, "detach"):
        import torch
        x = x.detach().to("cpu").to(torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def head_rows(*args, **kw):
    """Oracle rows of one head (see Oracle.head_rows)."""
    return _load().head_rows(*args, **kw)


def fwd(q1, q2, k1, k2, v, lam, *, causal: bool, lambda_init: float = 0.8,
        eps: float = 1e-5, pre_norm: bool = False):
    """Whole prefill: q*, k* [B,H,N*,d], v [B,H,Nk,dv], lam per head ([H] or
    scalar).  Returns fp64 [B,H,Nq,dv]."""
    q1, q2, k1, k2, v = (_f64(t) for t in (q1, q2, k1, k2, v))
    B, H, n_q, _ = q1.shape
    dv = v.shape[-1]
    lam = np.broadcast_to(_f64(lam).reshape(-1), (H,))
    out = np.empty((B, H, n_q, dv), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            out[b, h] = head_rows(q1[b, h], q2[b, h], k1[b, h], k2[b, h], v[b, h], None,
                                  causal=causal, lam=float(lam[h]),
                                  lambda_init=lambda_init, eps=eps, pre_norm=pre_norm)
    return out


def decode(q1, q2, k1, k2, v, lam, *, kv_len: Optional[int] = None,
           lambda_init: float = 0.8, eps: float = 1e-5, pre_norm: bool = False,
           heads: Optional[Sequence[tuple]] = None):
    """Decode: one query per (b, h) against the first kv_len cached keys, all
    visible.  q*: [B,H,d]; caches [B,H,L_cap,*].  ``heads`` restricts the work to
    a list of (b, h) pairs (the rest of the result is NaN).  Returns fp64
    [B,H,dv]."""
    B, H, d = tuple(q1.shape)
    dv = v.shape[-1]
    L = k1.shape[2] if kv_len is None else int(kv_len)
    lam = np.broadcast_to(_f64(lam).reshape(-1), (H,))
    out = np.full((B, H, dv), np.nan, dtype=np.float64)
    todo = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    for b, h in todo:
        o = head_rows(q1[b, h].reshape(1, d), q2[b, h].reshape(1, d),
                      k1[b, h, :L], k2[b, h, :L], v[b, h, :L], [0], causal=False,
                      lam=float(lam[h]), lambda_init=lambda_init, eps=eps, pre_norm=pre_norm)
        out[b, h] = o[0]
    return out


if __name__ == "__main__":  # pragma: no cover - manual build helper
    print(build(force=True))
    sys.exit(0)
