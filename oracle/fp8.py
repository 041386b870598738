"""fp64 CPU oracle for the Differential Attention forward with FP8 (E4M3)
query and key operands.

TEST INFRASTRUCTURE ONLY, like the rest of this package: only the tests, the
smoke check and the benchmark's CPU-baseline leg may use it, and it never
imports the GPU library.

The pages name FP8, beside INT8 and INT4, among the low-bit formats that
differential attention makes easier to use, because its attention logits
carry far smaller outliers (llmbytes.dev, "Solving the Quantization Crisis").
They give no quantisation scheme.  The reading taken here is the plainest one:
each of Q1, Q2, K1, K2 is stored as OCP FP8 E4M3 codes with one fp32 scale per
tensor, element = scale * value(code); V and the output stay bf16, and the
operator itself is unchanged.  So this oracle decodes the codes exactly to
fp64, multiplies by the scales, and hands the result to the forward oracle
(the DiffAttn formula and the GroupNorm step, see ``oracle/__init__.py``).

E4M3 as the OCP 8-bit floating point specification defines it: bit 7 sign,
bits 6..3 exponent e (bias 7), bits 2..0 mantissa m;
  e = 0:          (-1)^s * (m / 8) * 2^(1 - 7)          (zero and subnormals)
  e = 1..15:      (-1)^s * (1 + m / 8) * 2^(e - 7)
  e = 15, m = 7:  NaN (no infinities; the largest finite magnitude is 448).
"""
from __future__ import annotations

import numpy as np

import oracle


def e4m3_value(codes) -> np.ndarray:
    """Exact fp64 values of E4M3 codes (any integer array, or a torch uint8 /
    float8_e4m3fn tensor); NaN for the two NaN codes."""
    if hasattr(codes, "detach"):
        import torch
        t = codes.detach().to("cpu")
        if t.dtype != torch.uint8:
            t = t.view(torch.uint8)
        codes = t.numpy()
    c = np.asarray(codes).astype(np.int64) & 0xFF
    s = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 7
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** (1 - 7), (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


def dequantize(codes, scale: float) -> np.ndarray:
    """scale * value(code), fp64."""
    return float(scale) * e4m3_value(codes)


def fwd_fp8(q1, q2, k1, k2, v, scales, lam, *, causal: bool, lambda_init: float = 0.8,
            eps: float = 1e-5, pre_norm: bool = False):
    """Whole prefill from E4M3 codes q1, q2 [B,H,Nq,d], k1, k2 [B,H,Nk,d] with
    per-tensor scales (q1, q2, k1, k2), v [B,H,Nk,dv].  fp64 [B,H,Nq,dv]."""
    x = [dequantize(c, s) for c, s in zip((q1, q2, k1, k2), scales)]
    return oracle.fwd(*x, v, lam, causal=causal, lambda_init=lambda_init, eps=eps,
                      pre_norm=pre_norm)


def head_rows_fp8(q1, q2, k1, k2, v, scales, rows, *, causal: bool, lam: float,
                  lambda_init: float = 0.8, eps: float = 1e-5, pre_norm: bool = False):
    """Listed query rows of one head from E4M3 codes (see fwd_fp8)."""
    x = [dequantize(c, s) for c, s in zip((q1, q2, k1, k2), scales)]
    return oracle.head_rows(*x, v, rows, causal=causal, lam=lam, lambda_init=lambda_init,
                            eps=eps, pre_norm=pre_norm)
