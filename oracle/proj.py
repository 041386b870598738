"""fp64 CPU oracle for the split projections that feed Differential Attention.

TEST INFRASTRUCTURE ONLY, like the rest of this package: only the tests, the
smoke check and the benchmark's CPU-baseline leg may use it, and it never
imports the GPU library.

Step 1 of the operator (llmbytes.dev, "How Differential Attention Cancels
Common-Mode Noise"): for every head the input is projected into two queries
Q1, Q2, two keys K1, K2 and one value V.  The pages give no weight layout.
The reading taken here: one weight matrix W [H * (4 d + dv)][d_model] in the
layout of a linear layer (output features by input features), output feature
f belonging to head h = f // S (S = 4 d + dv) at offset o = f - h S, and the
offsets of a head in the order Q1 [0, d), Q2 [d, 2 d), K1 [2 d, 3 d),
K2 [3 d, 4 d), V [4 d, 4 d + dv).  With X [B][N][d_model] (tokens of each
batch entry in order), Y = X W^T, and the five outputs are Y's columns in
head-major order [B][H][N][channels] -- the layout the attention operator
reads.
"""
from __future__ import annotations

import numpy as np

SEGMENTS = ("q1", "q2", "k1", "k2", "v")


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):
        import torch
        x = x.detach().to("cpu").to(torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def segment_of(o: int, d: int, dv: int):
    """(output name, channel) of offset o within a head's 4 d + dv features."""
    if o < 0 or o >= 4 * d + dv:
        raise ValueError("offset outside the head")
    if o < 4 * d:
        return SEGMENTS[o // d], o % d
    return "v", o - 4 * d


def _split(y: np.ndarray, B: int, N: int, H: int, d: int, dv: int) -> dict:
    """Columns of y [B*N][H*(4d+dv)] into the five head-major outputs."""
    S = 4 * d + dv
    out = {n: np.empty((B, H, N, dv if n == "v" else d)) for n in SEGMENTS}
    yb = y.reshape(B, N, H, S)
    for o in range(S):
        name, ch = segment_of(o, d, dv)
        out[name][:, :, :, ch] = yb[:, :, :, o].transpose(0, 2, 1)
    return out


def qkv_proj(x, w, *, heads: int, head_dim: int, v_dim: int) -> dict:
    """x [B][N][d_model], w [H*(4d+dv)][d_model]: fp64 q1, q2, k1, k2 [B,H,N,d]
    and v [B,H,N,dv] of Y = X W^T."""
    x, w = _f64(x), _f64(w)
    B, N, dm = x.shape
    if w.shape != (heads * (4 * head_dim + v_dim), dm):
        raise ValueError("weight shape does not match heads, head_dim, v_dim, d_model")
    y = x.reshape(B * N, dm) @ w.T
    return _split(y, B, N, heads, head_dim, v_dim)


def qkv_proj_abs(x, w, *, heads: int, head_dim: int, v_dim: int) -> dict:
    """The same with |x| and |w|: for each output the sum over the
    contraction of |x_k w_k|, the scale of its summation error."""
    return qkv_proj(np.abs(_f64(x)), np.abs(_f64(w)), heads=heads, head_dim=head_dim,
                    v_dim=v_dim)
