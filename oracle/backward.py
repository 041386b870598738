"""fp64 CPU oracle for the gradient of the Differential Attention operator.

TEST INFRASTRUCTURE ONLY, like the rest of this package: only the tests, the
smoke check and the benchmark's CPU-baseline leg may use it, and it never
imports the GPU library.

The pages treat the operator as trained: lambda is a learnable scalar
(iloveeagents.com, "Mathematical Formula"), and the GroupNorm with the
(1 - lambda_init) scale of step 4 on llmbytes.dev ("How Differential Attention
Cancels Common-Mode Noise") is there for stable gradient flow.  The gradient
below is the chain rule taken through that same forward definition, written
out step by step in the forward's notation (per batch entry b and head h,
scale tau = 1/sqrt(d), c = 1 - lambda_init):

  forward:  S_k = tau Q_k K_k^T (causal: keys after the query masked),
            A_k = softmax_rows(S_k),  O_k = A_k V,  D = O_1 - lambda O_2,
            y = c (D - mu) / sigma   (mu, sigma^2 + eps: mean and population
            variance of each row of D over its dv channels);
  backward, given dy:
            dD = (1/sigma) (g - mean(g) - xhat mean(g xhat)),  g = c dy,
                 xhat = (D - mu)/sigma   (dD = dy when the output is D itself);
            dV = A_1^T dD - lambda A_2^T dD;
            dA_1 = dD V^T,  dA_2 = -lambda dD V^T;
            dS_k = A_k * (dA_k - rowsum(A_k * dA_k))     (softmax Jacobian);
            dQ_k = tau dS_k K_k,  dK_k = tau dS_k^T Q_k;
            dlambda = -sum(O_2 * dD)  (summed over rows; over b for the head).

Dense N x N maps are materialised, so this is for the small shapes the tests
use.  ``head_lse`` gives the natural-log log-sum-exp of each score row, the
per-row softmax statistic a training forward keeps for the backward.

Two diagnostics of the maps follow the quantities the pages report for trained
models -- the share of attention that lands on planted "needles"
(llmbytes.dev, "Benchmark Performance", multi-needle retrieval) and the top
attention logit (same page, "Solving the Quantization Crisis"):
``head_needles`` (each needle's weight in A1 and A2, and its query row's total
weight on all the head's needle keys) and ``head_row_max`` (each row's largest
scaled score).
"""
from __future__ import annotations

import numpy as np


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):
        import torch
        x = x.detach().to("cpu").to(torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _scores(q, k, causal: bool) -> np.ndarray:
    s = (q @ k.T) / np.sqrt(q.shape[1])
    if causal:
        nq, nk = s.shape
        s = np.where(np.arange(nk)[None, :] <= np.arange(nq)[:, None], s, -np.inf)
    return s


def _softmax_rows(s: np.ndarray) -> np.ndarray:
    e = np.exp(s - s.max(axis=1, keepdims=True))
    return e / e.sum(axis=1, keepdims=True)


def _norm_backward(D, dout, lambda_init: float, eps: float, pre_norm: bool) -> np.ndarray:
    """dD from dy through y = (1 - lambda_init) (D - mu) / sigma, row-wise
    (dD = dy when the output is D itself)."""
    if pre_norm:
        return dout
    mu = D.mean(axis=1, keepdims=True)
    sigma = np.sqrt(((D - mu) ** 2).mean(axis=1, keepdims=True) + eps)
    xhat = (D - mu) / sigma
    g = (1.0 - lambda_init) * dout
    return (g - g.mean(axis=1, keepdims=True)
            - xhat * (g * xhat).mean(axis=1, keepdims=True)) / sigma


def head_lse(q, k, *, causal: bool) -> np.ndarray:
    """log(sum_j exp(S_ij)) of each row of one map's scores, fp64 [Nq]."""
    s = _scores(_f64(q), _f64(k), causal)
    m = s.max(axis=1)
    return m + np.log(np.exp(s - m[:, None]).sum(axis=1))


def head_backward(q1, q2, k1, k2, v, lam: float, dout, *, causal: bool,
                  lambda_init: float = 0.8, eps: float = 1e-5, pre_norm: bool = False):
    """Gradients of sum(dout * out) for one head.  Returns
    (dq1, dq2, dk1, dk2, dv, dlam) in fp64; dlam is this head's scalar."""
    q1, q2, k1, k2, v, dout = (_f64(t) for t in (q1, q2, k1, k2, v, dout))
    d = q1.shape[1]
    tau = 1.0 / np.sqrt(d)
    a1 = _softmax_rows(_scores(q1, k1, causal))
    a2 = _softmax_rows(_scores(q2, k2, causal))
    o1, o2 = a1 @ v, a2 @ v
    D = o1 - lam * o2
    dD = _norm_backward(D, dout, lambda_init, eps, pre_norm)
    dv = a1.T @ dD - lam * (a2.T @ dD)
    da1 = dD @ v.T
    da2 = -lam * da1
    ds1 = a1 * (da1 - (a1 * da1).sum(axis=1, keepdims=True))
    ds2 = a2 * (da2 - (a2 * da2).sum(axis=1, keepdims=True))
    dq1, dq2 = tau * (ds1 @ k1), tau * (ds2 @ k2)
    dk1, dk2 = tau * (ds1.T @ q1), tau * (ds2.T @ q2)
    dlam = -float((o2 * dD).sum())
    return dq1, dq2, dk1, dk2, dv, dlam


def head_error_scales(q1, q2, k1, k2, v, lam: float, dout, *, causal: bool,
                      lambda_init: float = 0.8, eps: float = 1e-5, pre_norm: bool = False):
    """Per gradient element of one head, the error a computation with bf16
    factors can leave in it, in units of the format's unit roundoff u: the
    root-sum-square over the element's terms of each term's error scale,
    plus the part that cannot average out.  The model (fp32 sums, factors
    rounded to bf16, every rounding off by at most u relative):
      * dD: each entry off by u (|dD_ic| + s_i), s_i = rms_c dD_ic (its own
        rounding, and what it inherits through the normalisation's row
        statistics from the saved forward D);
      * dA_ij = sum_c dD_ic V_jc: off by u E_ij, E_ij = sqrt(sum_c
        (|dD_ic| + s_i)^2 V_jc^2) (independent errors over c);
      * A recomputed from the saved log-sum-exp: off by u relative, the same
        factor along a row (the row sum it comes from adds up rounded terms);
      * delta_i = sum_j A_ij dA_ij: off by u e_i, e_i = sqrt(sum_j A_ij^2
        E_ij^2) + |delta_i|;
      * dS_ij = A_ij (dA_ij - delta_i), rounded: off by u T_ij,
        T_ij = 2 |dS_ij| + A_ij (E_ij + e_i);
      * dQ_k,ic = tau c_k sum_j dS_ij K_jc: tau c_k (sqrt(sum_j T_ij^2
        K_jc^2) + |delta_i| |sum_j A_ij K_jc|), the last term being the row's
        common error of A, which does not average out over j;
        dK_k,jc: tau c_k sqrt(sum_i T_ij^2 Q_ic^2);
      * dV_jc = sum_i W_ij dD_ic, W = A_1 - lambda A_2 rounded:
        sqrt(sum_i ((A_1 + |lambda| A_2)_ij (3 |dD_ic| + s_i))^2);
    with c_1 = 1, c_2 = |lambda|.  The term errors are independent roundings,
    each of standard deviation at most u/sqrt(3) times its bound, so an
    element's error has a standard deviation of at most u R / sqrt(3) and a
    bound of 4 u R sits ~7 standard deviations out; the gradient's own
    rounding to bf16 adds u |g|.  Returns (rq1, rq2, rk1, rk2, rv)."""
    q1, q2, k1, k2, v, dout = (_f64(t) for t in (q1, q2, k1, k2, v, dout))
    d = q1.shape[1]
    tau = 1.0 / np.sqrt(d)
    a1 = _softmax_rows(_scores(q1, k1, causal))
    a2 = _softmax_rows(_scores(q2, k2, causal))
    dD = _norm_backward(a1 @ v - lam * (a2 @ v), dout, lambda_init, eps, pre_norm)
    s = np.sqrt((dD * dD).mean(axis=1, keepdims=True))
    e_dd = np.abs(dD) + s
    da = dD @ v.T
    E = np.sqrt((e_dd * e_dd) @ (v * v).T)
    out = []
    for a, c, q, k in ((a1, 1.0, q1, k1), (a2, abs(lam), q2, k2)):
        delta = (a * da).sum(axis=1, keepdims=True)
        e_delta = np.sqrt(((a * E) ** 2).sum(axis=1, keepdims=True)) + np.abs(delta)
        T = 2.0 * np.abs(a * (da - delta)) + a * (E + e_delta)
        rq = tau * c * (np.sqrt((T * T) @ (k * k)) + np.abs(delta) * np.abs(a @ k))
        rk = tau * c * np.sqrt((T * T).T @ (q * q))
        out.append((rq, rk))
    w = a1 + abs(lam) * a2
    tv = 3.0 * np.abs(dD) + s
    rv = np.sqrt((w * w).T @ (tv * tv))
    return out[0][0], out[1][0], out[0][1], out[1][1], rv


def head_dlambda_terms(q1, q2, k1, k2, v, lam: float, dout, *, causal: bool,
                       lambda_init: float = 0.8, eps: float = 1e-5, pre_norm: bool = False):
    """Per query row of one head: the row's share -O_2 . dD of dlambda and the
    sum over channels of |O_2 dD| (the size of the terms that cancel in it)."""
    q1, q2, k1, k2, v, dout = (_f64(t) for t in (q1, q2, k1, k2, v, dout))
    a1 = _softmax_rows(_scores(q1, k1, causal))
    a2 = _softmax_rows(_scores(q2, k2, causal))
    o2 = a2 @ v
    dD = _norm_backward(a1 @ v - lam * o2, dout, lambda_init, eps, pre_norm)
    return -(o2 * dD).sum(axis=1), np.abs(o2 * dD).sum(axis=1)


def backward(q1, q2, k1, k2, v, lam, dout, *, causal: bool, lambda_init: float = 0.8,
             eps: float = 1e-5, pre_norm: bool = False):
    """Whole batch: q*, k* [B,H,N,d], v and dout [B,H,N,dv], lam [H] (or a
    scalar).  Returns fp64 (dq1, dq2, dk1, dk2, dv [B,H,N,*], dlam [H])."""
    q1, q2, k1, k2, v, dout = (_f64(t) for t in (q1, q2, k1, k2, v, dout))
    B, H = q1.shape[:2]
    lam = np.broadcast_to(_f64(lam).reshape(-1), (H,))
    grads = [np.zeros_like(t) for t in (q1, q2, k1, k2, v)]
    dlam = np.zeros(H)
    for b in range(B):
        for h in range(H):
            r = head_backward(q1[b, h], q2[b, h], k1[b, h], k2[b, h], v[b, h], float(lam[h]),
                              dout[b, h], causal=causal, lambda_init=lambda_init, eps=eps,
                              pre_norm=pre_norm)
            for gbuf, gval in zip(grads, r[:5]):
                gbuf[b, h] = gval
            dlam[h] += r[5]
    return (*grads, dlam)


def lse(q, k, *, causal: bool) -> np.ndarray:
    """head_lse over a batch: q, k [B,H,N,d] -> fp64 [B,H,Nq]."""
    q, k = _f64(q), _f64(k)
    B, H = q.shape[:2]
    out = np.empty((B, H, q.shape[2]))
    for b in range(B):
        for h in range(H):
            out[b, h] = head_lse(q[b, h], k[b, h], causal=causal)
    return out


def _score_rows(q, k, rows, causal: bool) -> np.ndarray:
    """Scaled scores of the listed query rows against every key (-inf where
    the causal mask hides the key), [len(rows), Nk]."""
    rows = np.asarray(rows, dtype=np.int64)
    s = (q[rows] @ k.T) / np.sqrt(q.shape[1])
    if causal:
        s = np.where(np.arange(k.shape[0])[None, :] <= rows[:, None], s, -np.inf)
    return s


def head_row_max(q, k, *, causal: bool, rows=None) -> np.ndarray:
    """Largest scaled score S_ij = q_i . k_j / sqrt(d) over the keys row i sees
    (the row's top attention logit), fp64, for every row or the listed ones."""
    q, k = _f64(q), _f64(k)
    rows = np.arange(q.shape[0]) if rows is None else rows
    return _score_rows(q, k, rows, causal).max(axis=1)


def head_needles(q1, q2, k1, k2, needle_q, needle_k, *, causal: bool) -> np.ndarray:
    """For needle r (query needle_q[r], key needle_k[r]) of one head: A1 and A2
    at (query, key), and the query row's total A1 and A2 weight on all of the
    head's needle keys it sees.  Only the needles' query rows are formed.
    fp64 [n, 4]."""
    q1, q2, k1, k2 = (_f64(t) for t in (q1, q2, k1, k2))
    nq = np.asarray(needle_q, dtype=np.int64)
    nk = np.asarray(needle_k, dtype=np.int64)
    a1 = _softmax_rows(_score_rows(q1, k1, nq, causal))
    a2 = _softmax_rows(_score_rows(q2, k2, nq, causal))
    r = np.arange(len(nq))
    return np.stack([a1[r, nk], a2[r, nk], a1[:, nk].sum(axis=1), a2[:, nk].sum(axis=1)], axis=1)
