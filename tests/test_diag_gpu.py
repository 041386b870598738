"""GPU parity of the map diagnostics (diffattn_diag) against the fp64 oracle.

Tolerances, from the arithmetic:
* row max: the largest scaled score, formed from exact bf16 products summed
  in fp32 (d terms): within 1e-4 (1 + |oracle|);
* needle weights: exp(S - lse) with fp32 scores and the training forward's
  log-sum-exp, which is off by at most ~2^-8 (its row sum is taken over
  bf16-rounded probabilities): within 1e-2 relative + 1e-6.
"""
import numpy as np
import pytest
import torch

import transformer_attention_diffattn_amd as da
import workloads
from oracle import backward as obw

pytestmark = pytest.mark.gpu


def _needle_arrays(w):
    plans = workloads.needle_plan(w)
    nq = torch.tensor(np.stack([p[1] for p in plans]).reshape(w.B, w.H, -1), dtype=torch.int32)
    nk = torch.tensor(np.stack([p[0] for p in plans]).reshape(w.B, w.H, -1), dtype=torch.int32)
    return nq, nk


def _check_rowmax(got, x, w, heads=None, rows=None):
    got = got.double().cpu().numpy()
    heads = heads or [(b, h) for b in range(w.B) for h in range(w.H)]
    for (b, h) in heads:
        for m, (q, k) in enumerate((("q1", "k1"), ("q2", "k2"))):
            ref = obw.head_row_max(x[q][b, h], x[k][b, h], causal=w.causal)
            g = got[m, b, h]
            if rows is not None:
                ref, g = ref[rows], g[rows]
            assert np.all(np.abs(g - ref) <= 1e-4 * (1 + np.abs(ref))), (m, b, h)


@pytest.mark.parametrize("d,dv", [(32, 64), (64, 128), (128, 256)], ids=["d32", "d64", "d128"])
@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
@pytest.mark.parametrize("n", [1, 37, 129, 300])
def test_row_max_small(d, dv, causal, n):
    w = workloads.Workload("diag", "prefill", B=2, H=3, nq=n, nk=n, d=d, dv=dv, dtype="bf16",
                           causal=causal, dist="student_t3", lam=("const", 0.5), seed=700 + n + d)
    x = workloads.make_prefill(w)
    g = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    rm, nd = da.diag(g["q1"], g["q2"], g["k1"], g["k2"], g["v"], causal=causal)
    assert nd is None
    _check_rowmax(rm, x, w)


@pytest.mark.parametrize("d,dv", [(32, 64), (64, 128)], ids=["d32", "d64"])
def test_needles_small(d, dv):
    w = workloads.Workload("diag", "prefill", B=2, H=2, nq=600, nk=600, d=d, dv=dv, dtype="bf16",
                           causal=True, needles=8, lam=("const", 0.6), seed=710 + d)
    x = workloads.make_prefill(w)
    g = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    _, _, lse = da.fwd_train(g["q1"], g["q2"], g["k1"], g["k2"], g["v"], g["lam"], causal=True)
    nq, nk = _needle_arrays(w)
    rm, nd = da.diag(g["q1"], g["q2"], g["k1"], g["k2"], g["v"], causal=True, lse=lse,
                     needle_q=nq, needle_k=nk)
    nd = nd.double().cpu().numpy()
    for b in range(w.B):
        for h in range(w.H):
            ref = obw.head_needles(x["q1"][b, h], x["q2"][b, h], x["k1"][b, h], x["k2"][b, h],
                                   nq[b, h].numpy(), nk[b, h].numpy(), causal=True)
            assert np.all(np.abs(nd[b, h] - ref) <= 1e-2 * np.abs(ref) + 1e-6), (b, h)
    _check_rowmax(rm, x, w)


def test_needle_index_out_of_range_gives_nan():
    w = workloads.Workload("diag", "prefill", B=1, H=1, nq=64, nk=64, d=64, dv=128, dtype="bf16",
                           causal=True, lam=("const", 0.5), seed=720)
    x = workloads.make_prefill(w)
    g = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    _, _, lse = da.fwd_train(g["q1"], g["q2"], g["k1"], g["k2"], g["v"], g["lam"], causal=True)
    nq = torch.tensor([[[10, 64, -1, 20]]], dtype=torch.int32)
    nk = torch.tensor([[[3, 2, 1, 99]]], dtype=torch.int32)
    _, nd = da.diag(g["q1"], g["q2"], g["k1"], g["k2"], g["v"], causal=True, lse=lse,
                    needle_q=nq, needle_k=nk, row_max=False)
    nd = nd.cpu().numpy()[0, 0]
    assert np.all(np.isfinite(nd[0])) and np.all(np.isnan(nd[1:]))


def test_long_needles_workload():
    """The 32K needle workload: every needle of every head, and the row
    maxima of the needles' query rows and a few others."""
    w = workloads.get("long_needles_bf16")
    xg = workloads.make_prefill(w, device="cuda")
    _, _, lse = da.fwd_train(xg["q1"], xg["q2"], xg["k1"], xg["k2"], xg["v"], xg["lam"],
                             causal=True)
    nq, nk = _needle_arrays(w)
    rm, nd = da.diag(xg["q1"], xg["q2"], xg["k1"], xg["k2"], xg["v"], causal=True, lse=lse,
                     needle_q=nq, needle_k=nk)
    torch.cuda.synchronize()
    nd = nd.double().cpu().numpy()
    rm = rm.double().cpu().numpy()
    x = {k: xg[k].cpu() for k in ("q1", "q2", "k1", "k2")}
    del xg, lse
    torch.cuda.empty_cache()
    for h in range(w.H):
        q1, q2, k1, k2 = (x[k][0, h] for k in ("q1", "q2", "k1", "k2"))
        ref = obw.head_needles(q1, q2, k1, k2, nq[0, h].numpy(), nk[0, h].numpy(), causal=True)
        assert np.all(np.abs(nd[0, h] - ref) <= 1e-2 * np.abs(ref) + 1e-6), h
        rows = np.unique(np.concatenate([nq[0, h].numpy(), [0, 1, 100, 4095, w.nq - 1]]))
        for m, (q, k) in enumerate(((q1, k1), (q2, k2))):
            ref = obw.head_row_max(q, k, causal=True, rows=rows)
            assert np.all(np.abs(rm[m, 0, h, rows] - ref) <= 1e-4 * (1 + np.abs(ref))), (m, h)
