"""GPU parity of the fused projections (diffattn_qkv_proj) with the fp64
oracle (oracle/proj.py), through the C ABI.

Tolerance, from the arithmetic: the products of bf16 inputs are exact in
fp32 and summed in fp32 over d_model terms, then rounded once to bf16.  So
every element is within 2^-8 |oracle| (the rounding) plus d_model 2^-24
sum_k |x_k w_k| (a worst-case bound on fp32 summation), the second term
taken from the oracle's sums of absolute products.
"""
import numpy as np
import pytest
import torch

import oracle
import transformer_attention_diffattn_amd as da
import workloads
from oracle import proj as oproj
from tests.test_parity_gpu import assert_close

pytestmark = pytest.mark.gpu

NAMES = ("q1", "q2", "k1", "k2", "v")


def _w(B, N, H, d, dv, seed):
    return workloads.Workload("proj", "prefill", B=B, H=H, nq=N, nk=N, d=d, dv=dv, dtype="bf16",
                              causal=True, seed=seed)


def _check(got, x, wt, H, d, dv, rows=None):
    ref = oproj.qkv_proj(x, wt, heads=H, head_dim=d, v_dim=dv)
    absr = oproj.qkv_proj_abs(x, wt, heads=H, head_dim=d, v_dim=dv)
    dm = x.shape[-1]
    for name, g in zip(NAMES, got):
        g = g.detach().double().cpu().numpy()
        r, a = ref[name], absr[name]
        if rows is not None:
            g, r, a = g[:, :, rows], r[:, :, rows], a[:, :, rows]
        assert np.all(np.isfinite(g)), name
        bound = 2.0 ** -8 * np.abs(r) + dm * 2.0 ** -24 * a + 1e-30
        err = np.abs(g - r)
        i = np.unravel_index(np.argmax(err / bound), err.shape)
        assert np.all(err <= bound), (f"{name}: element {i} gpu {g[i]:.6f} oracle {r[i]:.6f} "
                                      f"bound {bound[i]:.2e}")


@pytest.mark.parametrize("d,dv", [(32, 64), (64, 128), (128, 256)], ids=["d32", "d64", "d128"])
@pytest.mark.parametrize("B,N,dm", [(1, 1, 32), (2, 37, 96), (1, 300, 256), (3, 129, 160)])
def test_proj_small(d, dv, B, N, dm):
    H = 3
    w = _w(B, N, H, d, dv, seed=900 + N + d)
    p = workloads.make_proj(w, d_model=dm)
    got = da.qkv_proj(p["x"].cuda(), p["w"].cuda(), H, d, dv)
    torch.cuda.synchronize()
    _check(got, p["x"], p["w"], H, d, dv)


def test_proj_ragged_tiles():
    """Token and feature counts that are not multiples of the 256 x 256 tile,
    and several tiles in both directions."""
    B, N, H, d, dv, dm = 2, 333, 5, 32, 64, 320
    w = _w(B, N, H, d, dv, seed=950)
    p = workloads.make_proj(w, d_model=dm)
    got = da.qkv_proj(p["x"].cuda(), p["w"].cuda(), H, d, dv)
    torch.cuda.synchronize()
    _check(got, p["x"], p["w"], H, d, dv)


def test_proj_headline_shape_sampled():
    """The headline attention shape's projections: B4 N2048 H16 d64 dv128
    from d_model 2048 (= H dv); every output of 40 sampled tokens."""
    w = workloads.get("causal_prefill_bf16")
    p = workloads.make_proj(w, device="cuda")
    got = da.qkv_proj(p["x"], p["w"], w.H, w.d, w.dv)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(5).choice(w.nq, 40, replace=False))
    rows = np.unique(np.concatenate([rows, [0, 255, 256, w.nq - 1]]))
    x = p["x"].cpu()
    _check([g.cpu() for g in got], x, p["w"].cpu(), w.H, w.d, w.dv, rows=rows)


def test_proj_then_attention_matches_oracle_chain():
    """Projections feeding the forward: the library's two calls against the
    oracle's projection followed by the forward oracle, on bf16-rounded
    projections (the forward reads bf16)."""
    B, N, H, d, dv = 2, 200, 4, 64, 128
    w = _w(B, N, H, d, dv, seed=960)
    p = workloads.make_proj(w)
    q1, q2, k1, k2, v = da.qkv_proj(p["x"].cuda(), p["w"].cuda(), H, d, dv)
    lam = torch.tensor([0.3, 0.5, 0.7, 0.2], dtype=torch.float32)
    out = da.fwd(q1, q2, k1, k2, v, lam.cuda(), causal=True)
    torch.cuda.synchronize()
    # the projections against the projection oracle, then the forward oracle
    # on the bf16 projections the GPU produced (what the forward read)
    _check((q1, q2, k1, k2, v), p["x"], p["w"], H, d, dv)
    ref = oracle.fwd(q1.cpu(), q2.cpu(), k1.cpu(), k2.cpu(), v.cpu(), lam, causal=True)
    assert_close(out, ref, torch.bfloat16, "projection then attention")


def test_proj_rejects_unsupported():
    x = torch.zeros((1, 4, 48), dtype=torch.bfloat16, device="cuda")
    wt = torch.zeros((2 * 256, 48), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):  # d_model not a multiple of 32
        da.qkv_proj(x, wt, 2, 32, 128)
    x = torch.zeros((1, 4, 64), dtype=torch.bfloat16, device="cuda")
    wt = torch.zeros((2 * (4 * 48 + 96), 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):  # head_dim 48 is not supported
        da.qkv_proj(x, wt, 2, 48, 96)
