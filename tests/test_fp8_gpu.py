"""GPU parity of the FP8 query/key prefill (diffattn_fwd_fp8) with the fp64
oracle, through the C ABI, at head_dim 64 and 128.

The oracle decodes the very E4M3 codes the GPU reads, multiplies by the same
per-tensor scales and runs the forward oracle on them.  Products of E4M3
values are exact in fp32 and the rest of the path is the bf16 prefill's, so
the bf16 bound applies: every element within 1.5e-2 + 2e-2 |oracle|.
"""
import numpy as np
import pytest
import torch

import transformer_attention_diffattn_amd as da
import workloads
from oracle import fp8 as of8
from tests.test_parity_gpu import _sample_rows, assert_close

pytestmark = pytest.mark.gpu


# head_dim 64 (one-sweep kernel) and head_dim 128 (two-sweep kernel)
DIMS = [(64, 128), (128, 256)]
DIM_IDS = ["d64", "d128"]


def _w(B, H, nq, nk, causal, seed, dist="normal", lam=("uniform", 0.2, 0.9), d=64, dv=128):
    return workloads.Workload("fp8", "prefill", B=B, H=H, nq=nq, nk=nk, d=d, dv=dv,
                              dtype="bf16", causal=causal, dist=dist, lam=lam, seed=seed)


def _run(x, w, pre_norm=False):
    g = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    out = da.fwd_fp8(g["q1"], g["q2"], g["k1"], g["k2"], g["v"], x["scales"], g["lam"],
                     lambda_init=w.lambda_init, causal=w.causal, eps=w.eps, pre_norm=pre_norm)
    torch.cuda.synchronize()
    return out


def _full_compare(w, pre_norm=False):
    x = workloads.make_prefill_fp8(w)
    out = _run(x, w, pre_norm)
    ref = of8.fwd_fp8(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], x["scales"], x["lam"],
                      causal=w.causal, lambda_init=w.lambda_init, eps=w.eps, pre_norm=pre_norm)
    assert_close(out, ref, torch.bfloat16, f"fp8 {w}")


@pytest.mark.parametrize("dims", DIMS, ids=DIM_IDS)
@pytest.mark.parametrize("dist", ["normal", "student_t3"])
@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
@pytest.mark.parametrize("n", [1, 37, 129, 300])
def test_fp8_small(dims, dist, causal, n):
    _full_compare(_w(2, 3, n, n, causal, seed=800 + n, dist=dist, d=dims[0], dv=dims[1]))


@pytest.mark.parametrize("dims", DIMS, ids=DIM_IDS)
@pytest.mark.parametrize("nq,nk", [(70, 200), (1, 513), (300, 33)])
def test_fp8_rectangular_noncausal(dims, nq, nk):
    _full_compare(_w(1, 2, nq, nk, False, seed=810 + nq, d=dims[0], dv=dims[1]))


@pytest.mark.parametrize("dims", DIMS, ids=DIM_IDS)
def test_fp8_pre_norm_output(dims):
    _full_compare(_w(1, 2, 150, 150, True, seed=820, d=dims[0], dv=dims[1]), pre_norm=True)


def test_fp8_d128_near_cancellation():
    """lambda near 1 and heavy-tailed Q/K with 3 degrees of freedom (the
    large-head workload's regime): the two maps nearly agree, D is a small
    difference, and the GroupNorm scales it back up."""
    _full_compare(_w(2, 4, 333, 333, True, seed=825, dist="student_t3", lam=("const", 0.95),
                     d=128, dv=256))


@pytest.mark.parametrize("dims", DIMS, ids=DIM_IDS)
@pytest.mark.parametrize("B,H,n", [(1, 600, 200), (3, 100, 700)])
def test_fp8_many_items_per_workgroup(dims, B, H, n):
    """More query tiles than compute units: each workgroup walks several."""
    w = _w(B, H, n, n, True, seed=830 + H, d=dims[0], dv=dims[1])
    x = workloads.make_prefill_fp8(w)
    out = _run(x, w).cpu()
    rng = np.random.default_rng(3)
    for bh in rng.choice(B * H, 6, replace=False):
        b, h = divmod(int(bh), H)
        ref = of8.head_rows_fp8(x["q1"][b, h], x["q2"][b, h], x["k1"][b, h], x["k2"][b, h],
                                x["v"][b, h], x["scales"], None, causal=True,
                                lam=float(x["lam"][h]), lambda_init=w.lambda_init, eps=w.eps)
        assert_close(out[b, h], ref, torch.bfloat16, f"b{b} h{h}")


@pytest.mark.parametrize("dims", DIMS, ids=DIM_IDS)
def test_fp8_equals_bf16_path_on_exact_values(dims):
    """Codes scaled by powers of two are exact in bf16: the FP8 entry point
    and the bf16 one then compute the same scores, so the outputs agree to
    fp32 summation order (and both to the oracle)."""
    w = _w(2, 4, 260, 260, True, seed=840, d=dims[0], dv=dims[1])
    x = workloads.make_prefill_fp8(w)
    x["scales"] = [2.0 ** -7, 2.0 ** -6, 2.0 ** -8, 2.0 ** -7]
    deq = {n: torch.from_numpy(of8.dequantize(x[n], s)).to(torch.bfloat16).cuda()
           for n, s in zip(("q1", "q2", "k1", "k2"), x["scales"])}
    assert all(np.array_equal(deq[n].double().cpu().numpy(), of8.dequantize(x[n], s))
               for n, s in zip(("q1", "q2", "k1", "k2"), x["scales"]))
    out8 = _run(x, w).double().cpu()
    out16 = da.fwd(deq["q1"], deq["q2"], deq["k1"], deq["k2"], x["v"].cuda(), x["lam"].cuda(),
                   causal=True).double().cpu()
    # two bf16 roundings of nearly equal fp32 values: a few bf16 ulps apart
    assert float((out8 - out16).abs().max()) <= 2e-2
    ref = of8.fwd_fp8(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], x["scales"], x["lam"],
                      causal=True)
    assert_close(out8, ref, torch.bfloat16, "fp8")


def test_fp8_headline_shape_sampled():
    """The headline prefill shape (B4 H16 N2048 d64 dv128, causal) with its
    Q and K quantised per tensor: sampled rows of 12 heads."""
    w = workloads.get("causal_prefill_bf16")
    xg = workloads.make_prefill_fp8(w, device="cuda")
    out = da.fwd_fp8(xg["q1"], xg["q2"], xg["k1"], xg["k2"], xg["v"], xg["scales"], xg["lam"],
                     lambda_init=w.lambda_init, causal=True, eps=w.eps)
    torch.cuda.synchronize()
    out = out.cpu()
    x = {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in xg.items()}
    del xg
    rng = np.random.default_rng(11)
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    for i in sorted(rng.choice(len(heads), 12, replace=False)):
        b, h = heads[i]
        rows = _sample_rows(w.nq, rng)
        ref = of8.head_rows_fp8(x["q1"][b, h], x["q2"][b, h], x["k1"][b, h], x["k2"][b, h],
                                x["v"][b, h], x["scales"], rows, causal=True,
                                lam=float(x["lam"][h]), lambda_init=w.lambda_init, eps=w.eps)
        assert_close(out[b, h, rows], ref, torch.bfloat16, f"b{b} h{h}")


def test_fp8_large_head_shape_sampled():
    """The head_dim-128 workload (B2 H32 N8192 d128 dv256, causal, Student-t
    Q/K, lambda 0.95) with Q and K quantised per tensor: sampled rows of 10
    heads."""
    w = workloads.get("large_head_bf16")
    xg = workloads.make_prefill_fp8(w, device="cuda")
    out = da.fwd_fp8(xg["q1"], xg["q2"], xg["k1"], xg["k2"], xg["v"], xg["scales"], xg["lam"],
                     lambda_init=w.lambda_init, causal=True, eps=w.eps)
    torch.cuda.synchronize()
    out = out.cpu()
    x = {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in xg.items()}
    del xg
    torch.cuda.empty_cache()
    rng = np.random.default_rng(13)
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    for i in sorted(rng.choice(len(heads), 10, replace=False)):
        b, h = heads[i]
        rows = _sample_rows(w.nq, rng)
        ref = of8.head_rows_fp8(x["q1"][b, h], x["q2"][b, h], x["k1"][b, h], x["k2"][b, h],
                                x["v"][b, h], x["scales"], rows, causal=True,
                                lam=float(x["lam"][h]), lambda_init=w.lambda_init, eps=w.eps)
        assert_close(out[b, h, rows], ref, torch.bfloat16, f"b{b} h{h}")


def test_fp8_long_sequence_sampled():
    """The 32K causal workload quantised: sampled rows of 3 heads (needle rows
    included)."""
    w = workloads.get("long_needles_bf16")
    xg = workloads.make_prefill_fp8(w, device="cuda")
    out = da.fwd_fp8(xg["q1"], xg["q2"], xg["k1"], xg["k2"], xg["v"], xg["scales"], xg["lam"],
                     lambda_init=w.lambda_init, causal=True, eps=w.eps)
    torch.cuda.synchronize()
    out = out.cpu()
    x = {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in xg.items()}
    del xg
    torch.cuda.empty_cache()
    plans = workloads.needle_plan(w)
    rng = np.random.default_rng(12)
    for h in (0, 7, 15):
        rows = _sample_rows(w.nq, rng, plans[h][1])
        ref = of8.head_rows_fp8(x["q1"][0, h], x["q2"][0, h], x["k1"][0, h], x["k2"][0, h],
                                x["v"][0, h], x["scales"], rows, causal=True,
                                lam=float(x["lam"][h]), lambda_init=w.lambda_init, eps=w.eps)
        assert_close(out[0, h, rows], ref, torch.bfloat16, f"h{h}")


def test_fp8_rejects_unsupported():
    w = _w(1, 1, 16, 16, True, seed=850)
    x = workloads.make_prefill_fp8(w)
    g = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    args = (g["q1"], g["q2"], g["k1"], g["k2"], g["v"])
    with pytest.raises(ValueError):  # a scale that is not > 0
        da.fwd_fp8(*args, [1.0, 0.0, 1.0, 1.0], g["lam"])
    with pytest.raises(ValueError):  # non-finite scale
        da.fwd_fp8(*args, [1.0, 1.0, float("inf"), 1.0], g["lam"])
    with pytest.raises(ValueError):  # causal with Nq != Nk
        da.fwd_fp8(g["q1"][:, :, :8].contiguous(), g["q2"][:, :, :8].contiguous(), g["k1"],
                   g["k2"], g["v"], x["scales"], g["lam"], causal=True)
    q32 = torch.zeros((1, 1, 16, 32), dtype=torch.float8_e4m3fn, device="cuda")
    v64 = torch.zeros((1, 1, 16, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):  # head_dim 32 is not supported
        da.fwd_fp8(q32, q32, q32, q32, v64, x["scales"], g["lam"])
    q128 = torch.zeros((1, 1, 16, 128), dtype=torch.float8_e4m3fn, device="cuda")
    v128 = torch.zeros((1, 1, 16, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):  # head_dim 128 pairs with v_dim 256 only
        da.fwd_fp8(q128, q128, q128, q128, v128, x["scales"], g["lam"])


@pytest.mark.parametrize("dims,nk", [((64, 128), 8_400_013), ((128, 256), 4_200_017)],
                         ids=DIM_IDS)
def test_fp8_keys_past_2gib_per_head(dims, nk):
    """V of the (batch, head) spans more than 2 GiB: per-tile descriptors,
    millions of keys with a ragged tail, sampled rows."""
    w = _w(1, 1, 40, nk, False, seed=860, d=dims[0], dv=dims[1])
    xg = workloads.make_prefill_fp8(w, device="cuda")
    out = da.fwd_fp8(xg["q1"], xg["q2"], xg["k1"], xg["k2"], xg["v"], xg["scales"], xg["lam"],
                     lambda_init=w.lambda_init, causal=False, eps=w.eps)
    torch.cuda.synchronize()
    out = out.cpu()
    x = {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in xg.items()}
    del xg
    torch.cuda.empty_cache()
    rows = [0, 17, 39]
    ref = of8.head_rows_fp8(x["q1"][0, 0], x["q2"][0, 0], x["k1"][0, 0], x["k2"][0, 0],
                            x["v"][0, 0], x["scales"], rows, causal=False,
                            lam=float(x["lam"][0]), lambda_init=w.lambda_init, eps=w.eps)
    assert_close(out[0, 0, rows], ref, torch.bfloat16, "fp8 past 2 GiB")
