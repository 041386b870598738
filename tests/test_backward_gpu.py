"""GPU parity of the training pair (diffattn_fwd_train, diffattn_bwd) against
the fp64 oracle (oracle/backward.py and the forward oracle), through the C ABI.

Tolerances, from the arithmetic (bf16 operands, fp32 accumulation):
* out: identical to diffattn_fwd (same kernel, same order of operations);
* D (fp32 save): the forward's bf16 bound, 1.5e-2 + 2e-2 |oracle|;
* log-sum-exp: 4e-3 absolute -- the row sum l is formed over probabilities
  rounded to bf16 (2^-9 relative each), so log l is off by at most ~2^-9;
* dQ, dK, dV: each element within 0.12 rms + 0.03 |oracle| + 1e-3, rms taken
  over that gradient tensor (the 1e-3 floor, about 1% of these gradients'
  rms, covers gradients that vanish exactly, e.g. dQ of a row that sees one
  key).  Every gradient is a sum of products one of whose
  factors (P, dS or dD) was rounded to bf16, and is itself stored in bf16; the
  observed worst element is ~6% of the rms, a wrong sign, index or missing
  term gives errors of the order of the rms itself;
* dQ, dK, dV as whole tensors: ||gpu - oracle|| <= 2e-2 ||oracle|| (Frobenius).
  The rounding errors of the bf16 factors (at most 2^-9 relative each,
  2^-9/sqrt(3) rms) are independent from term to term, so over a tensor they
  add in quadrature and its relative error is a small multiple of 1.1e-3
  (observed up to 3.9e-3 over these tests, dominated by dS = P (dP - delta),
  where dP and delta nearly cancel); 2e-2 keeps a margin of ~5 over that, while a wrong
  sign, a dropped term or a mis-scaled factor moves the whole tensor by the
  size of that term, tens of percent.  The per-element bound above catches
  large errors in a few elements, this one small systematic ones;
* dlambda: 3e-2 relative (a sum over all rows of fp32 row terms).
* Heavy-tailed inputs (Student-t with 3 degrees of freedom, the large-head
  workload's): a few keys carry entries a hundred times the typical one, and
  a gradient element can be a sum of large terms that nearly cancel (seen: a
  dQ element of 0.03 made of terms near 10, one key's entry at -135).  A bf16
  factor of each term is rounded (dD, the weights, dS), so the error of such
  an element scales with the sum of its terms' absolute values, M
  (oracle.backward.head_magnitudes), not with the tensor's rms: those tests
  add 2^-7 M (four roundings of 2^-9) to the per-element bound.  The observed
  worst is ~0.3 2^-9 M; the Frobenius bound is unchanged.
"""
import numpy as np
import pytest
import torch

import oracle
import transformer_attention_diffattn_amd as da
import workloads
from oracle import backward as obw

pytestmark = pytest.mark.gpu

NAMES = ("dq1", "dq2", "dk1", "dk2", "dv")


def _all_heads(x):
    B, H = x["q1"].shape[:2]
    return [(b, h) for b in range(B) for h in range(H)]


def _inputs(B, H, n, d, dv, causal, seed, dist="normal"):
    w = workloads.Workload("bwd", "prefill", B=B, H=H, nq=n, nk=n, d=d, dv=dv, dtype="bf16",
                           causal=causal, dist=dist, lam=("uniform", 0.2, 0.9), seed=seed)
    x = workloads.make_prefill(w)
    g = torch.Generator().manual_seed(seed + 1)
    dout = torch.randn((B, H, n, dv), generator=g, dtype=torch.float64).to(torch.bfloat16)
    return w, x, dout


def _gpu(x, dout, causal, pre_norm):
    g = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    out, d_save, lse = da.fwd_train(g["q1"], g["q2"], g["k1"], g["k2"], g["v"], g["lam"],
                                    causal=causal, pre_norm=pre_norm)
    grads = da.bwd(g["q1"], g["q2"], g["k1"], g["k2"], g["v"], g["lam"], dout.cuda(), d_save,
                   lse, causal=causal, pre_norm=pre_norm)
    plain = da.fwd(g["q1"], g["q2"], g["k1"], g["k2"], g["v"], g["lam"], causal=causal,
                   pre_norm=pre_norm)
    torch.cuda.synchronize()
    return out, d_save, lse, grads, plain


def _check_grad(name, got, ref, mag=None):
    """mag (heavy-tailed inputs only): oracle.backward.head_magnitudes of the
    same elements, adding 2^-7 mag to the bound (see the module docstring)."""
    got = got.detach().double().cpu().numpy()
    ref = np.asarray(ref, dtype=np.float64)
    assert np.all(np.isfinite(got)), f"{name}: non-finite"
    rms = float(np.sqrt((ref ** 2).mean()))
    err = np.abs(got - ref)
    bound = 0.12 * rms + 0.03 * np.abs(ref) + 1e-3
    if mag is not None:
        bound = bound + 2.0 ** -7 * np.asarray(mag, dtype=np.float64)
    i = np.unravel_index(np.argmax(err / bound), err.shape)
    assert np.all(err <= bound), (f"{name}: element {i} gpu {got[i]:.5f} oracle {ref[i]:.5f} "
                                  f"(rms {rms:.4f}, max err {err.max():.4f})")
    norm = float(np.linalg.norm(ref))
    fro = float(np.linalg.norm(got - ref))
    if norm > 1e-6:
        print(f"[grad] {name}: relative Frobenius error {fro / norm:.2e}")
        assert fro <= 2e-2 * norm, f"{name}: relative Frobenius error {fro / norm:.3e} > 2e-2"
    else:  # a gradient that vanishes exactly (one visible key)
        assert fro <= 1e-3 * np.sqrt(ref.size)


def _dlam_noise(x, dout, causal, pre_norm, heads_b):
    """Per head: sqrt(sum over rows of (sum_c |O_2 dD|)^2), the size of the
    terms whose bf16 rounding (dD enters the kernels in bf16) sets dlambda's
    error floor."""
    lam = x["lam"].double().numpy()
    out = {}
    for (b, h) in heads_b:
        _, a = obw.head_dlambda_terms(x["q1"][b, h], x["q2"][b, h], x["k1"][b, h], x["k2"][b, h],
                                      x["v"][b, h], float(lam[h]), dout[b, h], causal=causal,
                                      pre_norm=pre_norm)
        out[h] = out.get(h, 0.0) + float((a ** 2).sum())
    return {h: np.sqrt(v) for h, v in out.items()}


def _check_dlam(got, ref, noise):
    """dlambda sums per-row terms of both signs that can cancel (for one
    visible key it is exactly 0: dD is orthogonal to D), so beside 3e-2
    relative it gets 2^-6 of the terms' size (about 4x bf16's 2^-8 per row,
    summed as a random walk) as an absolute floor."""
    got = got.detach().double().cpu().numpy()
    floor = np.array([noise[h] for h in sorted(noise)]) * 2.0 ** -6
    assert np.all(np.abs(got - ref) <= 3e-2 * np.abs(ref) + floor), (got, ref, floor)


DIMS = [(32, 64), (64, 128), (128, 256)]
DIM_IDS = ["d32", "d64", "d128"]


@pytest.mark.parametrize("d,dv", DIMS, ids=DIM_IDS)
@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
@pytest.mark.parametrize("n", [1, 7, 64, 129, 300])
def test_backward_small(d, dv, causal, n):
    w, x, dout = _inputs(2, 3, n, d, dv, causal, seed=500 + n + d)
    out, d_save, lse, grads, plain = _gpu(x, dout, causal, False)
    assert torch.equal(out, plain), "training forward output differs from the forward"
    D = oracle.fwd(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], x["lam"], causal=causal,
                   pre_norm=True)
    Dg = d_save.double().cpu().numpy()
    assert np.all(np.abs(Dg - D) <= 1.5e-2 + 2e-2 * np.abs(D)), "saved D"
    for k, (q, kk) in enumerate((("q1", "k1"), ("q2", "k2"))):
        ref_lse = obw.lse(x[q], x[kk], causal=causal)
        assert np.abs(lse[k].double().cpu().numpy() - ref_lse).max() <= 4e-3, f"lse of map {k + 1}"
    ref = obw.backward(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], x["lam"], dout, causal=causal)
    for name, gg, rr in zip(NAMES, grads[:5], ref[:5]):
        _check_grad(f"{name} d{d} n{n} causal={causal}", gg, rr)
    _check_dlam(grads[5], ref[5], _dlam_noise(x, dout, causal, False, _all_heads(x)))


@pytest.mark.parametrize("d,dv,causal", [(64, 128, True), (32, 64, False), (128, 256, True)])
def test_backward_pre_norm_output(d, dv, causal):
    w, x, dout = _inputs(1, 2, 150, d, dv, causal, seed=77)
    out, d_save, lse, grads, plain = _gpu(x, dout, causal, True)
    assert torch.equal(out, plain)
    ref = obw.backward(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], x["lam"], dout, causal=causal,
                       pre_norm=True)
    for name, gg, rr in zip(NAMES, grads[:5], ref[:5]):
        _check_grad(name, gg, rr)
    _check_dlam(grads[5], ref[5], _dlam_noise(x, dout, causal, True, _all_heads(x)))


@pytest.mark.parametrize("d,dv,nq,nk", [(64, 128, 70, 200), (128, 256, 70, 200),
                                         (128, 256, 300, 33)])
def test_backward_rectangular_noncausal(d, dv, nq, nk):
    B, H = 1, 2
    w = workloads.Workload("bwd", "prefill", B=B, H=H, nq=nq, nk=nk, d=d, dv=dv, dtype="bf16",
                           causal=False, lam=("uniform", 0.2, 0.9), seed=91)
    x = workloads.make_prefill(w)
    dout = torch.randn((B, H, nq, dv), generator=torch.Generator().manual_seed(92),
                       dtype=torch.float64).to(torch.bfloat16)
    out, d_save, lse, grads, plain = _gpu(x, dout, False, False)
    ref = obw.backward(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], x["lam"], dout, causal=False)
    for name, gg, rr in zip(NAMES, grads[:5], ref[:5]):
        _check_grad(name, gg, rr)
    _check_dlam(grads[5], ref[5], _dlam_noise(x, dout, False, False, _all_heads(x)))


@pytest.mark.parametrize("d,dv", [(64, 128), (128, 256)], ids=["d64", "d128"])
def test_backward_deterministic(d, dv):
    w, x, dout = _inputs(1, 4, 300, d, dv, True, seed=93)
    a = _gpu(x, dout, True, False)[3]
    b = _gpu(x, dout, True, False)[3]
    for ga, gb in zip(a, b):
        assert torch.equal(ga, gb)


def test_backward_rejects_unsupported_and_small_workspace():
    w, x, dout = _inputs(1, 1, 16, 32, 128, True, seed=94)
    g = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    with pytest.raises(ValueError):
        da.fwd_train(g["q1"], g["q2"], g["k1"], g["k2"], g["v"], g["lam"], causal=True)
    w, x, dout = _inputs(1, 2, 64, 64, 128, True, seed=95)
    g = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    out, d_save, lse = da.fwd_train(g["q1"], g["q2"], g["k1"], g["k2"], g["v"], g["lam"],
                                    causal=True)
    small = torch.empty((16,), dtype=torch.uint8, device="cuda")
    with pytest.raises(da.DiffAttnError):
        da.bwd(g["q1"], g["q2"], g["k1"], g["k2"], g["v"], g["lam"], dout.cuda(), d_save, lse,
               causal=True, workspace=small)


def test_backward_headline_shape_sampled_heads():
    """The headline prefill shape (B4 H16 N2048 d64 dv128, causal): the GPU
    computes every head; three heads are checked in full, and dlambda of two
    heads over the whole batch."""
    w = workloads.get("causal_prefill_bf16")
    x = workloads.make_prefill(w)
    dout = torch.randn((w.B, w.H, w.nq, w.dv), generator=torch.Generator().manual_seed(96),
                       dtype=torch.float64).to(torch.bfloat16)
    out, d_save, lse, grads, plain = _gpu(x, dout, True, False)
    grads = [g.cpu() for g in grads]
    lam = x["lam"].double().numpy()
    for (b, h) in [(0, 0), (1, 7), (3, 15)]:
        r = obw.head_backward(x["q1"][b, h], x["q2"][b, h], x["k1"][b, h], x["k2"][b, h],
                              x["v"][b, h], float(lam[h]), dout[b, h], causal=True)
        for name, gg, rr in zip(NAMES, grads[:5], r[:5]):
            _check_grad(f"{name} b{b} h{h}", gg[b, h], rr)
    for h in (3, 12):
        tot = sum(obw.head_backward(x["q1"][b, h], x["q2"][b, h], x["k1"][b, h], x["k2"][b, h],
                                    x["v"][b, h], float(lam[h]), dout[b, h], causal=True)[5]
                  for b in range(w.B))
        noise = _dlam_noise(x, dout, True, False, [(b, h) for b in range(w.B)])
        _check_dlam(grads[5][h:h + 1], np.array([tot]), noise)


def test_backward_large_head_near_cancellation():
    """The head_dim-128 regime of the large-head workload at a size the
    oracle checks in full: Student-t Q/K with 3 degrees of freedom, lambda
    0.95 (the two maps nearly agree), causal, three query tiles with a ragged
    end."""
    w = workloads.Workload("bwd", "prefill", B=1, H=3, nq=333, nk=333, d=128, dv=256,
                           dtype="bf16", causal=True, dist="student_t3", lam=("const", 0.95),
                           seed=97)
    x = workloads.make_prefill(w)
    dout = torch.randn((1, 3, 333, 256), generator=torch.Generator().manual_seed(98),
                       dtype=torch.float64).to(torch.bfloat16)
    out, d_save, lse, grads, plain = _gpu(x, dout, True, False)
    assert torch.equal(out, plain)
    ref = obw.backward(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], x["lam"], dout, causal=True)
    mags = [np.stack([obw.head_magnitudes(x["q1"][0, h], x["q2"][0, h], x["k1"][0, h],
                                          x["k2"][0, h], x["v"][0, h], 0.95, dout[0, h],
                                          causal=True)[i] for h in range(3)])[None]
            for i in range(5)]
    for name, gg, rr, mm in zip(NAMES, grads[:5], ref[:5], mags):
        _check_grad(name, gg, rr, mm)
    _check_dlam(grads[5], ref[5], _dlam_noise(x, dout, True, False, _all_heads(x)))


def test_backward_large_head_shape_sampled_heads():
    """The large-head workload (B2 H32 N8192 d128 dv256, causal, Student-t,
    lambda 0.95): the GPU computes every head; two heads are checked in full
    and dlambda of one head over the batch."""
    w = workloads.get("large_head_bf16")
    x = workloads.make_prefill(w)
    dout = torch.randn((w.B, w.H, w.nq, w.dv), generator=torch.Generator().manual_seed(99),
                       dtype=torch.float64).to(torch.bfloat16)
    out, d_save, lse, grads, plain = _gpu(x, dout, True, False)
    grads = [g.cpu() for g in grads]
    del out, d_save, lse, plain
    torch.cuda.empty_cache()
    lam = x["lam"].double().numpy()
    for (b, h) in [(0, 5), (1, 30)]:
        hx = (x["q1"][b, h], x["q2"][b, h], x["k1"][b, h], x["k2"][b, h], x["v"][b, h],
              float(lam[h]), dout[b, h])
        r = obw.head_backward(*hx, causal=True)
        m = obw.head_magnitudes(*hx, causal=True)
        for name, gg, rr, mm in zip(NAMES, grads[:5], r[:5], m):
            _check_grad(f"{name} b{b} h{h}", gg[b, h], rr, mm)
        del r, m
    h = 17
    tot = sum(obw.head_dlambda_terms(x["q1"][b, h], x["q2"][b, h], x["k1"][b, h], x["k2"][b, h],
                                     x["v"][b, h], float(lam[h]), dout[b, h], causal=True)[0].sum()
              for b in range(w.B))
    noise = _dlam_noise(x, dout, True, False, [(b, h) for b in range(w.B)])
    _check_dlam(grads[5][h:h + 1], np.array([tot]), noise)
