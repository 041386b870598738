"""GPU parity of the training pair (diffattn_fwd_train, diffattn_bwd) against
the fp64 oracle (oracle/backward.py and the forward oracle), through the C ABI.

Tolerances, from the arithmetic (bf16 operands, fp32 accumulation):
* out: identical to diffattn_fwd (same kernel, same order of operations);
* D (fp32 save): the forward's bf16 bound, 1.5e-2 + 2e-2 |oracle|;
* log-sum-exp: 4e-3 absolute -- the row sum l is formed over probabilities
  rounded to bf16 (2^-8 relative each at most), so log l is off by at most
  ~2^-8;
* dQ, dK, dV, element by element: |gpu - oracle| <= 4 u R + u |oracle| + 1e-6,
  u = 2^-8 (bf16's unit roundoff), R from oracle.backward.head_error_scales:
  the root-sum-square over the element's terms of the error each term can
  carry when its factors (dD, the weights, dS) are bf16 and the sums fp32,
  plus the row-common part of the recomputed weights' error.  The term
  errors are independent roundings, so an element's error has a standard
  deviation of at most u R / sqrt(3) and 4 u R is ~7 of them; u |oracle| is
  the gradient's own rounding to bf16, and 1e-6 covers gradients that
  vanish exactly.  The model is pinned on the CPU against an exact emulation
  of a bf16-factor backward (tests/test_oracle_backward_pins.py), which it
  bounds with room to spare and which breaks it once the factors lose half
  their bits.  It holds for normal and heavy-tailed inputs alike: on the GPU
  the worst element of these tests uses 0.36 of the bound (~1.4 u R), and the
  bound is 2-4x tighter than a fixed fraction of the tensor's rms
  (0.12 rms + 0.03 |oracle|) at the median element;
* dQ, dK, dV as whole tensors: ||gpu - oracle|| <= 2e-2 ||oracle|| (Frobenius).
  The rounding errors are independent from term to term, so over a tensor
  they add in quadrature and its relative error is a small multiple of 2^-8
  (observed up to 3.9e-3 over these tests); a wrong sign, a dropped term or a
  mis-scaled factor moves the whole tensor by the size of that term, tens of
  percent.  The per-element bound catches errors in a few elements, this one
  small systematic ones;
* dlambda: 3e-2 relative (a sum over all rows of fp32 row terms).
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


U = 2.0 ** -8  # bf16's unit roundoff


def _error_scales(x, dout, causal, pre_norm=False, heads=None):
    """oracle.backward.head_error_scales for every head (or the listed
    (b, h) heads, stacked in that order), one array per gradient."""
    lam = x["lam"].double().numpy()
    heads = heads or _all_heads(x)
    per = [obw.head_error_scales(x["q1"][b, h], x["q2"][b, h], x["k1"][b, h], x["k2"][b, h],
                                 x["v"][b, h], float(lam[h]), dout[b, h], causal=causal,
                                 pre_norm=pre_norm) for (b, h) in heads]
    if heads == _all_heads(x):
        B, H = x["q1"].shape[:2]
        return [np.stack([p[i] for p in per]).reshape(B, H, *per[0][i].shape) for i in range(5)]
    return [np.stack([p[i] for p in per]) for i in range(5)]


def _check_grad(name, got, ref, scale):
    """Every element within 4 u R + u |oracle| + 1e-6, R = scale (see the
    module docstring), and the whole tensor within 2e-2 (Frobenius)."""
    got = got.detach().double().cpu().numpy()
    ref = np.asarray(ref, dtype=np.float64)
    assert np.all(np.isfinite(got)), f"{name}: non-finite"
    err = np.abs(got - ref)
    bound = 4 * U * np.asarray(scale, dtype=np.float64) + U * np.abs(ref) + 1e-6
    i = np.unravel_index(np.argmax(err / bound), err.shape)
    print(f"[grad] {name}: worst element at {err[i] / bound[i]:.3f} of its bound")
    assert np.all(err <= bound), (f"{name}: element {i} gpu {got[i]:.5f} oracle {ref[i]:.5f} "
                                  f"bound {bound[i]:.5f} (max err {err.max():.4f})")
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
    for name, gg, rr, sc in zip(NAMES, grads[:5], ref[:5], _error_scales(x, dout, causal)):
        _check_grad(f"{name} d{d} n{n} causal={causal}", gg, rr, sc)
    _check_dlam(grads[5], ref[5], _dlam_noise(x, dout, causal, False, _all_heads(x)))


@pytest.mark.parametrize("d,dv,causal", [(64, 128, True), (32, 64, False), (128, 256, True)])
def test_backward_pre_norm_output(d, dv, causal):
    w, x, dout = _inputs(1, 2, 150, d, dv, causal, seed=77)
    out, d_save, lse, grads, plain = _gpu(x, dout, causal, True)
    assert torch.equal(out, plain)
    ref = obw.backward(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], x["lam"], dout, causal=causal,
                       pre_norm=True)
    for name, gg, rr, sc in zip(NAMES, grads[:5], ref[:5], _error_scales(x, dout, causal, True)):
        _check_grad(name, gg, rr, sc)
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
    for name, gg, rr, sc in zip(NAMES, grads[:5], ref[:5], _error_scales(x, dout, False)):
        _check_grad(name, gg, rr, sc)
    _check_dlam(grads[5], ref[5], _dlam_noise(x, dout, False, False, _all_heads(x)))


@pytest.mark.parametrize("d,dv", [(64, 128), (128, 256)], ids=["d64", "d128"])
def test_backward_deterministic(d, dv):
    w, x, dout = _inputs(1, 4, 300, d, dv, True, seed=93)
    a = _gpu(x, dout, True, False)[3]
    b = _gpu(x, dout, True, False)[3]
    for ga, gb in zip(a, b):
        assert torch.equal(ga, gb)


# No stray writes: every gradient goes into the middle of a guard-banded
# buffer through the C ABI, with ragged query and key counts (333 = 2 x 128 +
# 77 keys, 10 x 32 + 13 queries); the results equal the binding's and the
# bands stay untouched.
@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
@pytest.mark.parametrize("d,dv", DIMS, ids=DIM_IDS)
def test_backward_canary(d, dv, causal):
    import ctypes
    w, x, dout = _inputs(1, 3, 333, d, dv, causal, seed=97)
    g = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    dout = dout.cuda()
    out, d_save, lse = da.fwd_train(g["q1"], g["q2"], g["k1"], g["k2"], g["v"], g["lam"],
                                    causal=causal)
    ref = da.bwd(g["q1"], g["q2"], g["k1"], g["k2"], g["v"], g["lam"], dout, d_save, lse,
                 causal=causal)
    guard = 2048
    bufs, views = [], []
    for t in (g["q1"], g["q2"], g["k1"], g["k2"], g["v"]):
        b = torch.full((guard + t.numel() + guard,), 7.0, dtype=t.dtype, device=t.device)
        bufs.append(b)
        views.append(b[guard:guard + t.numel()].view(t.shape))
    dl_buf = torch.full((guard + 3 + guard,), 7.0, dtype=torch.float32, device="cuda")
    dlam = dl_buf[guard:guard + 3]
    B, H, N = 1, 3, 333
    dims = da.Dims(B, H, N, N, d, dv, da._dtype_code(g["q1"]), 1e-5, da._flags(False, False))
    need = int(da.lib().diffattn_bwd_workspace_size(ctypes.byref(dims)))
    ws = torch.empty((max(need, 16),), dtype=torch.uint8, device="cuda")
    lam_t = da._lam_tensor(g["lam"], H, g["q1"].device)
    st = da.lib().diffattn_bwd(g["q1"].data_ptr(), g["q2"].data_ptr(), g["k1"].data_ptr(),
                               g["k2"].data_ptr(), g["v"].data_ptr(), lam_t.data_ptr(), 0.8,
                               int(causal), dout.data_ptr(), d_save.data_ptr(), lse.data_ptr(),
                               *[v_.data_ptr() for v_ in views], dlam.data_ptr(), ws.data_ptr(),
                               ws.numel(), ctypes.byref(dims), da._stream_ptr(g["q1"].device))
    assert st == 0, st
    torch.cuda.synchronize()
    for name, got, want, b in zip(("dq1", "dq2", "dk1", "dk2", "dv"), views, ref[:5], bufs):
        assert torch.equal(got, want), name
        assert bool((b[:guard] == 7.0).all()), f"{name}: write before the output"
        assert bool((b[guard + got.numel():] == 7.0).all()), f"{name}: write past the output"
    assert torch.equal(dlam, ref[5])
    assert bool((dl_buf[:guard] == 7.0).all()) and bool((dl_buf[guard + 3:] == 7.0).all())


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
        hx = (x["q1"][b, h], x["q2"][b, h], x["k1"][b, h], x["k2"][b, h], x["v"][b, h],
              float(lam[h]), dout[b, h])
        r = obw.head_backward(*hx, causal=True)
        sc = obw.head_error_scales(*hx, causal=True)
        for name, gg, rr, ss in zip(NAMES, grads[:5], r[:5], sc):
            _check_grad(f"{name} b{b} h{h}", gg[b, h], rr, ss)
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
    for name, gg, rr, sc in zip(NAMES, grads[:5], ref[:5], _error_scales(x, dout, True)):
        _check_grad(name, gg, rr, sc)
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
        sc = obw.head_error_scales(*hx, causal=True)
        for name, gg, rr, ss in zip(NAMES, grads[:5], r[:5], sc):
            _check_grad(f"{name} b{b} h{h}", gg[b, h], rr, ss)
        del r, sc
    h = 17
    tot = sum(obw.head_dlambda_terms(x["q1"][b, h], x["q2"][b, h], x["k1"][b, h], x["k2"][b, h],
                                     x["v"][b, h], float(lam[h]), dout[b, h], causal=True)[0].sum()
              for b in range(w.B))
    noise = _dlam_noise(x, dout, True, False, [(b, h) for b in range(w.B)])
    _check_dlam(grads[5][h:h + 1], np.array([tot]), noise)
