"""Pins of the fp64 backward oracle (oracle/backward.py) to facts other than
itself (CPU only).

* torch's autograd, differentiating the forward assembled from library
  routines only -- scaled_dot_product_attention for each softmax map (the
  DiffAttn formula, iloveeagents.com "Mathematical Formula") and group_norm
  with one group per head for step 4 on llmbytes.dev -- must give the same six
  gradients, causal and not, with and without the normalisation;
* central finite differences of the C forward oracle along random directions
  (every input tensor and lambda) must match the directional derivatives;
* exp(S - lse) applied to V must equal scaled_dot_product_attention, and each
  such row must sum to one;
* lambda = 0 leaves map 2 without any gradient.

A separate test plants mistakes in copies of the backward oracle and requires
each copy to fail the autograd comparison.
"""
import os
import types

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import backward as obw

SRC = os.path.join(os.path.dirname(oracle.__file__), "backward.py")


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _case(nq, d, dv, seed):
    return dict(q1=_rand((nq, d), seed), q2=_rand((nq, d), seed + 1), k1=_rand((nq, d), seed + 2),
                k2=_rand((nq, d), seed + 3), v=_rand((nq, dv), seed + 4),
                dout=_rand((nq, dv), seed + 5))


def _autograd(c, lam, causal, lambda_init, eps, pre_norm):
    t = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True) for k, v in c.items()
         if k != "dout"}
    lam_t = torch.tensor(lam, dtype=torch.float64, requires_grad=True)
    o1 = F.scaled_dot_product_attention(t["q1"][None], t["k1"][None], t["v"][None], is_causal=causal)[0]
    o2 = F.scaled_dot_product_attention(t["q2"][None], t["k2"][None], t["v"][None], is_causal=causal)[0]
    D = o1 - lam_t * o2
    y = D if pre_norm else (1.0 - lambda_init) * F.group_norm(D, 1, eps=eps)
    (y * torch.tensor(c["dout"])).sum().backward()
    return [t[k].grad.numpy() for k in ("q1", "q2", "k1", "k2", "v")] + [float(lam_t.grad)]


def check_against_autograd(bw):
    for (nq, d, dv, lam, causal, pre_norm, seed) in [
            (9, 4, 6, 0.5, False, False, 1), (9, 4, 6, 0.5, True, False, 2),
            (17, 8, 16, 0.8, True, False, 3), (17, 8, 16, -0.3, False, True, 4),
            (12, 6, 10, 1.2, True, True, 5), (1, 4, 6, 0.7, True, False, 6)]:
        c = _case(nq, d, dv, seed)
        got = bw.head_backward(c["q1"], c["q2"], c["k1"], c["k2"], c["v"], lam, c["dout"],
                               causal=causal, lambda_init=0.8, eps=1e-5, pre_norm=pre_norm)
        want = _autograd(c, lam, causal, 0.8, 1e-5, pre_norm)
        for name, g, w in zip(("dq1", "dq2", "dk1", "dk2", "dv", "dlam"), got, want):
            np.testing.assert_allclose(g, w, rtol=1e-9, atol=1e-11,
                                       err_msg=f"{name} nq={nq} causal={causal} pre_norm={pre_norm}")


def test_backward_matches_autograd_of_library_forward():
    check_against_autograd(obw)


@pytest.mark.parametrize("causal,pre_norm", [(True, False), (False, False), (True, True)])
def test_backward_matches_finite_differences_of_c_oracle(causal, pre_norm):
    nq, d, dv, lam = 11, 5, 7, 0.6
    c = _case(nq, d, dv, 40)

    def loss(x, lam_):
        out = oracle.head_rows(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], None, causal=causal,
                               lam=lam_, lambda_init=0.8, eps=1e-5, pre_norm=pre_norm)
        return float((out * c["dout"]).sum())

    grads = obw.head_backward(c["q1"], c["q2"], c["k1"], c["k2"], c["v"], lam, c["dout"],
                              causal=causal, pre_norm=pre_norm)
    rng = np.random.default_rng(41)
    h = 1e-6
    for i, name in enumerate(("q1", "q2", "k1", "k2", "v")):
        u = rng.standard_normal(c[name].shape)
        xp = dict(c); xp[name] = c[name] + h * u
        xm = dict(c); xm[name] = c[name] - h * u
        fd = (loss(xp, lam) - loss(xm, lam)) / (2 * h)
        an = float((grads[i] * u).sum())
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)
    fd = (loss(c, lam + h) - loss(c, lam - h)) / (2 * h)
    assert abs(fd - grads[5]) <= 1e-6 * max(1.0, abs(grads[5])), ("lambda", fd, grads[5])


@pytest.mark.parametrize("causal", [True, False])
def test_lse_reproduces_standard_attention(causal):
    q, k, v = _rand((13, 8), 50), _rand((13, 8), 51), _rand((13, 5), 52)
    lse = obw.head_lse(q, k, causal=causal)
    s = (q @ k.T) / np.sqrt(8)
    if causal:
        s = np.where(np.tril(np.ones((13, 13))) > 0, s, -np.inf)
    w = np.exp(s - lse[:, None])
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=1e-13)
    t = [torch.tensor(x)[None] for x in (q, k, v)]
    want = F.scaled_dot_product_attention(*t, is_causal=causal)[0].numpy()
    np.testing.assert_allclose(w @ v, want, rtol=1e-12, atol=1e-13)


def test_lambda_zero_leaves_map_two_without_gradient():
    c = _case(10, 4, 6, 60)
    g = obw.head_backward(c["q1"], c["q2"], c["k1"], c["k2"], c["v"], 0.0, c["dout"], causal=True)
    assert np.all(g[1] == 0) and np.all(g[3] == 0)


def test_batch_wrapper_sums_dlambda_over_batch():
    rng = np.random.default_rng(70)
    B, H, N, d, dv = 2, 3, 6, 4, 5
    x = {k: rng.standard_normal((B, H, N, dv if k in ("v", "dout") else d))
         for k in ("q1", "q2", "k1", "k2", "v", "dout")}
    lam = np.array([0.2, 0.5, 0.9])
    r = obw.backward(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], lam, x["dout"], causal=True)
    for h in range(H):
        tot = sum(obw.head_backward(x["q1"][b, h], x["q2"][b, h], x["k1"][b, h], x["k2"][b, h],
                                    x["v"][b, h], lam[h], x["dout"][b, h], causal=True)[5]
                  for b in range(B))
        assert r[5][h] == pytest.approx(tot, rel=1e-14)


def test_dlambda_terms_sum_to_dlambda():
    c = _case(14, 6, 9, 80)
    for pre_norm in (False, True):
        r, a = obw.head_dlambda_terms(c["q1"], c["q2"], c["k1"], c["k2"], c["v"], 0.7, c["dout"],
                                      causal=True, pre_norm=pre_norm)
        full = obw.head_backward(c["q1"], c["q2"], c["k1"], c["k2"], c["v"], 0.7, c["dout"],
                                 causal=True, pre_norm=pre_norm)[5]
        assert r.sum() == pytest.approx(full, rel=1e-12)
        assert np.all(a >= np.abs(r))


def _round_bits(x, bits):
    """x rounded to nearest with `bits` significand bits (8: bf16's)."""
    m, e = np.frexp(np.asarray(x, dtype=np.float64))
    return np.ldexp(np.round(m * 2.0 ** bits) / 2.0 ** bits, e)


def _emulated_backward(c, lam, causal, pre_norm, bits=8):
    """The gradient as a kernel with `bits`-bit factors and exact sums forms
    it: the forward's row sums over rounded probabilities (so the saved
    log-sum-exp and D carry their rounding), dD rounded, dS and the combined
    weights W = A_1 - lambda A_2 rounded, every gradient rounded at the end."""
    r = lambda x: _round_bits(x, bits)
    q1, q2, k1, k2, v, dout = (c[k] for k in ("q1", "q2", "k1", "k2", "v", "dout"))
    tau = 1.0 / np.sqrt(q1.shape[1])
    a, o = [], []
    for q, k in ((q1, k1), (q2, k2)):
        s = obw._scores(q, k, causal)
        m = s.max(axis=1, keepdims=True)
        pr = r(np.exp(s - m))
        l = pr.sum(axis=1, keepdims=True)
        o.append(pr @ v / l)
        a.append(np.exp(s - (m + np.log(l))))
    dD = r(obw._norm_backward(o[0] - lam * o[1], dout, 0.8, 1e-5, pre_norm))
    da = dD @ v.T
    g = []
    for ak, ck, q, k in ((a[0], 1.0, q1, k1), (a[1], -lam, q2, k2)):
        delta = (ak * da).sum(axis=1, keepdims=True)
        ds = r(ck * ak * (da - delta))
        g.append((r(tau * (ds @ k)), r(tau * (ds.T @ q))))
    dv = r(r(a[0] - lam * a[1]).T @ dD)
    return g[0][0], g[1][0], g[0][1], g[1][1], dv


def _error_ratios(c, lam, causal, pre_norm, bits):
    """max over elements of |emulated - exact| / (4 u R + u |exact|), u = 2^-8,
    and of |emulated - exact| / (u R), per gradient."""
    u = 2.0 ** -8
    args = (c["q1"], c["q2"], c["k1"], c["k2"], c["v"], lam, c["dout"])
    exact = obw.head_backward(*args, causal=causal, pre_norm=pre_norm)[:5]
    scales = obw.head_error_scales(*args, causal=causal, pre_norm=pre_norm)
    emu = _emulated_backward(c, lam, causal, pre_norm, bits)
    out = []
    for e, x, rr in zip(emu, exact, scales):
        err = np.abs(e - x)
        out.append(((err / (4 * u * rr + u * np.abs(x) + 1e-300)).max(),
                    (err / (u * rr + 1e-300)).max()))
    return out


@pytest.mark.parametrize("causal,pre_norm", [(True, False), (False, False), (True, True)])
def test_error_scales_bound_an_emulated_bf16_backward(causal, pre_norm):
    """head_error_scales against the errors a bf16-factor computation really
    makes (emulated exactly on the CPU): every element of every gradient
    within 4 u R + u |g|, for normal and heavy-tailed (Student-t, 3 degrees
    of freedom) inputs and lambda near one; and R is not vacuous: the worst
    element of each gradient uses at least 2% of u R."""
    for seed, heavy, lam in ((70, False, 0.5), (71, True, 0.95), (72, True, 0.3)):
        c = _case(48, 16, 32, seed)
        if heavy:
            rng = np.random.default_rng(seed + 7)
            for k in ("q1", "q2", "k1", "k2", "v"):
                c[k] = rng.standard_t(3, size=c[k].shape) / np.sqrt(3.0)
        for name, (ratio, used) in zip(("dq1", "dq2", "dk1", "dk2", "dv"),
                                       _error_ratios(c, lam, causal, pre_norm, 8)):
            assert ratio <= 1.0, f"{name} seed {seed}: {ratio:.3f} of the bound"
            assert used >= 0.02, f"{name} seed {seed}: worst error only {used:.4f} u R"


def test_error_scales_catch_a_coarser_computation():
    """With factors rounded to 4 significand bits instead of 8 (a kernel that
    lost half of them somewhere), the same bound fails on every gradient."""
    c = _case(48, 16, 32, 73)
    for name, (ratio, _) in zip(("dq1", "dq2", "dk1", "dk2", "dv"),
                                _error_ratios(c, 0.5, True, False, 4)):
        assert ratio > 1.0, f"{name}: {ratio:.3f}"


MUTANTS = [
    ("dv = a1.T @ dD - lam * (a2.T @ dD)", "dv = a1.T @ dD + lam * (a2.T @ dD)"),
    ("da2 = -lam * da1", "da2 = lam * da1"),
    ("- xhat * (g * xhat).mean(axis=1, keepdims=True)) / sigma",
     "+ xhat * (g * xhat).mean(axis=1, keepdims=True)) / sigma"),
    ("sigma = np.sqrt(((D - mu) ** 2).mean(axis=1, keepdims=True) + eps)",
     "sigma = np.sqrt(((D - mu) ** 2).mean(axis=1, keepdims=True)) + eps"),
    ("g = (1.0 - lambda_init) * dout", "g = dout"),
    ("dq1, dq2 = tau * (ds1 @ k1), tau * (ds2 @ k2)", "dq1, dq2 = ds1 @ k1, tau * (ds2 @ k2)"),
    ("dlam = -float((o2 * dD).sum())", "dlam = float((o2 * dD).sum())"),
    ("ds1 = a1 * (da1 - (a1 * da1).sum(axis=1, keepdims=True))", "ds1 = a1 * da1"),
    ("dk1, dk2 = tau * (ds1.T @ q1), tau * (ds2.T @ q2)",
     "dk1, dk2 = tau * (ds1.T @ q2), tau * (ds2.T @ q1)"),
    ("g - g.mean(axis=1, keepdims=True)", "g"),
    ("o1, o2 = a1 @ v, a2 @ v", "o1, o2 = a1 @ v, a1 @ v"),
]


@pytest.mark.parametrize("old,new", MUTANTS, ids=[str(i) for i in range(len(MUTANTS))])
def test_planted_backward_mistake_is_caught(old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, old
    mod = types.ModuleType("mutant_backward")
    exec(compile(src.replace(old, new), "mutant_backward", "exec"), mod.__dict__)
    with pytest.raises(AssertionError):
        check_against_autograd(mod)


@pytest.mark.parametrize("causal", [True, False])
def test_diagnostics_match_library_softmax_and_max(causal):
    n, d = 40, 16
    q1, q2, k1, k2 = (_rand((n, d), 90 + i) for i in range(4))
    nk = np.array([3, 17, 25, 39])
    nq = np.array([5, 30, 25, 39])  # each at or after its key
    got = obw.head_needles(q1, q2, k1, k2, nq, nk, causal=causal)
    mask = torch.tril(torch.ones(n, n, dtype=torch.bool)) if causal else None
    for col, (q, k) in enumerate(((q1, k1), (q2, k2))):
        s = torch.tensor(q) @ torch.tensor(k).T / np.sqrt(d)
        if causal:
            s = s.masked_fill(~mask, float("-inf"))
        a = torch.softmax(s, dim=-1).numpy()
        np.testing.assert_allclose(got[:, col], a[nq, nk], rtol=1e-12)
        np.testing.assert_allclose(got[:, 2 + col], a[nq][:, nk].sum(axis=1), rtol=1e-12)
        np.testing.assert_allclose(obw.head_row_max(q, k, causal=causal),
                                   torch.amax(s, dim=-1).numpy(), rtol=1e-13)
    # row subsets agree with the whole rows
    sub = np.array([0, 7, 39])
    np.testing.assert_allclose(obw.head_row_max(q1, k1, causal=causal, rows=sub),
                               obw.head_row_max(q1, k1, causal=causal)[sub], rtol=0)
    # the top logit never exceeds the row's log-sum-exp, nor falls more than
    # log(visible keys) below it
    lse = obw.head_lse(q1, k1, causal=causal)
    mx = obw.head_row_max(q1, k1, causal=causal)
    vis = np.arange(1, n + 1) if causal else np.full(n, n)
    assert np.all(mx <= lse + 1e-12) and np.all(mx >= lse - np.log(vis) - 1e-12)
