"""Pins of the fp64 oracle to facts other than itself (CPU only).

Each check ties one part of the operator to something the pages or the
mathematics fix independently of the oracle's own code:

* lambda = 0 reduces the operator to standard softmax attention, the formula
  both iloveeagents.com ("Detail") and llmbytes.dev ("The Mathematical Flaw in
  Standard Softmax Attention") print -- checked against torch's
  scaled_dot_product_attention (a library routine), causal and not;
* a zero Q1 makes map 1 uniform, which isolates map 2 and the sign of lambda;
* every softmax row sums to 1, so each row of A1 - lambda*A2 sums to 1 - lambda
  (llmbytes.dev steps 2-3), and V = ones gives D = 1 - lambda;
* identical maps with lambda = 1 cancel exactly (the common-mode argument of
  "Why Subtraction Induces Clean Sparsity");
* the GroupNorm-and-scale step (llmbytes.dev step 4) equals torch's group_norm
  with one group per head, and its output moments have a closed form;
* the causal row 0, swap symmetry at lambda = 1, equal keys, hand-worked
  examples with exact rational answers (tests/golden/hand_examples.json), and a
  50-digit mpmath brute force on tiny inputs.

``test_oracle_mutants.py`` runs the same checks against copies of the oracle
with planted mistakes and requires each copy to fail at least one of them.
"""
import json
import math
import os
from fractions import Fraction

import mpmath
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _sdpa(q, k, v, causal):
    t = [torch.from_numpy(np.ascontiguousarray(x)).to(torch.float64) for x in (q, k, v)]
    return F.scaled_dot_product_attention(t[0][None], t[1][None], t[2][None],
                                          is_causal=causal)[0].numpy()


# ---------------------------------------------------------------------------
# checks: each takes an oracle handle and raises AssertionError on a mismatch
# ---------------------------------------------------------------------------

def check_lambda_zero_is_standard_attention(orc):
    for causal in (False, True):
        for nq, nk, d, dv in ((37, 37, 8, 12), (64, 64, 32, 64), (5, 5, 3, 2)):
            q1, q2 = _rand((nq, d), 1), _rand((nq, d), 2)
            k1, k2 = _rand((nk, d), 3), _rand((nk, d), 4)
            v = _rand((nk, dv), 5)
            got = orc.head_rows(q1, q2, k1, k2, v, None, causal=causal, lam=0.0,
                                pre_norm=True)
            np.testing.assert_allclose(got, _sdpa(q1, k1, v, causal), rtol=0, atol=1e-12)


def check_uniform_map1_isolates_map2(orc):
    # Q1 = 0 makes every score of map 1 zero, so A1 is uniform over the visible
    # keys; what is left of D is mean(V) - lambda * Attention(Q2, K2, V).
    n, d, dv, lam = 29, 16, 24, 0.7
    q1 = np.zeros((n, d))
    q2, k1, k2, v = _rand((n, d), 7), _rand((n, d), 8), _rand((n, d), 9), _rand((n, dv), 10)
    for causal in (False, True):
        got = orc.head_rows(q1, q2, k1, k2, v, None, causal=causal, lam=lam, pre_norm=True)
        if causal:
            mean_v = np.cumsum(v, axis=0) / np.arange(1, n + 1)[:, None]
        else:
            mean_v = np.broadcast_to(v.mean(axis=0), (n, dv))
        want = mean_v - lam * _sdpa(q2, k2, v, causal)
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def check_row_sum_is_one_minus_lambda(orc):
    n, d, dv = 33, 8, 16
    q1, q2, k1, k2 = (_rand((n, d), s, 2.0) for s in (11, 12, 13, 14))
    v = _rand((n, dv), 15)
    ones = np.ones((n, dv))
    for causal in (False, True):
        for lam in (0.0, 0.35, 1.0, -0.4, 2.5):
            _, rs = orc.head_rows(q1, q2, k1, k2, v, None, causal=causal, lam=lam,
                                  pre_norm=True, want_rowsum=True)
            np.testing.assert_allclose(rs, 1.0 - lam, rtol=0, atol=1e-13)
            # with V all ones, D is that same row sum in every channel
            got = orc.head_rows(q1, q2, k1, k2, ones, None, causal=causal, lam=lam,
                                pre_norm=True)
            np.testing.assert_allclose(got, 1.0 - lam, rtol=0, atol=1e-13)


def check_identical_maps_cancel_at_lambda_one(orc):
    n, d, dv = 40, 16, 32
    q, k, v = _rand((n, d), 21), _rand((n, d), 22), _rand((n, dv), 23)
    for causal in (False, True):
        got = orc.head_rows(q, q, k, k, v, None, causal=causal, lam=1.0, pre_norm=True)
        assert np.max(np.abs(got)) == 0.0
        out = orc.head_rows(q, q, k, k, v, None, causal=causal, lam=1.0)
        assert np.max(np.abs(out)) == 0.0


def check_groupnorm_step_matches_library(orc):
    B, H, n, d, dv = 2, 3, 19, 8, 12
    lam = np.array([0.2, 0.55, 0.9])
    lambda_init, eps = 0.7, 1e-3
    rng = np.random.default_rng(31)
    q1, q2, k1, k2 = (rng.standard_normal((B, H, n, d)) for _ in range(4))
    v = rng.standard_normal((B, H, n, dv)) * 0.05
    for causal in (False, True):
        D = np.empty((B, H, n, dv))
        out = np.empty((B, H, n, dv))
        for b in range(B):
            for h in range(H):
                args = (q1[b, h], q2[b, h], k1[b, h], k2[b, h], v[b, h], None)
                D[b, h] = orc.head_rows(*args, causal=causal, lam=lam[h], pre_norm=True)
                out[b, h] = orc.head_rows(*args, causal=causal, lam=lam[h],
                                          lambda_init=lambda_init, eps=eps)
        # tokens as the batch axis, heads as the groups of the channel axis
        x = torch.from_numpy(D).permute(0, 2, 1, 3).reshape(B * n, H * dv)
        want = F.group_norm(x, num_groups=H, eps=eps) * (1.0 - lambda_init)
        want = want.reshape(B, n, H, dv).permute(0, 2, 1, 3).numpy()
        np.testing.assert_allclose(out, want, rtol=0, atol=1e-12)


def check_groupnorm_output_moments(orc):
    n, d, dv = 23, 8, 64
    lambda_init, eps = 0.8, 1e-5
    q1, q2, k1, k2 = (_rand((n, d), s) for s in (41, 42, 43, 44))
    v = _rand((n, dv), 45)
    D = orc.head_rows(q1, q2, k1, k2, v, None, causal=True, lam=0.5, pre_norm=True)
    out = orc.head_rows(q1, q2, k1, k2, v, None, causal=True, lam=0.5,
                        lambda_init=lambda_init, eps=eps)
    sig2 = D.var(axis=1)
    np.testing.assert_allclose(out.mean(axis=1), 0.0, atol=1e-14)
    np.testing.assert_allclose(out.var(axis=1), (1 - lambda_init) ** 2 * sig2 / (sig2 + eps),
                               rtol=1e-12)


def check_causal_row0_closed_form(orc):
    # causal row 0 sees only key 0: both maps put weight 1 on it
    n, d, dv, lam, li, eps = 17, 8, 16, 0.3, 0.8, 1e-5
    q1, q2, k1, k2 = (_rand((n, d), s, 3.0) for s in (51, 52, 53, 54))
    v = _rand((n, dv), 55)
    got = orc.head_rows(q1, q2, k1, k2, v, [0], causal=True, lam=lam,
                        lambda_init=li, eps=eps)[0]
    Dd = (1 - lam) * v[0]
    want = (1 - li) * (Dd - Dd.mean()) / math.sqrt(Dd.var() + eps)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-13)


def check_swap_symmetry_at_lambda_one(orc):
    n, d, dv = 21, 8, 16
    q1, q2, k1, k2 = (_rand((n, d), s) for s in (61, 62, 63, 64))
    v = _rand((n, dv), 65)
    for causal in (False, True):
        a = orc.head_rows(q1, q2, k1, k2, v, None, causal=causal, lam=1.0)
        b = orc.head_rows(q2, q1, k2, k1, v, None, causal=causal, lam=1.0)
        np.testing.assert_allclose(a, -b, rtol=0, atol=1e-12)


def check_equal_keys_give_uniform_maps(orc):
    # non-causal, every key row equal: both maps are uniform, D = (1-lam) mean(V)
    n, d, dv, lam = 13, 8, 8, 0.45
    q1, q2 = _rand((n, d), 71), _rand((n, d), 72)
    k1 = np.tile(_rand((1, d), 73), (n, 1))
    k2 = np.tile(_rand((1, d), 74), (n, 1))
    v = _rand((n, dv), 75)
    got = orc.head_rows(q1, q2, k1, k2, v, None, causal=False, lam=lam, pre_norm=True)
    np.testing.assert_allclose(got, np.broadcast_to((1 - lam) * v.mean(axis=0), (n, dv)),
                               rtol=0, atol=1e-13)


def _golden_value(s):
    s = s.strip()
    for tag, base in (("ln3", math.log(3.0)), ("ln4", math.log(4.0))):
        if s.endswith(tag):
            k = s[:-3]
            return (float(Fraction(k)) if k else 1.0) * base
    return float(Fraction(s))


def _golden_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


def check_hand_worked_examples(orc):
    for case in _golden_cases():
        arr = lambda key: np.array([[_golden_value(x) for x in row] for row in case[key]])
        q1, q2, k1, k2, v = (arr(k) for k in ("q1", "q2", "k1", "k2", "v"))
        lam, li, eps = (float(Fraction(case[k])) for k in ("lam", "lambda_init", "eps"))
        D = orc.head_rows(q1, q2, k1, k2, v, None, causal=case["causal"], lam=lam,
                          pre_norm=True)
        D_want = arr("D")
        np.testing.assert_allclose(D, D_want, rtol=0, atol=1e-14, err_msg=case["name"])
        out = orc.head_rows(q1, q2, k1, k2, v, None, causal=case["causal"], lam=lam,
                            lambda_init=li, eps=eps)
        mean = np.array([float(Fraction(m)) for m in case["mean"]])
        var = np.array([float(Fraction(m)) for m in case["var"]])
        want = (1 - li) * (D_want - mean[:, None]) / np.sqrt(var[:, None] + eps)
        np.testing.assert_allclose(out, want, rtol=0, atol=1e-14, err_msg=case["name"])


def _mp_brute(q1, q2, k1, k2, v, causal, lam, li, eps):
    """50-digit brute force straight from the formula, one query row at a time."""
    mpmath.mp.dps = 50
    nq, d = q1.shape
    nk, dv = v.shape
    M = lambda a: [[mpmath.mpf(float(x)) for x in row] for row in a]
    Q1, Q2, K1, K2, V = M(q1), M(q2), M(k1), M(k2), M(v)
    rt = mpmath.sqrt(d)
    lam, li, eps = mpmath.mpf(lam), mpmath.mpf(li), mpmath.mpf(eps)
    res = []
    for i in range(nq):
        js = range(i + 1) if causal else range(nk)
        e1 = [mpmath.exp(mpmath.fsum(Q1[i][t] * K1[j][t] for t in range(d)) / rt) for j in js]
        e2 = [mpmath.exp(mpmath.fsum(Q2[i][t] * K2[j][t] for t in range(d)) / rt) for j in js]
        z1, z2 = mpmath.fsum(e1), mpmath.fsum(e2)
        w = [a / z1 - lam * b / z2 for a, b in zip(e1, e2)]
        D = [mpmath.fsum(w[n] * V[j][c] for n, j in enumerate(js)) for c in range(dv)]
        mu = mpmath.fsum(D) / dv
        var = mpmath.fsum((x - mu) ** 2 for x in D) / dv
        res.append([float((1 - li) * (x - mu) / mpmath.sqrt(var + eps)) for x in D])
    return np.array(res)


def check_mpmath_bruteforce_tiny(orc):
    for causal in (False, True):
        for seed in (0, 1):
            rng = np.random.default_rng(100 + seed)
            n, d, dv = 7, 4, 6
            q1, q2, k1, k2 = (rng.standard_normal((n, d)) * 1.5 for _ in range(4))
            v = rng.standard_normal((n, dv))
            lam = float(rng.uniform(0.1, 0.9))
            got = orc.head_rows(q1, q2, k1, k2, v, None, causal=causal, lam=lam,
                                lambda_init=0.8, eps=1e-5)
            want = _mp_brute(q1, q2, k1, k2, v, causal, lam, 0.8, 1e-5)
            np.testing.assert_allclose(got, want, rtol=0, atol=1e-13)


CHECKS = [
    check_lambda_zero_is_standard_attention,
    check_uniform_map1_isolates_map2,
    check_row_sum_is_one_minus_lambda,
    check_identical_maps_cancel_at_lambda_one,
    check_groupnorm_step_matches_library,
    check_groupnorm_output_moments,
    check_causal_row0_closed_form,
    check_swap_symmetry_at_lambda_one,
    check_equal_keys_give_uniform_maps,
    check_hand_worked_examples,
    check_mpmath_bruteforce_tiny,
]


@pytest.mark.parametrize("check", CHECKS, ids=lambda c: c.__name__[len("check_"):])
def test_oracle_pin(check):
    check(oracle._load())


# ---------------------------------------------------------------------------
# oracle-level helpers that are not checks of the arithmetic itself
# ---------------------------------------------------------------------------

def test_decode_is_last_row_of_causal_prefill():
    L, d, dv = 50, 16, 32
    rng = np.random.default_rng(81)
    q1, q2, k1, k2 = (rng.standard_normal((1, 1, L, d)) for _ in range(4))
    v = rng.standard_normal((1, 1, L, dv))
    lam = np.array([0.6])
    pre = oracle.fwd(q1, q2, k1, k2, v, lam, causal=True)
    dec = oracle.decode(q1[:, :, -1], q2[:, :, -1], k1, k2, v, lam)
    np.testing.assert_allclose(dec[0, 0], pre[0, 0, -1], rtol=0, atol=1e-13)
    # and a shorter valid length inside a larger cache
    dec7 = oracle.decode(q1[:, :, 6], q2[:, :, 6], k1, k2, v, lam, kv_len=7)
    np.testing.assert_allclose(dec7[0, 0], pre[0, 0, 6], rtol=0, atol=1e-13)


def test_fwd_accepts_bf16_tensors_exactly():
    # bf16 -> fp64 is exact, so feeding bf16 tensors equals feeding their fp64 copies
    g = torch.Generator().manual_seed(5)
    t = [torch.randn(1, 2, 9, 8, generator=g).to(torch.bfloat16) for _ in range(4)]
    v = torch.randn(1, 2, 9, 16, generator=g).to(torch.bfloat16)
    lam = torch.tensor([0.3, 0.6])
    a = oracle.fwd(*t, v, lam, causal=True)
    b = oracle.fwd(*(x.double().numpy() for x in t), v.double().numpy(), lam.numpy(),
                   causal=True)
    assert np.array_equal(a, b)


def test_rejects_bad_arguments():
    z = np.zeros((4, 2))
    with pytest.raises(ValueError):
        oracle.head_rows(z, z, z, z, z, [4], causal=False, lam=0.5)
    with pytest.raises(ValueError):
        oracle.head_rows(z, z, np.zeros((3, 2)), np.zeros((3, 2)), np.zeros((3, 2)), None,
                         causal=True, lam=0.5)
