"""Pins of the projection oracle (oracle/proj.py) to facts other than itself
(CPU only).

* Brute force: every output element recomputed with plain Python loops, going
  the other way through the layout -- from (output, head, channel) to the
  weight row h (4 d + dv) + offset -- on tiny shapes;
* one-hot weights: a single 1 at (feature f, input k) must put column k of X
  at exactly the (output, head, channel) the layout names for f, and zeros
  everywhere else;
* an identity weight (d_model = H (4 d + dv)) returns slices of X.
Planted mistakes in copies of the oracle must each fail one of these.
"""
import itertools
import os
import types

import numpy as np
import pytest

from oracle import proj

SRC = os.path.join(os.path.dirname(proj.__file__), "proj.py")
OFFSET = {"q1": lambda d, dv: 0, "q2": lambda d, dv: d, "k1": lambda d, dv: 2 * d,
          "k2": lambda d, dv: 3 * d, "v": lambda d, dv: 4 * d}


def _case(B, N, H, d, dv, dm, seed):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((B, N, dm)), rng.standard_normal((H * (4 * d + dv), dm))


def check_brute_force(mod):
    for (B, N, H, d, dv, dm, seed) in [(2, 3, 2, 2, 3, 5, 1), (1, 4, 3, 1, 2, 3, 2)]:
        x, w = _case(B, N, H, d, dv, dm, seed)
        got = mod.qkv_proj(x, w, heads=H, head_dim=d, v_dim=dv)
        S = 4 * d + dv
        for name in ("q1", "q2", "k1", "k2", "v"):
            width = dv if name == "v" else d
            assert got[name].shape == (B, H, N, width)
            for b, h, n, c in itertools.product(range(B), range(H), range(N), range(width)):
                f = h * S + OFFSET[name](d, dv) + c
                want = sum(float(x[b, n, k]) * float(w[f, k]) for k in range(dm))
                assert abs(got[name][b, h, n, c] - want) <= 1e-12 * (1 + abs(want)), (name, b, h, n, c)


def check_one_hot(mod):
    B, N, H, d, dv, dm = 2, 3, 3, 2, 4, 6
    x, _ = _case(B, N, H, d, dv, dm, 3)
    S = 4 * d + dv
    for f, k in [(0, 0), (d, 1), (2 * d + 1, 2), (3 * d, 3), (4 * d + dv - 1, 4), (S + 1, 5),
                 (2 * S + 4 * d, 0)]:
        w = np.zeros((H * S, dm))
        w[f, k] = 1.0
        got = mod.qkv_proj(x, w, heads=H, head_dim=d, v_dim=dv)
        h, o = divmod(f, S)
        name = ("q1", "q2", "k1", "k2")[o // d] if o < 4 * d else "v"
        c = o - OFFSET[name](d, dv)
        for nm, t in got.items():
            expect = np.zeros_like(t)
            if nm == name:
                expect[:, h, :, c] = x[:, :, k]
            assert np.array_equal(t, expect), (f, k, nm)


def check_identity(mod):
    B, N, H, d, dv = 2, 5, 2, 3, 4
    S = 4 * d + dv
    x, _ = _case(B, N, H, d, dv, H * S, 4)
    got = mod.qkv_proj(x, np.eye(H * S), heads=H, head_dim=d, v_dim=dv)
    for h in range(H):
        for name in ("q1", "q2", "k1", "k2", "v"):
            lo = h * S + OFFSET[name](d, dv)
            width = dv if name == "v" else d
            assert np.array_equal(got[name][:, h], x[:, :, lo:lo + width])


CHECKS = [check_brute_force, check_one_hot, check_identity]


@pytest.mark.parametrize("check", CHECKS, ids=lambda c: c.__name__)
def test_projection_oracle(check):
    check(proj)


def test_abs_bound_dominates():
    x, w = _case(2, 3, 2, 2, 3, 5, 6)
    a = proj.qkv_proj(x, w, heads=2, head_dim=2, v_dim=3)
    b = proj.qkv_proj_abs(x, w, heads=2, head_dim=2, v_dim=3)
    for n in a:
        assert np.all(b[n] >= np.abs(a[n]))


def test_rejects_mismatched_weight():
    x, w = _case(1, 2, 2, 2, 3, 5, 7)
    with pytest.raises(ValueError):
        proj.qkv_proj(x, w[1:], heads=2, head_dim=2, v_dim=3)


MUTANTS = [
    ('SEGMENTS = ("q1", "q2", "k1", "k2", "v")', 'SEGMENTS = ("q1", "k1", "q2", "k2", "v")'),
    ("yb = y.reshape(B, N, H, S)", "yb = y.reshape(B, N, S, H)"),
    ("y = x.reshape(B * N, dm) @ w.T", "y = x.transpose(1, 0, 2).reshape(B * N, dm) @ w.T"),
    ("= yb[:, :, :, o].transpose(0, 2, 1)", "= yb[:, :, :, o].reshape(B, H, N)"),
    ('return "v", o - 4 * d', 'return "v", o - 3 * d - dv'),
    ("return SEGMENTS[o // d], o % d", "return SEGMENTS[o % 4], o // 4"),
]


@pytest.mark.parametrize("old,new", MUTANTS, ids=[str(i) for i in range(len(MUTANTS))])
def test_planted_projection_mistake_is_caught(old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, old
    mod = types.ModuleType("mutant_proj")
    exec(compile(src.replace(old, new), "mutant_proj", "exec"), mod.__dict__)
    failed = 0
    for check in CHECKS:
        try:
            check(mod)
        except Exception:
            failed += 1
    assert failed > 0
