"""The seeded input generators (CPU only): determinism, shapes, structure."""
import math

import numpy as np
import pytest
import torch

import workloads


def _small(name, **kw):
    w = workloads.get(name)
    shrink = dict(B=min(w.B, 2), H=min(w.H, 3))
    if w.kind == "decode":
        shrink.update(nk=96)
    else:
        shrink.update(nq=80, nk=80)
    shrink.update(kw)
    return w.with_(**shrink)


@pytest.mark.parametrize("name", sorted(workloads.WORKLOADS))
def test_same_seed_same_bytes(name):
    w = _small(name)
    a = workloads.make(w)
    b = workloads.make(w)
    for k in ("q1", "q2", "k1", "k2", "v", "lam"):
        assert torch.equal(a[k], b[k]), k
    c = workloads.make(w, seed=w.seed + 100)
    assert not torch.equal(a["k1"], c["k1"])


@pytest.mark.parametrize("name", sorted(workloads.WORKLOADS))
def test_shapes_and_dtypes(name):
    w = _small(name)
    x = workloads.make(w)
    if w.kind == "decode":
        assert x["q1"].shape == (w.B, w.H, w.d)
        assert x["k1"].shape == (w.B, w.H, w.nk, w.d)
        assert x["v"].shape == (w.B, w.H, w.nk, w.dv)
    else:
        assert x["q1"].shape == (w.B, w.H, w.nq, w.d)
        assert x["k2"].shape == (w.B, w.H, w.nk, w.d)
        assert x["v"].shape == (w.B, w.H, w.nk, w.dv)
    assert x["q1"].dtype == w.torch_dtype
    assert x["lam"].dtype == torch.float32 and x["lam"].shape == (w.H,)


def test_one_head_regenerates_alone():
    # each (b, h) has its own stream: a larger batch keeps the earlier heads' values
    w = _small("causal_prefill_bf16", B=1, H=2)
    w2 = w.with_(B=2)
    a, b = workloads.make(w), workloads.make(w2)
    assert torch.equal(a["q1"][0], b["q1"][0])


def test_lambda_rules():
    w = workloads.get("causal_prefill_bf16")
    lam = workloads.make(w.with_(B=1, nq=8, nk=8))["lam"].numpy()
    assert np.all((lam >= 0.2) & (lam <= 0.8)) and len(np.unique(lam)) == w.H
    w = workloads.get("large_head_bf16")
    lam = workloads.make(w.with_(B=1, H=2, nq=8, nk=8))["lam"].numpy()
    assert np.all(lam == np.float32(0.95))


def test_needles_point_at_their_queries():
    w = workloads.get("long_needles_bf16").with_(H=2, nq=512, nk=512)
    x = workloads.make(w, device="cpu")
    aux = np.random.default_rng(workloads._children(w)[-1])
    workloads._lambdas(w, aux)
    plans = workloads._needle_plan(w, aux, w.nq, w.nk)
    for h, (keys, queries, _) in enumerate(plans):
        assert len(set(keys.tolist())) == w.needles
        assert np.all(queries >= keys)
        for j, i in zip(keys, queries):
            u = x["q1"][0, h, i].double()
            k = x["k1"][0, h, j].double()
            cos = float(u @ k / (u.norm() * k.norm()))
            assert abs(cos - 0.9) < 0.02  # 0.9 before bf16 rounding


def test_student_t_scaled_to_unit_variance():
    w = workloads.get("large_head_bf16").with_(B=1, H=2, nq=4096, nk=4096)
    x = workloads.make(w)
    v = x["v"].double().flatten()
    # t(3) has heavy tails; its sample variance converges slowly, so the check
    # is loose, but the tails must be there
    assert 0.6 < float(v.var()) < 1.6
    assert float(v.abs().max()) > 8.0


def test_work_counts():
    w = workloads.get("causal_prefill_bf16")
    assert w.pairs() == 4 * 16 * 2048 * 2049 // 2
    assert w.exec_flops() == 4 * (64 + 128) * w.pairs()
    assert w.algorithmic_bytes() == 2 * (2 * 4 * 16 * 2048 * 64 * 2 + 2 * 4 * 16 * 2048 * 128)
    d = workloads.get("decode_bf16")
    assert d.algorithmic_bytes() == 8_590_983_168
