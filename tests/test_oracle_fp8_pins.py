"""Pins of the FP8 oracle (oracle/fp8.py) to facts other than itself (CPU).

* The E4M3 decoder, written from the format's definition, must agree with
  torch's float8_e4m3fn -> float64 conversion (a library routine) on all 256
  codes, NaN codes included, and with closed-form values of the format: 1.0,
  the largest finite value 448, the smallest normal 2^-6, the smallest
  subnormal 2^-9, signed zero.
* The FP8 forward must equal the operator assembled from library routines on
  the same dequantised inputs -- torch's scaled_dot_product_attention for each
  map and group_norm with one group per head (iloveeagents.com, "Mathematical
  Formula"; llmbytes.dev, "How Differential Attention Cancels Common-Mode
  Noise", steps 1-4) -- with dequantisation through torch's conversion.
* Moving a factor between a query scale and its key scale leaves the output
  unchanged (the score only sees their product).
Planted mistakes in copies of the decoder must each fail one of these.
"""
import os
import types

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import workloads
from oracle import fp8 as of8

SRC = os.path.join(os.path.dirname(of8.__file__), "fp8.py")
ALL = np.arange(256)


def _torch_values():
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def check_decoder(mod):
    got, want = mod.e4m3_value(ALL), _torch_values()
    assert np.array_equal(np.isnan(got), np.isnan(want)), "NaN codes"
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok]), "values"
    assert np.array_equal(np.signbit(got[ok]), np.signbit(want[ok])), "signs"


def check_closed_forms(mod):
    v = mod.e4m3_value(np.array([0x38, 0x7E, 0x08, 0x01, 0x07, 0xB8, 0x00, 0x80, 0x7F, 0xFF, 0x3C]))
    want = [1.0, 448.0, 2.0 ** -6, 2.0 ** -9, 7 * 2.0 ** -9, -1.0, 0.0, -0.0]
    assert list(v[:8]) == want
    assert np.signbit(v[7]) and not np.signbit(v[6])
    assert np.isnan(v[8]) and np.isnan(v[9])
    assert v[10] == 1.5
    # positive finite codes are strictly increasing
    pos = mod.e4m3_value(np.arange(0x7F))
    assert np.all(np.diff(pos) > 0)


def test_decoder_matches_library_conversion():
    check_decoder(of8)


def test_decoder_closed_forms():
    check_closed_forms(of8)


def test_decoder_accepts_torch_tensors():
    c = torch.tensor([0x38, 0xC0, 0x01], dtype=torch.uint8)
    assert list(of8.e4m3_value(c)) == [1.0, -2.0, 2.0 ** -9]
    assert list(of8.e4m3_value(c.view(torch.float8_e4m3fn))) == [1.0, -2.0, 2.0 ** -9]


def _library_forward(x, scales, lam, causal, lambda_init, eps):
    deq = [x[n].to(torch.float64) * s for n, s in zip(("q1", "q2", "k1", "k2"), scales)]
    v = x["v"].to(torch.float64)
    B, H = v.shape[:2]
    out = torch.empty(B, H, deq[0].shape[2], v.shape[3], dtype=torch.float64)
    for h in range(H):
        o1 = F.scaled_dot_product_attention(deq[0][:, h], deq[2][:, h], v[:, h], is_causal=causal)
        o2 = F.scaled_dot_product_attention(deq[1][:, h], deq[3][:, h], v[:, h], is_causal=causal)
        D = o1 - float(lam[h]) * o2
        out[:, h] = (1 - lambda_init) * F.group_norm(D.reshape(-1, D.shape[-1]), 1,
                                                     eps=eps).reshape(D.shape)
    return out.numpy()


@pytest.mark.parametrize("causal,dist", [(True, "normal"), (False, "student_t3")])
def test_fp8_forward_matches_library_forward(causal, dist):
    w = workloads.Workload("fp8pin", "prefill", B=2, H=3, nq=23, nk=23, d=16, dv=12, dtype="bf16",
                           causal=causal, dist=dist, lam=("uniform", 0.2, 0.9), seed=31)
    x = workloads.make_prefill_fp8(w)
    got = of8.fwd_fp8(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], x["scales"], x["lam"],
                      causal=causal)
    want = _library_forward(x, x["scales"], x["lam"].double().numpy(), causal, 0.8, 1e-5)
    np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-11)


def test_scale_moves_between_query_and_key():
    w = workloads.Workload("fp8pin", "prefill", B=1, H=2, nq=17, nk=17, d=8, dv=6, dtype="bf16",
                           causal=True, lam=("const", 0.5), seed=32)
    x = workloads.make_prefill_fp8(w)
    s = list(x["scales"])
    a = of8.fwd_fp8(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], s, x["lam"], causal=True)
    t = [s[0] * 3.0, s[1] / 5.0, s[2] / 3.0, s[3] * 5.0]
    b = of8.fwd_fp8(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], t, x["lam"], causal=True)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)
    # while a change of one product does change it
    t = [s[0] * 3.0, s[1], s[2], s[3]]
    c = of8.fwd_fp8(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], t, x["lam"], causal=True)
    assert np.abs(a - c).max() > 1e-3


def test_quantizer_round_trip():
    """The input quantiser keeps every element within half an E4M3 step."""
    g = torch.Generator().manual_seed(5)
    x = (torch.randn(4000, generator=g, dtype=torch.float64) * 3).to(torch.bfloat16)
    codes, scale = workloads.quantize_e4m3(x)
    back = of8.dequantize(codes, scale)
    xs = x.double().numpy()
    assert np.all(np.isfinite(back))
    assert np.abs(back).max() <= 448 * scale * (1 + 1e-12)
    # relative step 2^-3 for normals; absolute 2^-9 * scale for subnormals
    assert np.all(np.abs(back - xs) <= np.maximum(2.0 ** -4 * np.abs(xs), 2.0 ** -10 * scale)
                  * (1 + 1e-9))


DECODER_MUTANTS = [
    ("np.exp2(e - 7.0)", "np.exp2(e - 8.0)"),
    ("(m / 8.0) * 2.0 ** (1 - 7)", "(1.0 + m / 8.0) * 2.0 ** (1 - 7)"),
    ("(m / 8.0) * 2.0 ** (1 - 7)", "(m / 8.0) * 2.0 ** (0 - 7)"),
    ("(1.0 + m / 8.0) * np.exp2", "(1.0 + m / 16.0) * np.exp2"),
    ("return np.where(s == 1, -mag, mag)", "return mag"),
    ("e = (c >> 3) & 0xF", "e = (c >> 4) & 0x7"),
    ("(e == 15) & (m == 7)", "(e == 15)"),
]


@pytest.mark.parametrize("old,new", DECODER_MUTANTS, ids=[str(i) for i in range(len(DECODER_MUTANTS))])
def test_planted_decoder_mistake_is_caught(old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, old
    mod = types.ModuleType("mutant_fp8")
    mod.__dict__["__name__"] = "mutant_fp8"
    exec(compile(src.replace(old, new), "mutant_fp8", "exec"), mod.__dict__)
    with pytest.raises(AssertionError):
        check_decoder(mod)
        check_closed_forms(mod)
