"""Seeded synthetic inputs for the Differential Attention forward operator.

This module only draws numbers: it holds none of the operator's arithmetic, and
it is the one piece of code that both the HIP path's callers and the fp64
oracle's callers share.  Every tensor is drawn in a fixed order from a seed, so
any run can be repeated exactly.

Shapes follow the operator's definition on the llmbytes.dev page ("How
Differential Attention Cancels Common-Mode Noise", step 1): for every head
there are two queries Q1, Q2, two keys K1, K2 and one value V.  Storage layout
is [batch, heads, seq, dim], last dimension unit-stride.

Two generators are provided:

* ``device="cpu"``: NumPy PCG64 streams spawned from ``SeedSequence(seed)``, one
  child per (b, h) and one more for the per-head scalars and the needle
  choices.  Values are drawn in float64 and cast to the storage dtype with
  round-to-nearest-even.  Any single head can be regenerated on its own.
* ``device="cuda"`` (or any torch device): one ``torch.Generator`` seeded with
  ``seed`` on that device draws the five full tensors in the same order in
  float32, then casts to the storage dtype.  It is used for the large workloads,
  whose inputs would take minutes to draw on the host.  Its values differ from
  the CPU generator's for the same seed; both are deterministic.

Per-head lambda values and the needle positions are always drawn on the host
with NumPy, so they do not depend on the device.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np
import torch

__all__ = ["Workload", "WORKLOADS", "get", "make_prefill", "make_decode", "make", "needle_plan",
           "quantize_e4m3", "make_prefill_fp8", "make_proj"]


@dataclass(frozen=True)
class Workload:
    """One synthetic workload of the operator.

    kind: "prefill" (Nq query rows per head against Nk keys) or "decode" (one
    query token per sequence against a KV cache of length ``nk``).
    dist: "normal" (i.i.d. N(0,1) times ``scale``) or "student_t3" (Student-t
    with 3 degrees of freedom divided by sqrt(3), i.e. unit variance).
    lam: ("const", value) or ("uniform", lo, hi), one value per head.
    needles: number of planted needle keys per head (0 = none); see
    ``_plant_needles``.
    """

    name: str
    kind: str
    B: int
    H: int
    nq: int
    nk: int
    d: int
    dv: int
    dtype: str
    causal: bool
    dist: str = "normal"
    scale: float = 1.0
    lam: tuple = ("const", 0.5)
    lambda_init: float = 0.8
    eps: float = 1e-5
    seed: int = 0
    needles: int = 0
    needle_cos: float = 0.9
    description: str = ""

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)

    @property
    def torch_dtype(self) -> torch.dtype:
        return {"f32": torch.float32, "bf16": torch.bfloat16}[self.dtype]

    def pairs(self) -> int:
        """Number of unmasked (query, key) pairs over all heads."""
        if self.kind == "decode":
            return self.B * self.H * self.nk
        if self.causal:
            # query i sees keys 0..i (Nq == Nk for causal prefill)
            per_head = self.nq * (self.nq + 1) // 2
        else:
            per_head = self.nq * self.nk
        return self.B * self.H * per_head

    def exec_flops(self) -> int:
        """Flops the fused one-sweep method executes: 2 QK^T + 2 P.V per pair."""
        return 4 * (self.d + self.dv) * self.pairs()

    def formula_flops(self) -> int:
        """Flops of the formula read literally: 2 QK^T + one (A1 - lam*A2).V."""
        return (4 * self.d + 2 * self.dv) * self.pairs()

    def algorithmic_bytes(self) -> int:
        """Read Q1, Q2, K1, K2, V once and write the output once."""
        es = 4 if self.dtype == "f32" else 2
        nq = 1 if self.kind == "decode" else self.nq
        q = 2 * self.B * self.H * nq * self.d
        k = 2 * self.B * self.H * self.nk * self.d
        v = self.B * self.H * self.nk * self.dv
        o = self.B * self.H * nq * self.dv
        return es * (q + k + v + o)


_S2 = 1.0 / math.sqrt(2.0)

WORKLOADS = {
    w.name: w
    for w in [
        Workload(
            "tiny_noncausal_f32", "prefill", B=1, H=2, nq=128, nk=128, d=32, dv=64,
            dtype="f32", causal=False, lam=("const", 0.5), seed=1,
            description="non-causal prefill, fp32, B1 H2 N128 d32 dv64, N(0,1), lambda 0.5"),
        Workload(
            "causal_prefill_bf16", "prefill", B=4, H=16, nq=2048, nk=2048, d=64, dv=128,
            dtype="bf16", causal=True, scale=_S2, lam=("uniform", 0.2, 0.8), seed=2,
            description="causal prefill, bf16, B4 H16 N2048 d64 dv128, N(0,1)/sqrt2, "
                        "lambda U(0.2,0.8) per head"),
        Workload(
            "long_needles_bf16", "prefill", B=1, H=16, nq=32768, nk=32768, d=64, dv=128,
            dtype="bf16", causal=True, lam=("const", 0.6), seed=3, needles=8,
            description="long causal prefill, bf16, B1 H16 N32768 d64 dv128, N(0,1) with "
                        "8 planted K1 needles per head, lambda 0.6"),
        Workload(
            "decode_bf16", "decode", B=64, H=32, nq=1, nk=8192, d=64, dv=128,
            dtype="bf16", causal=False, lam=("uniform", 0.3, 0.8), seed=4,
            description="KV-cache decode, bf16, B64 H32 L8192 d64 dv128, N(0,1), "
                        "lambda U(0.3,0.8) per head"),
        Workload(
            "large_head_bf16", "prefill", B=2, H=32, nq=8192, nk=8192, d=128, dv=256,
            dtype="bf16", causal=True, dist="student_t3", lam=("const", 0.95), seed=5,
            description="large-head causal prefill, bf16, B2 H32 N8192 d128 dv256, "
                        "Student-t(3)/sqrt3, lambda 0.95"),
    ]
}


def get(name: str) -> Workload:
    return WORKLOADS[name]


# --------------------------------------------------------------------------
# host (NumPy) drawing
# --------------------------------------------------------------------------

def _np_draw(rng: np.random.Generator, dist: str, shape, scale: float) -> np.ndarray:
    if dist == "normal":
        return rng.standard_normal(shape) * scale
    if dist == "student_t3":
        return rng.standard_t(3, shape) / math.sqrt(3.0) * scale
    raise ValueError(f"unknown distribution {dist!r}")


def _lambdas(w: Workload, rng: np.random.Generator) -> np.ndarray:
    kind = w.lam[0]
    if kind == "const":
        return np.full(w.H, float(w.lam[1]), dtype=np.float32)
    if kind == "uniform":
        return rng.uniform(w.lam[1], w.lam[2], w.H).astype(np.float32)
    raise ValueError(f"unknown lambda rule {w.lam!r}")


def _children(w: Workload):
    ss = np.random.SeedSequence(w.seed)
    # one stream per (b, h) for the tensors, plus one for scalars and needles
    return ss.spawn(w.B * w.H + 1)


def _needle_plan(w: Workload, rng: np.random.Generator, n_q: int, n_k: int):
    """Per head: 8 distinct key positions, a query at or after each, and a
    unit direction to mix in.  Returns a list over heads of (keys, queries,
    gaussian vectors) in NumPy."""
    plans = []
    for _ in range(w.B * w.H):
        keys = rng.choice(n_k, size=w.needles, replace=False)
        queries = np.array([rng.integers(j, n_q) for j in keys], dtype=np.int64)
        gauss = rng.standard_normal((w.needles, w.d))
        plans.append((keys.astype(np.int64), queries, gauss))
    return plans


def _plant_needles(q1: torch.Tensor, k1: torch.Tensor, plan, cos: float) -> None:
    """Align K1 at each needle key with the direction of Q1 at its query.

    For needle key j and query i (i >= j, so a causal mask admits the pair):
    u = Q1[i]/|Q1[i]|, w = a Gaussian vector with its u-component removed and
    normalised, and K1[j] <- |K1[j]| * (cos*u + sqrt(1-cos^2)*w).  K2 is left as
    noise.  Works in float32 on whatever device the tensors live on; q1 and k1
    are [N, d] views of one head, modified in place.
    """
    keys, queries, gauss = plan
    dev = k1.device
    for j, i, g in zip(keys.tolist(), queries.tolist(), gauss):
        u = q1[i].float()
        u = u / u.norm()
        gv = torch.from_numpy(g).to(device=dev, dtype=torch.float32)
        gv = gv - (gv @ u) * u
        gv = gv / gv.norm()
        norm = k1[j].float().norm()
        k1[j] = (norm * (cos * u + math.sqrt(1.0 - cos * cos) * gv)).to(k1.dtype)


def needle_plan(w: Workload):
    """The needle positions make_prefill plants for workload w, per head
    (flattened b*H + h): a list of (key positions, query positions, gaussian
    vectors).  Empty when the workload has no needles."""
    if not w.needles:
        return []
    aux = np.random.default_rng(_children(w)[-1])
    _lambdas(w, aux)  # same draw order as make_prefill
    return _needle_plan(w, aux, w.nq, w.nk)


def make_prefill(w: Workload, device: str | torch.device = "cpu", seed: Optional[int] = None):
    """Inputs of a prefill workload.

    Returns a dict with q1, q2 [B,H,Nq,d], k1, k2 [B,H,Nk,d], v [B,H,Nk,dv] in the
    workload's storage dtype on ``device``, lam (float32 [H], same device), and
    the scalars lambda_init, eps, causal.
    """
    if seed is not None:
        w = w.with_(seed=seed)
    if w.kind != "prefill":
        raise ValueError("make_prefill needs a prefill workload")
    kids = _children(w)
    aux = np.random.default_rng(kids[-1])
    lam = _lambdas(w, aux)
    dt = w.torch_dtype
    shapes = [(w.nq, w.d), (w.nq, w.d), (w.nk, w.d), (w.nk, w.d), (w.nk, w.dv)]
    names = ["q1", "q2", "k1", "k2", "v"]
    dev = torch.device(device)
    if dev.type == "cpu":
        out = {n: torch.empty((w.B, w.H) + s, dtype=dt) for n, s in zip(names, shapes)}
        for bh in range(w.B * w.H):
            b, h = divmod(bh, w.H)
            rng = np.random.default_rng(kids[bh])
            for n, s in zip(names, shapes):
                out[n][b, h] = torch.from_numpy(_np_draw(rng, w.dist, s, w.scale)).to(dt)
    else:
        out = _device_draw(w, dev, names, shapes)
    if w.needles:
        plans = _needle_plan(w, aux, w.nq, w.nk)
        for bh, plan in enumerate(plans):
            b, h = divmod(bh, w.H)
            _plant_needles(out["q1"][b, h], out["k1"][b, h], plan, w.needle_cos)
    out["lam"] = torch.from_numpy(lam).to(dev)
    out["lambda_init"] = w.lambda_init
    out["eps"] = w.eps
    out["causal"] = w.causal
    return out


def make_decode(w: Workload, device: str | torch.device = "cpu", seed: Optional[int] = None):
    """Inputs of a decode workload: q1, q2 [B,H,d]; k1, k2 caches [B,H,L,d];
    v cache [B,H,L,dv]; lam float32 [H]; scalars lambda_init, eps."""
    if seed is not None:
        w = w.with_(seed=seed)
    if w.kind != "decode":
        raise ValueError("make_decode needs a decode workload")
    kids = _children(w)
    aux = np.random.default_rng(kids[-1])
    lam = _lambdas(w, aux)
    dt = w.torch_dtype
    shapes = [(w.d,), (w.d,), (w.nk, w.d), (w.nk, w.d), (w.nk, w.dv)]
    names = ["q1", "q2", "k1", "k2", "v"]
    dev = torch.device(device)
    if dev.type == "cpu":
        out = {n: torch.empty((w.B, w.H) + s, dtype=dt) for n, s in zip(names, shapes)}
        for bh in range(w.B * w.H):
            b, h = divmod(bh, w.H)
            rng = np.random.default_rng(kids[bh])
            for n, s in zip(names, shapes):
                out[n][b, h] = torch.from_numpy(_np_draw(rng, w.dist, s, w.scale)).to(dt)
    else:
        out = _device_draw(w, dev, names, shapes)
    out["lam"] = torch.from_numpy(lam).to(dev)
    out["lambda_init"] = w.lambda_init
    out["eps"] = w.eps
    return out


def make(w: Workload, device="cpu", seed: Optional[int] = None):
    return make_decode(w, device, seed) if w.kind == "decode" else make_prefill(w, device, seed)


def _device_draw(w: Workload, dev: torch.device, names, shapes):
    g = torch.Generator(device=dev)
    g.manual_seed(int(w.seed))
    dt = w.torch_dtype
    out = {}
    for n, s in zip(names, shapes):
        full = (w.B, w.H) + s
        if w.dist == "normal":
            x = torch.randn(full, generator=g, device=dev, dtype=torch.float32)
            x.mul_(w.scale)
        elif w.dist == "student_t3":
            # t_3 = Z / sqrt(chi2_3 / 3), chi2_3 = sum of three squared normals;
            # divided by sqrt(3) for unit variance: Z / sqrt(chi2_3)
            x = torch.randn(full, generator=g, device=dev, dtype=torch.float32)
            chi = torch.zeros_like(x)
            for _ in range(3):
                z = torch.randn(full, generator=g, device=dev, dtype=torch.float32)
                chi.addcmul_(z, z)
                del z
            x.div_(chi.sqrt_())
            del chi
            x.mul_(w.scale)
        else:
            raise ValueError(f"unknown distribution {w.dist!r}")
        out[n] = x.to(dt)
        del x
    return out


# --------------------------------------------------------------------------
# FP8 (E4M3) query/key inputs
# --------------------------------------------------------------------------

E4M3_MAX = 448.0


def quantize_e4m3(x: torch.Tensor):
    """Per-tensor E4M3 codes of x: scale = max|x| / 448 (1 if x is all zero),
    codes = x / scale rounded by torch's float8_e4m3fn conversion (nearest,
    ties to even).  Returns (codes as float8_e4m3fn, scale as a Python float).
    Input preparation only: whoever consumes the codes decodes them itself."""
    amax = float(x.abs().max().float()) if x.numel() else 0.0
    scale = amax / E4M3_MAX if amax > 0 else 1.0
    codes = (x.float() / scale).clamp_(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)
    return codes, scale


def make_prefill_fp8(w: Workload, device: str | torch.device = "cpu", seed: Optional[int] = None):
    """Inputs of a prefill workload with FP8 queries and keys: the tensors of
    make_prefill (bf16 V), with q1, q2, k1, k2 replaced by their E4M3 codes and
    ``scales`` = [s_q1, s_q2, s_k1, s_k2]."""
    x = make_prefill(w, device, seed)
    scales = []
    for n in ("q1", "q2", "k1", "k2"):
        x[n], s = quantize_e4m3(x[n])
        scales.append(s)
    x["scales"] = scales
    return x


# --------------------------------------------------------------------------
# inputs of the Q/K/V projection
# --------------------------------------------------------------------------

def make_proj(w: Workload, d_model: Optional[int] = None, device: str | torch.device = "cpu",
              seed: Optional[int] = None):
    """Hidden states and projection weight for workload w's attention shapes:
    x [B][N][d_model] ~ N(0, 1) and wt [H (4 d + dv)][d_model] ~ N(0, 1/d_model)
    (unit-variance outputs), both in w's storage dtype.  d_model defaults to
    H dv.  One torch.Generator seeded with the workload's seed (plus 1000) on
    ``device`` draws x, then wt."""
    dm = d_model if d_model is not None else w.H * w.dv
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(int(w.seed if seed is None else seed) + 1000)
    dt = w.torch_dtype
    x = torch.randn((w.B, w.nq, dm), generator=g, device=dev, dtype=torch.float32).to(dt)
    wt = torch.randn((w.H * (4 * w.d + w.dv), dm), generator=g, device=dev, dtype=torch.float32)
    wt = wt.mul_(1.0 / math.sqrt(dm)).to(dt)
    return {"x": x, "w": wt, "d_model": dm}
