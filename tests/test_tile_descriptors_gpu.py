"""The large-tensor load path at small sizes (GPU, through the C ABI).

The prefill, training-forward and backward kernels address their K/V (or
Q/dD) tiles through one buffer descriptor per tensor while a (batch, head)
slice spans less than 2 GiB, and through one descriptor per tile beyond that.
Only the second form serves slices of 2 GiB or more; test_parity_gpu.py
allocates such a slice for the head_dim-32/64 non-causal forward only (over
8.4M keys), and DIFFATTN_FLAG_TILE_DESCRIPTORS selects the form at any size
for every other kernel and mode.  The two forms load the same bytes into the
same LDS places and do the same arithmetic, so their results must be bitwise
equal -- and the one-descriptor results are checked against the oracle by
the other GPU tests (one case here is also checked against the oracle
directly).  Shapes: several tiles with a
ragged end, causal and not, rectangular, and a (batch * heads) count that is
not a multiple of 8 (the grid-order fallback).
"""
import pytest
import torch

import oracle
import transformer_attention_diffattn_amd as da
import workloads
from tests.test_parity_gpu import assert_close

pytestmark = pytest.mark.gpu

DIMS = [(32, 64), (64, 128), (128, 256)]
DIM_IDS = ["d32", "d64", "d128"]


def _inputs(B, H, nq, nk, d, dv, causal, seed, dist="normal"):
    w = workloads.Workload("tiles", "prefill", B=B, H=H, nq=nq, nk=nk, d=d, dv=dv, dtype="bf16",
                           causal=causal, dist=dist, lam=("uniform", 0.2, 0.9), seed=seed)
    x = workloads.make_prefill(w)
    g = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    return w, x, g


@pytest.mark.parametrize("dims", DIMS, ids=DIM_IDS)
@pytest.mark.parametrize("causal,nq,nk", [(True, 300, 300), (False, 300, 300), (False, 70, 513)],
                         ids=["causal", "full", "rect"])
def test_forward_tile_descriptors_match(dims, causal, nq, nk):
    d, dv = dims
    w, x, g = _inputs(2, 3, nq, nk, d, dv, causal, seed=1200 + nq + d)
    args = (g["q1"], g["q2"], g["k1"], g["k2"], g["v"], g["lam"])
    one = da.fwd(*args, causal=causal)
    tiles = da.fwd(*args, causal=causal, tile_descriptors=True)
    torch.cuda.synchronize()
    assert torch.equal(one, tiles), f"d{d} causal={causal} {nq}x{nk}"


def test_forward_tile_descriptors_against_oracle():
    w, x, g = _inputs(1, 2, 257, 257, 128, 256, True, seed=1210, dist="student_t3")
    out = da.fwd(g["q1"], g["q2"], g["k1"], g["k2"], g["v"], g["lam"], causal=True,
                 tile_descriptors=True)
    ref = oracle.fwd(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], x["lam"], causal=True)
    assert_close(out, ref, torch.bfloat16, "tile descriptors, d128 student-t")


@pytest.mark.parametrize("dims", [(64, 128), (128, 256)], ids=["d64", "d128"])
@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
def test_fp8_tile_descriptors_match(dims, causal):
    d, dv = dims
    w = workloads.Workload("tiles8", "prefill", B=2, H=3, nq=300, nk=300, d=d, dv=dv,
                           dtype="bf16", causal=causal, lam=("uniform", 0.2, 0.9), seed=1220 + d)
    x = workloads.make_prefill_fp8(w)
    g = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    args = (g["q1"], g["q2"], g["k1"], g["k2"], g["v"], x["scales"], g["lam"])
    one = da.fwd_fp8(*args, causal=causal)
    tiles = da.fwd_fp8(*args, causal=causal, tile_descriptors=True)
    torch.cuda.synchronize()
    assert torch.equal(one, tiles)


@pytest.mark.parametrize("dims", DIMS, ids=DIM_IDS)
@pytest.mark.parametrize("causal,nq,nk", [(True, 300, 300), (False, 300, 33)],
                         ids=["causal", "rect"])
def test_training_tile_descriptors_match(dims, causal, nq, nk):
    d, dv = dims
    w, x, g = _inputs(1, 3, nq, nk, d, dv, causal, seed=1230 + d)
    dout = torch.randn((1, 3, nq, dv), generator=torch.Generator().manual_seed(1231),
                       dtype=torch.float64).to(torch.bfloat16).cuda()
    args = (g["q1"], g["q2"], g["k1"], g["k2"], g["v"], g["lam"])
    res = {}
    for flag in (False, True):
        out, d_save, lse = da.fwd_train(*args, causal=causal, tile_descriptors=flag)
        grads = da.bwd(*args, dout, d_save, lse, causal=causal, tile_descriptors=flag)
        torch.cuda.synchronize()
        res[flag] = (out, d_save, lse, *grads)
    names = ("out", "d_save", "lse", "dq1", "dq2", "dk1", "dk2", "dv", "dlambda")
    for name, a, b in zip(names, res[False], res[True]):
        assert torch.equal(a, b), f"{name} d{d} causal={causal}"
