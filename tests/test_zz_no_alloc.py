"""diffattn_decode_noalloc (the decode entry point that allocates nothing and
keeps its split-K partials in the library's fixed scratch array) against
diffattn_decode with a caller workspace: same kernels, same split count, so
the outputs must be bit-identical.  Two calls in a row, the second smaller,
so the second reads records the first call left behind only if it is wrong."""
import pytest
import torch

import transformer_attention_diffattn_amd as da
import workloads

pytestmark = pytest.mark.gpu


def _case(B, H, L, seed):
    w = workloads.Workload("noalloc", "decode", B=B, H=H, nq=1, nk=L, d=64, dv=128,
                           dtype="bf16", causal=False, lam=("uniform", 0.3, 0.8), seed=seed)
    return {k: (v.cuda() if isinstance(v, torch.Tensor) else v)
            for k, v in workloads.make_decode(w, device="cpu").items()}


@pytest.mark.parametrize("pre_norm", [False, True])
def test_noalloc_decode_matches_workspace_decode(pre_norm):
    for (B, H, L, splits, seed) in [(8, 16, 4096, 8, 1), (2, 4, 1000, 3, 2)]:
        x = _case(B, H, L, seed)
        args = (x["q1"], x["q2"], x["k1"], x["k2"], x["v"], x["lam"])
        want = da.decode(*args, num_splits=splits, pre_norm=pre_norm)
        out = torch.full_like(want, 7.0)
        got = da.decode_noalloc(*args, num_splits=splits, pre_norm=pre_norm, out=out)
        torch.cuda.synchronize()
        assert got.data_ptr() == out.data_ptr()
        assert torch.equal(got, want), (B, H, L, splits)


def test_noalloc_decode_ragged_and_default_splits():
    x = _case(5, 2, 700, 3)
    lens = torch.tensor([700, 1, 0, 333, 129], dtype=torch.int32, device="cuda")
    args = (x["q1"], x["q2"], x["k1"], x["k2"], x["v"], x["lam"])
    for splits in (0, 4):
        want = da.decode(*args, kv_lens=lens, num_splits=splits)
        got = da.decode_noalloc(*args, kv_lens=lens, num_splits=splits)
        assert torch.equal(got, want), splits


def test_noalloc_decode_rejects_partials_past_the_scratch():
    x = _case(64, 32, 2048, 4)
    args = (x["q1"], x["q2"], x["k1"], x["k2"], x["v"], x["lam"])
    # 2048 (b, h) x 16 splits x 1040-byte records > 16 MiB: refused, nothing launched
    assert 2048 * 16 * (4 + 2 * 128) * 4 > da.NOALLOC_SCRATCH_BYTES
    out = torch.full((64, 32, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(da.DiffAttnError) as e:
        da.decode_noalloc(*args, num_splits=16, out=out)
    assert e.value.status == da.ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
