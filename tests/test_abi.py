"""The C-ABI library loads, exports what include/diffattn.h declares, and
rejects bad arguments before touching the GPU (CPU only: no kernel is
launched by any call here)."""
import ctypes
import subprocess

import pytest

import transformer_attention_diffattn_amd as da

A = 4096  # a fake, 16-byte aligned device address; never dereferenced here


def _dims(**kw):
    base = dict(batch=2, heads=3, seq_q=16, seq_k=16, head_dim=64, v_dim=128, dtype=da.BF16,
                eps=1e-5, flags=0)
    base.update(kw)
    return da.Dims(**base)


def _fwd(dims, ptrs=None, lambda_init=0.8, causal=1):
    p = ptrs or [A] * 7
    return da.lib().diffattn_fwd(p[0], p[1], p[2], p[3], p[4], p[5], lambda_init, causal, p[6],
                                 ctypes.byref(dims) if dims is not None else None, None)


def _decode(dims, cap=16, ws=None, ws_bytes=0, splits=1, ptrs=None, lens=None, lambda_init=0.8):
    p = ptrs or [A] * 7
    return da.lib().diffattn_decode(p[0], p[1], p[2], p[3], p[4], cap, lens, p[5], lambda_init,
                                    p[6], ws, ws_bytes, splits,
                                    ctypes.byref(dims) if dims is not None else None, None)


def test_library_loads_and_reports_version():
    assert da.abi_version() == 2


def test_exports_every_declared_function():
    names = da.header_functions()
    assert set(names) >= {"diffattn_fwd", "diffattn_decode", "diffattn_decode_workspace_size",
                          "diffattn_decode_default_splits", "diffattn_status_string",
                          "diffattn_abi_version"}
    out = subprocess.run(["nm", "-D", "--defined-only", da.library_path()], check=True,
                         capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for n in names:
        assert n in exported, n
        assert hasattr(da.lib(), n)


def test_status_strings():
    s = da.lib().diffattn_status_string
    assert s(0) == b"ok"
    for code in (1, 2, 3, 4):
        assert s(code) and s(code) != b"ok"
    assert s(99) == b"unknown status"


@pytest.mark.parametrize("i", range(7))
def test_fwd_rejects_null_pointers(i):
    p = [A] * 7
    p[i] = None
    assert _fwd(_dims(), p) == da.ERR_INVALID


@pytest.mark.parametrize("i", range(7))
def test_fwd_rejects_misaligned_pointers(i):
    p = [A] * 7
    p[i] = A + 8
    assert _fwd(_dims(), p) == da.ERR_INVALID


@pytest.mark.parametrize("field,value,code", [
    ("batch", 0, da.ERR_INVALID), ("heads", -1, da.ERR_INVALID), ("seq_q", 0, da.ERR_INVALID),
    ("seq_k", 0, da.ERR_INVALID), ("head_dim", 0, da.ERR_INVALID), ("v_dim", 0, da.ERR_INVALID),
    ("eps", -1e-3, da.ERR_INVALID), ("eps", float("nan"), da.ERR_INVALID),
    ("eps", float("inf"), da.ERR_INVALID), ("flags", 4, da.ERR_INVALID),
    ("dtype", 7, da.ERR_UNSUPPORTED), ("head_dim", 48, da.ERR_UNSUPPORTED),
    ("v_dim", 64, da.ERR_UNSUPPORTED), ("seq_k", (1 << 30) + 1, da.ERR_UNSUPPORTED),
])
def test_fwd_rejects_bad_dims(field, value, code):
    assert _fwd(_dims(**{field: value})) == code


def test_fwd_rejects_null_dims_and_bad_scalars():
    assert _fwd(None) == da.ERR_INVALID
    assert _fwd(_dims(), lambda_init=float("nan")) == da.ERR_INVALID
    assert _fwd(_dims(), lambda_init=float("inf")) == da.ERR_INVALID


def test_fwd_causal_needs_square():
    assert _fwd(_dims(seq_q=8, seq_k=16), causal=1) == da.ERR_UNSUPPORTED


def test_decode_argument_checks():
    assert _decode(_dims(seq_q=2)) == da.ERR_UNSUPPORTED
    assert _decode(_dims(seq_q=1), cap=15) == da.ERR_INVALID
    assert _decode(_dims(seq_q=1), splits=-1) == da.ERR_INVALID
    assert _decode(None) == da.ERR_INVALID
    p = [A] * 7
    p[2] = None
    assert _decode(_dims(seq_q=1), ptrs=p) == da.ERR_INVALID
    assert _decode(_dims(seq_q=1), lens=A + 2) == da.ERR_INVALID
    assert _decode(_dims(seq_q=1), lambda_init=float("nan")) == da.ERR_INVALID


def test_decode_workspace_checks():
    d = _dims(seq_q=1, seq_k=4096)
    need = da.lib().diffattn_decode_workspace_size(ctypes.byref(d), 4)
    assert need == 2 * 3 * 4 * (4 + 2 * 128) * 4
    assert _decode(d, cap=4096, splits=4) == da.ERR_WORKSPACE
    assert _decode(d, cap=4096, splits=4, ws=A, ws_bytes=need - 1) == da.ERR_WORKSPACE
    assert _decode(d, cap=4096, splits=4, ws=A + 4, ws_bytes=need) == da.ERR_WORKSPACE


@pytest.mark.parametrize("L,asked,used", [
    (8192, 1, 1), (8192, 4, 4), (8192, 3, 3), (200, 4, 2), (128, 8, 1), (129, 8, 2),
    (1, 5, 1), (100000, 7, 7),
])
def test_decode_split_plan(L, asked, used):
    # each split covers a whole number of 128-key blocks; unused splits are dropped
    d = _dims(seq_q=1, seq_k=L)
    ws = da.lib().diffattn_decode_workspace_size(ctypes.byref(d), asked)
    rec = (4 + 2 * 128) * 4
    assert ws == (0 if used == 1 else 2 * 3 * used * rec)


def test_python_binding_validates_before_the_library():
    import torch
    x = torch.zeros(1, 1, 4, 64)
    with pytest.raises(ValueError):
        da.fwd(x, x, x, x, torch.zeros(1, 1, 4, 128), 0.5)  # CPU tensors are refused
