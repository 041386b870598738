"""MI355X (gfx950) Differential Attention forward: Python binding.

A thin ctypes layer over ``libdiffattn.so`` (the HIP kernels behind the C ABI
in ``include/diffattn.h``).  It only checks and marshals arguments: every step
of the operator runs in the library's kernels.  PyTorch supplies device memory
and the current stream.  There is no fallback: if the library is not built,
every call raises.

The operator (iloveeagents.com, "Mathematical Formula"; llmbytes.dev, "How
Differential Attention Cancels Common-Mode Noise", steps 1-4):

    out = (1 - lambda_init) * GroupNorm_h((softmax(Q1 K1^T / sqrt(d))
                                           - lambda_h softmax(Q2 K2^T / sqrt(d))) V)

with one GroupNorm group per head over its dv channels (population variance,
eps inside the square root, no affine parameters).
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional, Sequence, Union

import torch

__all__ = [
    "fwd", "fwd_fp8", "fwd_train", "qkv_proj", "bwd", "bwd_workspace_size", "diag", "decode",
    "decode_noalloc", "NOALLOC_SCRATCH_BYTES",
    "decode_workspace_size", "decode_default_splits", "abi_version", "library_path",
    "prefill_kernel_name", "DiffAttnError", "SUPPORTED_DIMS", "FLAG_PRE_NORM",
    "FLAG_TILE_DESCRIPTORS",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
# DIFFATTN_LIBRARY: another build of the same library (the host-sanitized one)
_LIB_PATH = os.environ.get("DIFFATTN_LIBRARY") or os.path.join(_HERE, "_lib", "libdiffattn.so")
_HEADER = os.path.join(os.path.dirname(_HERE), "include", "diffattn.h")

SUPPORTED_DIMS = ((32, 64), (64, 128), (128, 256))
F32, BF16 = 0, 1
FLAG_PRE_NORM = 1
FLAG_TILE_DESCRIPTORS = 2
OK, ERR_INVALID, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = 0, 1, 2, 3, 4
NOALLOC_SCRATCH_BYTES = 16 << 20  # DIFFATTN_NOALLOC_SCRATCH_BYTES


class DiffAttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


class Dims(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("seq_q", ctypes.c_int32),
        ("seq_k", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("v_dim", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("eps", ctypes.c_float), ("flags", ctypes.c_uint32),
    ]


_lib = None


def library_path() -> str:
    return _LIB_PATH


def prefill_kernel_name(d: int, dv: int, dtype: str = "bf16") -> str:
    """Name of the kernel diffattn_fwd launches for these sizes (as a profiler
    lists it), so measurements can be matched to kernels."""
    if dtype == "f32":
        return "prefill_f32_kernel"
    return "prefill_bf16_twopass_kernel" if (d, dv) == (128, 256) else "prefill_bf16_kernel"


def lib():
    """The loaded C library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(
                f"{_LIB_PATH} is missing: build it with "
                "`python -m transformer_attention_diffattn_amd.build`")
        L = ctypes.CDLL(_LIB_PATH)
        P, I, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
        DP = ctypes.POINTER(Dims)
        L.diffattn_abi_version.restype = I
        L.diffattn_abi_version.argtypes = []
        L.diffattn_status_string.restype = ctypes.c_char_p
        L.diffattn_status_string.argtypes = [I]
        L.diffattn_fwd.restype = I
        L.diffattn_fwd.argtypes = [P, P, P, P, P, P, F, I, P, DP, P]
        L.diffattn_decode.restype = I
        L.diffattn_decode.argtypes = [P, P, P, P, P, ctypes.c_int32, P, P, F, P, P,
                                      ctypes.c_size_t, ctypes.c_int32, DP, P]
        L.diffattn_decode_noalloc.restype = I
        L.diffattn_decode_noalloc.argtypes = [P, P, P, P, P, ctypes.c_int32, P, P, F, P,
                                              ctypes.c_int32, DP, P]
        L.diffattn_decode_default_splits.restype = ctypes.c_int32
        L.diffattn_decode_default_splits.argtypes = [DP]
        L.diffattn_decode_workspace_size.restype = ctypes.c_size_t
        L.diffattn_decode_workspace_size.argtypes = [DP, ctypes.c_int32]
        L.diffattn_fwd_fp8.restype = I
        L.diffattn_fwd_fp8.argtypes = [P, P, P, P, P, ctypes.POINTER(ctypes.c_float), P, F, I, P,
                                       DP, P]
        i32 = ctypes.c_int32
        L.diffattn_qkv_proj.restype = I
        L.diffattn_qkv_proj.argtypes = [P, P, i32, i32, i32, i32, i32, i32, P, P, P, P, P, P]
        L.diffattn_fwd_train.restype = I
        L.diffattn_fwd_train.argtypes = [P, P, P, P, P, P, F, I, P, P, P, DP, P]
        L.diffattn_bwd_workspace_size.restype = ctypes.c_size_t
        L.diffattn_bwd_workspace_size.argtypes = [DP]
        L.diffattn_bwd.restype = I
        L.diffattn_bwd.argtypes = [P, P, P, P, P, P, F, I, P, P, P, P, P, P, P, P, P, P,
                                   ctypes.c_size_t, DP, P]
        L.diffattn_diag.restype = I
        L.diffattn_diag.argtypes = [P, P, P, P, P, I, P, P, ctypes.c_int32, P, P, DP, P]
        _lib = L
    return _lib


def header_functions() -> list:
    """Names of the functions include/diffattn.h declares."""
    with open(_HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(diffattn_[a-z0-9_]+)\s*\(", text)))


def abi_version() -> int:
    return int(lib().diffattn_abi_version())


def _check(status: int):
    if status != OK:
        msg = lib().diffattn_status_string(status).decode()
        if status in (ERR_INVALID, ERR_UNSUPPORTED):
            raise ValueError(f"diffattn: {msg} (status {status})")
        raise DiffAttnError(status, f"diffattn: {msg}")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise ValueError(f"unsupported dtype {t.dtype}; use bfloat16 or float32")


def _stream_ptr(device: torch.device) -> Optional[int]:
    return torch.cuda.current_stream(device).cuda_stream


def _lam_tensor(lam, H: int, device) -> torch.Tensor:
    if isinstance(lam, torch.Tensor):
        t = lam.to(device=device, dtype=torch.float32).reshape(-1)
    else:
        t = torch.as_tensor(lam, dtype=torch.float32).reshape(-1).to(device)
    if t.numel() == 1:
        t = t.expand(H)
    if t.numel() != H:
        raise ValueError(f"lambda must have 1 or {H} values, got {t.numel()}")
    return t.contiguous()


def _flags(pre_norm: bool, tile_descriptors: bool) -> int:
    """DIFFATTN_FLAG_* bits: pre_norm writes D itself; tile_descriptors makes
    the kernels address every tile through its own buffer descriptor, as they
    do for (batch, head) slices of 2 GiB or more (same results)."""
    return (FLAG_PRE_NORM if pre_norm else 0) | (FLAG_TILE_DESCRIPTORS if tile_descriptors else 0)


def _require(ok: bool, msg: str):
    if not ok:
        raise ValueError(msg)


def fwd(q1: torch.Tensor, q2: torch.Tensor, k1: torch.Tensor, k2: torch.Tensor,
        v: torch.Tensor, lam: Union[float, Sequence[float], torch.Tensor],
        lambda_init: float = 0.8, causal: bool = True, eps: float = 1e-5,
        out: Optional[torch.Tensor] = None, pre_norm: bool = False,
        tile_descriptors: bool = False) -> torch.Tensor:
    """Fused prefill.  q1, q2 [B,H,Nq,d]; k1, k2 [B,H,Nk,d]; v [B,H,Nk,dv]; all
    bf16 or all fp32, contiguous, on one GPU.  lam: scalar or [H].  Returns
    out [B,H,Nq,dv] in the input dtype.  pre_norm=True returns
    D = (A1 - lam A2) V without the GroupNorm and scale; tile_descriptors, see
    _flags."""
    ts = (q1, q2, k1, k2, v)
    _require(all(t.is_cuda for t in ts), "inputs must be GPU tensors")
    _require(all(t.device == q1.device for t in ts), "inputs must share one device")
    _require(all(t.dtype == q1.dtype for t in ts), "inputs must share one dtype")
    _require(all(t.dim() == 4 for t in ts), "inputs must be [B,H,N,dim]")
    _require(all(t.is_contiguous() for t in ts), "inputs must be contiguous")
    B, H, Nq, d = q1.shape
    Nk, dv = k1.shape[2], v.shape[3]
    _require(q2.shape == (B, H, Nq, d), "q2 shape must equal q1 shape")
    _require(k1.shape == (B, H, Nk, d) and k2.shape == (B, H, Nk, d), "k1/k2 shape mismatch")
    _require(v.shape == (B, H, Nk, dv), "v shape mismatch")
    if out is None:
        out = torch.empty((B, H, Nq, dv), dtype=q1.dtype, device=q1.device)
    _require(out.shape == (B, H, Nq, dv) and out.dtype == q1.dtype and out.is_contiguous()
             and out.device == q1.device, "out must be a contiguous [B,H,Nq,dv] tensor")
    lam_t = _lam_tensor(lam, H, q1.device)
    dims = Dims(B, H, Nq, Nk, d, dv, _dtype_code(q1), float(eps),
                _flags(pre_norm, tile_descriptors))
    st = lib().diffattn_fwd(q1.data_ptr(), q2.data_ptr(), k1.data_ptr(), k2.data_ptr(),
                            v.data_ptr(), lam_t.data_ptr(), float(lambda_init), int(bool(causal)),
                            out.data_ptr(), ctypes.byref(dims), _stream_ptr(q1.device))
    _check(st)
    return out


def fwd_fp8(q1: torch.Tensor, q2: torch.Tensor, k1: torch.Tensor, k2: torch.Tensor,
            v: torch.Tensor, qk_scales: Sequence[float],
            lam: Union[float, Sequence[float], torch.Tensor], lambda_init: float = 0.8,
            causal: bool = True, eps: float = 1e-5, out: Optional[torch.Tensor] = None,
            pre_norm: bool = False, tile_descriptors: bool = False) -> torch.Tensor:
    """Prefill with e4m3 queries and keys: q1, q2, k1, k2 are
    torch.float8_e4m3fn (or uint8 codes) [B,H,N,d], v bf16 [B,H,Nk,dv] with
    (d, dv) = (64, 128) or (128, 256); qk_scales the four per-tensor
    dequantisation scales (q1, q2, k1, k2).  Returns out [B,H,Nq,dv] bf16."""
    qs = (q1, q2, k1, k2)
    _require(all(t.dtype in (torch.float8_e4m3fn, torch.uint8) for t in qs),
             "q1, q2, k1, k2 must be float8_e4m3fn (or uint8 codes)")
    _require(v.dtype == torch.bfloat16, "v must be bfloat16")
    ts = qs + (v,)
    _require(all(t.is_cuda for t in ts), "inputs must be GPU tensors")
    _require(all(t.device == q1.device for t in ts), "inputs must share one device")
    _require(all(t.dim() == 4 for t in ts), "inputs must be [B,H,N,dim]")
    _require(all(t.is_contiguous() for t in ts), "inputs must be contiguous")
    B, H, Nq, d = q1.shape
    Nk, dv = k1.shape[2], v.shape[3]
    _require(q2.shape == (B, H, Nq, d), "q2 shape must equal q1 shape")
    _require(k1.shape == (B, H, Nk, d) and k2.shape == (B, H, Nk, d), "k1/k2 shape mismatch")
    _require(v.shape == (B, H, Nk, dv), "v shape mismatch")
    sc = [float(x) for x in qk_scales]
    _require(len(sc) == 4, "qk_scales must hold 4 values (q1, q2, k1, k2)")
    if out is None:
        out = torch.empty((B, H, Nq, dv), dtype=torch.bfloat16, device=q1.device)
    _require(out.shape == (B, H, Nq, dv) and out.dtype == torch.bfloat16 and out.is_contiguous()
             and out.device == q1.device, "out must be a contiguous bf16 [B,H,Nq,dv] tensor")
    lam_t = _lam_tensor(lam, H, q1.device)
    dims = Dims(B, H, Nq, Nk, d, dv, BF16, float(eps), _flags(pre_norm, tile_descriptors))
    scales = (ctypes.c_float * 4)(*sc)
    st = lib().diffattn_fwd_fp8(q1.data_ptr(), q2.data_ptr(), k1.data_ptr(), k2.data_ptr(),
                                v.data_ptr(), scales, lam_t.data_ptr(), float(lambda_init),
                                int(bool(causal)), out.data_ptr(), ctypes.byref(dims),
                                _stream_ptr(q1.device))
    _check(st)
    return out


def qkv_proj(x: torch.Tensor, w: torch.Tensor, heads: int, head_dim: int, v_dim: int,
             out: Optional[Sequence[torch.Tensor]] = None):
    """Fused projections: x [B,N,d_model] bf16, w [heads*(4 d + dv), d_model]
    bf16 (per head the Q1, Q2, K1, K2, V output rows in that order).  Returns
    (q1, q2, k1, k2, v) with q*, k* [B,H,N,d] and v [B,H,N,dv], ready for
    ``fwd``."""
    _require(x.is_cuda and w.is_cuda and x.device == w.device, "x and w must be on one GPU")
    _require(x.dtype == torch.bfloat16 and w.dtype == torch.bfloat16, "x and w must be bfloat16")
    _require(x.dim() == 3 and w.dim() == 2, "x must be [B,N,d_model] and w [n_out,d_model]")
    _require(x.is_contiguous() and w.is_contiguous(), "x and w must be contiguous")
    B, N, dm = x.shape
    H, d, dv = int(heads), int(head_dim), int(v_dim)
    _require(w.shape == (H * (4 * d + dv), dm), "w must be [heads*(4 d + dv), d_model]")
    shapes = [(B, H, N, d)] * 4 + [(B, H, N, dv)]
    if out is None:
        out = [torch.empty(s, dtype=torch.bfloat16, device=x.device) for s in shapes]
    _require(len(out) == 5 and all(o.shape == s and o.dtype == torch.bfloat16
                                   and o.is_contiguous() and o.device == x.device
                                   for o, s in zip(out, shapes)),
             "out must be five contiguous bf16 tensors of the output shapes")
    st = lib().diffattn_qkv_proj(x.data_ptr(), w.data_ptr(), B, N, H, d, dv, dm,
                                 *[o.data_ptr() for o in out], _stream_ptr(x.device))
    _check(st)
    return tuple(out)


def _check_inputs(q1, q2, k1, k2, v):
    ts = (q1, q2, k1, k2, v)
    _require(all(t.is_cuda for t in ts), "inputs must be GPU tensors")
    _require(all(t.device == q1.device for t in ts), "inputs must share one device")
    _require(all(t.dtype == q1.dtype for t in ts), "inputs must share one dtype")
    _require(all(t.dim() == 4 for t in ts), "inputs must be [B,H,N,dim]")
    _require(all(t.is_contiguous() for t in ts), "inputs must be contiguous")
    B, H, Nq, d = q1.shape
    Nk, dv = k1.shape[2], v.shape[3]
    _require(q2.shape == (B, H, Nq, d), "q2 shape must equal q1 shape")
    _require(k1.shape == (B, H, Nk, d) and k2.shape == (B, H, Nk, d), "k1/k2 shape mismatch")
    _require(v.shape == (B, H, Nk, dv), "v shape mismatch")
    return B, H, Nq, Nk, d, dv


def fwd_train(q1: torch.Tensor, q2: torch.Tensor, k1: torch.Tensor, k2: torch.Tensor,
              v: torch.Tensor, lam: Union[float, Sequence[float], torch.Tensor],
              lambda_init: float = 0.8, causal: bool = True, eps: float = 1e-5,
              pre_norm: bool = False, tile_descriptors: bool = False):
    """Training forward (bf16, d = 32, 64 or 128): returns (out, d_save, lse) with
    d_save = D [B,H,Nq,dv] fp32 and lse [2,B,H,Nq] fp32 (natural-log
    log-sum-exp of each map's score rows), the inputs of ``bwd``."""
    B, H, Nq, Nk, d, dv = _check_inputs(q1, q2, k1, k2, v)
    dev = q1.device
    out = torch.empty((B, H, Nq, dv), dtype=q1.dtype, device=dev)
    d_save = torch.empty((B, H, Nq, dv), dtype=torch.float32, device=dev)
    lse = torch.empty((2, B, H, Nq), dtype=torch.float32, device=dev)
    lam_t = _lam_tensor(lam, H, dev)
    dims = Dims(B, H, Nq, Nk, d, dv, _dtype_code(q1), float(eps),
                _flags(pre_norm, tile_descriptors))
    st = lib().diffattn_fwd_train(q1.data_ptr(), q2.data_ptr(), k1.data_ptr(), k2.data_ptr(),
                                  v.data_ptr(), lam_t.data_ptr(), float(lambda_init),
                                  int(bool(causal)), out.data_ptr(), d_save.data_ptr(),
                                  lse.data_ptr(), ctypes.byref(dims), _stream_ptr(dev))
    _check(st)
    return out, d_save, lse


def bwd_workspace_size(B: int, H: int, Nq: int, Nk: int, d: int, dv: int) -> int:
    """Bytes of device workspace ``bwd`` needs (bf16 sizes)."""
    dims = Dims(B, H, Nq, Nk, d, dv, BF16, 1e-5, 0)
    return int(lib().diffattn_bwd_workspace_size(ctypes.byref(dims)))


def bwd(q1: torch.Tensor, q2: torch.Tensor, k1: torch.Tensor, k2: torch.Tensor,
        v: torch.Tensor, lam: Union[float, Sequence[float], torch.Tensor], dout: torch.Tensor,
        d_save: torch.Tensor, lse: torch.Tensor, lambda_init: float = 0.8, causal: bool = True,
        eps: float = 1e-5, pre_norm: bool = False, workspace: Optional[torch.Tensor] = None,
        tile_descriptors: bool = False):
    """Backward of ``fwd_train`` (same arguments): gradients of sum(dout * out).
    Returns (dq1, dq2, dk1, dk2, dv) in the input dtype and dlambda [H] fp32
    (summed over batch and rows; sum it for a scalar lambda)."""
    B, H, Nq, Nk, d, dv = _check_inputs(q1, q2, k1, k2, v)
    dev = q1.device
    _require(dout.shape == (B, H, Nq, dv) and dout.dtype == q1.dtype and dout.is_contiguous()
             and dout.device == dev, "dout must be a contiguous [B,H,Nq,dv] tensor like out")
    _require(d_save.shape == (B, H, Nq, dv) and d_save.dtype == torch.float32
             and d_save.is_contiguous(), "d_save must be the fp32 [B,H,Nq,dv] from fwd_train")
    _require(lse.shape == (2, B, H, Nq) and lse.dtype == torch.float32 and lse.is_contiguous(),
             "lse must be the fp32 [2,B,H,Nq] from fwd_train")
    grads = [torch.empty_like(t) for t in (q1, q2, k1, k2, v)]
    dlam = torch.empty((H,), dtype=torch.float32, device=dev)
    dims = Dims(B, H, Nq, Nk, d, dv, _dtype_code(q1), float(eps),
                _flags(pre_norm, tile_descriptors))
    need = int(lib().diffattn_bwd_workspace_size(ctypes.byref(dims)))
    if workspace is None:
        workspace = torch.empty((max(need, 16),), dtype=torch.uint8, device=dev)
    lam_t = _lam_tensor(lam, H, dev)
    st = lib().diffattn_bwd(q1.data_ptr(), q2.data_ptr(), k1.data_ptr(), k2.data_ptr(),
                            v.data_ptr(), lam_t.data_ptr(), float(lambda_init), int(bool(causal)),
                            dout.data_ptr(), d_save.data_ptr(), lse.data_ptr(),
                            *[g.data_ptr() for g in grads], dlam.data_ptr(), workspace.data_ptr(),
                            workspace.numel() * workspace.element_size(), ctypes.byref(dims),
                            _stream_ptr(dev))
    _check(st)
    return (*grads, dlam)


def diag(q1: torch.Tensor, q2: torch.Tensor, k1: torch.Tensor, k2: torch.Tensor,
         v: torch.Tensor, causal: bool = True, lse: Optional[torch.Tensor] = None,
         needle_q: Optional[torch.Tensor] = None, needle_k: Optional[torch.Tensor] = None,
         row_max: bool = True):
    """Diagnostics of the two maps (bf16).  Returns (row_max [2,B,H,Nq] fp32 or
    None, needles [B,H,n,4] fp32 or None).  needle_q/needle_k: int [B,H,n]
    (query, key) pairs; needles need ``lse`` from ``fwd_train``.  v only
    supplies dv for the size checks."""
    B, H, Nq, Nk, d, dv = _check_inputs(q1, q2, k1, k2, v)
    dev = q1.device
    rm = torch.empty((2, B, H, Nq), dtype=torch.float32, device=dev) if row_max else None
    nd = None
    n = 0
    if needle_q is not None:
        _require(lse is not None and lse.shape == (2, B, H, Nq) and lse.dtype == torch.float32,
                 "needles need the fp32 [2,B,H,Nq] lse of fwd_train")
        needle_q = needle_q.to(device=dev, dtype=torch.int32).contiguous()
        needle_k = needle_k.to(device=dev, dtype=torch.int32).contiguous()
        _require(needle_q.dim() == 3 and needle_q.shape[:2] == (B, H)
                 and needle_k.shape == needle_q.shape, "needle_q/needle_k must be [B,H,n]")
        n = needle_q.shape[2]
        nd = torch.empty((B, H, n, 4), dtype=torch.float32, device=dev)
    dims = Dims(B, H, Nq, Nk, d, dv, _dtype_code(q1), 1e-5, 0)
    st = lib().diffattn_diag(q1.data_ptr(), q2.data_ptr(), k1.data_ptr(), k2.data_ptr(),
                             lse.data_ptr() if (lse is not None and nd is not None) else None,
                             int(bool(causal)),
                             needle_q.data_ptr() if nd is not None else None,
                             needle_k.data_ptr() if nd is not None else None, n,
                             rm.data_ptr() if rm is not None else None,
                             nd.data_ptr() if nd is not None else None,
                             ctypes.byref(dims), _stream_ptr(dev))
    _check(st)
    return rm, nd


def _decode_dims(B, H, L, d, dv, dtype_code, eps, pre_norm) -> Dims:
    return Dims(B, H, 1, L, d, dv, dtype_code, float(eps), FLAG_PRE_NORM if pre_norm else 0)


def decode_default_splits(B: int, H: int, L: int, d: int, dv: int) -> int:
    """Split count the library picks for these sizes on the current device."""
    return int(lib().diffattn_decode_default_splits(
        ctypes.byref(_decode_dims(B, H, L, d, dv, BF16, 1e-5, False))))


def decode_workspace_size(B: int, H: int, L: int, d: int, dv: int, num_splits: int = 0) -> int:
    return int(lib().diffattn_decode_workspace_size(
        ctypes.byref(_decode_dims(B, H, L, d, dv, BF16, 1e-5, False)), int(num_splits)))


def _decode_prep(q1, q2, k1_cache, k2_cache, v_cache, lam, kv_len, kv_lens, eps, out, pre_norm):
    ts = (q1, q2, k1_cache, k2_cache, v_cache)
    _require(all(t.is_cuda for t in ts), "inputs must be GPU tensors")
    _require(all(t.device == q1.device for t in ts), "inputs must share one device")
    _require(all(t.dtype == q1.dtype for t in ts), "inputs must share one dtype")
    _require(all(t.is_contiguous() for t in ts), "inputs must be contiguous")
    _require(q1.dim() == 3 and k1_cache.dim() == 4 and v_cache.dim() == 4, "bad ranks")
    B, H, d = q1.shape
    cap, dv = k1_cache.shape[2], v_cache.shape[3]
    _require(q2.shape == (B, H, d), "q2 shape must equal q1 shape")
    _require(k1_cache.shape == (B, H, cap, d) and k2_cache.shape == (B, H, cap, d),
             "k caches shape mismatch")
    _require(v_cache.shape == (B, H, cap, dv), "v cache shape mismatch")
    L = cap if kv_len is None else int(kv_len)
    if kv_lens is not None:
        _require(kv_lens.is_cuda and kv_lens.dtype == torch.int32 and kv_lens.numel() == B
                 and kv_lens.is_contiguous(), "kv_lens must be a contiguous int32 [B] GPU tensor")
    if out is None:
        out = torch.empty((B, H, dv), dtype=q1.dtype, device=q1.device)
    _require(out.shape == (B, H, dv) and out.dtype == q1.dtype and out.is_contiguous(),
             "out must be a contiguous [B,H,dv] tensor")
    lam_t = _lam_tensor(lam, H, q1.device)
    dims = _decode_dims(B, H, L, d, dv, _dtype_code(q1), eps, pre_norm)
    return cap, out, lam_t, dims


def decode(q1: torch.Tensor, q2: torch.Tensor, k1_cache: torch.Tensor, k2_cache: torch.Tensor,
           v_cache: torch.Tensor, lam, lambda_init: float = 0.8, kv_len: Optional[int] = None,
           kv_lens: Optional[torch.Tensor] = None, num_splits: int = 0, eps: float = 1e-5,
           out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
           pre_norm: bool = False) -> torch.Tensor:
    """KV-cache decode.  q1, q2 [B,H,d]; caches [B,H,cap,d] / [B,H,cap,dv].
    kv_len: cache length used (default: cap); kv_lens: optional int32 [B] of
    per-sequence lengths (clamped to [0, kv_len]).  Returns out [B,H,dv]."""
    cap, out, lam_t, dims = _decode_prep(q1, q2, k1_cache, k2_cache, v_cache, lam, kv_len,
                                         kv_lens, eps, out, pre_norm)
    need = int(lib().diffattn_decode_workspace_size(ctypes.byref(dims), int(num_splits)))
    ws_ptr, ws_bytes = None, 0
    if need > 0:
        if workspace is None or workspace.numel() * workspace.element_size() < need:
            workspace = torch.empty(need, dtype=torch.uint8, device=q1.device)
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    st = lib().diffattn_decode(q1.data_ptr(), q2.data_ptr(), k1_cache.data_ptr(),
                               k2_cache.data_ptr(), v_cache.data_ptr(), cap,
                               kv_lens.data_ptr() if kv_lens is not None else None,
                               lam_t.data_ptr(), float(lambda_init), out.data_ptr(), ws_ptr,
                               ws_bytes, int(num_splits), ctypes.byref(dims),
                               _stream_ptr(q1.device))
    _check(st)
    return out


def decode_noalloc(q1: torch.Tensor, q2: torch.Tensor, k1_cache: torch.Tensor,
                   k2_cache: torch.Tensor, v_cache: torch.Tensor, lam, lambda_init: float = 0.8,
                   kv_len: Optional[int] = None, kv_lens: Optional[torch.Tensor] = None,
                   num_splits: int = 0, eps: float = 1e-5, out: Optional[torch.Tensor] = None,
                   pre_norm: bool = False) -> torch.Tensor:
    """As decode, through diffattn_decode_noalloc: no workspace; the library's
    fixed scratch array (NOALLOC_SCRATCH_BYTES per GPU) holds the split-K
    partials.  Pass `out` (and a device lambda) for a call that allocates
    nothing at all."""
    cap, out, lam_t, dims = _decode_prep(q1, q2, k1_cache, k2_cache, v_cache, lam, kv_len,
                                         kv_lens, eps, out, pre_norm)
    st = lib().diffattn_decode_noalloc(q1.data_ptr(), q2.data_ptr(), k1_cache.data_ptr(),
                                       k2_cache.data_ptr(), v_cache.data_ptr(), cap,
                                       kv_lens.data_ptr() if kv_lens is not None else None,
                                       lam_t.data_ptr(), float(lambda_init), out.data_ptr(),
                                       int(num_splits), ctypes.byref(dims),
                                       _stream_ptr(q1.device))
    _check(st)
    return out
