"""Python binding of libattn.so, the gfx950 attention library (C ABI in include/attn.h).

The functions named like the C entry points (``attn_fwd``, ``attn_fwd_qk``,
``attn_fwd_splitkv`` and its two size helpers, ``attn_fwd_splitkv_noalloc``, ``attn_fwd_fp8``, ``attn_bwd``, ``attn_bwd_qk``,
``attn_bwd_preprocess``, ``attn_bwd_dkdv``, ``attn_bwd_dq``, ``attn_bwd_dq_delta``,
``attn_status_string``) only marshal arguments: tensors become device
pointers, ``stream=None`` becomes the current PyTorch stream of the tensors'
device, and a nonzero status becomes :class:`AttnError`.  Every step of the
computation runs in the library's HIP kernels; there is no fallback.  If the
library has not been built the first call raises.

``fwd`` and ``bwd`` are conveniences that check dtypes, devices and
contiguity and allocate the outputs with ``torch.empty``; q may have a
different number of rows than k and v (causal masks then align to the
bottom-right corner) and a multiple of their number of heads (grouped-query
attention).  ``fwd_fp8`` does the same for 8-bit (e4m3) inputs with per-head
scales.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libattn.so")

ATTN_OK = 0
ATTN_ERR_NULLPTR = 1
ATTN_ERR_BAD_SHAPE = 2
ATTN_ERR_UNSUPPORTED_D = 3
ATTN_ERR_MISALIGNED = 4
ATTN_ERR_BAD_SCALE = 5
ATTN_ERR_BAD_ARG = 6
ATTN_ERR_ALIAS = 7
ATTN_ERR_HIP = 8
ATTN_ERR_WORKSPACE = 9
ATTN_ERR_SCRATCH = 10
# bytes of the static device buffer attn_fwd_splitkv_noalloc keeps its pieces in
ATTN_NOALLOC_SCRATCH_BYTES = 16 << 20

_lock = threading.Lock()
_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float

_SIGNATURES = {
    "attn_fwd": [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _P],
    "attn_fwd_qk": [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _P],
    "attn_bwd_qk": [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _P],
    "attn_fwd_splitkv": [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _I, _P, ctypes.c_longlong, _P],
    "attn_fwd_splitkv_noalloc": [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _I, _P],
    "attn_fwd_fp8": [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _P],
    "attn_bwd": [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _P],
    "attn_bwd_preprocess": [_P, _P, _P, _I, _I, _I, _I, _P],
    "attn_bwd_dkdv": [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _P],
    "attn_bwd_dq": [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _P],
    "attn_bwd_dq_delta": [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _P],
}


class AttnError(RuntimeError):
    def __init__(self, name: str, status: int):
        self.status = status
        msg = "%s failed with status %d: %s" % (name, status, attn_status_string(status))
        if status == ATTN_ERR_HIP:
            msg += " (hipError_t %d)" % library().attn_last_hip_error()
        super().__init__(msg)


def library() -> ctypes.CDLL:
    """Load libattn.so (once).  Raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError("libattn.so is not built (%s); build it with "
                                   "`python -m tiled_online_softmax_02_amd.build`" % LIB_PATH)
            lib = ctypes.CDLL(LIB_PATH)
            for name, args in _SIGNATURES.items():
                fn = getattr(lib, name)
                fn.argtypes = args
                fn.restype = _I
            lib.attn_status_string.argtypes = [_I]
            lib.attn_status_string.restype = ctypes.c_char_p
            lib.attn_last_hip_error.argtypes = []
            lib.attn_last_hip_error.restype = _I
            lib.attn_fwd_splitkv_workspace_size.argtypes = [_I, _I, _I, _I, _I]
            lib.attn_fwd_splitkv_workspace_size.restype = ctypes.c_longlong
            lib.attn_fwd_splitkv_default_splits.argtypes = [_I, _I, _I, _I, _I]
            lib.attn_fwd_splitkv_default_splits.restype = _I
            lib.attn_fwd_splitkv_default_splits_qk.argtypes = [_I, _I, _I, _I, _I, _I]
            lib.attn_fwd_splitkv_default_splits_qk.restype = _I
            _lib = lib
    return _lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, torch.Tensor):
        return x.data_ptr() or None
    return int(x) or None


def _stream(stream, *tensors):
    if stream is not None:
        return stream.cuda_stream if isinstance(stream, torch.cuda.Stream) else int(stream)
    for t in tensors:
        if isinstance(t, torch.Tensor) and t.is_cuda:
            return torch.cuda.current_stream(t.device).cuda_stream
    return None


def _call(name: str, *args) -> None:
    rc = getattr(library(), name)(*args)
    if rc != ATTN_OK:
        raise AttnError(name, rc)


def attn_status_string(status: int) -> str:
    return library().attn_status_string(int(status)).decode()


def attn_fwd(q, k, v, o, lse, B, H, N, d, causal, scale, stream=None) -> None:
    _call("attn_fwd", _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d, int(causal), float(scale),
          _stream(stream, q, o))


def attn_fwd_qk(q, k, v, o, lse, B, H, Hk, Nq, Nk, d, causal, scale, stream=None) -> None:
    _call("attn_fwd_qk", _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Hk, Nq, Nk, d, int(causal),
          float(scale), _stream(stream, q, o))


def attn_fwd_splitkv(q, k, v, o, lse, B, H, Hk, Nq, Nk, d, causal, scale, num_splits, workspace, workspace_bytes,
                     stream=None) -> None:
    _call("attn_fwd_splitkv", _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Hk, Nq, Nk, d, int(causal),
          float(scale), int(num_splits), _ptr(workspace), int(workspace_bytes), _stream(stream, q, o))


def attn_fwd_splitkv_noalloc(q, k, v, o, lse, B, H, Hk, Nq, Nk, d, causal, scale, num_splits, stream=None) -> None:
    _call("attn_fwd_splitkv_noalloc", _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Hk, Nq, Nk, d,
          int(causal), float(scale), int(num_splits), _stream(stream, q, o))


def attn_fwd_splitkv_workspace_size(B, H, Nq, d, num_splits) -> int:
    return int(library().attn_fwd_splitkv_workspace_size(B, H, Nq, d, num_splits))


def attn_fwd_splitkv_default_splits(B, H, Nq, Nk, d) -> int:
    return int(library().attn_fwd_splitkv_default_splits(B, H, Nq, Nk, d))


def attn_fwd_splitkv_default_splits_qk(B, H, Hk, Nq, Nk, d) -> int:
    return int(library().attn_fwd_splitkv_default_splits_qk(B, H, Hk, Nq, Nk, d))


def attn_fwd_fp8(q, k, v, descale_q, descale_k, descale_v, o, lse, B, H, Hk, Nq, Nk, d, causal, scale,
                 stream=None) -> None:
    _call("attn_fwd_fp8", _ptr(q), _ptr(k), _ptr(v), _ptr(descale_q), _ptr(descale_k), _ptr(descale_v), _ptr(o),
          _ptr(lse), B, H, Hk, Nq, Nk, d, int(causal), float(scale), _stream(stream, q, o))


def attn_bwd_qk(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, Hk, Nq, Nk, d, causal, scale, stream=None) -> None:
    _call("attn_bwd_qk", _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
          _ptr(delta), B, H, Hk, Nq, Nk, d, int(causal), float(scale), _stream(stream, q, dq, dk))


def attn_bwd(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, N, d, causal, scale, stream=None) -> None:
    _call("attn_bwd", _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
          _ptr(delta), B, H, N, d, int(causal), float(scale), _stream(stream, q, dq))


def attn_bwd_preprocess(o, dout, delta, B, H, N, d, stream=None) -> None:
    _call("attn_bwd_preprocess", _ptr(o), _ptr(dout), _ptr(delta), B, H, N, d, _stream(stream, o, delta))


def attn_bwd_dkdv(q, k, v, dout, lse, delta, dk, dv, B, H, N, d, causal, scale, stream=None) -> None:
    _call("attn_bwd_dkdv", _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(lse), _ptr(delta), _ptr(dk), _ptr(dv),
          B, H, N, d, int(causal), float(scale), _stream(stream, q, dk))


def attn_bwd_dq(q, k, v, dout, lse, delta, dq, B, H, N, d, causal, scale, stream=None) -> None:
    _call("attn_bwd_dq", _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(lse), _ptr(delta), _ptr(dq), B, H, N, d,
          int(causal), float(scale), _stream(stream, q, dq))


def attn_bwd_dq_delta(q, k, v, o, dout, lse, delta, dq, B, H, N, d, causal, scale, stream=None) -> None:
    _call("attn_bwd_dq_delta", _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(delta), _ptr(dq),
          B, H, N, d, int(causal), float(scale), _stream(stream, q, dq))


def _check_inputs(q, k, v, *q_like):
    """q (and o, dO) are [B, H, Nq, d]; k and v are [B, Hk, Nk, d] with H a multiple of Hk."""
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("expected [B, H, N, d] tensors")
    for t in (q, k, v, *q_like):
        if t.dtype != torch.bfloat16:
            raise TypeError("tensors must be bfloat16")
        if not t.is_cuda or t.device != q.device:
            raise ValueError("tensors must be on the same GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    B, H, _, d = q.shape
    Hk = k.shape[1]
    if k.shape[0] != B or k.shape[3] != d or v.shape != k.shape or Hk < 1 or H % Hk:
        raise ValueError("k and v must be [B, Hk, Nk, d] with the B and d of q and H a multiple of Hk")
    for t in q_like:
        if t.shape != q.shape:
            raise ValueError("o and dO must have the shape of q")


def default_scale(d: int) -> float:
    import numpy as np
    return float(np.float32(1.0 / (d ** 0.5)))


def fwd(q, k, v, causal: bool = False, scale: float | None = None, stream=None):
    """Forward pass; returns (o bf16 [B,H,Nq,d], lse fp32 [B,H,Nq])."""
    _check_inputs(q, k, v)
    B, H, Nq, d = q.shape
    Hk, Nk = k.shape[1], k.shape[2]
    scale = default_scale(d) if scale is None else scale
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    if Nq == Nk and H == Hk:
        attn_fwd(q, k, v, o, lse, B, H, Nq, d, causal, scale, stream)
    else:
        attn_fwd_qk(q, k, v, o, lse, B, H, Hk, Nq, Nk, d, causal, scale, stream)
    return o, lse


def fwd_splitkv(q, k, v, causal: bool = False, scale: float | None = None, num_splits: int | None = None,
                stream=None):
    """Split-key forward (few query rows, many keys); returns (o, lse) like ``fwd``.  The
    workspace for the pieces is a ``torch.empty`` uint8 buffer of the size the library asks for."""
    _check_inputs(q, k, v)
    B, H, Nq, d = q.shape
    Hk, Nk = k.shape[1], k.shape[2]
    scale = default_scale(d) if scale is None else scale
    if num_splits is None:
        num_splits = attn_fwd_splitkv_default_splits_qk(B, H, Hk, Nq, Nk, d)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    nbytes = attn_fwd_splitkv_workspace_size(B, H, Nq, d, num_splits)
    if nbytes < 0:
        raise ValueError("invalid arguments for the split-key forward")
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    attn_fwd_splitkv(q, k, v, o, lse, B, H, Hk, Nq, Nk, d, causal, scale, num_splits, ws, nbytes, stream)
    return o, lse


def bwd(q, k, v, o, dout, lse, causal: bool = False, scale: float | None = None, stream=None):
    """Backward pass; returns (dq [B,H,Nq,d], dk, dv [B,Hk,Nk,d]), bf16."""
    _check_inputs(q, k, v, o, dout)
    B, H, Nq, d = q.shape
    Hk, Nk = k.shape[1], k.shape[2]
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, Nq) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, H, Nq] tensor")
    scale = default_scale(d) if scale is None else scale
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    delta = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    if Nq == Nk and H == Hk:
        attn_bwd(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, Nq, d, causal, scale, stream)
    else:
        attn_bwd_qk(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, Hk, Nq, Nk, d, causal, scale, stream)
    return dq, dk, dv


def fwd_fp8(q8, k8, v8, descale_q, descale_k, descale_v, causal: bool = False, scale: float | None = None,
            stream=None):
    """Forward pass on e4m3 inputs: q8 [B,H,Nq,d], k8 and v8 [B,Hk,Nk,d] (torch.float8_e4m3fn or uint8
    codes), descale_q [B,H], descale_k and descale_v [B,Hk] (float32, the per-head scales).
    Returns (o bf16 [B,H,Nq,d], lse fp32 [B,H,Nq])."""
    if q8.dim() != 4 or k8.dim() != 4 or v8.dim() != 4:
        raise ValueError("expected [B, H, N, d] tensors")
    for t in (q8, k8, v8):
        if t.dtype not in (torch.float8_e4m3fn, torch.uint8):
            raise TypeError("8-bit inputs must be float8_e4m3fn (or their uint8 codes)")
    for t in (q8, k8, v8, descale_q, descale_k, descale_v):
        if not t.is_cuda or t.device != q8.device:
            raise ValueError("tensors must be on the same GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    B, H, Nq, d = q8.shape
    Hk, Nk = k8.shape[1], k8.shape[2]
    if k8.shape[0] != B or k8.shape[3] != d or v8.shape != k8.shape or Hk < 1 or H % Hk:
        raise ValueError("k8 and v8 must be [B, Hk, Nk, d] with the B and d of q8 and H a multiple of Hk")
    for t, heads in ((descale_q, H), (descale_k, Hk), (descale_v, Hk)):
        if t.dtype != torch.float32 or tuple(t.shape) != (B, heads):
            raise ValueError("descale_q must be float32 [B, H], descale_k and descale_v float32 [B, Hk]")
    scale = default_scale(d) if scale is None else scale
    o = torch.empty((B, H, Nq, d), dtype=torch.bfloat16, device=q8.device)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q8.device)
    attn_fwd_fp8(q8, k8, v8, descale_q, descale_k, descale_v, o, lse, B, H, Hk, Nq, Nk, d, causal, scale, stream)
    return o, lse
