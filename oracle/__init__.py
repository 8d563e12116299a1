"""TEST INFRASTRUCTURE ONLY: ctypes binding of the fp64 CPU attention oracle.

The oracle (``attn_oracle.c`` beside this file) is a plain, slow, obviously
correct implementation of exact scaled-dot-product attention in fp64.  Only
``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package; the GPU library never does, and the two
share no code.

Every array is a C-contiguous float64 numpy array.  Shapes: q, dO, o, dq
``[B, H, nq, d]``; k, v, dk, dv ``[B, H, nk, d]``; lse and D ``[B, H, nq]``.

The functions follow these pages (cited by title and section):

* "digest_existing.txt" (xtrax package), answer q02_flashattention, sections 1
  and 2: materialised S and P; the running max / exp-sum merge rule;
  initialisation l = 0, m = -inf, O = 0.
* "GPU Programming and Kernel Optimization" (ai.engineer), items 51, 57, 58,
  59 and 60: row softmax, the online normaliser, blockwise rescaling of the
  outputs, bottom-right causal alignment with zero output for fully masked
  rows, and the -inf guards.
* 8-bit inputs: "FlashAttention v3 (Tri Dao et al.)", section "What it is" (FP8
  input types); "CUTLASS WGMMA Atom Skeleton", table "Atom Family Names Seen In
  CUTLASS" (FP8 products take e4m3 or e5m2); [gpko] item 33 (affine
  quantisation, real value = scale * (code - zero point)).  The e4m3 code itself
  is decoded by its OCP definition, written out in ``attn_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

_D = ctypes.POINTER(ctypes.c_double)
_L = ctypes.POINTER(ctypes.c_long)


def build(force: bool = False) -> str:
    """Compile ``attn_oracle.c`` into ``liboracle.so`` with gcc (fp64, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-pthread", "-fno-fast-math",
               _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB_PATH)
            lib.oracle_softmax_rows.argtypes = [_D, ctypes.c_long, ctypes.c_long, _D, _D]
            lib.oracle_online_merge.argtypes = [_D, ctypes.c_long, _L, ctypes.c_long, _D, _D]
            lib.oracle_online_normalizer.argtypes = [_D, ctypes.c_long, _D, _D]
            lib.oracle_attn_fwd.argtypes = [_D, _D, _D, _D, _D, _D, ctypes.c_long, ctypes.c_long, ctypes.c_long,
                                            ctypes.c_long, ctypes.c_long, ctypes.c_int, ctypes.c_double, ctypes.c_int]
            lib.oracle_attn_fwd_rows.argtypes = [_D, _L, ctypes.c_long, _D, _D, ctypes.c_long, ctypes.c_long,
                                                 ctypes.c_long, ctypes.c_int, ctypes.c_double, _D, _D]
            lib.oracle_attn_fwd_blockwise.argtypes = [_D, _D, _D, ctypes.c_long, ctypes.c_long, ctypes.c_long,
                                                      ctypes.c_int, ctypes.c_double, ctypes.c_long, ctypes.c_long,
                                                      _D, _D, _D, _D]
            lib.oracle_attn_bwd.argtypes = [_D, _D, _D, _D, _D, _D, _D, _D, ctypes.c_long, ctypes.c_long,
                                            ctypes.c_long, ctypes.c_long, ctypes.c_long, ctypes.c_int,
                                            ctypes.c_double, ctypes.c_int]
            lib.oracle_fp8_e4m3_decode.argtypes = [ctypes.POINTER(ctypes.c_ubyte), ctypes.c_long, _D]
            for name in ("oracle_softmax_rows", "oracle_online_merge", "oracle_online_normalizer",
                         "oracle_attn_fwd", "oracle_attn_fwd_rows", "oracle_attn_fwd_blockwise",
                         "oracle_attn_bwd", "oracle_fp8_e4m3_decode"):
                getattr(lib, name).restype = ctypes.c_int
            _lib = lib
    return _lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _p(a):
    return None if a is None else a.ctypes.data_as(_D)


def _check(rc: int, name: str) -> None:
    if rc != 0:
        raise ValueError("oracle %s rejected its arguments (status %d)" % (name, rc))


def default_threads() -> int:
    return max(1, min(os.cpu_count() or 1, 16))


def softmax_rows(x):
    """Row softmax of a 2-D array; returns (P, lse).  Rows of all -inf give zeros and lse = -inf."""
    x = _f64(x)
    rows, cols = x.shape
    p = np.empty_like(x)
    lse = np.empty(rows)
    _check(_load().oracle_softmax_rows(_p(x), rows, cols, _p(p), _p(lse)), "softmax_rows")
    return p, lse


def online_merge(x, cuts):
    """Max and exp-sum of vector x, built block by block with the merge rule."""
    x = _f64(x).ravel()
    c = np.ascontiguousarray(np.asarray(cuts, dtype=np.int64))
    m, l = ctypes.c_double(), ctypes.c_double()
    _check(_load().oracle_online_merge(_p(x), x.size, c.ctypes.data_as(_L), c.size, ctypes.byref(m),
                                       ctypes.byref(l)), "online_merge")
    return m.value, l.value


def online_normalizer(x):
    """Max and exp-sum of vector x by the element-at-a-time online normaliser."""
    x = _f64(x).ravel()
    m, d = ctypes.c_double(), ctypes.c_double()
    _check(_load().oracle_online_normalizer(_p(x), x.size, ctypes.byref(m), ctypes.byref(d)), "online_normalizer")
    return m.value, d.value


def attn_fwd(q, k, v, causal: bool, scale: float, want_p: bool = False, nthreads: int | None = None):
    """Forward pass by the definition.  Returns (O, lse) or (O, lse, P)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, nq, d = q.shape
    nk = k.shape[2]
    assert k.shape == (B, H, nk, d) and v.shape == (B, H, nk, d)
    o = np.empty((B, H, nq, d))
    lse = np.empty((B, H, nq))
    p = np.empty((B, H, nq, nk)) if want_p else None
    _check(_load().oracle_attn_fwd(_p(q), _p(k), _p(v), _p(o), _p(lse), _p(p), B, H, nq, nk, d, int(bool(causal)),
                                   float(scale), nthreads or default_threads()), "attn_fwd")
    return (o, lse, p) if want_p else (o, lse)


def attn_fwd_rows(q_rows, row_idx, k_head, v_head, nq: int, causal: bool, scale: float):
    """Forward pass for selected query rows of one head.

    q_rows [R, d] are the query vectors of rows ``row_idx`` (0-based, < nq);
    k_head, v_head [nk, d].  Returns (O_rows [R, d], lse_rows [R])."""
    q_rows, k_head, v_head = _f64(q_rows), _f64(k_head), _f64(v_head)
    idx = np.ascontiguousarray(np.asarray(row_idx, dtype=np.int64))
    R, d = q_rows.shape
    nk = k_head.shape[0]
    o = np.empty((R, d))
    lse = np.empty(R)
    _check(_load().oracle_attn_fwd_rows(_p(q_rows), idx.ctypes.data_as(_L), R, _p(k_head), _p(v_head), nq, nk, d,
                                        int(bool(causal)), float(scale), _p(o), _p(lse)), "attn_fwd_rows")
    return o, lse


def attn_fwd_blockwise(q_head, k_head, v_head, causal: bool, scale: float, br: int, bc: int):
    """FlashAttention's blockwise forward for one head ([nq,d], [nk,d], [nk,d]).

    Returns (O, lse, m, l) with the final running statistics."""
    q, k, v = _f64(q_head), _f64(k_head), _f64(v_head)
    nq, d = q.shape
    nk = k.shape[0]
    o = np.empty((nq, d))
    lse, m, l = np.empty(nq), np.empty(nq), np.empty(nq)
    _check(_load().oracle_attn_fwd_blockwise(_p(q), _p(k), _p(v), nq, nk, d, int(bool(causal)), float(scale),
                                             br, bc, _p(o), _p(lse), _p(m), _p(l)), "attn_fwd_blockwise")
    return o, lse, m, l


def attn_bwd(q, k, v, dout, causal: bool, scale: float, nthreads: int | None = None):
    """Backward pass by the chain rule of the definition.  Returns (dQ, dK, dV, D)."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, H, nq, d = q.shape
    nk = k.shape[2]
    assert dout.shape == q.shape and k.shape == (B, H, nk, d) and v.shape == k.shape
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    dvec = np.empty((B, H, nq))
    _check(_load().oracle_attn_bwd(_p(q), _p(k), _p(v), _p(dout), _p(dq), _p(dk), _p(dv), _p(dvec), B, H, nq, nk,
                                   d, int(bool(causal)), float(scale), nthreads or default_threads()), "attn_bwd")
    return dq, dk, dv, dvec


def attn_bwd_matmul(q, k, v, dout, causal: bool, scale: float, nthreads: int | None = None):
    """The same backward formulas as :func:`attn_bwd`, with each product done by numpy's fp64 matmul.

    P comes from the definitional forward pass (:func:`attn_fwd` with ``want_p``); then, per head,
    dV = P^T dO, dP = dO V^T, D = rowsum(P * dP), dS = P * (dP - D), dQ = scale dS K,
    dK = scale dS^T Q.  Used for large heads, where the plain loops of :func:`attn_bwd` are slow.
    Returns (dQ, dK, dV, D)."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, H, nq, d = q.shape
    nk = k.shape[2]
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    dvec = np.empty((B, H, nq))
    for b in range(B):
        for h in range(H):
            sl = (slice(b, b + 1), slice(h, h + 1))
            _, _, p = attn_fwd(q[sl], k[sl], v[sl], causal, scale, want_p=True, nthreads=1)
            p = p[0, 0]
            g = dout[b, h]
            dv[b, h] = p.T @ g
            dp = g @ v[b, h].T
            D = (p * dp).sum(axis=1)
            ds = p * (dp - D[:, None])
            dq[b, h] = scale * (ds @ k[b, h])
            dk[b, h] = scale * (ds.T @ q[b, h])
            dvec[b, h] = D
    return dq, dk, dv, dvec


def fp8_e4m3_decode(codes) -> np.ndarray:
    """Exact values of e4m3 codes (any integer array of bytes, same shape out, float64)."""
    c = np.ascontiguousarray(np.asarray(codes, dtype=np.uint8))
    out = np.empty(c.shape, dtype=np.float64)
    _check(_load().oracle_fp8_e4m3_decode(c.ctypes.data_as(ctypes.POINTER(ctypes.c_ubyte)), c.size, _p(out)),
           "fp8_e4m3_decode")
    return out


def attn_fwd_fp8(q8, k8, v8, descale_q, descale_k, descale_v, causal: bool, scale: float, nthreads: int | None = None):
    """Forward pass on 8-bit inputs by the definition.

    q8 ``[B, H, nq, d]``, k8 and v8 ``[B, H, nk, d]`` are e4m3 codes (uint8); descale_q, descale_k and
    descale_v ``[B, H]`` are the per-head scales.  The real inputs are descale * decoded code; S and P
    follow from them exactly as in :func:`attn_fwd` (with the same softmax ``scale``).
    Returns (O, lse) in float64."""
    dq, dk, dv = (np.asarray(x, dtype=np.float64) for x in (descale_q, descale_k, descale_v))
    q = fp8_e4m3_decode(q8) * dq[:, :, None, None]
    k = fp8_e4m3_decode(k8) * dk[:, :, None, None]
    v = fp8_e4m3_decode(v8) * dv[:, :, None, None]
    return attn_fwd(q, k, v, causal, scale, nthreads=nthreads)
