"""Seeded synthetic inputs and the named workloads.

This module only draws numbers and describes shapes: it holds none of the
attention arithmetic, so both the GPU path's tests and the CPU oracle can take
their inputs from it.

Recipe (the same for every workload): one CPU ``torch.Generator`` seeded with
``seed``; ``torch.randn`` in float32 for Q, K, V and (for a backward pass) dO,
drawn in that order, each rounded to bfloat16 (round-to-nearest-even).  For the
long-sequence workload every query row whose 0-based index is a multiple of 64
is multiplied by 8 after rounding (exact in bfloat16), which makes the running
row maximum jump and forces rescaling of the accumulators.  The softmax scale is
1/sqrt(d) rounded to float32.

8-bit workloads draw the same float32 numbers (same generator, same order, the
boost applied in float32) and store each (batch, head) slice of Q, K and V as
e4m3 codes with its own scale: scale = max|x| / 448 over the slice (448 being the
largest e4m3 value), codes = e4m3(x / scale), rounded to nearest even.  The
scales are float32.
"""
from __future__ import annotations

import hashlib
import math
from dataclasses import dataclass, field

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    causal: bool
    backward: bool = False
    boost_every: int = 0      # multiply query rows i % boost_every == 0 by `boost`
    boost: float = 8.0
    seed: int = 0
    Nk: int | None = None     # key length when it differs from the query length
    fp8: bool = False         # Q, K, V as e4m3 codes with per-head scales
    Hk: int | None = None     # K/V heads when fewer than the query heads (grouped-query attention)
    note: str = field(default="", compare=False)

    @property
    def nq(self) -> int:
        return self.N

    @property
    def nk(self) -> int:
        return self.N if self.Nk is None else self.Nk

    @property
    def hk(self) -> int:
        return self.H if self.Hk is None else self.Hk

    @property
    def scale(self) -> float:
        return softmax_scale(self.d)

    def describe(self) -> str:
        kind = ("fwd+bwd" if self.backward else "fwd") + (" e4m3" if self.fp8 else "")
        mask = "causal" if self.causal else "non-causal"
        s = "%s %s B=%d H=%d N=%d d=%d" % (kind, mask, self.B, self.H, self.N, self.d)
        if self.Hk is not None:
            s += " Hk=%d" % self.Hk
        if self.Nk is not None:
            s += " Nk=%d" % self.Nk
        if self.boost_every:
            s += " (every %dth query row x%g)" % (self.boost_every, self.boost)
        return s


WORKLOADS = {
    "c1": Workload("c1", 1, 1, 256, 64, False, note="single head forward, seed 0"),
    "c2": Workload("c2", 4, 16, 2048, 64, False),
    "c3": Workload("c3", 2, 32, 4096, 128, True),
    "c4": Workload("c4", 1, 16, 16384, 128, True, boost_every=64),
    "c5": Workload("c5", 2, 16, 4096, 128, True, backward=True),
    # decoding (widening beyond the five configurations): one query row per head against a
    # long key/value cache of 1 GiB; causal with bottom-right alignment, so the row sees every
    # key.  32 heads alone would occupy 32 of the 256 compute units without splitting.
    "dec": Workload("dec", 2, 16, 1, 128, True, Nk=65536, note="decoding, split-key forward"),
    # 8-bit forward (widening): the shapes of c3 and c4 with e4m3 inputs
    "c3f8": Workload("c3f8", 2, 32, 4096, 128, True, fp8=True, note="8-bit forward"),
    "c4f8": Workload("c4f8", 1, 16, 16384, 128, True, boost_every=64, fp8=True, note="8-bit forward"),
    # the other widened rows at the size of c5: grouped heads (4 query heads per K/V head),
    # head dimension 256, and half as many queries as keys (bottom-right causal alignment)
    "c5g": Workload("c5g", 2, 16, 4096, 128, True, backward=True, Hk=4, note="grouped-query attention"),
    "c5d256": Workload("c5d256", 2, 16, 4096, 256, True, backward=True, note="head dimension 256"),
    "c5u": Workload("c5u", 2, 16, 2048, 128, True, backward=True, Nk=4096, note="unequal lengths"),
    # informational: the forward workload of FlashAttention v3's own ablation table (B=4, N=8448,
    # H=16, d=128, non-causal), whose times the pages report on an H100 in FP16
    "fa3": Workload("fa3", 4, 16, 8448, 128, False, note="FlashAttention v3 ablation workload"),
}


def softmax_scale(d: int) -> float:
    """1/sqrt(d) rounded to float32 (returned as the Python float of that value)."""
    return float(np.float32(1.0 / math.sqrt(d)))


def make_inputs(B: int, H: int, nq: int, d: int, *, nk: int | None = None, seed: int = 0,
                backward: bool = False, boost_every: int = 0, boost: float = 8.0, Hk: int | None = None) -> dict:
    """Draw Q, K, V (and dO when ``backward``) as bfloat16 CPU tensors.

    Shapes: q and do ``[B, H, nq, d]``; k and v ``[B, Hk, nk, d]`` (Hk = H unless given)."""
    nk = nq if nk is None else nk
    Hk = H if Hk is None else Hk
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, H, nq, d, generator=g, dtype=torch.float32).to(torch.bfloat16)
    k = torch.randn(B, Hk, nk, d, generator=g, dtype=torch.float32).to(torch.bfloat16)
    v = torch.randn(B, Hk, nk, d, generator=g, dtype=torch.float32).to(torch.bfloat16)
    out = {"q": q, "k": k, "v": v}
    if backward:
        out["do"] = torch.randn(B, H, nq, d, generator=g, dtype=torch.float32).to(torch.bfloat16)
    if boost_every:
        out["q"][:, :, ::boost_every, :] *= boost
    return out


def make_fp8_inputs(B: int, H: int, nq: int, d: int, *, nk: int | None = None, Hk: int | None = None,
                    seed: int = 0, boost_every: int = 0, boost: float = 8.0) -> dict:
    """Draw Q, K, V in float32 and store them as per-head scaled e4m3 codes.

    Returns q8 ``[B, H, nq, d]``, k8 and v8 ``[B, Hk, nk, d]`` (torch.float8_e4m3fn CPU tensors) and
    descale_q ``[B, H]``, descale_k and descale_v ``[B, Hk]`` (float32): the real input is
    descale * code value."""
    nk = nq if nk is None else nk
    Hk = H if Hk is None else Hk
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, H, nq, d, generator=g, dtype=torch.float32)
    k = torch.randn(B, Hk, nk, d, generator=g, dtype=torch.float32)
    v = torch.randn(B, Hk, nk, d, generator=g, dtype=torch.float32)
    if boost_every:
        q[:, :, ::boost_every, :] *= boost
    out = {}
    for name, x in (("q", q), ("k", k), ("v", v)):
        amax = x.abs().amax(dim=(2, 3)) if x.numel() else torch.zeros(x.shape[:2])
        ds = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax)).to(torch.float32)
        codes = (x / ds[:, :, None, None]).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
        out[name + "8"] = codes
        out["descale_" + name] = ds
    return out


def workload_inputs(w: Workload) -> dict:
    if w.fp8:
        return make_fp8_inputs(w.B, w.H, w.nq, w.d, nk=w.nk, seed=w.seed, boost_every=w.boost_every, boost=w.boost)
    return make_inputs(w.B, w.H, w.nq, w.d, nk=w.nk, seed=w.seed, backward=w.backward,
                       boost_every=w.boost_every, boost=w.boost, Hk=w.Hk)


def inputs_sha256(tensors: dict) -> str:
    """SHA-256 over the raw bytes of the tensors, in key order q, k, v, do."""
    h = hashlib.sha256()
    for key in ("q", "k", "v", "do", "q8", "k8", "v8", "descale_q", "descale_k", "descale_v"):
        if key in tensors:
            t = tensors[key].contiguous()
            h.update(t.view(torch.uint8).numpy().tobytes())
    return h.hexdigest()
