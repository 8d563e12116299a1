"""Unequal query and key lengths on the GPU (attn_fwd_qk / attn_bwd_qk through the C ABI),
against the fp64 oracle.

The causal mask is aligned to the bottom-right corner: query i sees keys j <= i + (Nk - Nq)
("GPU Programming and Kernel Optimization", item 59).  With Nq > Nk the first Nq - Nk
queries see no key: their O is 0 and their lse is -inf (the oracle's reading of that
passage), their dQ is 0, and they add nothing to dK and dV.  Tolerances are those of the
equal-length parity tests.
"""
import numpy as np
import pytest
import torch

import oracle
import tiled_online_softmax_02_amd as A
from tiled_online_softmax_02_amd.inputs import make_inputs, softmax_scale

pytestmark = pytest.mark.gpu

O_TOL = 2e-2
G_TOL = 2e-2
LSE_RTOL = 1e-3
DEV = "cuda:0"

CASES = [
    # B, H, Nq, Nk, d, causal
    (1, 2, 100, 300, 64, True),
    (1, 2, 300, 100, 128, True),    # queries 0..199 see no key
    (2, 1, 65, 257, 128, False),
    (1, 1, 257, 65, 64, False),
    (1, 2, 1, 200, 128, True),      # one query that sees every key
    (1, 1, 200, 1, 64, True),       # only the last query sees the one key
    (1, 1, 640, 384, 128, True),    # several query and key blocks, 256 fully masked rows
    (1, 2, 384, 640, 64, True),
]


def note(msg):
    print("[unequal] " + msg, flush=True)


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def lse_check(lse_gpu, lse_ref, what):
    masked = np.isneginf(lse_ref)
    assert np.all(np.isneginf(lse_gpu[masked])), (what, "rows without keys must have lse = -inf")
    fin = ~masked
    rel = (np.abs(lse_gpu[fin] - lse_ref[fin]) / np.abs(lse_ref[fin])).max() if fin.any() else 0.0
    assert np.all(np.isfinite(lse_gpu[fin]))
    return rel


@pytest.mark.parametrize("B,H,Nq,Nk,d,causal", CASES)
def test_forward_unequal_lengths(B, H, Nq, Nk, d, causal):
    note("fwd B=%d H=%d Nq=%d Nk=%d d=%d causal=%d seed=21" % (B, H, Nq, Nk, d, causal))
    scale = softmax_scale(d)
    inp = make_inputs(B, H, Nq, d, nk=Nk, seed=21)
    q, k, v = (inp[n].to(DEV) for n in "qkv")
    o, lse = A.fwd(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attn_fwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), causal, scale)
    err = np.abs(f64(o) - o_ref).max()
    rel = lse_check(f64(lse), lse_ref, "fwd")
    note("  max|dO|=%.3e  max rel lse=%.3e  rows without keys=%d" % (err, rel, int(np.isneginf(lse_ref).sum())))
    assert np.all(np.isfinite(f64(o)))
    assert err <= O_TOL
    assert rel <= LSE_RTOL


@pytest.mark.parametrize("B,H,Nq,Nk,d,causal", CASES)
def test_backward_unequal_lengths(B, H, Nq, Nk, d, causal):
    note("bwd B=%d H=%d Nq=%d Nk=%d d=%d causal=%d seed=22" % (B, H, Nq, Nk, d, causal))
    scale = softmax_scale(d)
    inp = make_inputs(B, H, Nq, d, nk=Nk, seed=22, backward=True)
    q, k, v, do = (inp[n].to(DEV) for n in ("q", "k", "v", "do"))
    o, lse = A.fwd(q, k, v, causal=causal, scale=scale)
    dq, dk, dv = A.bwd(q, k, v, o, do, lse, causal=causal, scale=scale)
    torch.cuda.synchronize()
    ref = oracle.attn_bwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(inp["do"]), causal, scale)
    for name, got, r in (("Q", dq, ref[0]), ("K", dk, ref[1]), ("V", dv, ref[2])):
        g = f64(got)
        err = np.abs(g - r).max()
        note("  max|d%s err|=%.3e" % (name, err))
        assert np.all(np.isfinite(g)), name
        assert err <= G_TOL, (name, err)


@pytest.mark.parametrize("d,causal", [(64, False), (128, True)])
def test_no_keys(d, causal):
    """Nk = 0: every query sees no key, so O = 0, lse = -inf and dQ = 0."""
    note("Nk=0 d=%d causal=%d" % (d, causal))
    inp = make_inputs(1, 2, 130, d, nk=0, seed=23, backward=True)
    q, k, v, do = (inp[n].to(DEV) for n in ("q", "k", "v", "do"))
    o, lse = A.fwd(q, k, v, causal=causal, scale=softmax_scale(d))
    dq, dk, dv = A.bwd(q, k, v, o, do, lse, causal=causal, scale=softmax_scale(d))
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))
    assert torch.all(dq == 0) and dk.numel() == 0 and dv.numel() == 0


@pytest.mark.parametrize("d,causal", [(64, True), (128, False)])
def test_no_queries(d, causal):
    """Nq = 0: no query sees any key, so dK = dV = 0 and the forward writes nothing."""
    note("Nq=0 d=%d causal=%d" % (d, causal))
    inp = make_inputs(1, 2, 0, d, nk=200, seed=24, backward=True)
    q, k, v, do = (inp[n].to(DEV) for n in ("q", "k", "v", "do"))
    o, lse = A.fwd(q, k, v, causal=causal, scale=softmax_scale(d))
    dq, dk, dv = A.bwd(q, k, v, o, do, lse, causal=causal, scale=softmax_scale(d))
    torch.cuda.synchronize()
    assert o.numel() == 0 and lse.numel() == 0 and dq.numel() == 0
    assert torch.all(dk == 0) and torch.all(dv == 0)
