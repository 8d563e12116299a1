"""Grouped-query and multi-query attention on the GPU (H query heads over Hk K/V heads,
through attn_fwd_qk, attn_bwd_qk and attn_fwd_splitkv) against the fp64 oracle.

By definition query head h attends with K/V head h // (H // Hk), so the forward equals
multi-head attention on K and V with each head repeated H // Hk times, and the gradient of
a shared K/V head is the sum of the gradients of its copies (the chain rule through the
repetition).  The oracle is run on the repeated heads and its dK, dV summed per group.
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
    # B, H, Hk, Nq, Nk, d, causal
    (1, 4, 2, 200, 200, 128, True),
    (2, 8, 1, 130, 130, 64, False),     # multi-query
    (1, 6, 3, 100, 300, 128, True),     # grouped and unequal lengths
    (1, 4, 4, 64, 64, 64, True),        # one query head per K/V head
    (1, 8, 2, 300, 257, 64, True),      # rows without keys in every group
]


def note(msg):
    print("[gqa] " + msg, flush=True)


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def draw(B, H, Hk, Nq, Nk, d, seed, backward=False):
    """q (and dO) with H heads, k and v with Hk heads, from the shared seeded recipe."""
    qi = make_inputs(B, H, Nq, d, nk=0, seed=seed, backward=backward)
    kv = make_inputs(B, Hk, 0, d, nk=Nk, seed=seed + 1)
    out = {"q": qi["q"], "k": kv["k"], "v": kv["v"]}
    if backward:
        out["do"] = qi["do"]
    return out


def check_fwd(o, lse, o_ref, lse_ref, what):
    o, lse = f64(o), f64(lse)
    masked = np.isneginf(lse_ref)
    assert np.all(np.isneginf(lse[masked])), what
    fin = ~masked
    rel = (np.abs(lse[fin] - lse_ref[fin]) / np.abs(lse_ref[fin])).max() if fin.any() else 0.0
    err = np.abs(o - o_ref).max()
    note("  %s: max|dO|=%.3e  max rel lse=%.3e" % (what, err, rel))
    assert np.all(np.isfinite(o)) and err <= O_TOL and rel <= LSE_RTOL, (what, err, rel)


@pytest.mark.parametrize("B,H,Hk,Nq,Nk,d,causal", CASES)
def test_grouped_heads_forward_and_backward(B, H, Hk, Nq, Nk, d, causal):
    note("B=%d H=%d Hk=%d Nq=%d Nk=%d d=%d causal=%d seed=41" % (B, H, Hk, Nq, Nk, d, causal))
    G = H // Hk
    scale = softmax_scale(d)
    inp = draw(B, H, Hk, Nq, Nk, d, 41, backward=True)
    q, k, v, do = (inp[n].to(DEV) for n in ("q", "k", "v", "do"))
    o, lse = A.fwd(q, k, v, causal=causal, scale=scale)
    dq, dk, dv = A.bwd(q, k, v, o, do, lse, causal=causal, scale=scale)
    o_s, lse_s = A.fwd_splitkv(q, k, v, causal=causal, scale=scale, num_splits=3)
    torch.cuda.synchronize()
    k_rep = inp["k"].repeat_interleave(G, dim=1)
    v_rep = inp["v"].repeat_interleave(G, dim=1)
    o_ref, lse_ref = oracle.attn_fwd(f64(inp["q"]), f64(k_rep), f64(v_rep), causal, scale)
    check_fwd(o, lse, o_ref, lse_ref, "fwd")
    check_fwd(o_s, lse_s, o_ref, lse_ref, "split fwd")
    dq_ref, dk_rep, dv_rep, _ = oracle.attn_bwd(f64(inp["q"]), f64(k_rep), f64(v_rep), f64(inp["do"]), causal, scale)
    dk_ref = dk_rep.reshape(B, Hk, G, Nk, d).sum(axis=2)
    dv_ref = dv_rep.reshape(B, Hk, G, Nk, d).sum(axis=2)
    assert tuple(dk.shape) == (B, Hk, Nk, d)
    for name, got, r in (("Q", dq, dq_ref), ("K", dk, dk_ref), ("V", dv, dv_ref)):
        g = f64(got)
        err = np.abs(g - r).max()
        note("  max|d%s err|=%.3e" % (name, err))
        assert np.all(np.isfinite(g)) and err <= G_TOL, (name, err)
