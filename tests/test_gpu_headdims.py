"""Head dimensions 192 and 256 on the GPU against the fp64 oracle: forward, backward (the
dK/dV kernel splits the columns of dK and dV between two waves that share the keys), the
split-key forward, unequal lengths and grouped heads, on small and ragged shapes."""
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
    (1, 2, 2, 200, 200, 192, True),
    (2, 1, 1, 130, 130, 192, False),
    (1, 2, 2, 257, 257, 256, True),
    (1, 1, 1, 64, 64, 256, False),
    (1, 2, 1, 100, 300, 256, True),     # grouped heads, more keys than queries
    (1, 4, 2, 300, 129, 192, True),     # grouped heads, rows without keys
]


def note(msg):
    print("[headdim] " + msg, flush=True)


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


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
def test_large_head_dims(B, H, Hk, Nq, Nk, d, causal):
    note("B=%d H=%d Hk=%d Nq=%d Nk=%d d=%d causal=%d seed=51" % (B, H, Hk, Nq, Nk, d, causal))
    G = H // Hk
    scale = softmax_scale(d)
    qi = make_inputs(B, H, Nq, d, nk=0, seed=51, backward=True)
    kv = make_inputs(B, Hk, 0, d, nk=Nk, seed=52)
    inp = {"q": qi["q"], "do": qi["do"], "k": kv["k"], "v": kv["v"]}
    q, k, v, do = (inp[n].to(DEV) for n in ("q", "k", "v", "do"))
    o, lse = A.fwd(q, k, v, causal=causal, scale=scale)
    dq, dk, dv = A.bwd(q, k, v, o, do, lse, causal=causal, scale=scale)
    o_s, lse_s = A.fwd_splitkv(q, k, v, causal=causal, scale=scale, num_splits=2)
    torch.cuda.synchronize()
    k_rep = inp["k"].repeat_interleave(G, dim=1)
    v_rep = inp["v"].repeat_interleave(G, dim=1)
    o_ref, lse_ref = oracle.attn_fwd(f64(inp["q"]), f64(k_rep), f64(v_rep), causal, scale)
    check_fwd(o, lse, o_ref, lse_ref, "fwd")
    check_fwd(o_s, lse_s, o_ref, lse_ref, "split fwd")
    dq_ref, dk_rep, dv_rep, _ = oracle.attn_bwd(f64(inp["q"]), f64(k_rep), f64(v_rep), f64(inp["do"]), causal, scale)
    dk_ref = dk_rep.reshape(B, Hk, G, Nk, d).sum(axis=2)
    dv_ref = dv_rep.reshape(B, Hk, G, Nk, d).sum(axis=2)
    for name, got, r in (("Q", dq, dq_ref), ("K", dk, dk_ref), ("V", dv, dv_ref)):
        g = f64(got)
        err = np.abs(g - r).max()
        note("  max|d%s err|=%.3e" % (name, err))
        assert np.all(np.isfinite(g)) and err <= G_TOL, (name, err)
