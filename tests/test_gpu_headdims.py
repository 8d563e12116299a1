"""Head dimensions 192 and 256 on the GPU against the fp64 oracle: forward, backward (one wave per
SIMD in every kernel, each dK/dV wave doing all four products for its keys), the split-key forward,
unequal lengths and grouped heads, on small and ragged shapes; and inputs whose row maxima grow
along the keys, so that the forward moves its running offset and rescales O many times per row
(the online-softmax recurrence of "digest_existing.txt", answer q02_flashattention; a row's offset
moves only when its maximum outgrows it by more than 2^8 in exp2 units)."""
import numpy as np
import pytest
import torch

import oracle
import tiled_online_softmax_02_amd as A
from parity_util import check_grad
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


RESCALE_CASES = [
    # B, H, Nq, Nk, d, causal
    (1, 2, 300, 300, 192, True),
    (1, 2, 300, 300, 192, False),
    (1, 2, 257, 257, 256, True),
    (1, 1, 200, 450, 256, False),
]


@pytest.mark.parametrize("B,H,Nq,Nk,d,causal", RESCALE_CASES)
def test_large_head_dims_growing_maxima(B, H, Nq, Nk, d, causal):
    """Every 7th query row scaled by 8 and key row j by 1 + j / 64 (then rounded to bf16): the
    scores of later key blocks are several times larger, so each row's maximum grows past the
    offset block after block (by up to ~100 in exp2 units for the scaled rows).  V is halved: with
    so peaked a softmax an output row is close to a single row of V, and halving keeps |O| below
    2.5, where the bf16 output rounding (at most 0.0078) leaves room for the arithmetic under the
    2e-2 bar (full-size V rows reach |O| >= 4, where the rounding alone can take 0.0156).  The
    backward recomputes P from the large lse of these rows, with dO scaled by 1/8 (exact in
    bf16) and the gradient bound of the other tests (2e-2, plus the element's own half bf16 ulp
    from |x| = 4).  At full-size dO these magnified Q rows and keys make the bf16 rounding that
    every such backward has move dQ and dK by up to 0.045 and 0.095 (the four cases in order:
    dQ 0.030, 0.045, 0.019, 0.044; dK 0.036, 0.095, 0.048, 0.040), almost all of it from D =
    rowsum(dO O) formed from the bf16 O the forward wrote: in rows whose softmax is this peaked,
    dS = P (dP - D) cancels, and the rows scaled by 8 carry D's rounding into dK eightfold.  An
    fp64 emulation of just those roundings (O and then D, P and dS where they enter the
    products) on the CPU gives these figures, and the kernels give the same (0.0239 for dK in
    the second case at 1/4 dO).  The 2e-2 bar is set for N(0,1) inputs; the gradients are linear
    in dO, so at 1/8 the same roundings stay inside it."""
    note("growing maxima: B=%d H=%d Nq=%d Nk=%d d=%d causal=%d seed=53" % (B, H, Nq, Nk, d, causal))
    scale = softmax_scale(d)
    qi = make_inputs(B, H, Nq, d, nk=0, seed=53, backward=True)
    kv = make_inputs(B, H, 0, d, nk=Nk, seed=54)
    q32 = qi["q"].float()
    q32[:, :, ::7, :] *= 8.0
    ramp = 1.0 + torch.arange(Nk, dtype=torch.float32) / 64.0
    k32 = kv["k"].float() * ramp[None, None, :, None]
    qb, kb, vb = q32.to(torch.bfloat16), k32.to(torch.bfloat16), kv["v"] * 0.5
    q, k, v = qb.to(DEV), kb.to(DEV), vb.to(DEV)
    o, lse = A.fwd(q, k, v, causal=causal, scale=scale)
    o_s, lse_s = A.fwd_splitkv(q, k, v, causal=causal, scale=scale, num_splits=3)
    do_b = qi["do"] * 0.125
    do = do_b.to(DEV)
    dq, dk, dv = A.bwd(q, k, v, o, do, lse, causal=causal, scale=scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attn_fwd(f64(qb), f64(kb), f64(vb), causal, scale)
    # the inputs do what they are for: some row's maximum grows by more than 2^8 (exp2 units)
    # past the maximum of its first 64 keys
    s = np.einsum("bhid,bhjd->bhij", f64(qb), f64(kb)) * scale * np.log2(np.e)
    if causal:
        s = np.where(np.arange(Nk)[None, :] > np.arange(Nq)[:, None] + (Nk - Nq), -np.inf, s)
    first = s[..., :64].max(axis=-1)
    growth = s.max(axis=-1) - first
    note("  largest growth of a row maximum past its first 64 keys: %.1f (exp2 units)" % np.nanmax(growth[np.isfinite(growth)]))
    assert np.nanmax(growth[np.isfinite(growth)]) > 64.0
    check_fwd(o, lse, o_ref, lse_ref, "fwd")
    check_fwd(o_s, lse_s, o_ref, lse_ref, "split fwd")
    rdq, rdk, rdv, _ = oracle.attn_bwd_matmul(f64(qb), f64(kb), f64(vb), f64(do_b), causal, scale)
    for name, got, ref in (("dQ", dq, rdq), ("dK", dk, rdk), ("dV", dv, rdv)):
        ok, margin, report = check_grad(f64(got), ref)
        note("  %s: margin %.3e; %s" % (name, margin, report))
        assert ok, (name, margin)
