"""The dK/dV kernel (d <= 128) when its grid is persistent: with more key blocks than the chip
has CUs and a head count that is a multiple of 8, 256 workgroups take the (head, key block)
items in passes, every other pass in reverse order within each XCD.

B = 1, H = 8, N = 4097, d = 128, causal: 33 key blocks of 128 per head (the last holds one
key), 264 items: the first pass over the workgroups is full and the second (reversed) holds
8.  Every element of dQ, dK and dV of every head is compared with the fp64 oracle's backward
(the gradient formulas of the backward pass in "digest_existing.txt", answer
q02_flashattention) at the bf16 bar of 2e-2; an item taken twice or never would leave a whole
key block wrong.
"""
import numpy as np
import pytest
import torch

import oracle
import tiled_online_softmax_02_amd as A
from parity_util import check_grad
from tiled_online_softmax_02_amd.inputs import make_inputs, softmax_scale

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
G_TOL = 2e-2


def note(msg):
    print("[persistent dK/dV] " + msg, flush=True)


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def test_persistent_dkdv_two_passes_ragged():
    B, H, N, d, causal = 1, 8, 4097, 128, True
    scale = softmax_scale(d)
    note("B=%d H=%d N=%d d=%d causal=%d: %d items on 256 workgroups" % (B, H, N, d, causal, B * H * ((N + 127) // 128)))
    inp = make_inputs(B, H, N, d, seed=41, backward=True)
    q, k, v, do = (inp[n].to(DEV) for n in ("q", "k", "v", "do"))
    o, lse = A.fwd(q, k, v, causal=causal, scale=scale)
    dq, dk, dv = A.bwd(q, k, v, o, do, lse, causal=causal, scale=scale)
    torch.cuda.synchronize()
    rdq, rdk, rdv, _ = oracle.attn_bwd_matmul(*(f64(inp[n]) for n in ("q", "k", "v", "do")), causal, scale)
    for name, got, ref in (("Q", f64(dq), rdq), ("K", f64(dk), rdk), ("V", f64(dv), rdv)):
        err = np.abs(got - ref)
        # the worst key block of any head, so that a block taken twice or never is named
        per_block = np.pad(err.max(axis=3), ((0, 0), (0, 0), (0, (-N) % 128))).reshape(B, H, -1, 128).max(axis=3)
        note("  d%s: max err %.3e (worst key block %s)" % (name, err.max(), np.unravel_index(per_block.argmax(), per_block.shape)))
        assert np.all(np.isfinite(got)) and err.max() <= G_TOL, (name, err.max())


def test_persistent_dkdv_grouped_heads_two_passes():
    """Grouped K/V heads on the persistent grid: B = 2, H = 16 query heads over Hk = 8 K/V heads,
    N = 4096, causal: 512 items, two full passes (key blocks 0..15 of every head in the first,
    16..31 in the reversed second), each item looping over its G = 2 query heads.  One whole K/V
    head's dK and dV, and its query heads' dQ, against the oracle (for the K/V head: the sum over
    its query heads, by the chain rule), each element within 2e-2, plus its own half bf16 ulp where
    |x| >= 4 (as for every grouped-head gradient); on every K/V head, sum_j dK_j = 0 and
    sum_j dV_j = the sum of dO over the query rows of the heads that read it."""
    B, H, Hk, N, d, causal = 2, 16, 8, 4096, 128, True
    G = H // Hk
    scale = softmax_scale(d)
    note("B=%d H=%d Hk=%d N=%d d=%d causal=%d: %d items on 256 workgroups" % (B, H, Hk, N, d, causal, B * Hk * (N // 128)))
    inp = make_inputs(B, H, N, d, seed=43, backward=True, Hk=Hk)
    q, k, v, do = (inp[n].to(DEV) for n in ("q", "k", "v", "do"))
    o, lse = A.fwd(q, k, v, causal=causal, scale=scale)
    dq, dk, dv = A.bwd(q, k, v, o, do, lse, causal=causal, scale=scale)
    torch.cuda.synchronize()
    q64, k64, v64, do64 = (f64(inp[n]) for n in ("q", "k", "v", "do"))
    b, hk = 1, 5
    heads = list(range(hk * G, (hk + 1) * G))
    kk = np.repeat(k64[b:b + 1, hk:hk + 1], G, axis=1)
    vv = np.repeat(v64[b:b + 1, hk:hk + 1], G, axis=1)
    rdq, rdk, rdv, _ = oracle.attn_bwd_matmul(q64[b:b + 1, heads], kk, vv, do64[b:b + 1, heads], causal, scale)
    for name, got, ref in (("Q", f64(dq)[b, heads], rdq[0]), ("K", f64(dk)[b, hk], rdk[0].sum(axis=0)),
                           ("V", f64(dv)[b, hk], rdv[0].sum(axis=0))):
        ok, margin, report = check_grad(got, ref)
        note("  K/V head (%d,%d) d%s: worst margin to the bound %.3e; %s" % (b, hk, name, margin, report))
        assert ok, (name, margin)
    dk64, dv64 = f64(dk), f64(dv)
    sk = np.abs(dk64.sum(axis=2))
    sv = np.abs(dv64.sum(axis=2) - do64.reshape(B, Hk, G, N, d).sum(axis=(2, 3)))
    tk = 16 * np.sqrt((dk64 ** 2).sum(axis=2)) * 2.0 ** -9 + 1e-2
    tv = 16 * np.sqrt((dv64 ** 2).sum(axis=2)) * 2.0 ** -9 + 1e-2
    note("  invariants: max|sum dK|=%.3e  max|sum dV - sum dO|=%.3e" % (sk.max(), sv.max()))
    assert np.all(sk <= tk) and np.all(sv <= tv)
