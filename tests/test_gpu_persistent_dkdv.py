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
from tiled_online_softmax_02_amd.inputs import make_inputs, softmax_scale

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
G_TOL = 2e-2


def note(msg):
    print("[persistent dK/dV] " + msg, flush=True)


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def test_persistent_dkdv_two_rounds_ragged():
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
