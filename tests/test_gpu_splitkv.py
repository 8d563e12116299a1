"""Split-key forward (attn_fwd_splitkv through the C ABI) against the fp64 oracle.

The key range is cut into pieces whose normalised outputs and log-sum-exps are merged by
a second kernel ("GPU Programming and Kernel Optimization", item 59, small-query attention
split across thread blocks with a combining kernel; the merge rule is that of the running
maxima and sums of the FlashAttention answer in "digest_existing.txt", q02 section 2).
Cases include decoding shapes (one query row, thousands of keys), pieces that hold no key
(more pieces than key blocks, causal pieces past a row's last key) and rows that see no key.
"""
import numpy as np
import pytest
import torch

import oracle
import tiled_online_softmax_02_amd as A
from tiled_online_softmax_02_amd.inputs import make_inputs, softmax_scale

pytestmark = pytest.mark.gpu

O_TOL = 2e-2
LSE_RTOL = 1e-3
DEV = "cuda:0"

CASES = [
    # B, H, Nq, Nk, d, causal, num_splits
    (2, 4, 1, 2000, 128, False, 8),
    (1, 8, 1, 4096, 64, True, 16),
    (1, 2, 17, 1000, 128, True, 5),
    (2, 2, 40, 777, 64, False, 3),
    (1, 1, 300, 100, 128, True, 4),     # rows 0..199 see no key; some pieces are empty
    (1, 2, 5, 64, 64, False, 8),        # more pieces than key blocks
    (1, 1, 260, 520, 128, True, 2),     # two query blocks
    (1, 3, 33, 3000, 128, False, 1),    # one piece: the merge of a single piece
]


def note(msg):
    print("[splitkv] " + msg, flush=True)


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def check(o, lse, o_ref, lse_ref, what):
    o, lse = f64(o), f64(lse)
    masked = np.isneginf(lse_ref)
    assert np.all(np.isneginf(lse[masked])), what
    fin = ~masked
    rel = (np.abs(lse[fin] - lse_ref[fin]) / np.abs(lse_ref[fin])).max() if fin.any() else 0.0
    err = np.abs(o - o_ref).max()
    note("  %s: max|dO|=%.3e  max rel lse=%.3e" % (what, err, rel))
    assert np.all(np.isfinite(o))
    assert err <= O_TOL, (what, err)
    assert rel <= LSE_RTOL, (what, rel)


@pytest.mark.parametrize("B,H,Nq,Nk,d,causal,ns", CASES)
def test_splitkv_matches_oracle(B, H, Nq, Nk, d, causal, ns):
    note("B=%d H=%d Nq=%d Nk=%d d=%d causal=%d splits=%d seed=31" % (B, H, Nq, Nk, d, causal, ns))
    scale = softmax_scale(d)
    inp = make_inputs(B, H, Nq, d, nk=Nk, seed=31)
    q, k, v = (inp[n].to(DEV) for n in "qkv")
    o, lse = A.fwd_splitkv(q, k, v, causal=causal, scale=scale, num_splits=ns)
    o1, lse1 = A.fwd(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attn_fwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), causal, scale)
    check(o, lse, o_ref, lse_ref, "split")
    check(o1, lse1, o_ref, lse_ref, "one pass")


def test_splitkv_default_splits_and_repeat():
    note("default splits, B=4 H=8 Nq=1 Nk=8192 d=128, two calls")
    inp = make_inputs(4, 8, 1, 128, nk=8192, seed=32)
    q, k, v = (inp[n].to(DEV) for n in "qkv")
    ns = A.attn_fwd_splitkv_default_splits(4, 8, 1, 8192, 128)
    assert ns > 1
    o, lse = A.fwd_splitkv(q, k, v, causal=False, scale=softmax_scale(128))
    o2, lse2 = A.fwd_splitkv(q, k, v, causal=False, scale=softmax_scale(128))
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    o_ref, lse_ref = oracle.attn_fwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), False, softmax_scale(128))
    check(o, lse, o_ref, lse_ref, "default splits (%d)" % ns)


def test_splitkv_workspace_too_small_is_rejected():
    inp = make_inputs(1, 1, 2, 64, nk=256, seed=33)
    q, k, v = (inp[n].to(DEV) for n in "qkv")
    o = torch.empty_like(q)
    lse = torch.empty((1, 1, 2), dtype=torch.float32, device=DEV)
    need = A.attn_fwd_splitkv_workspace_size(1, 1, 2, 64, 4)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    with pytest.raises(A.AttnError) as e:
        A.attn_fwd_splitkv(q, k, v, o, lse, 1, 1, 1, 2, 256, 64, False, 0.125, 4, ws, need - 16)
    assert e.value.status == A.ATTN_ERR_WORKSPACE
