"""attn_fwd_splitkv_noalloc through the C ABI: the split-key forward whose pieces live in the
library's static device buffer instead of a caller-provided workspace.

Its kernels are those of attn_fwd_splitkv, so on the same inputs and number of pieces its outputs
must equal attn_fwd_splitkv's bit for bit.  Two calls in a row share the one buffer: the first
fills nearly all of it, the second (smaller, other head dimension, other causal setting) must not
see anything the first left behind.  A call past the buffer's size is rejected on the host and
leaves its outputs untouched.  The small call is also checked against the fp64 oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import tiled_online_softmax_02_amd as A
from tiled_online_softmax_02_amd.inputs import make_inputs, softmax_scale

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
O_TOL = 2e-2
LSE_RTOL = 1e-3

# B, H, Hk, Nq, Nk, d, causal, num_splits
BIG = (2, 4, 2, 1016, 5000, 128, True, 4)     # 16 775 168 bytes of pieces: the buffer is 16 777 216
SMALL = (1, 8, 8, 1, 3001, 64, False, 16)      # decoding: one query row, a ragged key count


def note(msg):
    print("[noalloc] " + msg, flush=True)


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def setup(case, seed):
    B, H, Hk, Nq, Nk, d, causal, ns = case
    inp = make_inputs(B, H, Nq, d, nk=Nk, Hk=Hk, seed=seed)
    q, k, v = (inp[n].to(DEV) for n in "qkv")
    return inp, q, k, v


def outputs(case):
    B, H, Hk, Nq, Nk, d, causal, ns = case
    o = torch.full((B, H, Nq, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((B, H, Nq), float("nan"), dtype=torch.float32, device=DEV)
    return o, lse


def with_workspace(case, q, k, v):
    B, H, Hk, Nq, Nk, d, causal, ns = case
    o, lse = outputs(case)
    nbytes = A.attn_fwd_splitkv_workspace_size(B, H, Nq, d, ns)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    A.attn_fwd_splitkv(q, k, v, o, lse, B, H, Hk, Nq, Nk, d, causal, softmax_scale(d), ns, ws, nbytes)
    return o, lse


def without_workspace(case, q, k, v, o, lse):
    B, H, Hk, Nq, Nk, d, causal, ns = case
    A.attn_fwd_splitkv_noalloc(q, k, v, o, lse, B, H, Hk, Nq, Nk, d, causal, softmax_scale(d), ns)


def same_bits(a, b):
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_noalloc_equals_the_workspace_entry_point_on_two_calls_in_a_row():
    assert A.attn_fwd_splitkv_workspace_size(*BIG[:2], BIG[3], BIG[5], BIG[7]) <= A.ATTN_NOALLOC_SCRATCH_BYTES
    note("big %s, small %s, seeds 41/42" % (BIG, SMALL))
    inp_b, qb, kb, vb = setup(BIG, 41)
    inp_s, qs, ks, vs = setup(SMALL, 42)
    ref_b = with_workspace(BIG, qb, kb, vb)
    ref_s = with_workspace(SMALL, qs, ks, vs)
    torch.cuda.synchronize()

    # the two calls back to back on one stream, no synchronisation between them
    got_b, got_s = outputs(BIG), outputs(SMALL)
    without_workspace(BIG, qb, kb, vb, *got_b)
    without_workspace(SMALL, qs, ks, vs, *got_s)
    torch.cuda.synchronize()
    for name, got, ref in (("big o", got_b[0], ref_b[0]), ("big lse", got_b[1], ref_b[1]),
                           ("small o", got_s[0], ref_s[0]), ("small lse", got_s[1], ref_s[1])):
        diff = (got.float() - ref.float()).abs()
        diff = diff[torch.isfinite(diff)]
        note("  %s: bitwise equal %s, max |diff| %.3e" % (name, same_bits(got, ref),
                                                             diff.max().item() if diff.numel() else 0.0))
        assert same_bits(got, ref), name

    # the small call against the oracle too (every row sees keys: no -inf here)
    B, H, Hk, Nq, Nk, d, causal, ns = SMALL
    o_ref, lse_ref = oracle.attn_fwd(f64(inp_s["q"]), np.repeat(f64(inp_s["k"]), H // Hk, axis=1),
                                     np.repeat(f64(inp_s["v"]), H // Hk, axis=1), causal, softmax_scale(d))
    err = np.abs(f64(got_s[0]) - o_ref).max()
    rel = (np.abs(f64(got_s[1]) - lse_ref) / np.abs(lse_ref)).max()
    note("  small vs oracle: max|dO|=%.3e  max rel lse=%.3e" % (err, rel))
    assert err <= O_TOL and rel <= LSE_RTOL


def test_noalloc_rejects_a_call_past_the_buffer_and_touches_nothing():
    case = (1, 1, 1, 8129, 64, 128, False, 4)   # 16 778 256 bytes of pieces
    _, q, k, v = setup(case, 43)
    o = torch.full((1, 1, 8129, 128), 3.0, dtype=torch.bfloat16, device=DEV)
    lse = torch.full((1, 1, 8129), 7.0, dtype=torch.float32, device=DEV)
    with pytest.raises(A.AttnError) as e:
        without_workspace(case, q, k, v, o, lse)
    assert e.value.status == A.ATTN_ERR_SCRATCH
    torch.cuda.synchronize()
    assert bool((o == 3.0).all()) and bool((lse == 7.0).all())


def test_noalloc_on_a_side_stream():
    case = (2, 2, 1, 7, 2100, 128, True, 5)
    note("side stream %s, seed 44" % (case,))
    _, q, k, v = setup(case, 44)
    ref = with_workspace(case, q, k, v)
    got = outputs(case)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        without_workspace(case, q, k, v, *got)
    s.synchronize()
    assert same_bits(got[0], ref[0]) and same_bits(got[1], ref[1])


def test_noalloc_under_graph_capture():
    """The callers this entry point is for include code under HIP graph capture.  A first eager call
    looks up the buffer's address and the device shape; the captured call then allocates nothing,
    and each replay (with eager work of other shapes, which also uses the buffer, between replays)
    must reproduce the eager result bit for bit."""
    case = (2, 4, 2, 33, 3000, 128, False, 6)
    other = (1, 2, 2, 5, 1500, 64, True, 3)
    note("graph capture %s, eager work between replays %s, seeds 45/46" % (case, other))
    _, q, k, v = setup(case, 45)
    _, q2, k2, v2 = setup(other, 46)
    ref = with_workspace(case, q, k, v)
    ref2 = with_workspace(other, q2, k2, v2)
    got = outputs(case)
    without_workspace(case, q, k, v, *got)      # eager first call: address and device shape cached
    torch.cuda.synchronize()
    assert same_bits(got[0], ref[0]) and same_bits(got[1], ref[1])
    got[0].fill_(float("nan"))
    got[1].fill_(float("nan"))
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            without_workspace(case, q, k, v, *got)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(4):
        g.replay()
        torch.cuda.synchronize()
        ok = same_bits(got[0], ref[0]) and same_bits(got[1], ref[1])
        note("  replay %d: bitwise equal %s" % (rep, ok))
        assert ok, rep
        # eager work in between that overwrites the shared buffer with another problem's pieces
        got2 = outputs(other)
        without_workspace(other, q2, k2, v2, *got2)
        torch.cuda.synchronize()
        assert same_bits(got2[0], ref2[0]) and same_bits(got2[1], ref2[1])
        got[0].fill_(float("nan"))
        got[1].fill_(float("nan"))
        torch.cuda.synchronize()
