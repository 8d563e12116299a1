"""The forward at the longest key length the library accepts (d = 128), checked by a closed form.

The library keeps per-head byte offsets in 32 bits, padding rows of the last tile included, so
it accepts key lengths with (Nk + 256) * d * 2 <= 2^32 - 1; test_boundary_cpu.py checks that
one more row is rejected.  Here Nk is exactly that limit (16776959 keys at d = 128, 4.3 GB of K
and of V per head, a ragged last block of 63 keys) and the kernels stream all of it.

Closed form (the softmax definition of the attention in "digest_existing.txt", answer
q02_flashattention, section 1): with Q = 0 every score is 0, so each row's weights are uniform
over the keys it sees, O is the mean of those rows of V and lse = ln(number of keys).  V holds
a ramp in the key index, V[j][c] = bf16(j / 2^24) in every column, so a row read from a wrong
offset moves the mean; the expected means are prefix sums of the same bf16 values in fp64 on
the CPU.  Causal rows align to the bottom-right corner: query i sees keys 0 .. i + Nk - Nq.

The running sum l adds ones and stays exact below 2^24; O accumulates in fp32 over 262141
key blocks, which is why the bound on O is relative (1e-3) rather than the bf16 rounding alone.
"""
import numpy as np
import pytest
import torch

import tiled_online_softmax_02_amd as A
from tiled_online_softmax_02_amd.inputs import softmax_scale

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
D = 128
NK_MAX = 0xFFFFFFFF // (2 * D) - 256   # the largest Nk with (Nk + 256) * d * 2 <= 2^32 - 1


def note(msg):
    print("[max-length] " + msg, flush=True)


@pytest.fixture(scope="module")
def kv():
    note("allocating K = 0 and a ramp V of %d x %d bf16 (%.1f GB each)" % (NK_MAX, D, NK_MAX * D * 2 / 1e9))
    ramp = (torch.arange(NK_MAX, dtype=torch.float64) / float(1 << 24)).to(torch.bfloat16)
    k = torch.zeros((1, 1, NK_MAX, D), dtype=torch.bfloat16, device=DEV)
    v = ramp.to(DEV).view(1, 1, NK_MAX, 1).expand(1, 1, NK_MAX, D).contiguous()
    prefix = np.cumsum(ramp.to(torch.float64).numpy())   # prefix[n - 1] = sum of the first n values
    yield k, v, prefix
    del k, v
    torch.cuda.empty_cache()


def expected(nq, causal, prefix):
    """Mean of V over the keys each query row sees, and ln of their count."""
    rows = np.arange(nq)
    n = (rows + NK_MAX - nq + 1) if causal else np.full(nq, NK_MAX)
    return prefix[n - 1] / n, np.log(n.astype(np.float64))


def check(o, lse, nq, causal, prefix, what):
    o_ref, lse_ref = expected(nq, causal, prefix)
    o = o.to("cpu", torch.float64).numpy().reshape(nq, D)
    lse = lse.to("cpu", torch.float64).numpy().reshape(nq)
    # every column holds the same ramp: each column of a row is held to the same mean
    rel_o = np.abs(o - o_ref[:, None]).max() / np.abs(o_ref).max()
    rel_lse = (np.abs(lse - lse_ref) / lse_ref).max()
    note("  %s: max rel |dO| = %.3e, max rel lse = %.3e (O ~ %.4f, lse ~ %.4f)"
         % (what, rel_o, rel_lse, o_ref[0], lse_ref[0]))
    assert rel_o <= 1e-3, (what, rel_o)
    assert rel_lse <= 1e-5, (what, rel_lse)


@pytest.mark.parametrize("causal", [False, True])
def test_forward_at_the_key_length_limit(kv, causal):
    k, v, prefix = kv
    nq = 64
    note("attn_fwd_qk B=1 H=1 Nq=%d Nk=%d d=%d causal=%d, Q = 0" % (nq, NK_MAX, D, causal))
    q = torch.zeros((1, 1, nq, D), dtype=torch.bfloat16, device=DEV)
    o = torch.empty_like(q)
    lse = torch.empty((1, 1, nq), dtype=torch.float32, device=DEV)
    A.attn_fwd_qk(q, k, v, o, lse, 1, 1, 1, nq, NK_MAX, D, causal, softmax_scale(D))
    torch.cuda.synchronize()
    check(o, lse, nq, causal, prefix, "causal=%d" % causal)


def test_split_key_forward_at_the_key_length_limit(kv):
    k, v, prefix = kv
    nq = 1
    ns = A.attn_fwd_splitkv_default_splits(1, 1, nq, NK_MAX, D)
    note("attn_fwd_splitkv B=1 H=1 Nq=%d Nk=%d d=%d causal=1 splits=%d, Q = 0" % (nq, NK_MAX, D, ns))
    q = torch.zeros((1, 1, nq, D), dtype=torch.bfloat16, device=DEV)
    o = torch.empty_like(q)
    lse = torch.empty((1, 1, nq), dtype=torch.float32, device=DEV)
    ws_bytes = A.attn_fwd_splitkv_workspace_size(1, 1, nq, D, ns)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=DEV)
    A.attn_fwd_splitkv(q, k, v, o, lse, 1, 1, 1, nq, NK_MAX, D, True, softmax_scale(D), ns, ws, ws_bytes)
    torch.cuda.synchronize()
    check(o, lse, nq, True, prefix, "split-key, %d pieces" % ns)



@pytest.mark.parametrize("causal", [False, True])
def test_backward_at_the_key_length_limit(kv, causal):
    """Backward at the same length, by the same closed form: with Q = 0 and K = 0, dQ and dK are
    exactly 0 (every product has a zero operand), and with dO = 1 each key's dV is the sum of the
    weights the query rows give it, sum over the rows i that see key j of 1 / n_i (the weights are
    rounded to bf16 for the dV product, hence a relative bound of 1e-2).  Every one of the
    16776959 rows of dK and dV is checked, so a row written at a wrong offset, or not at all,
    fails."""
    k, v, prefix = kv
    nq = 64
    scale = softmax_scale(D)
    note("attn_bwd_qk B=1 H=1 Nq=%d Nk=%d d=%d causal=%d, Q = K = 0, dO = 1" % (nq, NK_MAX, D, causal))
    q = torch.zeros((1, 1, nq, D), dtype=torch.bfloat16, device=DEV)
    do = torch.ones_like(q)
    o = torch.empty_like(q)
    lse = torch.empty((1, 1, nq), dtype=torch.float32, device=DEV)
    A.attn_fwd_qk(q, k, v, o, lse, 1, 1, 1, nq, NK_MAX, D, causal, scale)
    dq = torch.full_like(q, float("nan"))
    dk = torch.full_like(k, float("nan"))
    dv = torch.full_like(v, float("nan"))
    delta = torch.empty_like(lse)
    A.attn_bwd_qk(q, k, v, o, do, lse, dq, dk, dv, delta, 1, 1, 1, nq, NK_MAX, D, causal, scale)
    torch.cuda.synchronize()
    # expected dV row j: sum over the query rows that see key j of 1 / n_i
    rows = np.arange(nq)
    n = (rows + NK_MAX - nq + 1) if causal else np.full(nq, NK_MAX)
    w = 1.0 / n.astype(np.float64)
    if causal:
        # key j is seen by the rows i >= j - (NK_MAX - nq): a suffix of the rows
        first_row = np.clip(np.arange(NK_MAX) - (NK_MAX - nq), 0, nq)
        suffix = np.concatenate([np.cumsum(w[::-1])[::-1], [0.0]])
        dv_ref = suffix[first_row]
    else:
        dv_ref = np.full(NK_MAX, w.sum())
    dv_ref_t = torch.from_numpy(dv_ref).to(DEV)
    assert bool(torch.all(dq == 0)) and bool(torch.all(dk == 0))
    # every column of a row is held to the same value: compare the row's extremes
    hi, lo = dv[0, 0].amax(dim=-1).double(), dv[0, 0].amin(dim=-1).double()
    rel = max(((hi - dv_ref_t).abs() / dv_ref_t).max().item(), ((lo - dv_ref_t).abs() / dv_ref_t).max().item())
    note("  causal=%d: dQ, dK all zero; max rel |d dV| = %.3e (dV ~ %.3e)" % (causal, rel, dv_ref[0]))
    assert rel <= 1e-2, rel
