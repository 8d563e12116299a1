"""Pins of the fp64 CPU oracle against facts that do not come from the oracle itself.

Each test states the property it checks and where it comes from.  The pages
cited are "digest_existing.txt" (xtrax package, answer q02_flashattention) and
"GPU Programming and Kernel Optimization" (ai.engineer, numbered items).
Independent checks: closed forms, invariants, the merge rule of the digest
answer's section 2, PyTorch's own fp64 CPU routines (softmax, attention and
autograd: a separate implementation, never the GPU path), central finite
differences and golden fixtures under tests/golden/.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
RNG = np.random.default_rng(1234)


def rand(*shape, rng=RNG):
    return rng.standard_normal(shape)


def torch_attention(q, k, v, causal, scale):
    """Explicit fp64 attention in PyTorch (CPU): softmax(Q K^T * scale + mask) V, bottom-right aligned mask."""
    q, k, v = (torch.from_numpy(np.ascontiguousarray(a)) for a in (q, k, v))
    s = torch.matmul(q, k.transpose(-1, -2).contiguous()) * scale
    nq, nk = s.shape[-2], s.shape[-1]
    if causal:
        i = torch.arange(nq).unsqueeze(1)
        j = torch.arange(nk).unsqueeze(0)
        s = s.masked_fill(j > i + (nk - nq), float("-inf"))
    return s


# ---------------------------------------------------------------- softmax rows

def test_softmax_rows_sum_to_one_and_masked_rows_are_zero():
    x = rand(40, 33) * 5
    x[3, ::2] = -np.inf
    x[7, :] = -np.inf  # fully masked row
    p, lse = oracle.softmax_rows(x)
    live = [r for r in range(40) if r != 7]
    np.testing.assert_allclose(p[live].sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert np.all(p[3, ::2] == 0.0)
    assert np.all(p[7] == 0.0) and lse[7] == -np.inf
    assert np.all(p >= 0)


def test_softmax_rows_match_torch_on_irregular_1823x781():
    # "GPU Programming and Kernel Optimization", item 51: the fused-softmax test shape 1823x781
    # compared against torch.softmax.
    x = rand(1823, 781) * 3
    p, lse = oracle.softmax_rows(x)
    t = torch.from_numpy(x)
    np.testing.assert_allclose(p, torch.softmax(t, dim=1).numpy(), rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(lse, torch.logsumexp(t, dim=1).numpy(), rtol=1e-13, atol=0)


# ---------------------------------------------------------- online statistics

@pytest.mark.parametrize("n", [1, 2, 17, 64, 1000])
def test_merge_rule_over_random_splits_equals_direct(n):
    # digest q02 section 2: m(x) = max(m1, m2), l(x) = e^(m1-m) l1 + e^(m2-m) l2.
    x = rand(n) * 6
    m_direct = x.max()
    l_direct = np.exp(x - m_direct).sum()
    for trial in range(5):
        k = int(RNG.integers(0, min(n - 1, 9) + 1)) if n > 1 else 0
        cuts = np.sort(RNG.choice(np.arange(1, n), size=k, replace=False)) if k else np.array([], dtype=np.int64)
        m, l = oracle.online_merge(x, cuts)
        assert m == m_direct
        assert abs(l - l_direct) <= 1e-12 * l_direct


def test_merge_rule_with_fully_masked_blocks():
    x = rand(32)
    x[:8] = -np.inf   # the first block is entirely -inf
    x[20:24] = -np.inf
    m, l = oracle.online_merge(x, [8, 20, 24])
    live = x[np.isfinite(x)]
    assert m == live.max()
    assert abs(l - np.exp(live - live.max()).sum()) <= 1e-12 * l
    m, l = oracle.online_merge(np.full(5, -np.inf), [2])
    assert m == -np.inf and l == 0.0


def test_online_normalizer_equals_direct():
    # "GPU Programming and Kernel Optimization", item 57: m' = max(m, x), d' = d e^(m-m') + e^(x-m').
    for n in (1, 5, 4000):
        x = rand(n) * 4
        m, d = oracle.online_normalizer(x)
        assert m == x.max()
        assert abs(d - np.exp(x - x.max()).sum()) <= 1e-12 * d
    # a running maximum that keeps increasing forces a rescale at every step
    x = np.arange(50, dtype=np.float64)
    m, d = oracle.online_normalizer(x)
    assert m == 49.0 and abs(d - np.exp(x - 49.0).sum()) <= 1e-13 * d


# ------------------------------------------------------------ forward: pins

@pytest.mark.parametrize("nq,nk,d,br,bc,causal", [
    (16, 16, 8, 4, 4, False), (16, 16, 8, 4, 4, True), (37, 37, 5, 8, 6, True),
    (50, 23, 7, 16, 5, False), (23, 50, 7, 5, 16, True), (64, 64, 16, 64, 64, True),
    (9, 40, 3, 2, 7, True), (1, 1, 4, 1, 1, False),
])
def test_blockwise_online_equals_direct(nq, nk, d, br, bc, causal):
    # FlashAttention's blockwise recurrence (digest q02 section 2; GPU Programming item 58)
    # equals the materialised definition (digest q02 section 1).
    q, k, v = rand(nq, d), rand(nk, d), rand(nk, d)
    scale = 1.0 / math.sqrt(d)
    o_b, lse_b, m_b, l_b = oracle.attn_fwd_blockwise(q, k, v, causal, scale, br, bc)
    o_d, lse_d = oracle.attn_fwd(q[None, None], k[None, None], v[None, None], causal, scale)
    o_d, lse_d = o_d[0, 0], lse_d[0, 0]
    live = np.isfinite(lse_d)
    np.testing.assert_allclose(o_b[live], o_d[live], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse_b[live], lse_d[live], rtol=1e-12, atol=1e-13)
    assert np.all(o_b[~live] == 0) and np.all(lse_b[~live] == -np.inf)
    # the running statistics themselves: m = row max of the scores, l = sum exp(s - m)
    s = torch_attention(q[None, None], k[None, None], v[None, None], causal, scale)[0, 0].numpy()
    for i in np.nonzero(live)[0]:
        assert m_b[i] == pytest.approx(s[i].max(), rel=1e-14, abs=1e-14)
        assert l_b[i] == pytest.approx(np.exp(s[i] - s[i].max()).sum(), rel=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_rows_of_p_sum_to_one(causal):
    q, k, v = rand(2, 3, 31, 8), rand(2, 3, 31, 8), rand(2, 3, 31, 8)
    _, _, p = oracle.attn_fwd(q, k, v, causal, 0.3, want_p=True)
    np.testing.assert_allclose(p.sum(axis=-1), 1.0, rtol=0, atol=1e-12)
    if causal:
        assert np.all(np.triu(p[0, 0], 1) == 0.0)  # key j > query i carries no weight


@pytest.mark.parametrize("causal", [False, True])
def test_constant_v_returns_that_row(causal):
    q, k = rand(1, 2, 20, 6) * 3, rand(1, 2, 20, 6) * 3
    row = rand(6)
    v = np.broadcast_to(row, (1, 2, 20, 6)).copy()
    o, _ = oracle.attn_fwd(q, k, v, causal, 0.5)
    np.testing.assert_allclose(o, np.broadcast_to(row, o.shape), rtol=1e-13, atol=1e-13)


def test_causal_row_zero_is_v0_and_its_lse_is_the_single_score():
    q, k, v = rand(2, 2, 12, 5), rand(2, 2, 12, 5), rand(2, 2, 12, 5)
    scale = 0.37
    o, lse = oracle.attn_fwd(q, k, v, True, scale)
    np.testing.assert_allclose(o[:, :, 0], v[:, :, 0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse[:, :, 0], scale * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0]),
                               rtol=1e-14, atol=1e-15)


def test_zero_queries_give_uniform_weights_closed_form():
    # Q = 0 => every visible score is 0 => uniform weights.
    B, H, N, d = 1, 2, 24, 4
    q = np.zeros((B, H, N, d))
    k, v = rand(B, H, N, d), rand(B, H, N, d)
    o, lse = oracle.attn_fwd(q, k, v, False, 0.125)
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(axis=2, keepdims=True), o.shape), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse, math.log(N), rtol=1e-15)
    o, lse = oracle.attn_fwd(q, k, v, True, 0.125)
    cum = np.cumsum(v, axis=2) / np.arange(1, N + 1)[None, None, :, None]
    np.testing.assert_allclose(o, cum, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse, np.broadcast_to(np.log(np.arange(1, N + 1)), lse.shape), rtol=1e-15)
    # bottom-right alignment with more keys than queries: row i sees keys 0..i+(nk-nq)
    nq, nk = 5, 9
    q = np.zeros((1, 1, nq, d))
    k, v = rand(1, 1, nk, d), rand(1, 1, nk, d)
    o, lse = oracle.attn_fwd(q, k, v, True, 0.125)
    for i in range(nq):
        n_vis = i + (nk - nq) + 1
        np.testing.assert_allclose(o[0, 0, i], v[0, 0, :n_vis].mean(axis=0), rtol=1e-13, atol=1e-14)
        assert lse[0, 0, i] == pytest.approx(math.log(n_vis), rel=1e-15)


def test_permutations():
    q, k, v = rand(1, 1, 18, 7), rand(1, 1, 18, 7), rand(1, 1, 18, 7)
    o, lse = oracle.attn_fwd(q, k, v, False, 0.4)
    perm = RNG.permutation(18)
    o2, lse2 = oracle.attn_fwd(q, k[:, :, perm], v[:, :, perm], False, 0.4)  # keys and values together
    np.testing.assert_allclose(o2, o, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse2, lse, rtol=1e-14)
    o3, lse3 = oracle.attn_fwd(q[:, :, perm], k, v, False, 0.4)  # queries: rows move with them
    np.testing.assert_allclose(o3, o[:, :, perm], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(lse3, lse[:, :, perm], rtol=1e-15)


@pytest.mark.parametrize("nq,nk,causal", [(33, 33, False), (33, 33, True), (20, 45, True), (45, 20, False)])
def test_forward_matches_torch_fp64(nq, nk, causal):
    # An independent implementation: PyTorch's fp64 CPU matmul + softmax (the "math" path
    # that upcasts, "GPU Programming and Kernel Optimization" item 31).
    B, H, d = 2, 3, 16
    q, k, v = rand(B, H, nq, d), rand(B, H, nk, d), rand(B, H, nk, d)
    scale = 0.25
    o, lse = oracle.attn_fwd(q, k, v, causal, scale)
    s = torch_attention(q, k, v, causal, scale)
    ref = torch.matmul(torch.softmax(s, dim=-1), torch.from_numpy(v)).numpy()
    ref_lse = torch.logsumexp(s, dim=-1).numpy()
    live = np.isfinite(ref_lse)
    np.testing.assert_allclose(o[live], ref[live], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse[live], ref_lse[live], rtol=1e-13, atol=1e-14)
    if nq == nk:
        sdpa = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), is_causal=causal, scale=scale)
        np.testing.assert_allclose(o, sdpa.numpy(), rtol=1e-12, atol=1e-13)


def test_rows_entry_point_equals_full_forward():
    B, H, nq, nk, d = 1, 2, 40, 40, 8
    q, k, v = rand(B, H, nq, d), rand(B, H, nk, d), rand(B, H, nk, d)
    o, lse = oracle.attn_fwd(q, k, v, True, 0.3)
    rows = np.array([0, 1, 17, 39])
    for h in range(H):
        o_r, lse_r = oracle.attn_fwd_rows(q[0, h, rows], rows, k[0, h], v[0, h], nq, True, 0.3)
        np.testing.assert_array_equal(o_r, o[0, h, rows])
        np.testing.assert_array_equal(lse_r, lse[0, h, rows])


def test_fully_masked_rows_golden_bottom_right_example():
    with open(os.path.join(GOLDEN, "causal_bottom_right_5q_2k.json")) as f:
        g = json.load(f)
    nq, nk, d = g["nq"], g["nk"], 4
    q, k, v = rand(1, 1, nq, d), rand(1, 1, nk, d), rand(1, 1, nk, d)
    o, lse, p = oracle.attn_fwd(q, k, v, True, 0.5, want_p=True)
    visible = (p[0, 0] > 0).astype(int).tolist()
    assert visible == g["visible"]
    for i in g["zero_output_rows"]:
        assert np.all(o[0, 0, i] == 0.0) and lse[0, 0, i] == -np.inf
    # the blockwise recurrence agrees, including the empty rows
    o_b, lse_b, _, _ = oracle.attn_fwd_blockwise(q[0, 0], k[0, 0], v[0, 0], True, 0.5, 2, 1)
    np.testing.assert_allclose(o_b, o[0, 0], rtol=1e-13, atol=1e-15)
    assert np.all(lse_b[g["zero_output_rows"]] == -np.inf)
    dq, dk, dv, D = oracle.attn_bwd(q, k, v, rand(1, 1, nq, d), True, 0.5)
    assert np.all(dq[0, 0, g["zero_output_rows"]] == 0.0)


# ----------------------------------------------------------- backward: pins

def loss(q, k, v, dout, causal, scale):
    o, _ = oracle.attn_fwd(q, k, v, causal, scale, nthreads=1)
    return float((o * dout).sum())


@pytest.mark.parametrize("nq,nk,d,causal", [(6, 6, 4, False), (6, 6, 4, True), (5, 8, 3, True), (7, 4, 3, False)])
def test_backward_matches_central_finite_differences(nq, nk, d, causal):
    # dL/dX for L = sum(O * dO), every element of Q, K and V, step 1e-6, fp64.
    q, k, v, dout = rand(1, 1, nq, d), rand(1, 1, nk, d), rand(1, 1, nk, d), rand(1, 1, nq, d)
    scale = 0.45
    dq, dk, dv, _ = oracle.attn_bwd(q, k, v, dout, causal, scale, nthreads=1)
    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        fd = np.empty_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args = {"q": q, "k": k, "v": v}
            lp = loss(**{**args, name: xp}, dout=dout, causal=causal, scale=scale)
            lm = loss(**{**args, name: xm}, dout=dout, causal=causal, scale=scale)
            fd[idx] = (lp - lm) / (2 * h)
        err = np.abs(fd - g).max() / max(np.abs(g).max(), 1e-30)
        assert err <= 1e-6, (name, err)


@pytest.mark.parametrize("nq,nk,causal", [(24, 24, False), (24, 24, True), (13, 30, True)])
def test_backward_matches_torch_autograd_fp64(nq, nk, causal):
    B, H, d = 2, 2, 8
    q, k, v, dout = rand(B, H, nq, d), rand(B, H, nk, d), rand(B, H, nk, d), rand(B, H, nq, d)
    scale = 0.35
    dq, dk, dv, D = oracle.attn_bwd(q, k, v, dout, causal, scale)
    tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    s = torch.matmul(tq, tk.transpose(-1, -2)) * scale
    if causal:
        i = torch.arange(nq).unsqueeze(1)
        j = torch.arange(nk).unsqueeze(0)
        s = s.masked_fill(j > i + (nk - nq), float("-inf"))
    o = torch.matmul(torch.softmax(s, dim=-1), tv)
    o.backward(torch.from_numpy(dout))
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-11, atol=1e-12)


def test_backward_identities():
    # D_i = sum_j P_ij dP_ij equals <dO_i, O_i>; sum_j dK_j = 0 (rows of dS sum to zero);
    # sum_j dV_j = sum_i dO_i (rows of P sum to one).
    B, H, N, d = 1, 3, 29, 6
    q, k, v, dout = rand(B, H, N, d), rand(B, H, N, d), rand(B, H, N, d), rand(B, H, N, d)
    for causal in (False, True):
        o, _ = oracle.attn_fwd(q, k, v, causal, 0.4)
        dq, dk, dv, D = oracle.attn_bwd(q, k, v, dout, causal, 0.4)
        np.testing.assert_allclose(D, (dout * o).sum(-1), rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(dk.sum(axis=2), 0.0, rtol=0, atol=1e-12)
        np.testing.assert_allclose(dv.sum(axis=2), dout.sum(axis=2), rtol=1e-12, atol=1e-12)


def test_argument_errors_are_reported():
    with pytest.raises(ValueError):
        oracle.attn_fwd_blockwise(rand(4, 2), rand(4, 2), rand(4, 2), False, 1.0, 0, 2)
    with pytest.raises(ValueError):
        oracle.online_merge(rand(5), [3, 2])


@pytest.mark.parametrize("nq,nk,causal", [(6, 6, True), (5, 8, True), (7, 4, False)])
def test_matmul_backward_matches_finite_differences_and_loops(nq, nk, causal):
    d = 3
    q, k, v, dout = rand(1, 1, nq, d), rand(1, 1, nk, d), rand(1, 1, nk, d), rand(1, 1, nq, d)
    scale = 0.45
    ref = oracle.attn_bwd(q, k, v, dout, causal, scale, nthreads=1)
    got = oracle.attn_bwd_matmul(q, k, v, dout, causal, scale)
    for a, b in zip(got, ref):
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)
    h = 1e-6
    for name, x, g in (("q", q, got[0]), ("k", k, got[1]), ("v", v, got[2])):
        fd = np.empty_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args = {"q": q, "k": k, "v": v}
            fd[idx] = (loss(**{**args, name: xp}, dout=dout, causal=causal, scale=scale)
                       - loss(**{**args, name: xm}, dout=dout, causal=causal, scale=scale)) / (2 * h)
        assert np.abs(fd - g).max() <= 1e-6 * np.abs(g).max()


def test_matmul_backward_matches_loops_on_a_multi_head_case():
    B, H, N, d = 2, 2, 40, 16
    q, k, v, dout = rand(B, H, N, d), rand(B, H, N, d), rand(B, H, N, d), rand(B, H, N, d)
    for causal in (False, True):
        ref = oracle.attn_bwd(q, k, v, dout, causal, 0.25)
        got = oracle.attn_bwd_matmul(q, k, v, dout, causal, 0.25)
        for a, b in zip(got, ref):
            np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------- 8-bit inputs

def test_fp8_decode_matches_torch_e4m3fn_for_all_codes():
    """Every e4m3 code decodes to PyTorch's float8_e4m3fn value (an independent library
    implementation of the OCP format); the NaN codes are exactly 0x7f and 0xff."""
    codes = np.arange(256, dtype=np.uint8)
    mine = oracle.fp8_e4m3_decode(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(mine)
    assert np.array_equal(nan, np.isnan(ref))
    assert sorted(np.nonzero(nan)[0].tolist()) == [0x7F, 0xFF]
    assert np.array_equal(mine[~nan], ref[~nan])
    assert np.array_equal(np.signbit(mine[~nan]), np.signbit(ref[~nan]))


def test_fp8_decode_closed_form_values():
    """Values that follow from the format's fields alone: 1.0 (exponent field 7), the largest
    finite value 1.75 * 2^8 = 448, the smallest subnormal 2^-9, the largest subnormal 7 * 2^-9,
    the smallest normal 2^-6, and the sign bit."""
    got = oracle.fp8_e4m3_decode(np.array([0x38, 0x7E, 0x01, 0x07, 0x08, 0xB8, 0x00, 0x80], np.uint8))
    assert got.tolist() == [1.0, 448.0, 2.0**-9, 7 * 2.0**-9, 2.0**-6, -1.0, 0.0, -0.0]


def _fp8_case(B=2, H=3, nq=13, nk=21, d=16, seed=5):
    rng = np.random.default_rng(seed)
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    q8 = rng.choice(finite, size=(B, H, nq, d))
    k8 = rng.choice(finite, size=(B, H, nk, d))
    v8 = rng.choice(finite, size=(B, H, nk, d))
    ds = [np.exp2(rng.integers(-9, -5, size=(B, H))).astype(np.float64) * rng.uniform(0.5, 1.0, size=(B, H))
          for _ in range(3)]
    return q8, k8, v8, ds


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_attention_is_attention_of_the_scaled_decoded_inputs(causal):
    """Per head (b, h) the real inputs are descale[b, h] * value(code): PyTorch's e4m3 decode,
    scaled head by head, fed to PyTorch's own fp64 softmax attention, gives the same O and lse.
    A descale applied to the wrong tensor or the wrong head fails this."""
    q8, k8, v8, (dq, dk, dv) = _fp8_case()
    scale = 0.25
    o, lse = oracle.attn_fwd_fp8(q8, k8, v8, dq, dk, dv, causal, scale)
    dec = lambda c: torch.from_numpy(c.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    q = dec(q8) * dq[:, :, None, None]
    k = dec(k8) * dk[:, :, None, None]
    v = dec(v8) * dv[:, :, None, None]
    s = torch_attention(q, k, v, causal, scale)
    ref_lse = torch.logsumexp(s, dim=-1).numpy()
    ref_o = torch.matmul(torch.softmax(s, dim=-1), torch.from_numpy(v)).numpy()
    np.testing.assert_allclose(o, ref_o, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-12, atol=1e-12)


def test_fp8_attention_scale_invariances():
    """Doubling the value scale doubles O and leaves lse; moving a factor 2 from the key scale to
    the query scale changes nothing (the scores are bilinear in the two scales); a value tensor
    whose rows all hold the same codes returns those values for every query."""
    q8, k8, v8, (dq, dk, dv) = _fp8_case(seed=6)
    o, lse = oracle.attn_fwd_fp8(q8, k8, v8, dq, dk, dv, True, 0.5)
    o2, lse2 = oracle.attn_fwd_fp8(q8, k8, v8, dq, dk, 2 * dv, True, 0.5)
    np.testing.assert_allclose(o2, 2 * o, rtol=1e-14, atol=0)
    np.testing.assert_array_equal(lse2, lse)
    o3, lse3 = oracle.attn_fwd_fp8(q8, k8, v8, 2 * dq, dk / 2, dv, True, 0.5)
    np.testing.assert_allclose(o3, o, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse3, lse, rtol=1e-12, atol=1e-14)
    vconst = np.broadcast_to(v8[:, :, :1, :], v8.shape).copy()
    o4, _ = oracle.attn_fwd_fp8(q8, k8, vconst, dq, dk, dv, False, 0.5)
    row = oracle.fp8_e4m3_decode(v8[:, :, :1, :]) * dv[:, :, None, None]
    np.testing.assert_allclose(o4, np.broadcast_to(row, o4.shape), rtol=1e-12, atol=0)
