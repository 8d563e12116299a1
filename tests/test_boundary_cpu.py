"""The C ABI without a GPU: the library loads, exports what include/attn.h declares, and
rejects bad arguments on the host before any HIP call.

Every call below fails validation, so nothing is ever launched (fake pointers are never
dereferenced).  Calls that would pass validation are not made here.
"""
import os
import re

import pytest

import tiled_online_softmax_02_amd as A

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

# fake, 16-byte aligned, never dereferenced device addresses (distinct, non-overlapping)
P = [0x7f0000000000 + i * (1 << 36) for i in range(12)]


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(A.LIB_PATH):
        from tiled_online_softmax_02_amd import build
        build.build()
    return A.library()


def declared_functions():
    text = open(HEADER).read()
    # declarations start at column 0 with their return type; comment lines start with "/*" or " *"
    return sorted(set(re.findall(r"^[a-z][\w ]*?[\s*](attn_\w+)\s*\(", text, re.M)))


def test_header_declares_the_expected_entry_points():
    assert declared_functions() == sorted([
        "attn_fwd", "attn_fwd_qk", "attn_fwd_splitkv", "attn_fwd_splitkv_workspace_size", "attn_fwd_splitkv_noalloc",
        "attn_fwd_splitkv_default_splits", "attn_fwd_splitkv_default_splits_qk", "attn_fwd_fp8", "attn_bwd", "attn_bwd_qk", "attn_bwd_preprocess", "attn_bwd_dkdv",
        "attn_bwd_dq", "attn_bwd_dq_delta", "attn_status_string", "attn_last_hip_error"])


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code in range(0, 11):
        s = A.attn_status_string(code)
        assert s and s != "unknown status"
    assert A.attn_status_string(99) == "unknown status"
    assert lib.attn_last_hip_error() == 0


def fwd(lib, q=P[0], k=P[1], v=P[2], o=P[3], lse=P[4], B=1, H=1, N=64, d=64, causal=0, scale=0.125):
    return lib.attn_fwd(q, k, v, o, lse, B, H, N, d, causal, scale, None)


@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), A.ATTN_ERR_BAD_SHAPE),
    (dict(H=-3), A.ATTN_ERR_BAD_SHAPE),
    (dict(N=-1), A.ATTN_ERR_BAD_SHAPE),
    (dict(d=96), A.ATTN_ERR_UNSUPPORTED_D),
    (dict(d=0), A.ATTN_ERR_UNSUPPORTED_D),
    (dict(d=320), A.ATTN_ERR_UNSUPPORTED_D),
    (dict(d=160), A.ATTN_ERR_UNSUPPORTED_D),
    (dict(N=1 << 24, d=128), A.ATTN_ERR_BAD_SHAPE),   # (N+256)*d*2 > 2^32
    (dict(N=(1 << 24) - 200, d=128), A.ATTN_ERR_BAD_SHAPE),  # (N+256)*d*2 just above 2^32
    (dict(N=2**31 - 1, d=64), A.ATTN_ERR_BAD_SHAPE),   # INT_MAX rows: N + 256 is formed in 64 bits
    (dict(N=2**31 - 200, d=64), A.ATTN_ERR_BAD_SHAPE),
    (dict(B=2**31 - 1, H=2**31 - 1, N=2**31 - 1, d=256), A.ATTN_ERR_BAD_SHAPE),
    (dict(causal=2), A.ATTN_ERR_BAD_ARG),
    (dict(causal=-1), A.ATTN_ERR_BAD_ARG),
    (dict(scale=0.0), A.ATTN_ERR_BAD_SCALE),
    (dict(scale=-0.125), A.ATTN_ERR_BAD_SCALE),
    (dict(scale=float("nan")), A.ATTN_ERR_BAD_SCALE),
    (dict(scale=float("inf")), A.ATTN_ERR_BAD_SCALE),
    (dict(q=None), A.ATTN_ERR_NULLPTR),
    (dict(lse=None), A.ATTN_ERR_NULLPTR),
    (dict(k=P[1] + 2), A.ATTN_ERR_MISALIGNED),
    (dict(o=P[3] + 8), A.ATTN_ERR_MISALIGNED),
    (dict(o=P[0]), A.ATTN_ERR_ALIAS),                  # o == q
    (dict(lse=P[2] + 64), A.ATTN_ERR_ALIAS),           # lse inside v
    (dict(o=P[2] + 8192 - 16), A.ATTN_ERR_ALIAS),      # o overlaps the tail of v (64*64*2 bytes)
])
def test_forward_argument_checks(lib, kw, status):
    assert fwd(lib, **kw) == status


def test_empty_problems_are_valid_no_ops(lib):
    # nothing is launched, pointers may be NULL
    assert fwd(lib, q=None, k=None, v=None, o=None, lse=None, B=0) == A.ATTN_OK
    assert fwd(lib, q=None, k=None, v=None, o=None, lse=None, N=0) == A.ATTN_OK
    assert lib.attn_bwd(*([None] * 10), 1, 0, 64, 128, 1, 0.1, None) == A.ATTN_OK
    assert lib.attn_bwd_preprocess(None, None, None, 0, 1, 1, 64, None) == A.ATTN_OK
    # an empty problem is still checked for d, causal and scale
    assert fwd(lib, B=0, d=80) == A.ATTN_ERR_UNSUPPORTED_D
    assert fwd(lib, N=0, scale=0.0) == A.ATTN_ERR_BAD_SCALE


def test_backward_argument_checks(lib):
    args = [P[0], P[1], P[2], P[3], P[4], P[5], P[6], P[7], P[8], P[9]]

    def bwd(**kw):
        a = list(args)
        for i, val in kw.get("ptr", {}).items():
            a[i] = val
        return lib.attn_bwd(*a, kw.get("B", 2), kw.get("H", 2), kw.get("N", 128), kw.get("d", 128),
                            kw.get("causal", 1), kw.get("scale", 0.088), None)

    assert bwd(d=32) == A.ATTN_ERR_UNSUPPORTED_D
    assert bwd(scale=float("nan")) == A.ATTN_ERR_BAD_SCALE
    assert bwd(causal=5) == A.ATTN_ERR_BAD_ARG
    assert bwd(ptr={9: None}) == A.ATTN_ERR_NULLPTR      # delta workspace
    assert bwd(ptr={6: P[0]}) == A.ATTN_ERR_ALIAS        # dq == q
    assert bwd(ptr={7: P[6]}) == A.ATTN_ERR_ALIAS        # dk == dq
    assert bwd(ptr={9: P[5]}) == A.ATTN_ERR_ALIAS        # delta == lse
    assert bwd(ptr={8: P[8] + 4}) == A.ATTN_ERR_MISALIGNED
    # the three step entry points check their own arguments
    assert lib.attn_bwd_preprocess(P[0], P[1], P[0], 1, 1, 64, 64, None) == A.ATTN_ERR_ALIAS
    assert lib.attn_bwd_preprocess(P[0], None, P[2], 1, 1, 64, 64, None) == A.ATTN_ERR_NULLPTR
    assert lib.attn_bwd_dkdv(P[0], P[1], P[2], P[3], P[4], P[5], P[6], P[6], 1, 1, 64, 64, 0, 0.125,
                             None) == A.ATTN_ERR_ALIAS
    assert lib.attn_bwd_dq(P[0], P[1], P[2], P[3], P[4], P[5], P[6], 1, 1, 64, 64, 0, 0.0,
                           None) == A.ATTN_ERR_BAD_SCALE
    assert lib.attn_bwd_dq(P[0], P[1], P[2], P[3], P[4], P[5], P[6], 1, 1, 64, 100, 0, 0.1,
                           None) == A.ATTN_ERR_UNSUPPORTED_D
    # attn_bwd_dq_delta: q, k, v, o, dout, lse in; delta, dq out
    dqd = lambda *p, d=64, scale=0.125: lib.attn_bwd_dq_delta(*p, 1, 1, 64, d, 0, scale, None)
    assert dqd(P[0], P[1], P[2], P[3], P[4], P[5], P[6], P[7], scale=0.0) == A.ATTN_ERR_BAD_SCALE
    assert dqd(P[0], P[1], P[2], P[3], P[4], P[5], P[6], P[7], d=100) == A.ATTN_ERR_UNSUPPORTED_D
    assert dqd(P[0], P[1], P[2], None, P[4], P[5], P[6], P[7]) == A.ATTN_ERR_NULLPTR       # o
    assert dqd(P[0], P[1], P[2], P[3], P[4], P[5], P[3], P[7]) == A.ATTN_ERR_ALIAS         # delta == o
    assert dqd(P[0], P[1], P[2], P[3], P[4], P[5], P[6], P[6]) == A.ATTN_ERR_ALIAS         # dq == delta
    assert dqd(P[0], P[1], P[2], P[3], P[4], P[5], P[6], P[7] + 4) == A.ATTN_ERR_MISALIGNED


def test_python_binding_raises_with_status(lib):
    with pytest.raises(A.AttnError) as e:
        A.attn_fwd(P[0], P[1], P[2], P[3], P[4], 1, 1, 64, 64, False, -1.0)
    assert e.value.status == A.ATTN_ERR_BAD_SCALE


def fwd_qk(lib, q=P[0], k=P[1], v=P[2], o=P[3], lse=P[4], B=1, H=1, Hk=None, Nq=64, Nk=128, d=64, causal=1,
           scale=0.125):
    return lib.attn_fwd_qk(q, k, v, o, lse, B, H, H if Hk is None else Hk, Nq, Nk, d, causal, scale, None)


@pytest.mark.parametrize("kw,status", [
    (dict(Nq=-1), A.ATTN_ERR_BAD_SHAPE),
    (dict(Nk=-1), A.ATTN_ERR_BAD_SHAPE),
    (dict(Nk=1 << 24, d=128), A.ATTN_ERR_BAD_SHAPE),    # (Nk+256)*d*2 > 2^32
    (dict(Nk=16776960, d=128), A.ATTN_ERR_BAD_SHAPE),   # one row past the longest accepted key length
    (dict(Nq=1 << 24, d=128), A.ATTN_ERR_BAD_SHAPE),
    (dict(Nq=2**31 - 1), A.ATTN_ERR_BAD_SHAPE),         # INT_MAX lengths: no signed overflow in the checks
    (dict(Nk=2**31 - 1), A.ATTN_ERR_BAD_SHAPE),
    (dict(d=96), A.ATTN_ERR_UNSUPPORTED_D),
    (dict(causal=3), A.ATTN_ERR_BAD_ARG),
    (dict(k=None), A.ATTN_ERR_NULLPTR),                 # Nk > 0: k is required
    (dict(o=None), A.ATTN_ERR_NULLPTR),
    (dict(v=P[2] + 4), A.ATTN_ERR_MISALIGNED),
    (dict(o=P[1] + 16384 - 16), A.ATTN_ERR_ALIAS),      # inside k, whose size is Nk*d*2 = 16384
    (dict(lse=P[0] + 8192 - 16), A.ATTN_ERR_ALIAS),     # inside q, whose size is Nq*d*2 = 8192
    (dict(H=4, Hk=3), A.ATTN_ERR_BAD_SHAPE),             # H must be a multiple of Hk
    (dict(H=4, Hk=0), A.ATTN_ERR_BAD_SHAPE),
    (dict(H=4, Hk=-1), A.ATTN_ERR_BAD_SHAPE),
    (dict(H=4, Hk=8), A.ATTN_ERR_BAD_SHAPE),
    (dict(H=4, Hk=2, o=P[1] + 2 * 16384 - 16), A.ATTN_ERR_ALIAS),   # k holds Hk = 2 heads of 16384 B
])
def test_forward_qk_argument_checks(lib, kw, status):
    assert fwd_qk(lib, **kw) == status


def test_qk_empty_problems(lib):
    # no query rows: the forward has nothing to write and accepts NULL everywhere
    assert fwd_qk(lib, q=None, k=None, v=None, o=None, lse=None, Nq=0, Nk=64) == A.ATTN_OK
    # the backward with Nq = Nk = 0 is empty
    assert lib.attn_bwd_qk(*([None] * 10), 1, 1, 1, 0, 0, 64, 1, 0.125, None) == A.ATTN_OK


def test_backward_qk_argument_checks(lib):
    args = [P[0], P[1], P[2], P[3], P[4], P[5], P[6], P[7], P[8], P[9]]

    def bwd(Nq=64, Nk=96, **kw):
        a = list(args)
        for i, val in kw.get("ptr", {}).items():
            a[i] = val
        return lib.attn_bwd_qk(*a, 1, 2, kw.get("Hk", 2), Nq, Nk, 64, 1, 0.125, None)

    assert bwd(Nq=-2) == A.ATTN_ERR_BAD_SHAPE
    assert bwd(ptr={9: None}) == A.ATTN_ERR_NULLPTR     # delta
    assert bwd(ptr={1: None}) == A.ATTN_ERR_NULLPTR     # k with Nk > 0
    assert bwd(ptr={7: P[1]}) == A.ATTN_ERR_ALIAS       # dk == k
    assert bwd(ptr={6: P[3] + 16384 - 16}) == A.ATTN_ERR_ALIAS  # dq inside o (Nq rows: 2*64*64*2 B)
    assert bwd(ptr={8: P[2] + 24576 - 16}) == A.ATTN_ERR_ALIAS  # dv inside v (Nk rows: 2*96*64*2 B)
    assert bwd(Hk=3) == A.ATTN_ERR_BAD_SHAPE                   # 2 query heads over 3 K/V heads


def test_splitkv_workspace_size_and_default_splits(lib):
    assert A.attn_fwd_splitkv_workspace_size(2, 3, 5, 128, 4) == 4 * 2 * 3 * 5 * 129 * 4
    assert A.attn_fwd_splitkv_workspace_size(1, 1, 1, 64, 1) == 65 * 4
    assert A.attn_fwd_splitkv_workspace_size(1, 1, 1, 96, 1) == -1
    assert A.attn_fwd_splitkv_workspace_size(1, 1, 1, 64, 0) == -1
    assert A.attn_fwd_splitkv_workspace_size(1, 1, -1, 64, 2) == -1
    # decoding: 1 query row per head -> enough pieces for ~512 workgroups of the decoding kernel
    assert A.attn_fwd_splitkv_default_splits(4, 16, 1, 16384, 128) == 8     # 64 heads
    assert A.attn_fwd_splitkv_default_splits(2, 16, 1, 65536, 128) == 16    # 32 heads
    # grouped heads: the rows of a K/V head share workgroups (up to 4 rows each), so fewer items
    assert A.attn_fwd_splitkv_default_splits_qk(2, 32, 8, 1, 32768, 128) == 32   # 16 items
    assert A.attn_fwd_splitkv_default_splits_qk(2, 64, 8, 1, 32768, 128) == 16   # 8 rows: 2 groups
    assert A.attn_fwd_splitkv_default_splits_qk(2, 16, 16, 1, 65536, 128) == \
        A.attn_fwd_splitkv_default_splits(2, 16, 1, 65536, 128)
    assert A.attn_fwd_splitkv_default_splits_qk(2, 16, 3, 1, 4096, 128) == 1     # Hk must divide H
    # d = 192 and more than 4 rows per head: matrix-instruction pieces, ~256 workgroups
    assert A.attn_fwd_splitkv_default_splits(2, 16, 1, 65536, 192) == 8
    assert A.attn_fwd_splitkv_default_splits(2, 16, 8, 65536, 128) == 8
    # few keys: at least two 64-key blocks per piece
    assert A.attn_fwd_splitkv_default_splits(1, 1, 1, 256, 128) == 2
    assert A.attn_fwd_splitkv_default_splits(1, 1, 1, 64, 128) == 1
    # many heads and query blocks already fill the GPU
    assert A.attn_fwd_splitkv_default_splits(8, 64, 4096, 4096, 128) == 1


def splitkv(lib, q=P[0], k=P[1], v=P[2], o=P[3], lse=P[4], ws=P[5], wsb=None, B=1, H=2, Nq=4, Nk=512, d=64,
            causal=0, scale=0.125, ns=4):
    if wsb is None:
        wsb = ns * B * H * Nq * (d + 1) * 4
    return lib.attn_fwd_splitkv(q, k, v, o, lse, B, H, H, Nq, Nk, d, causal, scale, ns, ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(ns=0), A.ATTN_ERR_BAD_ARG),
    (dict(ns=257), A.ATTN_ERR_BAD_ARG),
    (dict(ws=None), A.ATTN_ERR_NULLPTR),
    (dict(ws=P[5] + 8), A.ATTN_ERR_MISALIGNED),
    (dict(wsb=4 * 2 * 4 * 65 * 4 - 1), A.ATTN_ERR_WORKSPACE),
    (dict(ws=P[3]), A.ATTN_ERR_ALIAS),                 # workspace over o
    (dict(ws=P[1] + 64), A.ATTN_ERR_ALIAS),            # workspace inside k
    (dict(Nk=-5), A.ATTN_ERR_BAD_SHAPE),
    (dict(d=80), A.ATTN_ERR_UNSUPPORTED_D),
    (dict(scale=0.0), A.ATTN_ERR_BAD_SCALE),
])
def test_splitkv_argument_checks(lib, kw, status):
    assert splitkv(lib, **kw) == status


def test_splitkv_empty_is_a_no_op(lib):
    assert splitkv(lib, q=None, k=None, v=None, o=None, lse=None, ws=None, Nq=0) == A.ATTN_OK


def splitkv_noalloc(lib, q=P[0], k=P[1], v=P[2], o=P[3], lse=P[4], B=1, H=2, Nq=4, Nk=512, d=64, causal=0,
                    scale=0.125, ns=4):
    return lib.attn_fwd_splitkv_noalloc(q, k, v, o, lse, B, H, H, Nq, Nk, d, causal, scale, ns, None)


@pytest.mark.parametrize("kw,status", [
    (dict(ns=0), A.ATTN_ERR_BAD_ARG),
    (dict(ns=257), A.ATTN_ERR_BAD_ARG),
    (dict(q=None), A.ATTN_ERR_NULLPTR),
    (dict(lse=P[4] + 4), A.ATTN_ERR_MISALIGNED),
    (dict(o=P[1] + 64), A.ATTN_ERR_ALIAS),
    (dict(Nk=-5), A.ATTN_ERR_BAD_SHAPE),
    (dict(d=80), A.ATTN_ERR_UNSUPPORTED_D),
    (dict(scale=0.0), A.ATTN_ERR_BAD_SCALE),
    (dict(causal=3), A.ATTN_ERR_BAD_ARG),
    # pieces of 64 heads x 4096 rows x 129 floats x 4 splits: far beyond the 16 MiB buffer
    (dict(H=64, Nq=4096, d=128), A.ATTN_ERR_SCRATCH),
    # the smallest single-head size past the buffer fails the same way, before any pointer is looked at
    (dict(q=None, H=1, Nq=8129, d=128, ns=4), A.ATTN_ERR_SCRATCH),
])
def test_splitkv_noalloc_argument_checks(lib, kw, status):
    assert splitkv_noalloc(lib, **kw) == status


def test_splitkv_noalloc_scratch_limit_matches_the_workspace_size(lib):
    # the largest single-head problem that fits: ns * Nq * (d + 1) * 4 <= 16 MiB
    assert A.attn_fwd_splitkv_workspace_size(1, 1, 8129, 128, 4) > A.ATTN_NOALLOC_SCRATCH_BYTES
    assert A.attn_fwd_splitkv_workspace_size(1, 1, 8128, 128, 4) <= A.ATTN_NOALLOC_SCRATCH_BYTES


def test_splitkv_noalloc_empty_is_a_no_op(lib):
    assert splitkv_noalloc(lib, q=None, k=None, v=None, o=None, lse=None, Nq=0) == A.ATTN_OK
    assert splitkv_noalloc(lib, q=None, k=None, v=None, o=None, lse=None, B=0) == A.ATTN_OK


def fwd8(lib, q=P[0], k=P[1], v=P[2], dq=P[5], dk=P[6], dv=P[7], o=P[3], lse=P[4], B=1, H=2, Hk=1, Nq=64, Nk=80,
         d=128, causal=1, scale=0.125):
    return lib.attn_fwd_fp8(q, k, v, dq, dk, dv, o, lse, B, H, Hk, Nq, Nk, d, causal, scale, None)


@pytest.mark.parametrize("kw,status", [
    (dict(d=192), A.ATTN_ERR_UNSUPPORTED_D),
    (dict(d=256), A.ATTN_ERR_UNSUPPORTED_D),
    (dict(d=32), A.ATTN_ERR_UNSUPPORTED_D),
    (dict(H=3, Hk=2), A.ATTN_ERR_BAD_SHAPE),
    (dict(Nk=-1), A.ATTN_ERR_BAD_SHAPE),
    (dict(causal=2), A.ATTN_ERR_BAD_ARG),
    (dict(scale=0.0), A.ATTN_ERR_BAD_SCALE),
    (dict(q=0), A.ATTN_ERR_NULLPTR),
    (dict(dq=0), A.ATTN_ERR_NULLPTR),
    (dict(dv=0), A.ATTN_ERR_NULLPTR),
    (dict(k=P[1] + 8), A.ATTN_ERR_MISALIGNED),
    (dict(dk=P[6] + 2), A.ATTN_ERR_MISALIGNED),
    (dict(o=P[0]), A.ATTN_ERR_ALIAS),
    (dict(lse=P[5]), A.ATTN_ERR_ALIAS),           # lse on top of the query scales
    (dict(o=P[7] - 64), A.ATTN_ERR_ALIAS),        # o runs into the value scales
])
def test_fp8_forward_argument_checks(lib, kw, status):
    assert fwd8(lib, **kw) == status


def test_fp8_forward_empty_is_a_no_op(lib):
    assert fwd8(lib, q=0, o=0, lse=0, Nq=0) == A.ATTN_OK
    assert fwd8(lib, B=0, q=0, k=0, v=0, dq=0, dk=0, dv=0, o=0, lse=0) == A.ATTN_OK
