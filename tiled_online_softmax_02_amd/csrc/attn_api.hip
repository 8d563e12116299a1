// attn_api.hip -- the C ABI declared in include/attn.h: host-side argument
// checks, then kernel launches on the caller's stream.  Nothing here allocates
// device memory, synchronises or prints.
#include <math.h>
#include <stdint.h>

#include <atomic>

#include "../../include/attn.h"
#include "attn_launch.h"

namespace {

thread_local int g_last_hip_error = 0;

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};

Range range_of(const void *p, long long bytes) { return Range{(uintptr_t)p, (uintptr_t)p + (uintptr_t)bytes}; }

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }  // empty ranges never overlap

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Shape rules shared by every entry point: H query heads and Hk K/V heads (H a multiple of
// Hk), Nq query rows and Nk key rows per head.  Sets *empty when there is nothing to compute.
int check_shape(int B, int H, int Hk, int Nq, int Nk, int d, bool *empty)
{
    if (B < 0 || H < 0 || Hk < 0 || Nq < 0 || Nk < 0) return ATTN_ERR_BAD_SHAPE;
    if (H > 0 && (Hk < 1 || H % Hk != 0)) return ATTN_ERR_BAD_SHAPE;
    if (d != 64 && d != 128 && d != 192 && d != 256) return ATTN_ERR_UNSUPPORTED_D;
    // B * H * N of three ints can pass 2^63: form the products with an overflow check
    long long rows_q = 0, rows_k = 0;
    if (__builtin_mul_overflow((long long)B * H, (long long)Nq, &rows_q) ||
        __builtin_mul_overflow((long long)B * Hk, (long long)Nk, &rows_k))
        return ATTN_ERR_BAD_SHAPE;
    if (rows_q > ((1LL << 62) - 1) / d || rows_k > ((1LL << 62) - 1) / d) return ATTN_ERR_BAD_SHAPE;  // B*H*N*d < 2^62
    // per-head byte offsets, including the padding rows of the last tile, are 32-bit
    if (((long long)Nq + 256) * d * 2 > 0xFFFFFFFFLL || ((long long)Nk + 256) * d * 2 > 0xFFFFFFFFLL)
        return ATTN_ERR_BAD_SHAPE;
    // work-group counts of the launches must fit a 32-bit grid
    if (attn::fwd_grid_size(B, H, Nq) >= (1LL << 31) || attn::bwd_dkdv_grid_size(B, Hk, Nk) >= (1LL << 31) ||
        attn::bwd_dq_grid_size(B, H, Nq) >= (1LL << 31) || rows_q / 16 >= (1LL << 31))
        return ATTN_ERR_BAD_SHAPE;
    *empty = (rows_q == 0 && rows_k == 0);
    return ATTN_OK;
}

int check_scale(float scale) { return (isfinite(scale) && scale > 0.f) ? ATTN_OK : ATTN_ERR_BAD_SCALE; }

int check_causal(int causal) { return (causal == 0 || causal == 1) ? ATTN_OK : ATTN_ERR_BAD_ARG; }

// Pointers: non-null and 16-byte aligned, except that a buffer of zero bytes may be NULL.
int check_ptrs(const void *const *ptrs, const long long *bytes, int n)
{
    for (int i = 0; i < n; ++i)
        if (!ptrs[i] && bytes[i] > 0) return ATTN_ERR_NULLPTR;
    for (int i = 0; i < n; ++i)
        if (!aligned16(ptrs[i])) return ATTN_ERR_MISALIGNED;
    return ATTN_OK;
}

// Every output range must be disjoint from every input range and from the other outputs.
int check_alias(const Range *in, int nin, const Range *out, int nout)
{
    for (int i = 0; i < nout; ++i) {
        for (int j = 0; j < nin; ++j)
            if (overlap(out[i], in[j])) return ATTN_ERR_ALIAS;
        for (int j = i + 1; j < nout; ++j)
            if (overlap(out[i], out[j])) return ATTN_ERR_ALIAS;
    }
    return ATTN_OK;
}

int hip_status(hipError_t e)
{
    if (e == hipSuccess) return ATTN_OK;
    g_last_hip_error = (int)e;
    return ATTN_ERR_HIP;
}

// Scratch of the no-allocation split-key forward: one static buffer per device, holding the pieces'
// partial outputs and log-sum-exps between the two launches.  In host code the array's name is only a
// stand-in; its device address on each device is looked up once (scratch_address) and used instead.
static __device__ __align__(256) char scratch[ATTN_NOALLOC_SCRATCH_BYTES];

// Compute units and XCDs of the device that `stream` belongs to (the current device for the null
// stream), queried once per device and then cached.
constexpr int kMaxDevices = 64;
std::atomic<long long> g_shape[kMaxDevices];  // (cus << 32) | nx, 0 until queried

int device_shape(void *stream, attn::DeviceShape *out)
{
    int dev = 0;
    hipError_t e = stream ? hipStreamGetDevice((hipStream_t)stream, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e);
    if (dev >= 0 && dev < kMaxDevices) {
        const long long v = g_shape[dev].load(std::memory_order_relaxed);
        if (v != 0) {
            out->cus = (int)(v >> 32);
            out->nx = (int)(v & 0xFFFFFFFF);
            return ATTN_OK;
        }
    }
    int cus = 0, nx = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_status(e);
    e = hipDeviceGetAttribute(&nx, hipDeviceAttributeNumberOfXccs, dev);
    if (e != hipSuccess) return hip_status(e);
    if (cus < 1 || nx < 1) return hip_status(hipErrorInvalidDevice);
    out->cus = cus;
    out->nx = nx;
    if (dev >= 0 && dev < kMaxDevices) g_shape[dev].store(((long long)cus << 32) | nx, std::memory_order_relaxed);
    return ATTN_OK;
}

// Device address of `scratch` on the device that `stream` belongs to, looked up once per device with
// that device current and then cached.
std::atomic<void *> g_scratch[kMaxDevices];

int scratch_address(void *stream, void **out)
{
    int dev = 0;
    hipError_t e = stream ? hipStreamGetDevice((hipStream_t)stream, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e);
    if (dev >= 0 && dev < kMaxDevices) {
        void *p = g_scratch[dev].load(std::memory_order_acquire);
        if (p) {
            *out = p;
            return ATTN_OK;
        }
    }
    int cur = 0;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return hip_status(e);
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return hip_status(e);
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
        const hipError_t e2 = hipSetDevice(cur);
        if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return hip_status(e);
    if (!p) return hip_status(hipErrorInvalidSymbol);
    if (dev >= 0 && dev < kMaxDevices) g_scratch[dev].store(p, std::memory_order_release);
    *out = p;
    return ATTN_OK;
}

#define RETURN_IF(x)               \
    do {                           \
        const int rc_ = (x);       \
        if (rc_ != ATTN_OK) return rc_; \
    } while (0)

int validate_common(int B, int H, int Hk, int Nq, int Nk, int d, int causal, float scale, bool *empty)
{
    RETURN_IF(check_shape(B, H, Hk, Nq, Nk, d, empty));
    RETURN_IF(check_causal(causal));
    RETURN_IF(check_scale(scale));
    return ATTN_OK;
}

// Byte sizes of one [B, H, rows, d] bf16 tensor and of one [B, H, rows] fp32 vector.
long long tensor_bytes(int B, int H, int rows, int d) { return (long long)B * H * rows * d * 2; }
long long vector_bytes(int B, int H, int rows) { return (long long)B * H * rows * 4; }

int fwd_impl(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H, int Hk, int Nq, int Nk,
             int d, int causal, float scale, void *stream)
{
    bool empty = false;
    RETURN_IF(validate_common(B, H, Hk, Nq, Nk, d, causal, scale, &empty));
    const long long qb = tensor_bytes(B, H, Nq, d), kb = tensor_bytes(B, Hk, Nk, d), lb = vector_bytes(B, H, Nq);
    if (qb == 0) return ATTN_OK;  // no query rows: nothing to write
    const void *ptrs[] = {q, k, v, o, lse};
    const long long sizes[] = {qb, kb, kb, qb, lb};
    RETURN_IF(check_ptrs(ptrs, sizes, 5));
    const Range in[] = {range_of(q, qb), range_of(k, kb), range_of(v, kb)};
    const Range out[] = {range_of(o, qb), range_of(lse, lb)};
    RETURN_IF(check_alias(in, 3, out, 2));
    attn::FwdArgs a{q, k, v, o, lse, B, H, Hk, Nq, Nk, d, causal, scale, stream, {}};
    RETURN_IF(device_shape(stream, &a.dev));
    return hip_status(attn::launch_fwd(a));
}

int fwd_split_impl(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H, int Hk, int Nq,
                   int Nk, int d, int causal, float scale, int num_splits, void *workspace,
                   long long workspace_bytes, void *stream)
{
    bool empty = false;
    RETURN_IF(validate_common(B, H, Hk, Nq, Nk, d, causal, scale, &empty));
    if (num_splits < 1 || num_splits > 256) return ATTN_ERR_BAD_ARG;
    const long long qb = tensor_bytes(B, H, Nq, d), kb = tensor_bytes(B, Hk, Nk, d), lb = vector_bytes(B, H, Nq);
    if (qb == 0) return ATTN_OK;  // no query rows: nothing to write
    if (attn::fwd_split_grid_size(B, H, Nq, num_splits) >= (1LL << 31)) return ATTN_ERR_BAD_SHAPE;
    const long long wb = attn::fwd_split_workspace_bytes(B, H, Nq, d, num_splits);
    if (wb < 0) return ATTN_ERR_BAD_SHAPE;
    const void *ptrs[] = {q, k, v, o, lse, workspace};
    const long long sizes[] = {qb, kb, kb, qb, lb, wb};
    RETURN_IF(check_ptrs(ptrs, sizes, 6));
    if (workspace_bytes < wb) return ATTN_ERR_WORKSPACE;
    const Range in[] = {range_of(q, qb), range_of(k, kb), range_of(v, kb)};
    const Range out[] = {range_of(o, qb), range_of(lse, lb), range_of(workspace, wb)};
    RETURN_IF(check_alias(in, 3, out, 3));
    attn::FwdArgs a{q, k, v, o, lse, B, H, Hk, Nq, Nk, d, causal, scale, stream, {}};
    RETURN_IF(device_shape(stream, &a.dev));
    return hip_status(attn::launch_fwd_split(a, num_splits, workspace));
}

// The split-key forward with its workspace in the static scratch buffer: the same checks without the
// workspace argument, and the workspace size against the buffer's.
int fwd_split_noalloc_impl(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H, int Hk,
                           int Nq, int Nk, int d, int causal, float scale, int num_splits, void *stream)
{
    bool empty = false;
    RETURN_IF(validate_common(B, H, Hk, Nq, Nk, d, causal, scale, &empty));
    if (num_splits < 1 || num_splits > 256) return ATTN_ERR_BAD_ARG;
    const long long qb = tensor_bytes(B, H, Nq, d), kb = tensor_bytes(B, Hk, Nk, d), lb = vector_bytes(B, H, Nq);
    if (qb == 0) return ATTN_OK;  // no query rows: nothing to write
    if (attn::fwd_split_grid_size(B, H, Nq, num_splits) >= (1LL << 31)) return ATTN_ERR_BAD_SHAPE;
    const long long wb = attn::fwd_split_workspace_bytes(B, H, Nq, d, num_splits);
    if (wb < 0) return ATTN_ERR_BAD_SHAPE;
    if (wb > ATTN_NOALLOC_SCRATCH_BYTES) return ATTN_ERR_SCRATCH;
    const void *ptrs[] = {q, k, v, o, lse};
    const long long sizes[] = {qb, kb, kb, qb, lb};
    RETURN_IF(check_ptrs(ptrs, sizes, 5));
    const Range in[] = {range_of(q, qb), range_of(k, kb), range_of(v, kb)};
    const Range out[] = {range_of(o, qb), range_of(lse, lb)};
    RETURN_IF(check_alias(in, 3, out, 2));
    void *ws = nullptr;
    RETURN_IF(scratch_address(stream, &ws));
    attn::FwdArgs a{q, k, v, o, lse, B, H, Hk, Nq, Nk, d, causal, scale, stream, {}};
    RETURN_IF(device_shape(stream, &a.dev));
    // every piece of every row is written by the first launch before the merge reads it, so the buffer
    // needs no clearing between calls
    return hip_status(attn::launch_fwd_split(a, num_splits, ws));
}

// Per-head scale arrays of the 8-bit forward: non-null (unless empty) and 4-byte aligned.
int check_scale_ptrs(const float *const *ptrs, const long long *bytes, int n)
{
    for (int i = 0; i < n; ++i)
        if (!ptrs[i] && bytes[i] > 0) return ATTN_ERR_NULLPTR;
    for (int i = 0; i < n; ++i)
        if (((uintptr_t)ptrs[i] & 3u) != 0) return ATTN_ERR_MISALIGNED;
    return ATTN_OK;
}

int fwd_fp8_impl(const void *q, const void *k, const void *v, const float *descale_q, const float *descale_k,
                 const float *descale_v, void *o, float *lse, int B, int H, int Hk, int Nq, int Nk, int d, int causal,
                 float scale, void *stream)
{
    bool empty = false;
    RETURN_IF(validate_common(B, H, Hk, Nq, Nk, d, causal, scale, &empty));
    if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED_D;
    const long long qb = tensor_bytes(B, H, Nq, d), kb = tensor_bytes(B, Hk, Nk, d), lb = vector_bytes(B, H, Nq);
    if (qb == 0) return ATTN_OK;  // no query rows: nothing to write
    // 8-bit inputs take half the bytes of the bf16 output
    const long long q8 = qb / 2, k8 = kb / 2;
    const long long sqb = (long long)B * H * 4, skb = (long long)B * Hk * 4;
    const void *ptrs[] = {q, k, v, o, lse};
    const long long sizes[] = {q8, k8, k8, qb, lb};
    RETURN_IF(check_ptrs(ptrs, sizes, 5));
    const float *sptrs[] = {descale_q, descale_k, descale_v};
    const long long ssizes[] = {sqb, skb, skb};
    RETURN_IF(check_scale_ptrs(sptrs, ssizes, 3));
    const Range in[] = {range_of(q, q8), range_of(k, k8), range_of(v, k8),
                        range_of(descale_q, sqb), range_of(descale_k, skb), range_of(descale_v, skb)};
    const Range out[] = {range_of(o, qb), range_of(lse, lb)};
    RETURN_IF(check_alias(in, 6, out, 2));
    attn::Fp8FwdArgs a{q, k, v, descale_q, descale_k, descale_v, o, lse, B, H, Hk, Nq, Nk, d, causal, scale, stream, {}};
    RETURN_IF(device_shape(stream, &a.dev));
    return hip_status(attn::launch_fwd_fp8(a));
}

int bwd_impl(const void *q, const void *k, const void *v, const void *o, const void *dout, const float *lse, void *dq,
             void *dk, void *dv, float *delta, int B, int H, int Hk, int Nq, int Nk, int d, int causal, float scale,
             void *stream)
{
    bool empty = false;
    RETURN_IF(validate_common(B, H, Hk, Nq, Nk, d, causal, scale, &empty));
    if (empty) return ATTN_OK;
    const long long qb = tensor_bytes(B, H, Nq, d), kb = tensor_bytes(B, Hk, Nk, d), lb = vector_bytes(B, H, Nq);
    const void *ptrs[] = {q, k, v, o, dout, lse, dq, dk, dv, delta};
    const long long sizes[] = {qb, kb, kb, qb, qb, lb, qb, kb, kb, lb};
    RETURN_IF(check_ptrs(ptrs, sizes, 10));
    const Range in[] = {range_of(q, qb), range_of(k, kb),    range_of(v, kb),
                        range_of(o, qb), range_of(dout, qb), range_of(lse, lb)};
    const Range out[] = {range_of(dq, qb), range_of(dk, kb), range_of(dv, kb), range_of(delta, lb)};
    RETURN_IF(check_alias(in, 6, out, 4));
    attn::BwdArgs a{q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, Hk, Nq, Nk, d, causal, scale, stream, {}};
    RETURN_IF(device_shape(stream, &a.dev));
    if (attn::bwd_dq_fuses_delta(d)) {
        // the dQ kernel forms D on the way (no preprocess launch), then dK/dV reads it
        RETURN_IF(hip_status(attn::launch_bwd_dq_delta(a)));
        return hip_status(attn::launch_bwd_dkdv(a));
    }
    RETURN_IF(hip_status(attn::launch_bwd_preprocess(a)));
    RETURN_IF(hip_status(attn::launch_bwd_dkdv(a)));
    return hip_status(attn::launch_bwd_dq(a));
}

}  // namespace

extern "C" {

int attn_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H, int N, int d, int causal,
             float scale, void *stream)
{
    return fwd_impl(q, k, v, o, lse, B, H, H, N, N, d, causal, scale, stream);
}

int attn_fwd_qk(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H, int Hk, int Nq, int Nk,
                int d, int causal, float scale, void *stream)
{
    return fwd_impl(q, k, v, o, lse, B, H, Hk, Nq, Nk, d, causal, scale, stream);
}

int attn_fwd_splitkv(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H, int Hk, int Nq,
                     int Nk, int d, int causal, float scale, int num_splits, void *workspace,
                     long long workspace_bytes, void *stream)
{
    return fwd_split_impl(q, k, v, o, lse, B, H, Hk, Nq, Nk, d, causal, scale, num_splits, workspace,
                          workspace_bytes, stream);
}

int attn_fwd_splitkv_noalloc(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H, int Hk,
                             int Nq, int Nk, int d, int causal, float scale, int num_splits, void *stream)
{
    return fwd_split_noalloc_impl(q, k, v, o, lse, B, H, Hk, Nq, Nk, d, causal, scale, num_splits, stream);
}

int attn_fwd_fp8(const void *q, const void *k, const void *v, const float *descale_q, const float *descale_k,
                 const float *descale_v, void *o, float *lse, int B, int H, int Hk, int Nq, int Nk, int d, int causal,
                 float scale, void *stream)
{
    return fwd_fp8_impl(q, k, v, descale_q, descale_k, descale_v, o, lse, B, H, Hk, Nq, Nk, d, causal, scale, stream);
}

long long attn_fwd_splitkv_workspace_size(int B, int H, int Nq, int d, int num_splits)
{
    bool empty = false;
    if (check_shape(B, H, H > 0 ? 1 : 0, Nq, 0, d, &empty) != ATTN_OK || num_splits < 1 || num_splits > 256) return -1;
    return attn::fwd_split_workspace_bytes(B, H, Nq, d, num_splits);
}

int attn_fwd_splitkv_default_splits_qk(int B, int H, int Hk, int Nq, int Nk, int d)
{
    bool empty = false;
    if (check_shape(B, H, Hk, Nq, Nk, d, &empty) != ATTN_OK) return 1;
    return attn::fwd_split_default(B, H, Hk, Nq, Nk, d);
}

int attn_fwd_splitkv_default_splits(int B, int H, int Nq, int Nk, int d)
{
    return attn_fwd_splitkv_default_splits_qk(B, H, H, Nq, Nk, d);
}

int attn_bwd_preprocess(const void *o, const void *dout, float *delta, int B, int H, int N, int d, void *stream)
{
    bool empty = false;
    RETURN_IF(check_shape(B, H, H, N, N, d, &empty));
    if (empty) return ATTN_OK;
    const long long tb = tensor_bytes(B, H, N, d), lb = vector_bytes(B, H, N);
    const void *ptrs[] = {o, dout, delta};
    const long long sizes[] = {tb, tb, lb};
    RETURN_IF(check_ptrs(ptrs, sizes, 3));
    const Range in[] = {range_of(o, tb), range_of(dout, tb)};
    const Range out[] = {range_of(delta, lb)};
    RETURN_IF(check_alias(in, 2, out, 1));
    attn::BwdArgs a{};
    a.o = o;
    a.dout = dout;
    a.delta = delta;
    a.B = B;
    a.H = H;
    a.Hk = H;
    a.Nq = a.Nk = N;
    a.d = d;
    a.stream = stream;
    RETURN_IF(device_shape(stream, &a.dev));
    return hip_status(attn::launch_bwd_preprocess(a));
}

int attn_bwd_dkdv(const void *q, const void *k, const void *v, const void *dout, const float *lse, const float *delta,
                  void *dk, void *dv, int B, int H, int N, int d, int causal, float scale, void *stream)
{
    bool empty = false;
    RETURN_IF(validate_common(B, H, H, N, N, d, causal, scale, &empty));
    if (empty) return ATTN_OK;
    const long long tb = tensor_bytes(B, H, N, d), lb = vector_bytes(B, H, N);
    const void *ptrs[] = {q, k, v, dout, lse, delta, dk, dv};
    const long long sizes[] = {tb, tb, tb, tb, lb, lb, tb, tb};
    RETURN_IF(check_ptrs(ptrs, sizes, 8));
    const Range in[] = {range_of(q, tb),    range_of(k, tb),     range_of(v, tb),
                        range_of(dout, tb), range_of(lse, lb),   range_of(delta, lb)};
    const Range out[] = {range_of(dk, tb), range_of(dv, tb)};
    RETURN_IF(check_alias(in, 6, out, 2));
    attn::BwdArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.dout = dout;
    a.lse = lse;
    a.delta = (float *)delta;
    a.dk = dk;
    a.dv = dv;
    a.B = B;
    a.H = H;
    a.Hk = H;
    a.Nq = a.Nk = N;
    a.d = d;
    a.causal = causal;
    a.scale = scale;
    a.stream = stream;
    RETURN_IF(device_shape(stream, &a.dev));
    return hip_status(attn::launch_bwd_dkdv(a));
}

int attn_bwd_dq(const void *q, const void *k, const void *v, const void *dout, const float *lse, const float *delta,
                void *dq, int B, int H, int N, int d, int causal, float scale, void *stream)
{
    bool empty = false;
    RETURN_IF(validate_common(B, H, H, N, N, d, causal, scale, &empty));
    if (empty) return ATTN_OK;
    const long long tb = tensor_bytes(B, H, N, d), lb = vector_bytes(B, H, N);
    const void *ptrs[] = {q, k, v, dout, lse, delta, dq};
    const long long sizes[] = {tb, tb, tb, tb, lb, lb, tb};
    RETURN_IF(check_ptrs(ptrs, sizes, 7));
    const Range in[] = {range_of(q, tb),    range_of(k, tb),   range_of(v, tb),
                        range_of(dout, tb), range_of(lse, lb), range_of(delta, lb)};
    const Range out[] = {range_of(dq, tb)};
    RETURN_IF(check_alias(in, 6, out, 1));
    attn::BwdArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.dout = dout;
    a.lse = lse;
    a.delta = (float *)delta;
    a.dq = dq;
    a.B = B;
    a.H = H;
    a.Hk = H;
    a.Nq = a.Nk = N;
    a.d = d;
    a.causal = causal;
    a.scale = scale;
    a.stream = stream;
    RETURN_IF(device_shape(stream, &a.dev));
    return hip_status(attn::launch_bwd_dq(a));
}

int attn_bwd_dq_delta(const void *q, const void *k, const void *v, const void *o, const void *dout, const float *lse,
                      float *delta, void *dq, int B, int H, int N, int d, int causal, float scale, void *stream)
{
    bool empty = false;
    RETURN_IF(validate_common(B, H, H, N, N, d, causal, scale, &empty));
    if (empty) return ATTN_OK;
    const long long tb = tensor_bytes(B, H, N, d), lb = vector_bytes(B, H, N);
    const void *ptrs[] = {q, k, v, o, dout, lse, delta, dq};
    const long long sizes[] = {tb, tb, tb, tb, tb, lb, lb, tb};
    RETURN_IF(check_ptrs(ptrs, sizes, 8));
    const Range in[] = {range_of(q, tb),    range_of(k, tb),    range_of(v, tb),
                        range_of(o, tb),    range_of(dout, tb), range_of(lse, lb)};
    const Range out[] = {range_of(delta, lb), range_of(dq, tb)};
    RETURN_IF(check_alias(in, 6, out, 2));
    attn::BwdArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.dout = dout;
    a.lse = lse;
    a.delta = delta;
    a.dq = dq;
    a.B = B;
    a.H = H;
    a.Hk = H;
    a.Nq = a.Nk = N;
    a.d = d;
    a.causal = causal;
    a.scale = scale;
    a.stream = stream;
    RETURN_IF(device_shape(stream, &a.dev));
    if (attn::bwd_dq_fuses_delta(d)) return hip_status(attn::launch_bwd_dq_delta(a));
    RETURN_IF(hip_status(attn::launch_bwd_preprocess(a)));
    return hip_status(attn::launch_bwd_dq(a));
}

int attn_bwd(const void *q, const void *k, const void *v, const void *o, const void *dout, const float *lse, void *dq,
             void *dk, void *dv, float *delta, int B, int H, int N, int d, int causal, float scale, void *stream)
{
    return bwd_impl(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, H, N, N, d, causal, scale, stream);
}

int attn_bwd_qk(const void *q, const void *k, const void *v, const void *o, const void *dout, const float *lse,
                void *dq, void *dk, void *dv, float *delta, int B, int H, int Hk, int Nq, int Nk, int d, int causal,
                float scale, void *stream)
{
    return bwd_impl(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, Hk, Nq, Nk, d, causal, scale, stream);
}

const char *attn_status_string(int status)
{
    switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULLPTR: return "a required pointer is NULL";
    case ATTN_ERR_BAD_SHAPE:
        return "bad shape: B, H, Hk and the lengths must be >= 0 and within the size limits, H a multiple of Hk";
    case ATTN_ERR_UNSUPPORTED_D: return "unsupported head dimension: d must be 64, 128, 192 or 256";
    case ATTN_ERR_MISALIGNED: return "a pointer is not 16-byte aligned";
    case ATTN_ERR_BAD_SCALE: return "scale must be finite and > 0";
    case ATTN_ERR_BAD_ARG: return "causal must be 0 or 1 and num_splits in 1..256";
    case ATTN_ERR_ALIAS: return "an output overlaps an input or another output";
    case ATTN_ERR_HIP: return "the HIP runtime reported an error at launch";
    case ATTN_ERR_WORKSPACE: return "the workspace is smaller than the size the call needs";
    case ATTN_ERR_SCRATCH: return "the call needs more than the library's static scratch buffer (16 MiB)";
    default: return "unknown status";
    }
}

int attn_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
