// attn_bwd.hip -- attention backward pass for gfx950: preprocess, dK/dV and dQ kernels.
//
// The backward pass regenerates the score tiles from the saved inputs and the
// per-row log-sum-exp instead of storing P ("GPU Programming and Kernel
// Optimization", item 58).  With P = exp(scale * Q K^T - lse) (masked entries
// 0) and dO the output gradient it computes
//   D_i  = sum_c dO_ic O_ic                (preprocess kernel)
//   dV   = P^T dO,  dP = dO V^T,  dS = P * (dP - D)
//   dK   = scale * dS^T Q                   (dK/dV kernel: one key block per
//                                            workgroup, loop over query blocks)
//   dQ   = scale * dS K                     (dQ kernel: one query block per
//                                            workgroup, loop over key blocks)
// Splitting dQ into its own kernel keeps every sum in registers of a single
// workgroup: no atomics, bitwise reproducible results.
//
// MFMA layouts follow attn_device.h.  In the dK/dV kernel the scores are
// computed as S = Q K^T (each lane: one key, 16 queries of a 32-query block),
// so P and dS feed dV^T += dO^T P and dK^T += Q^T dS from registers, with dO^T
// and Q^T read from LDS by transposing reads.  In the dQ kernel the scores are
// computed as S^T = K Q^T (each lane: one query), so lse and D are per-lane
// scalars and dS^T feeds dQ^T += K^T dS^T from registers.
#include "attn_device.h"
#include "attn_launch.h"

namespace attn {

namespace {

constexpr int kThreads = 256;

// ------------------------------------------------------------ preprocess

template <int D>
__global__ __launch_bounds__(kThreads) void bwd_preprocess_kernel(const bf16 *__restrict__ O,
                                                                  const bf16 *__restrict__ dO,
                                                                  float *__restrict__ Dl, long long rows)
{
    constexpr int CPR = D / 8;            // lanes per row, 8 elements each
    constexpr int RPB = kThreads / CPR;   // rows per workgroup
    const long long row = (long long)blockIdx.x * RPB + threadIdx.x / CPR;
    const int c = threadIdx.x % CPR;
    float acc = 0.f;
    if (row < rows) {
        const bf16x8 o = *(const bf16x8 *)(O + row * D + 8 * c);
        const bf16x8 g = *(const bf16x8 *)(dO + row * D + 8 * c);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = fmaf((float)o[e], (float)g[e], acc);
    }
#pragma unroll
    for (int off = CPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (row < rows && c == 0) Dl[row] = acc;
}

// ------------------------------------------------------------ dK / dV

constexpr int kKvBN = 128;  // keys per workgroup (32 per wave)
constexpr int kKvBM = 64;   // queries per streamed block

template <int D>
struct KvSmem {
    static constexpr int RS = D * 2 + 16;  // Q / dO row stride in bytes
    static constexpr int QBYTES = kKvBM * RS;
    static constexpr int OFF_DO = QBYTES;
    static constexpr int OFF_LSE = 2 * QBYTES;            // kKvBM floats: lse * log2(e)
    static constexpr int OFF_D = OFF_LSE + 4 * kKvBM;     // kKvBM floats: D
    static constexpr int STAGE = OFF_D + 4 * kKvBM;
    static constexpr int TOTAL = 2 * STAGE;
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void bwd_dkdv_kernel(
    const bf16 *__restrict__ Q, const bf16 *__restrict__ K, const bf16 *__restrict__ V, const bf16 *__restrict__ dO,
    const float *__restrict__ LSE, const float *__restrict__ Dl, bf16 *__restrict__ dK, bf16 *__restrict__ dV, int N,
    int n_ktiles, float scale, float c_log2)
{
    using L = KvSmem<D>;
    constexpr int NKS = D / 16;
    constexpr int NDB = D / 32;
    constexpr int CPR = D / 8;
    constexpr int RPP = kThreads / CPR;
    constexpr int NP = kKvBM / RPP;
    __shared__ __attribute__((aligned(16))) char smem_raw[L::TOTAL];
    lds_char *smem = (lds_char *)smem_raw;

    const int id = xcd_remap(blockIdx.x, gridDim.x);
    const int head = id / n_ktiles;
    const int ktile = id - head * n_ktiles;  // causal: key block 0 sees the most queries and goes first

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6, h = lane >> 5, c32 = lane & 31;
    const size_t hoff = (size_t)head * (size_t)N * D;
    const bf16 *Qh = Q + hoff, *Kh = K + hoff, *Vh = V + hoff, *dOh = dO + hoff;
    const float *LSEh = LSE + (size_t)head * N, *Dh = Dl + (size_t)head * N;

    const int k0 = ktile * kKvBN;
    const int kw0 = k0 + 32 * w;
    const int key = kw0 + c32;
    const bool key_ok = key < N;

    // K and V fragments (B operands of S = Q K^T and dP = dO V^T): lane holds row `key`.
    bf16x8 kf[NKS], vf[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
        if (key_ok) {
            kf[ks] = *(const bf16x8 *)(Kh + (size_t)key * D + 16 * ks + 8 * h);
            vf[ks] = *(const bf16x8 *)(Vh + (size_t)key * D + 16 * ks + 8 * h);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                kf[ks][e] = (bf16)0.f;
                vf[ks][e] = (bf16)0.f;
            }
        }
    }

    f32x16 dk[NDB], dv[NDB];
#pragma unroll
    for (int i = 0; i < NDB; ++i) {
        dk[i] = zero16();
        dv[i] = zero16();
    }

    const int q_start = CAUSAL ? (k0 / kKvBM) * kKvBM : 0;
    const int nsteps = (N > q_start) ? (N - q_start + kKvBM - 1) / kKvBM : 0;

    const int ld_row = tid / CPR, ld_chk = tid % CPR;
    u32x4 qreg[NP], oreg[NP];
    float lreg = 0.f, dreg = 0.f;
    auto gload = [&](int i) {
        const int qs = q_start + i * kKvBM;
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int row = qs + p * RPP + ld_row;
            if (row < N) {
                qreg[p] = *(const u32x4 *)(Qh + (size_t)row * D + 8 * ld_chk);
                oreg[p] = *(const u32x4 *)(dOh + (size_t)row * D + 8 * ld_chk);
            } else {
                qreg[p] = u32x4{0u, 0u, 0u, 0u};
                oreg[p] = u32x4{0u, 0u, 0u, 0u};
            }
        }
        if (tid < kKvBM) {
            const int row = qs + tid;
            // rows beyond N get lse = +inf so that their probabilities are exactly 0
            lreg = (row < N) ? LSEh[row] * kLog2e : __builtin_inff();
            dreg = (row < N) ? Dh[row] : 0.f;
        }
    };
    auto swrite = [&](int stage) {
        lds_char *base = smem + stage * L::STAGE;
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int r = p * RPP + ld_row;
            lds_write16(base, r * L::RS + 16 * ld_chk, qreg[p]);
            lds_write16(base + L::OFF_DO, r * L::RS + 16 * ld_chk, oreg[p]);
        }
        if (tid < kKvBM) {
            *(__attribute__((address_space(3))) float *)(base + L::OFF_LSE + 4 * tid) = lreg;
            *(__attribute__((address_space(3))) float *)(base + L::OFF_D + 4 * tid) = dreg;
        }
    };

    if (nsteps > 0) {
        gload(0);
        swrite(0);
    }
    __syncthreads();

    for (int i = 0; i < nsteps; ++i) {
        if (i + 1 < nsteps) gload(i + 1);
        const lds_char *qs_l = smem + (i & 1) * L::STAGE;
        const lds_char *do_l = qs_l + L::OFF_DO;
        const lds_char *lse_l = qs_l + L::OFF_LSE;
        const lds_char *d_l = qs_l + L::OFF_D;
        const int qs = q_start + i * kKvBM;
        // some query of this block sees some key of this wave
        const bool active = (kw0 < N) && (!CAUSAL || qs + kKvBM - 1 >= kw0);
        if (active) {
            // S = Q K^T and dP = dO V^T, two 32-query blocks
            f32x16 s[2] = {zero16(), zero16()};
            f32x16 dp[2] = {zero16(), zero16()};
#pragma unroll
            for (int kst = 0; kst < NKS; ++kst) {
#pragma unroll
                for (int qb = 0; qb < 2; ++qb) {
                    const int off = (32 * qb + c32) * L::RS + 32 * kst + 16 * h;
                    s[qb] = mfma(lds_read16(qs_l, off), kf[kst], s[qb]);
                    dp[qb] = mfma(lds_read16(do_l, off), vf[kst], dp[qb]);
                }
            }
            const bool need_mask = CAUSAL && (qs < kw0 + 31);
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int qloc = 32 * qb + 8 * g + 4 * h;  // first of 4 consecutive queries
                    const f32x4 l4 = *(const __attribute__((address_space(3))) f32x4 *)(lse_l + 4 * qloc);
                    const f32x4 d4 = *(const __attribute__((address_space(3))) f32x4 *)(d_l + 4 * qloc);
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const int r = 4 * g + u;
                        float p = fast_exp2(fmaf(s[qb][r], c_log2, -l4[u]));
                        if (need_mask && (qs + qloc + u < key)) p = 0.f;
                        s[qb][r] = p;
                        dp[qb][r] = p * (dp[qb][r] - d4[u]);
                    }
                }
            }
            // dV^T += dO^T P and dK^T += Q^T dS over 4 groups of 16 queries
#pragma unroll
            for (int t = 0; t < kKvBM / 16; ++t) {
                const bf16x8 pb = pack_bf16(s[t >> 1], t & 1);
                const bf16x8 sb = pack_bf16(dp[t >> 1], t & 1);
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    dv[db] = mfma(lds_read_tr_rows(do_l, L::RS, 16 * t, 32 * db, lane), pb, dv[db]);
                    dk[db] = mfma(lds_read_tr_rows(qs_l, L::RS, 16 * t, 32 * db, lane), sb, dk[db]);
                }
            }
        }
        if (i + 1 < nsteps) swrite((i + 1) & 1);
        __syncthreads();
    }

    if (key_ok) {
        bf16 *dkrow = dK + hoff + (size_t)key * D;
        bf16 *dvrow = dV + hoff + (size_t)key * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                bf16x4 kv4, vv4;
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    kv4[u] = (bf16)(dk[db][4 * g + u] * scale);
                    vv4[u] = (bf16)dv[db][4 * g + u];
                }
                *(bf16x4 *)(dkrow + 32 * db + 8 * g + 4 * h) = kv4;
                *(bf16x4 *)(dvrow + 32 * db + 8 * g + 4 * h) = vv4;
            }
        }
    }
}

// ------------------------------------------------------------ dQ

constexpr int kQBM = 128;  // queries per workgroup (32 per wave)
constexpr int kQBN = 64;   // keys per streamed block

template <int D>
struct QSmem {
    static constexpr int RS = D * 2 + 16;
    static constexpr int KBYTES = kQBN * RS;
    static constexpr int STAGE = 2 * KBYTES;  // K then V
    static constexpr int TOTAL = 2 * STAGE;
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void bwd_dq_kernel(
    const bf16 *__restrict__ Q, const bf16 *__restrict__ K, const bf16 *__restrict__ V, const bf16 *__restrict__ dO,
    const float *__restrict__ LSE, const float *__restrict__ Dl, bf16 *__restrict__ dQ, int N, int n_qtiles,
    float scale, float c_log2)
{
    using L = QSmem<D>;
    constexpr int NKS = D / 16;
    constexpr int NDB = D / 32;
    constexpr int CPR = D / 8;
    constexpr int RPP = kThreads / CPR;
    constexpr int NP = kQBN / RPP;
    __shared__ __attribute__((aligned(16))) char smem_raw[L::TOTAL];
    lds_char *smem = (lds_char *)smem_raw;

    const int id = xcd_remap(blockIdx.x, gridDim.x);
    const int head = id / n_qtiles;
    const int t_in = id - head * n_qtiles;
    const int qtile = CAUSAL ? (n_qtiles - 1 - t_in) : t_in;

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6, h = lane >> 5, c32 = lane & 31;
    const size_t hoff = (size_t)head * (size_t)N * D;
    const bf16 *Qh = Q + hoff, *Kh = K + hoff, *Vh = V + hoff, *dOh = dO + hoff;

    const int q0 = qtile * kQBM;
    const int qw0 = q0 + 32 * w;
    const int qrow = qw0 + c32;
    const bool row_ok = qrow < N;

    bf16x8 qf[NKS], gf[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
        if (row_ok) {
            qf[ks] = *(const bf16x8 *)(Qh + (size_t)qrow * D + 16 * ks + 8 * h);
            gf[ks] = *(const bf16x8 *)(dOh + (size_t)qrow * D + 16 * ks + 8 * h);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                qf[ks][e] = (bf16)0.f;
                gf[ks][e] = (bf16)0.f;
            }
        }
    }
    const float lse2 = row_ok ? LSE[(size_t)head * N + qrow] * kLog2e : __builtin_inff();
    const float dval = row_ok ? Dl[(size_t)head * N + qrow] : 0.f;

    f32x16 dq[NDB];
#pragma unroll
    for (int i = 0; i < NDB; ++i) dq[i] = zero16();

    const int kv_end = CAUSAL ? min(N, q0 + kQBM) : N;
    const int nt = (kv_end + kQBN - 1) / kQBN;

    const int ld_row = tid / CPR, ld_chk = tid % CPR;
    u32x4 kreg[NP], vreg[NP];
    auto gload = [&](int j) {
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int row = j * kQBN + p * RPP + ld_row;
            if (row < N) {
                kreg[p] = *(const u32x4 *)(Kh + (size_t)row * D + 8 * ld_chk);
                vreg[p] = *(const u32x4 *)(Vh + (size_t)row * D + 8 * ld_chk);
            } else {
                kreg[p] = u32x4{0u, 0u, 0u, 0u};
                vreg[p] = u32x4{0u, 0u, 0u, 0u};
            }
        }
    };
    auto swrite = [&](int stage) {
        lds_char *ks = smem + stage * L::STAGE;
        lds_char *vs = ks + L::KBYTES;
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int r = p * RPP + ld_row;
            lds_write16(ks, r * L::RS + 16 * ld_chk, kreg[p]);
            lds_write16(vs, r * L::RS + 16 * ld_chk, vreg[p]);
        }
    };

    gload(0);
    swrite(0);
    __syncthreads();

    for (int j = 0; j < nt; ++j) {
        if (j + 1 < nt) gload(j + 1);
        const lds_char *ks = smem + (j & 1) * L::STAGE;
        const lds_char *vs = ks + L::KBYTES;
        const int k0 = j * kQBN;
        const bool active = (qw0 < N) && (!CAUSAL || k0 <= qw0 + 31);
        if (active) {
            f32x16 s[2] = {zero16(), zero16()};
            f32x16 dp[2] = {zero16(), zero16()};
#pragma unroll
            for (int kst = 0; kst < NKS; ++kst) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const int off = (32 * kb + c32) * L::RS + 32 * kst + 16 * h;
                    s[kb] = mfma(lds_read16(ks, off), qf[kst], s[kb]);
                    dp[kb] = mfma(lds_read16(vs, off), gf[kst], dp[kb]);
                }
            }
            const bool need_mask = (CAUSAL && (k0 + kQBN - 1 > qw0)) || (k0 + kQBN > N);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float p = fast_exp2(fmaf(s[kb][r], c_log2, -lse2));
                    if (need_mask) {
                        const int kk = k0 + 32 * kb + 8 * (r >> 2) + 4 * h + (r & 3);
                        if ((CAUSAL && kk > qrow) || kk >= N) p = 0.f;
                    }
                    dp[kb][r] = p * (dp[kb][r] - dval);
                }
            }
            // dQ^T += K^T dS^T over 4 groups of 16 keys
#pragma unroll
            for (int t = 0; t < kQBN / 16; ++t) {
                const bf16x8 sb = pack_bf16(dp[t >> 1], t & 1);
#pragma unroll
                for (int db = 0; db < NDB; ++db)
                    dq[db] = mfma(lds_read_tr_rows(ks, L::RS, 16 * t, 32 * db, lane), sb, dq[db]);
            }
        }
        if (j + 1 < nt) swrite((j + 1) & 1);
        __syncthreads();
    }

    if (row_ok) {
        bf16 *qrow_p = dQ + hoff + (size_t)qrow * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                bf16x4 v4;
#pragma unroll
                for (int u = 0; u < 4; ++u) v4[u] = (bf16)(dq[db][4 * g + u] * scale);
                *(bf16x4 *)(qrow_p + 32 * db + 8 * g + 4 * h) = v4;
            }
        }
    }
}

template <int D>
hipError_t launch_pre_t(const BwdArgs &a)
{
    constexpr int RPB = kThreads / (D / 8);
    const long long rows = (long long)a.B * a.H * a.N;
    const long long G = (rows + RPB - 1) / RPB;
    hipLaunchKernelGGL((bwd_preprocess_kernel<D>), dim3((unsigned)G), dim3(kThreads), 0, (hipStream_t)a.stream,
                       (const bf16 *)a.o, (const bf16 *)a.dout, a.delta, rows);
    return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_dkdv_t(const BwdArgs &a)
{
    const int n_ktiles = (a.N + kKvBN - 1) / kKvBN;
    const long long G = (long long)a.B * a.H * n_ktiles;
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL>), dim3((unsigned)G), dim3(kThreads), 0, (hipStream_t)a.stream,
                       (const bf16 *)a.q, (const bf16 *)a.k, (const bf16 *)a.v, (const bf16 *)a.dout, a.lse,
                       (const float *)a.delta, (bf16 *)a.dk, (bf16 *)a.dv, a.N, n_ktiles, a.scale, a.scale * kLog2e);
    return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_dq_t(const BwdArgs &a)
{
    const int n_qtiles = (a.N + kQBM - 1) / kQBM;
    const long long G = (long long)a.B * a.H * n_qtiles;
    hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL>), dim3((unsigned)G), dim3(kThreads), 0, (hipStream_t)a.stream,
                       (const bf16 *)a.q, (const bf16 *)a.k, (const bf16 *)a.v, (const bf16 *)a.dout, a.lse,
                       (const float *)a.delta, (bf16 *)a.dq, a.N, n_qtiles, a.scale, a.scale * kLog2e);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_preprocess(const BwdArgs &a)
{
    return a.d == 64 ? launch_pre_t<64>(a) : launch_pre_t<128>(a);
}

hipError_t launch_bwd_dkdv(const BwdArgs &a)
{
    if (a.d == 64) return a.causal ? launch_dkdv_t<64, true>(a) : launch_dkdv_t<64, false>(a);
    return a.causal ? launch_dkdv_t<128, true>(a) : launch_dkdv_t<128, false>(a);
}

hipError_t launch_bwd_dq(const BwdArgs &a)
{
    if (a.d == 64) return a.causal ? launch_dq_t<64, true>(a) : launch_dq_t<64, false>(a);
    return a.causal ? launch_dq_t<128, true>(a) : launch_dq_t<128, false>(a);
}

long long bwd_dkdv_grid_size(int B, int H, int N) { return (long long)B * H * ((N + kKvBN - 1) / kKvBN); }
long long bwd_dq_grid_size(int B, int H, int N) { return (long long)B * H * ((N + kQBM - 1) / kQBM); }

}  // namespace attn
