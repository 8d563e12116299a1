// attn_fwd.hip -- fused tiled attention forward pass for gfx950.
//
// Method ("digest_existing.txt", answer q02_flashattention, sections 1-2;
// "GPU Programming and Kernel Optimization", items 41, 57, 58, 60): for each
// block of query rows, stream the key/value blocks through on-chip memory,
// keep per row a running maximum m and a running exponential sum l
// (initialised to -inf and 0), rescale the output accumulator by
// exp(m_old - m_new) whenever the maximum moves, and divide by l only once at
// the end.  S and P never leave the chip.
//
// gfx950 mapping:
//   * one workgroup of 4 waves per block of 128 query rows; each wave owns 32
//     rows and holds their Q fragments in VGPRs for the whole loop;
//   * key/value blocks of 64 rows are double-buffered through LDS with 16-byte
//     coalesced global loads issued one block ahead;
//   * scores are computed transposed, S^T = K Q^T, so each lane holds 32 keys
//     of a single query row: the row maximum needs one cross-half exchange and
//     the probabilities feed O^T += V^T P^T straight from registers;
//   * V^T is read from the row-major LDS tile with transposing LDS reads;
//   * exponentials are exp2 of scores pre-scaled by scale*log2(e) in fp32;
//   * causal: key blocks above the diagonal are never loaded, waves skip the
//     blocks that lie wholly above their own rows, and query blocks are issued
//     longest first.
#include "attn_device.h"
#include "attn_launch.h"

namespace attn {

namespace {

constexpr int kFwdBM = 128;  // query rows per workgroup
constexpr int kFwdBN = 64;   // keys per streamed block
constexpr int kThreads = 256;

template <int D>
struct FwdSmem {
    static constexpr int KRS = D * 2 + 16;  // K row stride in bytes
    static constexpr int VRS = D * 2 + 64;  // V row stride in bytes
    static constexpr int KBYTES = kFwdBN * KRS;
    static constexpr int VBYTES = kFwdBN * VRS;
    static constexpr int STAGE = KBYTES + VBYTES;
    static constexpr int TOTAL = 2 * STAGE;
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void fwd_kernel(const bf16 *__restrict__ Q, const bf16 *__restrict__ K,
                                                          const bf16 *__restrict__ V, bf16 *__restrict__ O,
                                                          float *__restrict__ LSE, int N, int n_qtiles, float scale,
                                                          float c_log2)
{
    using L = FwdSmem<D>;
    constexpr int NKS = D / 16;  // reduction steps over d for S^T
    constexpr int NDB = D / 32;  // 32-wide column blocks of O
    constexpr int CPR = D / 8;   // 16-byte chunks per row
    constexpr int RPP = kThreads / CPR;  // rows per load pass
    constexpr int NP = kFwdBN / RPP;     // load passes per block
    __shared__ __attribute__((aligned(16))) char smem_raw[L::TOTAL];
    lds_char *smem = (lds_char *)smem_raw;

    const int id = xcd_remap(blockIdx.x, gridDim.x);
    const int head = id / n_qtiles;
    const int t_in = id - head * n_qtiles;
    const int qtile = CAUSAL ? (n_qtiles - 1 - t_in) : t_in;  // causal: longest rows first

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6, h = lane >> 5, c32 = lane & 31;
    const size_t hoff = (size_t)head * (size_t)N * D;
    const bf16 *Qh = Q + hoff;
    const bf16 *Kh = K + hoff;
    const bf16 *Vh = V + hoff;

    const int q0 = qtile * kFwdBM;
    const int qw0 = q0 + 32 * w;
    const int qrow = qw0 + c32;
    const bool row_ok = qrow < N;

    // Q fragments: B operand of S^T = K Q^T, lane holds Q[qrow][16ks + 8h .. +7].
    bf16x8 qf[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
        if (row_ok) {
            qf[ks] = *(const bf16x8 *)(Qh + (size_t)qrow * D + 16 * ks + 8 * h);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) qf[ks][e] = (bf16)0.f;
        }
    }

    f32x16 oacc[NDB];
#pragma unroll
    for (int i = 0; i < NDB; ++i) oacc[i] = zero16();
    float m_run = -__builtin_inff();
    float l_run = 0.f;

    const int kv_end = CAUSAL ? min(N, q0 + kFwdBM) : N;
    const int nt = (kv_end + kFwdBN - 1) / kFwdBN;

    // Cooperative block loader: thread -> (row within pass, 16-byte chunk).
    const int ld_row = tid / CPR, ld_chk = tid % CPR;
    u32x4 kreg[NP], vreg[NP];
    auto gload = [&](int j) {
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int row = j * kFwdBN + p * RPP + ld_row;
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
            lds_write16(ks, r * L::KRS + 16 * ld_chk, kreg[p]);
            lds_write16(vs, r * L::VRS + 16 * ld_chk, vreg[p]);
        }
    };

    gload(0);
    swrite(0);
    __syncthreads();

    for (int j = 0; j < nt; ++j) {
        if (j + 1 < nt) gload(j + 1);
        const lds_char *ks = smem + (j & 1) * L::STAGE;
        const lds_char *vs = ks + L::KBYTES;
        const int k0 = j * kFwdBN;
        const bool active = (qw0 < N) && (!CAUSAL || k0 <= qw0 + 31);
        if (active) {
            // S^T block (64 keys x 32 queries) = K Q^T
            f32x16 s[2] = {zero16(), zero16()};
#pragma unroll
            for (int kst = 0; kst < NKS; ++kst) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const bf16x8 a = lds_read16(ks, (32 * kb + c32) * L::KRS + 32 * kst + 16 * h);
                    s[kb] = mfma(a, qf[kst], s[kb]);
                }
            }
            // mask keys beyond the causal diagonal or beyond N
            const bool need_mask = (CAUSAL && (k0 + kFwdBN - 1 > qw0)) || (k0 + kFwdBN > N);
            if (need_mask) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = k0 + 32 * kb + 8 * (r >> 2) + 4 * h + (r & 3);
                        if ((CAUSAL && key > qrow) || key >= N) s[kb][r] = -__builtin_inff();
                    }
                }
            }
            // online softmax update (scores in raw units; scale > 0)
            float mx = s[0][0];
#pragma unroll
            for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[1][r]);
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float m_new = fmaxf(m_run, mx);
            const bool empty = (m_new == -__builtin_inff());  // every key so far masked for this row
            const float alpha = empty ? 1.f : fast_exp2((m_run - m_new) * c_log2);
            const float msc = empty ? 0.f : m_new * c_log2;
            float rs = 0.f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float e = fast_exp2(fmaf(s[kb][r], c_log2, -msc));
                    s[kb][r] = e;
                    rs += e;
                }
            }
            l_run = l_run * alpha + rs;
            m_run = m_new;
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
            }
            // O^T += V^T P^T over 4 groups of 16 keys
#pragma unroll
            for (int t = 0; t < kFwdBN / 16; ++t) {
                const bf16x8 pb = pack_bf16(s[t >> 1], t & 1);
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const bf16x8 a = lds_read_tr_rows(vs, L::VRS, 16 * t, 32 * db, lane);
                    oacc[db] = mfma(a, pb, oacc[db]);
                }
            }
        }
        if (j + 1 < nt) swrite((j + 1) & 1);
        __syncthreads();
    }

    // epilogue: O = acc / l (bf16, nearest even), lse = m*scale + ln(l)
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    if (row_ok) {
        const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
        bf16 *orow = O + hoff + (size_t)qrow * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                bf16x4 ov;
#pragma unroll
                for (int i = 0; i < 4; ++i) ov[i] = (bf16)(oacc[db][4 * g + i] * inv);
                *(bf16x4 *)(orow + 32 * db + 8 * g + 4 * h) = ov;
            }
        }
        if (h == 0)
            LSE[(size_t)head * N + qrow] = (l_tot > 0.f) ? fmaf(m_run, scale, __logf(l_tot)) : -__builtin_inff();
    }
}

template <int D, bool CAUSAL>
hipError_t launch_fwd_t(const FwdArgs &a)
{
    const int n_qtiles = (a.N + kFwdBM - 1) / kFwdBM;
    const long long G = (long long)a.B * a.H * n_qtiles;
    const float c_log2 = a.scale * kLog2e;
    hipLaunchKernelGGL((fwd_kernel<D, CAUSAL>), dim3((unsigned)G), dim3(kThreads), 0, (hipStream_t)a.stream,
                       (const bf16 *)a.q, (const bf16 *)a.k, (const bf16 *)a.v, (bf16 *)a.o, a.lse, a.N, n_qtiles,
                       a.scale, c_log2);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd(const FwdArgs &a)
{
    if (a.d == 64) return a.causal ? launch_fwd_t<64, true>(a) : launch_fwd_t<64, false>(a);
    return a.causal ? launch_fwd_t<128, true>(a) : launch_fwd_t<128, false>(a);
}

long long fwd_grid_size(int B, int H, int N) { return (long long)B * H * ((N + kFwdBM - 1) / kFwdBM); }

}  // namespace attn
