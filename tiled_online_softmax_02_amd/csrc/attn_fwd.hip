// attn_fwd.hip -- fused tiled attention forward pass for gfx950.
//
// Method ("digest_existing.txt", answer q02_flashattention, sections 1-2;
// "GPU Programming and Kernel Optimization", items 41, 57, 58, 60): for each
// block of query rows, stream the key/value blocks through on-chip memory,
// keep per row a running maximum m and a running exponential sum l
// (initialised to -inf and 0), rescale the output accumulator by
// exp(m_old - m_new) when the maximum moves, and divide by l only once at the
// end.  S and P never leave the chip.
//
// gfx950 mapping:
//   * one workgroup of 4 waves per block of 128 query rows; each wave owns 32
//     rows and holds their Q fragments in VGPRs for the whole loop;
//   * key/value blocks of 64 rows are double-buffered through LDS with 16-byte
//     buffer loads (rows past N read as zeros); K runs one block ahead of V, so
//     the scores of block j+1 are computed on the matrix cores while the
//     vector units exponentiate block j;
//   * scores are computed transposed, S^T = K Q^T, so each lane holds 32 keys
//     of a single query row: the row maximum needs one cross-half exchange and
//     the probabilities feed O^T += V^T P^T straight from registers;
//   * V^T is read from the row-major LDS tile with transposing LDS reads;
//   * exponentials are exp2 of scores scaled by scale*log2(e) in fp32;
//   * the running maximum used as the exponent offset is only moved when the
//     row maximum exceeds it by more than 2^kRescaleLog2 in exp2 units
//     (conditional rescaling): probabilities stay <= 2^kRescaleLog2, the O
//     rescale is skipped on most blocks, and the final O = acc / l and
//     lse = m + ln l are unchanged because acc and l share the offset;
//   * causal: key blocks above the diagonal are never loaded, waves skip the
//     blocks that lie wholly above their own rows, masking runs only on blocks
//     that cross the diagonal, and query blocks are issued longest first.
#include "attn_device.h"
#include "attn_launch.h"

namespace attn {

namespace {

constexpr int kFwdBM = 128;  // query rows per workgroup
constexpr int kFwdBN = 64;   // keys per streamed block
constexpr int kThreads = 256;
constexpr float kRescaleLog2 = 8.0f;

template <int D>
struct FwdSmem {
    static constexpr int KRS = D * 2 + 16;  // K row stride in bytes
    static constexpr int VRS = D * 2 + 64;  // V row stride in bytes
    static constexpr int KBYTES = kFwdBN * KRS;
    static constexpr int VBYTES = kFwdBN * VRS;
    static constexpr int OFF_V = 2 * KBYTES;  // two K stages, then two V stages
    static constexpr int TOTAL = 2 * KBYTES + 2 * VBYTES;
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void fwd_kernel(const bf16 *__restrict__ Q, const bf16 *__restrict__ K,
                                                          const bf16 *__restrict__ V, bf16 *__restrict__ O,
                                                          float *__restrict__ LSE, int N, int n_qtiles, float scale,
                                                          float c_log2)
{
    using L = FwdSmem<D>;
    constexpr int NKS = D / 16;          // reduction steps over d for S^T
    constexpr int NDB = D / 32;          // 32-wide column blocks of O
    constexpr int CPR = D / 8;           // 16-byte chunks per row
    constexpr int RPP = kThreads / CPR;  // rows per load pass
    constexpr int NP = kFwdBN / RPP;     // load passes per block
    __shared__ __attribute__((aligned(16))) char smem_raw[L::TOTAL];
    lds_char *smem = (lds_char *)smem_raw;

    const int id = xcd_remap(blockIdx.x, gridDim.x);
    const int head = id / n_qtiles;
    const int t_in = id - head * n_qtiles;
    const int qtile = CAUSAL ? (n_qtiles - 1 - t_in) : t_in;  // causal: longest rows first

    const int tid = threadIdx.x;
    const int lane = tid & 63, h = lane >> 5, c32 = lane & 31;
    const int w = wave_uniform(tid >> 6);
    const size_t hoff = (size_t)head * (size_t)N * D;
    const uint32_t head_bytes = (uint32_t)N * D * 2;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(Q + hoff, head_bytes);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(K + hoff, head_bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(V + hoff, head_bytes);

    const int q0 = qtile * kFwdBM;
    const int qw0 = q0 + 32 * w;  // wave-uniform
    const int qrow = qw0 + c32;

    // Q fragments: B operand of S^T = K Q^T, lane holds Q[qrow][16ks + 8h .. +7] (zeros past N).
    bf16x8 qf[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
        qf[ks] = __builtin_bit_cast(bf16x8, buffer_load16(rq, (uint32_t)(qrow * D + 16 * ks + 8 * h) * 2u));

    f32x16 oacc[NDB];
#pragma unroll
    for (int i = 0; i < NDB; ++i) oacc[i] = zero16();
    float m_run = -__builtin_inff();  // exponent offset (raw score units)
    float msc = 0.f;                   // m_run * c_log2, 0 while m_run = -inf
    float l_run = 0.f;
    const float grow_thr = kRescaleLog2 / c_log2;

    const int kv_end = CAUSAL ? min(N, q0 + kFwdBM) : N;
    const int nt = (kv_end + kFwdBN - 1) / kFwdBN;

    // Cooperative block loader: thread -> (row within pass, 16-byte chunk).
    const int ld_row = tid / CPR, ld_chk = tid % CPR;
    u32x4 kreg[NP], vreg[NP];
    auto gload = [&](const __amdgpu_buffer_rsrc_t &r, int j, u32x4 *regs) {
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int row = j * kFwdBN + p * RPP + ld_row;
            regs[p] = buffer_load16(r, (uint32_t)(row * D + 8 * ld_chk) * 2u);
        }
    };
    auto swrite = [&](int off, int rs, const u32x4 *regs) {
#pragma unroll
        for (int p = 0; p < NP; ++p) lds_write16(smem + off, (p * RPP + ld_row) * rs + 16 * ld_chk, regs[p]);
    };
    auto kstage = [&](int j) { return smem + (j & 1) * L::KBYTES; };
    auto vstage = [&](int j) { return smem + L::OFF_V + (j & 1) * L::VBYTES; };

    // S^T block (64 keys x 32 queries) of key block j
    auto scores = [&](int j, f32x16 *s) {
        const lds_char *ks = kstage(j);
        s[0] = zero16();
        s[1] = zero16();
#pragma unroll
        for (int kst = 0; kst < NKS; ++kst) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const bf16x8 a = lds_read16(ks, (32 * kb + c32) * L::KRS + 32 * kst + 16 * h);
                s[kb] = mfma(a, qf[kst], s[kb]);
            }
        }
    };

    auto active = [&](int j) { return (qw0 < N) && (!CAUSAL || j * kFwdBN <= qw0 + 31); };

    // prologue: K0, V0 and K1 in LDS, scores of block 0 in registers
    gload(rk, 0, kreg);
    gload(rv, 0, vreg);
    swrite(0, L::KRS, kreg);
    swrite(L::OFF_V, L::VRS, vreg);
    if (nt > 1) {
        gload(rk, 1, kreg);
        swrite(L::KBYTES, L::KRS, kreg);
    }
    __syncthreads();
    f32x16 sa[2], sb[2];
    if (active(0)) scores(0, sa);

    // One pipeline step on key block j: scores of j are in `cur`, scores of j+1 go to `nxt`.
    auto step = [&](int j, f32x16 *cur, f32x16 *nxt) {
        const bool more = j + 1 < nt;
        if (j + 2 < nt) gload(rk, j + 2, kreg);
        if (more) gload(rv, j + 1, vreg);
        if (active(j)) {
            const int k0 = j * kFwdBN;
            if ((CAUSAL && (k0 + kFwdBN - 1 > qw0)) || (k0 + kFwdBN > N)) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = k0 + 32 * kb + 8 * (r >> 2) + 4 * h + (r & 3);
                        if ((CAUSAL && key > qrow) || key >= N) cur[kb][r] = -__builtin_inff();
                    }
                }
            }
            float mx = cur[0][0];
#pragma unroll
            for (int r = 1; r < 16; ++r) mx = fmaxf(mx, cur[0][r]);
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, cur[1][r]);
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            // move the offset only when some row's maximum outgrows it (or it is still -inf)
            const bool grow = mx > m_run + grow_thr;
            if (__builtin_amdgcn_ballot_w64(grow)) {
                const float m_new = grow ? mx : m_run;
                const float alpha = grow ? fast_exp2((m_run - m_new) * c_log2) : 1.f;
                m_run = m_new;
                msc = (m_run == -__builtin_inff()) ? 0.f : m_run * c_log2;
                l_run *= alpha;
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
                }
            }
            // scores of block j+1 on the matrix cores, probabilities of block j on the vector units
            scores(more ? j + 1 : j, nxt);
            float rs = 0.f;
            bf16x8 pb[kFwdBN / 16];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                                        const float e = fast_exp2(fmaf(cur[kb][r], c_log2, -msc));
                    rs += e;
                    pb[2 * kb + (r >> 3)][r & 7] = (bf16)e;
                }
            }
            l_run += rs;
            // O^T += V^T P^T over 4 groups of 16 keys
            const lds_char *vs = vstage(j);
#pragma unroll
            for (int t = 0; t < kFwdBN / 16; ++t) {
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const bf16x8 a = lds_read_tr_rows(vs, L::VRS, 16 * t, 32 * db, lane);
                    oacc[db] = mfma(a, pb[t], oacc[db]);
                }
            }
            // Issue order for the block above: each score MFMA is followed by the K read two
            // MFMAs ahead and a slice of the exponential work; the first V reads are issued
            // before the P V MFMAs, each of which then issues the reads two MFMAs ahead.
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
            for (int i = 0; i < 2 * NKS; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 128 / (2 * NKS), 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
            for (int i = 0; i < (kFwdBN / 16) * NDB; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);
            }
        }
        if (j + 2 < nt) swrite((j & 1) * L::KBYTES, L::KRS, kreg);
        if (more) swrite(L::OFF_V + ((j + 1) & 1) * L::VBYTES, L::VRS, vreg);
        __syncthreads();
    };

    int j = 0;
    for (; j + 1 < nt; j += 2) {
        step(j, sa, sb);
        step(j + 1, sb, sa);
    }
    if (j < nt) step(j, sa, sb);

    // epilogue: O = acc / l (bf16, nearest even), lse = m*scale + ln(l)
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    if (qrow < N) {
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
