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
// Two dK/dV kernels: bwd_dkdv2_kernel for d <= 128 splits each key block's work between the two
// waves of a SIMD (one computes P and dV, the other dS and dK); bwd_dkdv4_kernel for d = 192 and
// 256 runs one wave per SIMD with up to 512 registers, each wave doing all four products for its
// keys.
//
// MFMA layouts follow attn_device.h.  In the dK/dV kernels the scores are
// computed as S = Q K^T (each lane: one key, 16 queries of a 32-query block),
// so P and dS feed dV^T += dO^T P and dK^T += Q^T dS from registers, with dO^T
// and Q^T read from LDS by transposing reads.  In the dQ kernel the scores are
// computed as S^T = K Q^T (each lane: one query), so lse and D are per-lane
// scalars and dS^T feeds dQ^T += K^T dS^T from registers.
#include "attn_device.h"
#include "attn_launch.h"

#include <type_traits>

namespace attn {

namespace {

constexpr int kThreads = 256;

// ------------------------------------------------------------ preprocess

template <int D>
__global__ __launch_bounds__(kThreads) void bwd_preprocess_kernel(const bf16 *__restrict__ O,
                                                                  const bf16 *__restrict__ dO,
                                                                  float *__restrict__ Dl, long long rows)
{
    constexpr int CPR = D / 8;                              // 8-element chunks per row
    constexpr int LPR = CPR <= 8 ? 8 : CPR <= 16 ? 16 : 32;  // lanes per row (a power of two)
    constexpr int RPB = kThreads / LPR;                     // rows per workgroup
    const long long row = (long long)blockIdx.x * RPB + threadIdx.x / LPR;
    const int c = threadIdx.x % LPR;
    float acc = 0.f;
    if (row < rows && c < CPR) {
        const bf16x8 o = *(const bf16x8 *)(O + row * D + 8 * c);
        const bf16x8 g = *(const bf16x8 *)(dO + row * D + 8 * c);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = fmaf((float)o[e], (float)g[e], acc);
    }
#pragma unroll
    for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (row < rows && c == 0) Dl[row] = acc;
}

// ------------------------------------------------------------ dK / dV

// Keys per dK/dV workgroup: 128 for d <= 128 (paired-wave kernel below), 64 for d = 192 and 256.
template <int D>
constexpr int kv_bn() { return D >= 192 ? 64 : 128; }
constexpr int kKvBM = 64;   // queries per streamed block

// ------------------------------------------------------------ dK / dV, paired waves (d <= 128)

// Eight waves, two per SIMD: wave pair (w, w + 4) owns 32 keys (128 keys per workgroup) and
// splits the work on each query block between its two waves.  Wave w (the P wave) computes
// S = Q K^T, P = exp2(S scale log2e - lse log2e) and dV^T += dO^T P, and leaves P in LDS;
// wave w + 4 (the dS wave) works one block behind: dP = dO V^T, then with that P from LDS
// dS = P (dP - D) and dK^T += Q^T dS.  Each wave does 32 of the 64 matrix instructions of a
// block and holds one key-side operand and one accumulator, so two waves fit per SIMD, and
// within a step the two run independently (one barrier per step).  Query-block tiles live in
// three LDS stages (loading, P wave, dS wave), P in two.  P crosses in bf16, the precision
// the dV product uses anyway.
struct Dkdv2Args {
    const bf16 *Q, *K, *V, *dO;
    const float *LSE, *Dl;
    bf16 *dK, *dV;
    int Nq, Nk, H, G, n_ktiles, n_items, nx;
    float scale, c_log2;
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(512, 1) void bwd_dkdv2_kernel(const Dkdv2Args args)
{
    static_assert(D <= 128, "paired-wave dK/dV kernel: d <= 128");
    constexpr int NKS = D / 16;
    constexpr int NDB = D / 32;
    constexpr int TILE = kKvBM * D * 2;
    constexpr int kBN = 128;
    constexpr int PBUF = 4 * 4 * 64 * 16;  // P of the four pairs (4 KB each)
    __shared__ __attribute__((aligned(16))) char q0_raw[TILE], q1_raw[TILE], q2_raw[TILE];
    __shared__ __attribute__((aligned(16))) char g0_raw[TILE], g1_raw[TILE], g2_raw[TILE];
    __shared__ __attribute__((aligned(16))) float s0_raw[2 * kKvBM], s1_raw[2 * kKvBM], s2_raw[2 * kKvBM];  // lse, D
    __shared__ __attribute__((aligned(16))) char p0_raw[PBUF], p1_raw[PBUF];

    // Persistent when the grid is smaller than the item count: each workgroup takes items in
    // rounds (persistent_item), and the next item's loads start while the last one's stores drain.
    // Every step ends with a barrier and the epilogue reads no LDS, so a new item may refill
    // stage 0 at once.
    // The arguments are read again from the kernel-argument segment in each round (behind an
    // empty asm, so the loads stay in the loop): held across the rounds they would add two dozen
    // scalar registers to a loop body that already spills scalars to vector lanes.
    for (int r = 0;; ++r) {
        const __attribute__((address_space(4))) Dkdv2Args *ap =
            (const __attribute__((address_space(4))) Dkdv2Args *)__builtin_amdgcn_kernarg_segment_ptr();
        asm volatile("" : "+s"(ap));
        const bf16 *__restrict__ Q = ap->Q, *__restrict__ K = ap->K, *__restrict__ V = ap->V, *__restrict__ dO = ap->dO;
        const float *__restrict__ LSE = ap->LSE, *__restrict__ Dl = ap->Dl;
        bf16 *__restrict__ dK = ap->dK, *__restrict__ dV = ap->dV;
        const int Nq = ap->Nq, Nk = ap->Nk, H = ap->H, G = ap->G, n_ktiles = ap->n_ktiles, n_items = ap->n_items;
        const float scale = ap->scale, c_log2 = ap->c_log2;
        const int item = persistent_item(r, (int)blockIdx.x, (int)gridDim.x, ap->nx);
        if (item >= n_items) break;  // workgroup-uniform; later rounds hold only larger items
        int head, ktile;
        work_item_of(item, n_items, n_ktiles, ap->nx, head, ktile);
        const int Hk = H / G;
        const int qh0 = (head / Hk) * H + (head % Hk) * G;

        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));  // lane-derived values are formed per round, not held across
        const int lane = tid & 63, h = lane >> 5, c32 = lane & 31;
        const int w = wave_uniform(tid >> 6);
        const int pair = w & 3;
        const bool pwave = w < 4;  // wave-uniform role
        const size_t hoff = (size_t)head * (size_t)Nk * D;
        __amdgpu_buffer_rsrc_t rq, rg, rl, rd;
        auto bind_query_head = [&](int qh) __attribute__((always_inline)) {
            const size_t hoff_q = (size_t)qh * (size_t)Nq * D;
            rq = make_rsrc(Q + hoff_q, (uint32_t)Nq * D * 2);
            rg = make_rsrc(dO + hoff_q, (uint32_t)Nq * D * 2);
            rl = make_rsrc(LSE + (size_t)qh * Nq, (uint32_t)Nq * 4);
            rd = make_rsrc(Dl + (size_t)qh * Nq, (uint32_t)Nq * 4);
        };
        const int off = Nk - Nq;
        const int k0 = ktile * kBN;
        const int kw0 = k0 + 32 * pair;
        const int key = kw0 + c32;

        // key-side operand: K for the P wave (S = Q K^T), -V for the dS wave, whose product then
        // starts from D: D - dO V^T = -(dP - D), so that dS needs one multiply per element; its dK
        // accumulator holds -dK and is negated with the scale at the end
        bf16x8 kvf[NKS];
        {
            const __amdgpu_buffer_rsrc_t rkv = make_rsrc((pwave ? K : V) + hoff, (uint32_t)Nk * D * 2);
            const unsigned sign = pwave ? 0u : 0x80008000u;
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
                kvf[ks] = __builtin_bit_cast(bf16x8, buffer_load16(rkv, (uint32_t)(key * D + 16 * ks + 8 * h) * 2u) ^ sign);
        }

        f32x16 acc[NDB];  // dV (P wave) or dK (dS wave)
#pragma unroll
        for (int i = 0; i < NDB; ++i) acc[i] = zero16();

        const int q_start = CAUSAL ? (max(0, k0 - off) / kKvBM) * kKvBM : 0;
        const int nsteps = (Nq > q_start) ? (Nq - q_start + kKvBM - 1) / kKvBM : 0;

        auto qst = [&](auto st) __attribute__((always_inline)) {
            constexpr int v = decltype(st)::value;
            return (lds_char *)(v == 0 ? q0_raw : v == 1 ? q1_raw : q2_raw);
        };
        auto gst = [&](auto st) __attribute__((always_inline)) {
            constexpr int v = decltype(st)::value;
            return (lds_char *)(v == 0 ? g0_raw : v == 1 ? g1_raw : g2_raw);
        };
        auto sst = [&](auto st) __attribute__((always_inline)) {
            constexpr int v = decltype(st)::value;
            return (lds_char *)(v == 0 ? s0_raw : v == 1 ? s1_raw : s2_raw);
        };
        auto pst = [&](auto b) __attribute__((always_inline)) {
            return (lds_char *)(decltype(b)::value ? p1_raw : p0_raw) + pair * (4 * 64 * 16);
        };
        // lse of the block being loaded (wave 0, lanes 0..15): it goes to LDS in log2 units at the end
        // of the step, so that the P waves form each exponent with one fused multiply-add
        f32x4 lse_ld;
        constexpr int NLI = kKvBM * (D / 8) / 64 / 8;  // direct loads per wave and tile
        // load part j of block i: Q instructions, then dO instructions, then lse / D
        auto load_part = [&](int i, auto st, auto J) __attribute__((always_inline)) {
            constexpr int j = decltype(J)::value;
            const int qs = q_start + i * kKvBM;
            if constexpr (j < NLI) load_tile_lds_part<D, 8>(rq, qst(st), qs, w, lane, j);
            else if constexpr (j < 2 * NLI) load_tile_lds_part<D, 8>(rg, gst(st), qs, w, lane, j - NLI);
            else {
                if (w == 0 && lane < 16) lse_ld = __builtin_bit_cast(f32x4, buffer_load16(rl, (uint32_t)(qs + 4 * lane) * 4u));
                if (w == 1 && lane < 16) buffer_load_lds16(rd, sst(st) + 4 * kKvBM, (uint32_t)(qs + 4 * lane) * 4u);
            }
        };
        auto load_blk = [&](int i, auto st) __attribute__((always_inline)) {
            static_for<0, 2 * NLI + 1>([&](auto J) __attribute__((always_inline)) { load_part(i, st, J); });
        };
        auto store_lse = [&](auto st) __attribute__((always_inline)) {
            if (w == 0 && lane < 16)
                *(__attribute__((address_space(3))) f32x4 *)(sst(st) + 16 * lane) = lse_ld * kLog2e;
        };
        // A block that no query of it sees for this pair's keys (causal: the first block for the
        // later pairs) runs in full, masked to P = 0, so that the block index stays out of the
        // step's control flow.  The one exception is the P wave's step past the last block (only
        // zero tiles there, dO = 0): it skips its work, and the dS wave has the SIMD to itself.
        const bool keys_ok = kw0 < Nk;

        // Step i: the P wave works on block i (stage S = i % 3, P buffer B = i % 2), the dS wave on
        // block i - 1 (stage (S + 2) % 3, P buffer 1 - B); block i + 1 is loaded into stage (S + 1) % 3.
        // Each role runs its own copy of the loop (PW), so that the two roles' registers are never
        // live at the same time; both copies load and wait at the same barriers.
        auto run = [&](auto PW) __attribute__((always_inline)) {
            constexpr bool P_WAVE = decltype(PW)::value;
            auto step = [&](int i, auto S, auto B, auto FIRST) __attribute__((always_inline)) {
                constexpr int s_cur = decltype(S)::value;
                using SN = std::integral_constant<int, (s_cur + 1) % 3>;
                using SP = std::integral_constant<int, (s_cur + 2) % 3>;
                using BP = std::integral_constant<int, 1 - decltype(B)::value>;
                // past the last block: zeros into a free stage, never read.  A working wave issues the
                // loads one every second chunk from chunk 1 on, instead of all before its first matrix
                // instruction (B=2, H=16, N=4096 causal: dK/dV -1.3% at d = 128, -1% at d = 64)
                const bool work = (P_WAVE || !decltype(FIRST)::value) && keys_ok && (!P_WAVE || i < nsteps);
                if (!work) load_blk(i + 1, SN{});
                if constexpr (P_WAVE || !decltype(FIRST)::value) {
                    if (work) {
                        // P wave: rows of Q for S, dO^T for dV, on block i.  dS wave: rows of dO for dP,
                        // Q^T for dK, on block i - 1.
                        using SB = std::conditional_t<P_WAVE, decltype(S), SP>;
                        const lds_char *a_l = P_WAVE ? qst(SB{}) : gst(SB{});
                        const lds_char *t_l = P_WAVE ? gst(SB{}) : qst(SB{});
                        const lds_char *st_l = sst(SB{});
                        lds_char *p_l = P_WAVE ? pst(B) : pst(BP{});
                        const int qs = q_start + (P_WAVE ? i : i - 1) * kKvBM;
                        // NC chunks of one matrix instruction and a slice of vector work:
                        //   [0, HS): first product, queries 0..31     [HS, NS): first product, queries 32..63
                        //                                              | P or dS of queries 0..31
                        //   [NS, NS + NA/2): second product over 0..31 | P or dS of queries 32..63
                        //   [NS + NA/2, NC): second product over 32..63
                        constexpr int HS = NKS, NS = 2 * NKS, NA = 4 * NDB, NC = NS + NA, PF = 2;
                        const bool need_mask = P_WAVE && CAUSAL && (qs + off < kw0 + 31);
                        f32x16 sc[2] = {zero16(), zero16()};
                        bf16x8 pb[4];     // P (P wave) or -dS (dS wave), bf16, groups of 16 queries
                        f32x4 v4[2][4];   // lse * log2e of the lane's queries, per half (P wave)
                        if constexpr (!P_WAVE) {
                            // dS wave: the products start from D of the lane's queries 32 qb + 8 g + 4 h + u
#pragma unroll
                            for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
                                for (int g = 0; g < 4; ++g) {
                                    const f32x4 dv = *(const __attribute__((address_space(3))) f32x4 *)(
                                        st_l + 4 * (kKvBM + 32 * qb + 8 * g + 4 * h));
#pragma unroll
                                    for (int u = 0; u < 4; ++u) sc[qb][4 * g + u] = dv[u];
                                }
                            }
                        }
                        bf16x8 pv[2][2];  // P of the half read back from LDS (dS wave)
                        auto fetch = [&](auto C) __attribute__((always_inline)) {
                            constexpr int c = decltype(C)::value;
                            if constexpr (c < NS) {
                                constexpr int qb = c / HS, kst = c % HS;
                                return lds_read16(a_l, swz_off<D>(32 * qb + c32, 2 * kst + h));
                            } else {
                                constexpr int n = c - NS, t = n / NDB, db = n % NDB;
                                return lds_read_tr_rows_swz<D>(t_l, 16 * t, 32 * db, lane);
                            }
                        };
                        bf16x8 fr[PF + 1];
                        static_for<0, PF>([&](auto F) __attribute__((always_inline)) { fr[decltype(F)::value] = fetch(F); });
                        static_for<0, NC>([&](auto C) __attribute__((always_inline)) {
                            constexpr int c = decltype(C)::value;
                            if constexpr (c + PF < NC) fr[(c + PF) % (PF + 1)] = fetch(std::integral_constant<int, c + PF>{});
                            const bf16x8 fc = fr[c % (PF + 1)];
                            if constexpr (c < NS) {
                                constexpr int qb = c / HS, kst = c % HS;
                                sc[qb] = mfma(fc, kvf[kst], sc[qb]);
                            } else {
                                constexpr int n = c - NS, t = n / NDB, db = n % NDB;
                                acc[db] = mfma(fc, pb[t], acc[db]);
                            }
                            // vector work on half qb during window [w0, w0 + L)
                            constexpr int qb = (c >= HS && c < NS) ? 0 : (c >= NS && c < NS + NA / 2) ? 1 : -1;
                            if constexpr (qb >= 0) {
                                constexpr int w0 = qb == 0 ? HS : NS;
                                constexpr int L = qb == 0 ? NS - HS : NA / 2;
                                constexpr int k = c - w0;
                                if constexpr (k == 0) {
                                    // the half's lse (P wave) or P (dS wave) from LDS
                                    if constexpr (P_WAVE) {
#pragma unroll
                                        for (int g = 0; g < 4; ++g)
                                            v4[qb][g] = *(const __attribute__((address_space(3))) f32x4 *)(
                                                st_l + 4 * (32 * qb + 8 * g + 4 * h));
                                    }
                                    if constexpr (!P_WAVE) {
#pragma unroll
                                        for (int tt = 0; tt < 2; ++tt)
                                            pv[qb][tt] = __builtin_bit_cast(bf16x8, *(const __attribute__((address_space(3))) u32x4 *)(
                                                p_l + ((2 * qb + tt) * 64 + lane) * 16));
                                    }
                                    if (need_mask) {
                                        // scores of queries before this lane's key -> -inf (P = 0); a query that
                                        // sees no key has lse = -inf: keep exp2 away from -inf + inf
#pragma unroll
                                        for (int g = 0; g < 4; ++g) {
#pragma unroll
                                            for (int u = 0; u < 4; ++u) {
                                                v4[qb][g][u] = fmaxf(v4[qb][g][u], -1e30f);
                                                if (qs + 32 * qb + 8 * g + 4 * h + u + off < key) sc[qb][4 * g + u] = -__builtin_inff();
                                            }
                                        }
                                    }
                                }
                                static_for<k * 16 / L, (k + 1) * 16 / L>([&](auto RR) __attribute__((always_inline)) {
                                    constexpr int r = decltype(RR)::value, g = r >> 2, u = r & 3;
                                    if constexpr (P_WAVE)
                                        pb[2 * qb + (r >> 3)][r & 7] = (bf16)fast_exp2(fmaf(sc[qb][r], c_log2, -v4[qb][g][u]));
                                    else
                                        pb[2 * qb + (r >> 3)][r & 7] = (bf16)((float)pv[qb][r >> 3][r & 7] * sc[qb][r]);
                                });
                                if constexpr (P_WAVE && k == L - 1) {
#pragma unroll
                                    for (int tt = 0; tt < 2; ++tt)
                                        lds_write16(p_l, ((2 * qb + tt) * 64 + lane) * 16, __builtin_bit_cast(u32x4, pb[2 * qb + tt]));
                                }
                            }
                            if constexpr (c % 2 == 1 && c / 2 < 2 * NLI + 1)
                                load_part(i + 1, SN{}, std::integral_constant<int, c / 2>{});
                            __builtin_amdgcn_sched_barrier(0);
                        });
                    }
                }
                wait_vmem();
                store_lse(SN{});
                __syncthreads();
            };

            using I0 = std::integral_constant<int, 0>;
            using I1 = std::integral_constant<int, 1>;
            using I2 = std::integral_constant<int, 2>;
            using F = std::false_type;
            for (int gq = 0; gq < G; ++gq) {
                bind_query_head(qh0 + gq);
                load_blk(0, I0{});  // the previous query head's last step ended with a barrier
                wait_vmem();
                store_lse(I0{});
                __syncthreads();
                // steps 0 .. nsteps (the dS wave's last block is nsteps - 1); stage i % 3, P buffer
                // i % 2; in step 0 only the P wave works
                if (nsteps == 0) continue;
                step(0, I0{}, I0{}, std::true_type{});
                const int n = nsteps + 1;
                int i = 1;
                for (; i + 5 < n; i += 6) {
                    step(i, I1{}, I1{}, F{});
                    step(i + 1, I2{}, I0{}, F{});
                    step(i + 2, I0{}, I1{}, F{});
                    step(i + 3, I1{}, I0{}, F{});
                    step(i + 4, I2{}, I1{}, F{});
                    step(i + 5, I0{}, I0{}, F{});
                }
                if (i < n) step(i++, I1{}, I1{}, F{});
                if (i < n) step(i++, I2{}, I0{}, F{});
                if (i < n) step(i++, I0{}, I1{}, F{});
                if (i < n) step(i++, I1{}, I0{}, F{});
                if (i < n) step(i++, I2{}, I1{}, F{});
            }
        };
        if (pwave)
            run(std::true_type{});
        else
            run(std::false_type{});

        if (key < Nk) {
            bf16 *row = (pwave ? dV : dK) + hoff + (size_t)key * D;
            const float f = pwave ? 1.f : -scale;
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    bf16x4 v4;
#pragma unroll
                    for (int u = 0; u < 4; ++u) v4[u] = (bf16)(acc[db][4 * g + u] * f);
                    *(bf16x4 *)(row + 32 * db + 8 * g + 4 * h) = v4;
                }
            }
        }
    }
}

// ------------------------------------------------------------ dK / dV, one wave per SIMD (d = 192, 256)

// Four waves, one per SIMD with up to 512 registers.  Wave w owns 32 keys (128 per workgroup): it
// holds K and V of its keys over all of d, and both accumulators, dV^T and dK^T / scale (d columns
// by 32 keys each), which only the matrix instructions touch (the compiler keeps them in AGPRs).
// Per 32-query block it forms S - lse / scale and dP - D = dO V^T - D as two interleaved chains of
// matrix instructions with VGPR accumulators (mfma_vgpr), then P = exp2(S scale log2e -
// lse log2e) and dS = P (dP - D), then dV^T += dO^T P and dK^T += Q^T dS with dO^T and Q^T read
// by transposing reads.  Every wave does all four products for its keys: no partial sums or P pass
// between waves, one barrier per block, about 1 KB of LDS read per matrix instruction.  Q/dO tiles
// live in two LDS stages (working, loading).
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void bwd_dkdv4_kernel(
    const bf16 *__restrict__ Q, const bf16 *__restrict__ K, const bf16 *__restrict__ V, const bf16 *__restrict__ dO,
    const float *__restrict__ LSE, const float *__restrict__ Dl, bf16 *__restrict__ dK, bf16 *__restrict__ dV, int Nq,
    int Nk, int H, int G, int n_ktiles, float scale, float c_log2, int nx)
{
    static_assert(D == 192 || D == 256, "wide-head dK/dV kernel");
    constexpr int NKS = D / 16;  // reduction steps over d of S and dP
    constexpr int NDB = D / 32;  // 32-column blocks of dK and dV
    constexpr int BMQ = 32;      // queries per streamed block
    constexpr int TILE = BMQ * D * 2;
    constexpr int kBN = 128;     // keys per workgroup
    __shared__ __attribute__((aligned(1024))) char q0_raw[TILE], q1_raw[TILE];
    __shared__ __attribute__((aligned(1024))) char g0_raw[TILE], g1_raw[TILE];
    __shared__ __attribute__((aligned(16))) float s0_raw[2 * BMQ], s1_raw[2 * BMQ];  // -lse / scale, -D

    int head, ktile;
    work_item(blockIdx.x, n_ktiles, nx, head, ktile);
    const int Hk = H / G;
    const int qh0 = (head / Hk) * H + (head % Hk) * G;

    const int tid = threadIdx.x;
    const int lane = tid & 63, h = lane >> 5, c32 = lane & 31;
    const int w = wave_uniform(tid >> 6);
    const size_t hoff = (size_t)head * (size_t)Nk * D;
    __amdgpu_buffer_rsrc_t rq, rg, rl, rd;
    auto bind_query_head = [&](int qh) __attribute__((always_inline)) {
        const size_t hoff_q = (size_t)qh * (size_t)Nq * D;
        rq = make_rsrc(Q + hoff_q, (uint32_t)Nq * D * 2);
        rg = make_rsrc(dO + hoff_q, (uint32_t)Nq * D * 2);
        rl = make_rsrc(LSE + (size_t)qh * Nq, (uint32_t)Nq * 4);
        rd = make_rsrc(Dl + (size_t)qh * Nq, (uint32_t)Nq * 4);
    };
    const int off = Nk - Nq;
    const int k0 = ktile * kBN;
    const int kw0 = k0 + 32 * w;
    const int key = kw0 + c32;
    const bool keys_ok = kw0 < Nk;

    // K and V of the lane's key: B operands of S = Q K^T and of dO V^T - D = dP - D, whose
    // accumulator starts from -D, so that dS = P (dP - D) is one multiply per element
    bf16x8 kf[NKS], vf[NKS];
    {
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(K + hoff, (uint32_t)Nk * D * 2);
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(V + hoff, (uint32_t)Nk * D * 2);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            const uint32_t byte = (uint32_t)(key * D + 16 * ks + 8 * h) * 2u;
            kf[ks] = __builtin_bit_cast(bf16x8, buffer_load16(rk, byte));
            vf[ks] = __builtin_bit_cast(bf16x8, buffer_load16(rv, byte));
        }
    }
    f32x16 av[NDB], ak[NDB];  // dV^T and dK^T / scale: columns 32 db .. 32 db + 31, the lane's key
#pragma unroll
    for (int i = 0; i < NDB; ++i) {
        av[i] = zero16();
        ak[i] = zero16();
    }

    // The lane's byte offsets inside a swizzled Q / dO tile, computed once and kept opaque (each
    // LDS read is then one register plus a constant in the offset field).  The swizzle changes only
    // chunk bits 0..3 (d = 256) or 0..2 (d = 192), so chunk 2 kst + h lies at ao[kst % NAO] plus
    // (kst / NAO) 2 NAO chunks, and the transposed reads of column block db at to[db % NTO] plus
    // (db / NTO) 4 NTO chunks.
    constexpr int NAO = D == 256 ? 8 : 4;
    constexpr int NTO = D == 256 ? 4 : 2;
    int ao[NAO];      // A operand of S and dP: row c32, chunk 2 kst + h
    int to[NTO][2];   // transposed reads of column block db: rows 4 (G4 / 2) + s / 4 and + 8 of a 16-row group
#pragma unroll
    for (int kst = 0; kst < NAO; ++kst) {
        ao[kst] = swz_off<D>(c32, 2 * kst + h);
        asm volatile("" : "+v"(ao[kst]));
    }
    auto a_off = [&](int kst) __attribute__((always_inline)) { return ao[kst % NAO] + (kst / NAO) * 32 * NAO; };
    {
        const int G4 = lane >> 4, s16 = lane & 15;
        const int tr = 4 * (G4 >> 1) + (s16 >> 2);
#pragma unroll
        for (int db = 0; db < NTO; ++db) {
            const int byte = 2 * (32 * db + 16 * (G4 & 1) + 4 * (s16 & 3));
            to[db][0] = swz_off<D>(tr, byte >> 4) + (byte & 15);
            to[db][1] = swz_off<D>(tr + 8, byte >> 4) + (byte & 15);
            asm volatile("" : "+v"(to[db][0]));
            asm volatile("" : "+v"(to[db][1]));
        }
    }
    auto t_off = [&](int db, int j) __attribute__((always_inline)) { return to[db % NTO][j] + (db / NTO) * 64 * NTO; };

    const int q_start = CAUSAL ? (max(0, k0 - off) / BMQ) * BMQ : 0;
    const int nsteps = (Nq > q_start) ? (Nq - q_start + BMQ - 1) / BMQ : 0;

    auto qst = [&](auto st) __attribute__((always_inline)) { return (lds_char *)(decltype(st)::value ? q1_raw : q0_raw); };
    auto gst = [&](auto st) __attribute__((always_inline)) { return (lds_char *)(decltype(st)::value ? g1_raw : g0_raw); };
    auto sst = [&](auto st) __attribute__((always_inline)) { return (lds_char *)(decltype(st)::value ? s1_raw : s0_raw); };
    // block i: Q and dO tiles by all four waves; lse (wave 0) and D (wave 1) into registers, to LDS
    // once they have arrived as -lse / scale and -D, the starting values of the two first-product
    // accumulators: S - lse / scale comes out of the matrix instructions, so P = exp2((S - lse /
    // scale) scale log2e) is a multiply and an exponential (a row that sees no key, lse = -inf,
    // starts from 1e30 and is masked to -inf), and dO V^T - D = dP - D
    f32x4 sd_ld;
    auto load_blk = [&](int i, auto st) __attribute__((always_inline)) {
        const int qs = q_start + i * BMQ;
        load_tile_lds<D, 4, BMQ>(rq, qst(st), qs, w, lane);
        load_tile_lds<D, 4, BMQ>(rg, gst(st), qs, w, lane);
        if (w < 2 && lane < 8) sd_ld = __builtin_bit_cast(f32x4, buffer_load16(w == 0 ? rl : rd, (uint32_t)(qs + 4 * lane) * 4u));
    };
    auto store_lse = [&](auto st) __attribute__((always_inline)) {
        if (w < 2 && lane < 8) {
            f32x4 v = sd_ld * (w == 0 ? -1.f / scale : -1.f);
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] = fminf(v[u], 1e30f);
            *(__attribute__((address_space(3))) f32x4 *)(sst(st) + 4 * (w * BMQ + 4 * lane)) = v;
        }
    };

    // Step i on block i (stage S); block i + 1 loads into the other stage, which block i - 1 left
    // at the last barrier.
    auto step = [&](int i, auto S) __attribute__((always_inline)) {
        using SN = std::integral_constant<int, 1 - decltype(S)::value>;
        load_blk(i + 1, SN{});  // past the last block: zeros into the free stage, never read
        if (keys_ok) {
            const lds_char *ql = qst(S), *gl = gst(S), *sl = sst(S);
            const int qs = q_start + i * BMQ;
            // the accumulators start from -lse / scale and from -D of the lane's queries 8 g + 4 h + u
            f32x16 sc, dp;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f32x4 l4 = *(const __attribute__((address_space(3))) f32x4 *)(sl + 4 * (8 * g + 4 * h));
                const f32x4 d4 = *(const __attribute__((address_space(3))) f32x4 *)(sl + 4 * (BMQ + 8 * g + 4 * h));
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    sc[4 * g + u] = l4[u];
                    dp[4 * g + u] = d4[u];
                }
            }
            // first products: S - lse / scale and dP - D as two interleaved chains with VGPR
            // accumulators (the AGPRs all hold dV and dK); fragment c is Q (even c) or dO (odd c)
            // rows for reduction step c / 2, fetched PF instructions ahead
            constexpr int PF = 2, N1 = 2 * NKS;
            auto fetch1 = [&](auto C) __attribute__((always_inline)) {
                constexpr int c = decltype(C)::value;
                return lds_read16((c & 1) ? gl : ql, a_off(c >> 1));
            };
            bf16x8 fr[PF + 1];
            static_for<0, PF>([&](auto F) __attribute__((always_inline)) { fr[decltype(F)::value] = fetch1(F); });
            static_for<0, N1>([&](auto C) __attribute__((always_inline)) {
                constexpr int c = decltype(C)::value;
                if constexpr (c + PF < N1) fr[(c + PF) % (PF + 1)] = fetch1(std::integral_constant<int, c + PF>{});
                if constexpr (c & 1)
                    mfma_vgpr(dp, fr[c % (PF + 1)], vf[c >> 1]);
                else
                    mfma_vgpr(sc, fr[c % (PF + 1)], kf[c >> 1]);
                __builtin_amdgcn_sched_barrier(0);
            });
            mfma_vgpr_settle(sc, dp);
            if (CAUSAL && (qs + off < kw0 + 31)) {
                // scores of queries before this lane's key -> -inf (P = 0)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        if (qs + 8 * g + 4 * h + u + off < key) sc[4 * g + u] = -__builtin_inff();
                }
            }
            // P and dS in bf16, two groups of 16 queries
            bf16x8 pb[2], sb[2];
            auto form_p = [&](auto RR) __attribute__((always_inline)) {
                constexpr int r = decltype(RR)::value;
                sc[r] = fast_exp2(sc[r] * c_log2);
                pb[r >> 3][r & 7] = (bf16)sc[r];
            };
            auto form_ds = [&](auto RR) __attribute__((always_inline)) {
                constexpr int r = decltype(RR)::value;
                sb[r >> 3][r & 7] = (bf16)(sc[r] * dp[r]);
            };
            // second products: chunk n < 2 NDB is dV over query group n / NDB, column block n % NDB
            // (dO^T fragments); n >= 2 NDB is dK / scale likewise (Q^T fragments)
            constexpr int N2 = 4 * NDB;
            auto fetch2 = [&](auto NN) __attribute__((always_inline)) {
                constexpr int n = decltype(NN)::value, m = n % (2 * NDB), t = m / NDB, db = m % NDB;
                const lds_char *tl = n < 2 * NDB ? gl : ql;
                const bf16x4 lo = lds_read_tr(tl, t_off(db, 0) + 16 * t * 2 * D);
                const bf16x4 hi = lds_read_tr(tl, t_off(db, 1) + 16 * t * 2 * D);
                return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            };
            static_for<0, PF>([&](auto F) __attribute__((always_inline)) { fr[decltype(F)::value] = fetch2(F); });
            static_for<0, 8>(form_p);  // P of the first 16 queries before the products that read it
            static_for<0, N2>([&](auto NN) __attribute__((always_inline)) {
                constexpr int n = decltype(NN)::value, m = n % (2 * NDB), t = m / NDB, db = m % NDB;
                if constexpr (n + PF < N2) fr[(n + PF) % (PF + 1)] = fetch2(std::integral_constant<int, n + PF>{});
                if constexpr (n < 2 * NDB)
                    av[db] = mfma(fr[n % (PF + 1)], pb[t], av[db]);
                else
                    ak[db] = mfma(fr[n % (PF + 1)], sb[t], ak[db]);
                // vector work under the products: P of the second group and dS of the first during
                // dV over the first group, dS of the second during dV over the second
                if constexpr (n < NDB) {
                    static_for<8 + n * 8 / NDB, 8 + (n + 1) * 8 / NDB>(form_p);
                    static_for<n * 8 / NDB, (n + 1) * 8 / NDB>(form_ds);
                } else if constexpr (n < 2 * NDB) {
                    static_for<8 + (n - NDB) * 8 / NDB, 8 + (n - NDB + 1) * 8 / NDB>(form_ds);
                }
                __builtin_amdgcn_sched_barrier(0);
            });
        }
        wait_vmem();
        store_lse(SN{});
        __syncthreads();
    };

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    for (int gq = 0; gq < G; ++gq) {
        bind_query_head(qh0 + gq);
        load_blk(0, I0{});  // the previous query head's last step ended with a barrier and no load in flight
        wait_vmem();
        store_lse(I0{});
        __syncthreads();
        int i = 0;
        for (; i + 1 < nsteps; i += 2) {
            step(i, I0{});
            step(i + 1, I1{});
        }
        if (i < nsteps) step(i, I0{});
    }

    if (key < Nk) {
        bf16 *rv_ = dV + hoff + (size_t)key * D;
        bf16 *rk_ = dK + hoff + (size_t)key * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                bf16x4 v4, k4;
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    v4[u] = (bf16)av[db][4 * g + u];
                    k4[u] = (bf16)(ak[db][4 * g + u] * scale);
                }
                *(bf16x4 *)(rv_ + 32 * db + 8 * g + 4 * h) = v4;
                *(bf16x4 *)(rk_ + 32 * db + 8 * g + 4 * h) = k4;
            }
        }
    }
}

// ------------------------------------------------------------ dQ

// Waves per dQ workgroup (32 queries each): 8 for d <= 128, two per SIMD sharing every K/V block
// loaded into LDS; 4 for d = 192, 256, one per SIMD (their registers exceed 256).
template <int D>
constexpr int dq_waves() { return D <= 128 ? 8 : 4; }
constexpr int kQBM = 128;  // the smallest query block of a dQ workgroup (bounds the grid size)
constexpr int kQBN = 64;   // keys per streamed block

// FUSE_D: the kernel also forms D = rowsum(dO o O) of its own rows from O and writes it to Dl for
// the dK/dV kernel that runs after it, in place of the preprocess kernel.  The sum takes the
// preprocess kernel's order (8-element chunks by fused multiply-add, then the chunks pairwise at
// halving distances over a power-of-two count of chunks, the missing ones zero), so D is bitwise
// the same either way.
template <int D, bool CAUSAL, bool FUSE_D = false>
__global__ __launch_bounds__(64 * dq_waves<D>(), D >= 192 ? 1 : 8 / dq_waves<D>()) void bwd_dq_kernel(
    const bf16 *__restrict__ Q, const bf16 *__restrict__ K, const bf16 *__restrict__ V, const bf16 *__restrict__ dO,
    const float *__restrict__ LSE, float *__restrict__ Dl, bf16 *__restrict__ dQ, int Nq, int Nk, int H, int G,
    int n_qtiles, float scale, float c_log2, const bf16 *__restrict__ O, int nx)
{
    constexpr int NKS = D / 16;
    constexpr int NDB = D / 32;
    constexpr int TILE = kQBN * D * 2;
    __shared__ __attribute__((aligned(16))) char k0_raw[TILE], k1_raw[TILE], v0_raw[TILE], v1_raw[TILE];

    int head, t_in;
    work_item(blockIdx.x, n_qtiles, nx, head, t_in);
    const int qtile = CAUSAL ? (n_qtiles - 1 - t_in) : t_in;

    const int tid = threadIdx.x;
    const int lane = tid & 63, h = lane >> 5, c32 = lane & 31;
    const int w = wave_uniform(tid >> 6);
    const size_t hoff = (size_t)head * (size_t)Nq * D;    // Q, dO and dQ of this head
    // K and V of the query head's K/V head (grouped-query attention: G query heads per K/V head)
    const int kvh = (head / H) * (H / G) + (head % H) / G;
    const size_t hoff_k = (size_t)kvh * (size_t)Nk * D;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(Q + hoff, (uint32_t)Nq * D * 2);
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(dO + hoff, (uint32_t)Nq * D * 2);
    // Causal mask with bottom-right alignment: query i sees keys j <= i + off.
    const int off = Nk - Nq;

    constexpr int NW = dq_waves<D>();
    constexpr int BMQ = 32 * NW;  // queries per workgroup
    const int q0 = qtile * BMQ;
    const int qw0 = q0 + 32 * w;  // wave-uniform
    const int qrow = qw0 + c32;
    const bool row_ok = qrow < Nq;

    // dO is held negated, so that the dP product starts from D and yields D - dP; dS = P (dP - D)
    // is then one multiply per element and dQ accumulates with the opposite sign
    bf16x8 qf[NKS], gf[NKS];
    float dfused = 0.f;
    {
        // lane (c32, h) holds 8-element chunks 2 ks + h of its row, ks = 0 .. NKS-1; the preprocess
        // kernel sums 2 NKSP chunks, the ones past the row zero (d = 192: 24 of 32)
        constexpr int NKSP = NKS <= 4 ? 4 : NKS <= 8 ? 8 : 16;
        float a[NKSP];
#pragma unroll
        for (int ks = NKS; ks < NKSP; ++ks) a[ks] = 0.f;
        bf16x8 of[NKS];
        if constexpr (FUSE_D) {
            const __amdgpu_buffer_rsrc_t ro = make_rsrc(O + hoff, (uint32_t)Nq * D * 2);
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
                of[ks] = __builtin_bit_cast(bf16x8, buffer_load16(ro, (uint32_t)(qrow * D + 16 * ks + 8 * h) * 2u));
        }
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            qf[ks] = __builtin_bit_cast(bf16x8, buffer_load16(rq, (uint32_t)(qrow * D + 16 * ks + 8 * h) * 2u));
            const u32x4 graw = buffer_load16(rg, (uint32_t)(qrow * D + 16 * ks + 8 * h) * 2u);
            gf[ks] = __builtin_bit_cast(bf16x8, graw ^ 0x80008000u);
            if constexpr (FUSE_D) {
                const bf16x8 g = __builtin_bit_cast(bf16x8, graw);
                a[ks] = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) a[ks] = fmaf((float)of[ks][e], (float)g[e], a[ks]);
            }
        }
        if constexpr (FUSE_D) {
            // chunks j and j + CPR/2 (ks and ks + NKS/2) first, then halving distances; the last
            // step pairs the even chunks of lane half 0 with the odd ones of half 1
#pragma unroll
            for (int n = NKSP / 2; n >= 1; n >>= 1) {
#pragma unroll
                for (int ks = 0; ks < n; ++ks) a[ks] = a[ks] + a[ks + n];
            }
            dfused = a[0] + __shfl_xor(a[0], 32);
        }
    }
    // a row past Nq, or a query that sees no key (lse = -inf), gets lse2 = +inf and so P = 0
    const float lse_row = row_ok ? LSE[(size_t)head * Nq + qrow] : -__builtin_inff();
    const float lse2 = (lse_row == -__builtin_inff()) ? __builtin_inff() : lse_row * kLog2e;
    float dval;
    if constexpr (FUSE_D) {
        dval = row_ok ? dfused : 0.f;
        if (row_ok && h == 0) Dl[(size_t)head * Nq + qrow] = dfused;
    } else {
        dval = row_ok ? Dl[(size_t)head * Nq + qrow] : 0.f;
    }

    f32x16 dq[NDB];
#pragma unroll
    for (int i = 0; i < NDB; ++i) dq[i] = zero16();

    const int kv_end = CAUSAL ? min(Nk, max(0, q0 + BMQ + off)) : Nk;
    const int nt = (kv_end + kQBN - 1) / kQBN;

    auto kst_l = [&](auto par) __attribute__((always_inline)) { return (lds_char *)(decltype(par)::value ? k1_raw : k0_raw); };
    auto vst_l = [&](auto par) __attribute__((always_inline)) { return (lds_char *)(decltype(par)::value ? v1_raw : v0_raw); };
    // The lane's byte offsets inside a swizzled K/V tile are computed once and kept opaque, so
    // that every LDS read of the loop is one register plus a constant in the instruction's offset
    // field, and every direct load one register plus a buffer base moved by scalar arithmetic;
    // otherwise the compiler rebuilds the swizzled addresses at every use.
    constexpr int kLoadNI = kQBN * (D / 8) / 64 / NW;  // direct loads per wave and tile
    int ko[NKS], vo[NDB][2], go[kLoadNI];
    {
#pragma unroll
        for (int kst = 0; kst < NKS; ++kst) {
            ko[kst] = swz_off<D>(c32, 2 * kst + h);
            asm volatile("" : "+v"(ko[kst]));
        }
        const int G4 = lane >> 4, s16 = lane & 15;
        const int vr = 4 * (G4 >> 1) + (s16 >> 2);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            const int byte = 2 * (32 * db + 16 * (G4 & 1) + 4 * (s16 & 3));
            vo[db][0] = swz_off<D>(vr, byte >> 4) + (byte & 15);
            vo[db][1] = swz_off<D>(vr + 8, byte >> 4) + (byte & 15);
            asm volatile("" : "+v"(vo[db][0]));
            asm volatile("" : "+v"(vo[db][1]));
        }
#pragma unroll
        for (int i = 0; i < kLoadNI; ++i) {
            const int pchunk = 64 * (w * kLoadNI + i) + lane;
            const int row = pchunk / (D / 8);
            const int chunk = (pchunk - row * (D / 8)) ^ lds_swz<D>(row);
            go[i] = row * 2 * D + 16 * chunk;
            asm volatile("" : "+v"(go[i]));
        }
    }
    // direct load I of key block j: K instructions, then V instructions; rows past Nk read as zeros
    auto load_part = [&](int j, auto par, auto I) __attribute__((always_inline)) {
        constexpr int i = decltype(I)::value;
        const int r0 = min(j * kQBN, Nk);
        const __amdgpu_buffer_rsrc_t rj = make_rsrc((i < kLoadNI ? K : V) + hoff_k + (size_t)r0 * D, (uint32_t)(Nk - r0) * D * 2);
        buffer_load_lds16(rj, (i < kLoadNI ? kst_l(par) : vst_l(par)) + 1024 * (w * kLoadNI + i % kLoadNI), (uint32_t)go[i % kLoadNI]);
    };
    auto load_blk = [&](int j, auto par) __attribute__((always_inline)) {
        static_for<0, 2 * kLoadNI>([&](auto I) __attribute__((always_inline)) { load_part(j, par, I); });
    };

    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    load_blk(0, P0{});
    wait_vmem();
    __syncthreads();

    // The wave works on key blocks [0, ja) and only loads and waits on [ja, nt) (causal: the blocks
    // wholly above its rows); separate loops keep the block index out of the step.
    const int last_key = qw0 + 31 + off;
    const int ja = (qw0 >= Nq) ? 0 : (!CAUSAL ? nt : (last_key < 0 ? 0 : min(nt, last_key / kQBN + 1)));
    auto step_idle = [&](int j, auto par) __attribute__((always_inline)) {
        using PN = std::integral_constant<int, 1 - decltype(par)::value>;
        load_blk(j + 1, PN{});
        wait_vmem();
        __syncthreads();
    };
    // CH: an unmasked block, run as chunks (below); otherwise the plain step
    auto step = [&](int j, auto par, auto CH) __attribute__((always_inline)) {
        using PN = std::integral_constant<int, 1 - decltype(par)::value>;
        // past the last block: zeros into the free stage, never read; the chunked step issues the
        // loads one every second chunk from chunk 1 on
        if constexpr (!decltype(CH)::value) load_blk(j + 1, PN{});
        const lds_char *ks = kst_l(par);
        const lds_char *vs = vst_l(par);
        const int k0 = j * kQBN;
        // Only blocks that cross the diagonal or the end of the keys are masked: their masked
        // scores become -inf (P = 0) in a branch that the other blocks skip.
        const bool need_mask = (CAUSAL && (k0 + kQBN - 1 > qw0 + off)) || (k0 + kQBN > Nk);
        // Unmasked block: chunks of one matrix instruction and a slice of vector work,
        // so that one wave's exponentials run under its own products.  LDS fragments are fetched
        // two chunks ahead; scheduling barriers keep each chunk whole.
        if constexpr (decltype(CH)::value) {
            // Six phases of L = NKS chunks (2 NDB = NKS): S of keys 0..31 (half 0), dP of half 0,
            // S of keys 32..63 (half 1), dP of half 1, dQ over half 0, dQ over half 1.  The vector
            // work goes where its inputs are complete, about one element's P or dS per chunk
            // (a lane holds 16 elements of each half; elements 0..7 and 8..15 are the two
            // 16-key groups of dS that the dQ products read):
            //   phase 1 (dP, half 0):  P of elements 0..7 of half 0
            //   phase 2 (S, half 1):   P of elements 8..15 of half 0, dS of its elements 0..7
            //   phase 3 (dP, half 1):  dS of elements 8..15 of half 0, P of elements 0..7 of half 1
            //   phase 4 (dQ, half 0):  P of elements 8..15 of half 1, dS of its elements 0..7
            //   phase 5 (dQ, half 1):  dS of elements 8..15 of half 1 in the first L/2 chunks,
            //                          before the products that read them
            constexpr int L = NKS, NC = 6 * L, PF = 2;
            static_assert(2 * NDB == L, "dQ phases are as long as the score phases");
            f32x16 s[2] = {zero16(), zero16()};  // scores, then P in place
            f32x16 dp[2];                        // D - dP (dO is held negated)
#pragma unroll
            for (int r = 0; r < 16; ++r) dp[0][r] = dp[1][r] = dval;
            bf16x8 sb[4];
            auto fetch = [&](auto C) __attribute__((always_inline)) {
                constexpr int c = decltype(C)::value, ph = c / L, i = c % L;
                if constexpr (ph < 4) {
                    return lds_read16((ph & 1) ? vs : ks, ko[i] + 32 * (ph >> 1) * 2 * D);
                } else {
                    constexpr int t = 2 * (ph - 4) + i / NDB, db = i % NDB;
                    const bf16x4 lo = lds_read_tr(ks, vo[db][0] + 16 * t * 2 * D);
                    const bf16x4 hi = lds_read_tr(ks, vo[db][1] + 16 * t * 2 * D);
                    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                }
            };
            // P and dS of elements [e0, e1) of half kb (elements e and e + 8 share an 8-element
            // group of sb; 8 of them are one group)
            auto p_of = [&](auto KB, auto E0, auto E1) __attribute__((always_inline)) {
                constexpr int kb = decltype(KB)::value;
                static_for<decltype(E0)::value, decltype(E1)::value>([&](auto R) __attribute__((always_inline)) {
                    constexpr int r = decltype(R)::value;
                    s[kb][r] = fast_exp2(fmaf(s[kb][r], c_log2, -lse2));
                });
            };
            auto ds_of = [&](auto KB, auto E0, auto E1) __attribute__((always_inline)) {
                constexpr int kb = decltype(KB)::value;
                static_for<decltype(E0)::value, decltype(E1)::value>([&](auto R) __attribute__((always_inline)) {
                    constexpr int r = decltype(R)::value;
                    sb[2 * kb + (r >> 3)][r & 7] = (bf16)(s[kb][r] * dp[kb][r]);
                });
            };
            using K0 = std::integral_constant<int, 0>;
            using K1 = std::integral_constant<int, 1>;
            bf16x8 fr[PF + 1];
            static_for<0, PF>([&](auto F) __attribute__((always_inline)) { fr[decltype(F)::value] = fetch(F); });
            static_for<0, NC>([&](auto C) __attribute__((always_inline)) {
                constexpr int c = decltype(C)::value, ph = c / L, i = c % L;
                if constexpr (c + PF < NC) fr[(c + PF) % (PF + 1)] = fetch(std::integral_constant<int, c + PF>{});
                const bf16x8 fc = fr[c % (PF + 1)];
                if constexpr (ph < 4) {
                    constexpr int kb = ph >> 1;
                    if constexpr (ph & 1)
                        dp[kb] = mfma(fc, gf[i], dp[kb]);
                    else
                        s[kb] = mfma(fc, qf[i], s[kb]);
                } else {
                    constexpr int t = 2 * (ph - 4) + i / NDB, db = i % NDB;
                    dq[db] = mfma(fc, sb[t], dq[db]);
                }
                // 8 elements over the L chunks of a phase: chunk i takes [8 i / L, 8 (i + 1) / L)
                using A0 = std::integral_constant<int, 8 * i / L>;
                using A1 = std::integral_constant<int, 8 * (i + 1) / L>;
                using B0 = std::integral_constant<int, 8 + 8 * i / L>;
                using B1 = std::integral_constant<int, 8 + 8 * (i + 1) / L>;
                if constexpr (ph == 1) {
                    p_of(K0{}, A0{}, A1{});
                } else if constexpr (ph == 2) {
                    p_of(K0{}, B0{}, B1{});
                    ds_of(K0{}, A0{}, A1{});
                } else if constexpr (ph == 3) {
                    ds_of(K0{}, B0{}, B1{});
                    p_of(K1{}, A0{}, A1{});
                } else if constexpr (ph == 4) {
                    p_of(K1{}, B0{}, B1{});
                    ds_of(K1{}, A0{}, A1{});
                } else if constexpr (ph == 5 && i < L / 2) {
                    ds_of(K1{}, std::integral_constant<int, 8 + 16 * i / L>{}, std::integral_constant<int, 8 + 16 * (i + 1) / L>{});
                }
                if constexpr (c % 2 == 1 && c / 2 < 2 * kLoadNI) load_part(j + 1, PN{}, std::integral_constant<int, c / 2>{});
                __builtin_amdgcn_sched_barrier(0);
            });
        } else {
            f32x16 s[2] = {zero16(), zero16()};
            f32x16 dp[2];  // D - dP
#pragma unroll
            for (int r = 0; r < 16; ++r) dp[0][r] = dp[1][r] = dval;
#pragma unroll
            for (int kst = 0; kst < NKS; ++kst) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const int off = ko[kst] + 32 * kb * 2 * D;
                    s[kb] = mfma(lds_read16(ks, off), qf[kst], s[kb]);
                    dp[kb] = mfma(lds_read16(vs, off), gf[kst], dp[kb]);
                }
            }
            if (need_mask) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int kk = k0 + 32 * kb + 8 * (r >> 2) + 4 * h + (r & 3);
                        if ((CAUSAL && kk > qrow + off) || kk >= Nk) s[kb][r] = -__builtin_inff();
                    }
                }
            }
            bf16x8 sb[4];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p = fast_exp2(fmaf(s[kb][r], c_log2, -lse2));
                    sb[2 * kb + (r >> 3)][r & 7] = (bf16)(p * dp[kb][r]);
                }
            }
            // dQ^T += K^T dS^T over 4 groups of 16 keys
#pragma unroll
            for (int t = 0; t < kQBN / 16; ++t) {
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const bf16x4 lo = lds_read_tr(ks, vo[db][0] + 16 * t * 2 * D);
                    const bf16x4 hi = lds_read_tr(ks, vo[db][1] + 16 * t * 2 * D);
                    dq[db] = mfma(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), sb[t], dq[db]);
                }
            }
        }
        wait_vmem();
        __syncthreads();
    };

    // stage parity of key block j is j & 1.  Blocks [0, jm) need no mask and run as chunks;
    // [jm, ja) cross the diagonal or the end of the keys (the need for a mask only grows with j).
    // Separate loops keep the two bodies' registers apart.
    using CHK = std::true_type;
    using PLAIN = std::false_type;
    const int jm_c = CAUSAL ? (qw0 + off - (kQBN - 1) >= 0 ? (qw0 + off - (kQBN - 1)) / kQBN + 1 : 0) : ja;
    const int jm = max(0, min(ja, min(jm_c, Nk / kQBN)));
    int j = 0;
    for (; j + 1 < jm; j += 2) {
        step(j, P0{}, CHK{});
        step(j + 1, P1{}, CHK{});
    }
    if (j < jm) step(j++, P0{}, CHK{});
    if (j < ja && (j & 1)) step(j++, P1{}, PLAIN{});
    for (; j + 1 < ja; j += 2) {
        step(j, P0{}, PLAIN{});
        step(j + 1, P1{}, PLAIN{});
    }
    if (j < ja) step(j++, P0{}, PLAIN{});
    if (j < nt && (j & 1)) step_idle(j++, P1{});
    for (; j + 1 < nt; j += 2) {
        step_idle(j, P0{});
        step_idle(j + 1, P1{});
    }
    if (j < nt) step_idle(j, P0{});

    if (row_ok) {
        bf16 *qrow_p = dQ + hoff + (size_t)qrow * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                bf16x4 v4;
#pragma unroll
                for (int u = 0; u < 4; ++u) v4[u] = (bf16)(dq[db][4 * g + u] * -scale);
                *(bf16x4 *)(qrow_p + 32 * db + 8 * g + 4 * h) = v4;
            }
        }
    }
}

template <int D>
hipError_t launch_pre_t(const BwdArgs &a)
{
    constexpr int RPB = kThreads / (D / 8 <= 8 ? 8 : D / 8 <= 16 ? 16 : 32);
    const long long rows = (long long)a.B * a.H * a.Nq;
    const long long G = (rows + RPB - 1) / RPB;
    if (G == 0) return hipSuccess;
    hipLaunchKernelGGL((bwd_preprocess_kernel<D>), dim3((unsigned)G), dim3(kThreads), 0, (hipStream_t)a.stream,
                       (const bf16 *)a.o, (const bf16 *)a.dout, a.delta, rows);
    return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_dkdv2_t(const BwdArgs &a)
{
    const int n_ktiles = (a.Nk + 127) / 128;
    const long long n_items = (long long)a.B * a.Hk * n_ktiles;
    if (n_items == 0) return hipSuccess;
    // one workgroup per CU fits (LDS); with more items than CUs and heads spread evenly over the
    // XCDs, one persistent workgroup per CU takes them in rounds
    const long long P = persistent_grid(n_items, (long long)a.B * a.Hk, a.dev.cus, a.dev.nx);
    const long long G = P > 0 ? P : n_items;
    const Dkdv2Args args{(const bf16 *)a.q, (const bf16 *)a.k, (const bf16 *)a.v, (const bf16 *)a.dout, a.lse,
                         (const float *)a.delta, (bf16 *)a.dk, (bf16 *)a.dv, a.Nq, a.Nk, a.H, a.H / a.Hk, n_ktiles,
                         (int)n_items, a.dev.nx, a.scale, a.scale * kLog2e};
    hipLaunchKernelGGL((bwd_dkdv2_kernel<D, CAUSAL>), dim3((unsigned)G), dim3(512), 0, (hipStream_t)a.stream, args);
    return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_dkdv4_t(const BwdArgs &a)
{
    const int n_ktiles = (a.Nk + 127) / 128;
    const long long G = (long long)a.B * a.Hk * n_ktiles;
    if (G == 0) return hipSuccess;
    hipLaunchKernelGGL((bwd_dkdv4_kernel<D, CAUSAL>), dim3((unsigned)G), dim3(256), 0, (hipStream_t)a.stream,
                       (const bf16 *)a.q, (const bf16 *)a.k, (const bf16 *)a.v, (const bf16 *)a.dout, a.lse,
                       (const float *)a.delta, (bf16 *)a.dk, (bf16 *)a.dv, a.Nq, a.Nk, a.H, a.H / a.Hk, n_ktiles, a.scale,
                       a.scale * kLog2e, a.dev.nx);
    return hipGetLastError();
}

template <int D, bool CAUSAL, bool FUSE_D = false>
hipError_t launch_dq_t(const BwdArgs &a)
{
    const int n_qtiles = (a.Nq + 32 * dq_waves<D>() - 1) / (32 * dq_waves<D>());
    const long long G = (long long)a.B * a.H * n_qtiles;
    if (G == 0) return hipSuccess;
    hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL, FUSE_D>), dim3((unsigned)G), dim3(64 * dq_waves<D>()), 0, (hipStream_t)a.stream,
                       (const bf16 *)a.q, (const bf16 *)a.k, (const bf16 *)a.v, (const bf16 *)a.dout, a.lse,
                       a.delta, (bf16 *)a.dq, a.Nq, a.Nk, a.H, a.H / a.Hk, n_qtiles, a.scale, a.scale * kLog2e,
                       (const bf16 *)a.o, a.dev.nx);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_preprocess(const BwdArgs &a)
{
    switch (a.d) {
    case 64: return launch_pre_t<64>(a);
    case 128: return launch_pre_t<128>(a);
    case 192: return launch_pre_t<192>(a);
    default: return launch_pre_t<256>(a);
    }
}

hipError_t launch_bwd_dkdv(const BwdArgs &a)
{
    switch (a.d) {
    case 64: return a.causal ? launch_dkdv2_t<64, true>(a) : launch_dkdv2_t<64, false>(a);
    case 128: return a.causal ? launch_dkdv2_t<128, true>(a) : launch_dkdv2_t<128, false>(a);
    case 192: return a.causal ? launch_dkdv4_t<192, true>(a) : launch_dkdv4_t<192, false>(a);
    default: return a.causal ? launch_dkdv4_t<256, true>(a) : launch_dkdv4_t<256, false>(a);
    }
}

bool bwd_dq_fuses_delta(int d) { return d == 64 || d == 128 || d == 192 || d == 256; }

hipError_t launch_bwd_dq_delta(const BwdArgs &a)
{
    switch (a.d) {
    case 64: return a.causal ? launch_dq_t<64, true, true>(a) : launch_dq_t<64, false, true>(a);
    case 128: return a.causal ? launch_dq_t<128, true, true>(a) : launch_dq_t<128, false, true>(a);
    case 192: return a.causal ? launch_dq_t<192, true, true>(a) : launch_dq_t<192, false, true>(a);
    case 256: return a.causal ? launch_dq_t<256, true, true>(a) : launch_dq_t<256, false, true>(a);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_bwd_dq(const BwdArgs &a)
{
    switch (a.d) {
    case 64: return a.causal ? launch_dq_t<64, true>(a) : launch_dq_t<64, false>(a);
    case 128: return a.causal ? launch_dq_t<128, true>(a) : launch_dq_t<128, false>(a);
    case 192: return a.causal ? launch_dq_t<192, true>(a) : launch_dq_t<192, false>(a);
    default: return a.causal ? launch_dq_t<256, true>(a) : launch_dq_t<256, false>(a);
    }
}

long long bwd_dkdv_grid_size(int B, int Hk, int Nk) { return (long long)B * Hk * ((Nk + kv_bn<256>() - 1) / kv_bn<256>()); }
long long bwd_dq_grid_size(int B, int H, int Nq) { return (long long)B * H * ((Nq + kQBM - 1) / kQBM); }

}  // namespace attn
