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
//   * one workgroup of 8 waves (d = 128) or 4 waves (d = 64, 192, 256) per block
//     of query rows; each wave owns 32 rows and holds their Q fragments in VGPRs
//     for the whole loop; at d = 192 and 256 one wave per SIMD, with the O
//     accumulators in AGPRs and the score chains in VGPRs (mfma_vgpr);
//   * key/value blocks of 64 rows are double-buffered through swizzled LDS tiles
//     filled by direct global->LDS buffer loads (rows past the end read as zeros, no
//     staging registers, no LDS store instructions); K runs one block ahead of V, so
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
//     that cross the diagonal, and each workgroup takes a long and a short query
//     block (T-1-p and p of T), so that all workgroups carry equal work.
#include "attn_device.h"
#include "attn_launch.h"

#include <type_traits>

namespace attn {

namespace {

// Waves per workgroup (32 query rows each): 8 at d = 128, where two waves per SIMD come from
// the same workgroup and share each K/V block loaded into LDS; 4 otherwise.
template <int D>
constexpr int fwd_waves() { return D == 128 ? 8 : 4; }
// Workgroups per CU the launch bounds ask for: two waves per SIMD for d <= 128; one for
// d = 192 and 256, whose accumulators need more than 256 registers per wave.
template <int D>
constexpr int fwd_min_blocks() { return D >= 192 ? 1 : 8 / fwd_waves<D>(); }
template <int D>
constexpr int fwd_bm() { return 32 * fwd_waves<D>(); }
constexpr int kFwdBN = 64;                 // keys per streamed block
constexpr float kRescaleLog2 = 8.0f;

template <int D>
struct FwdSmem {
    static constexpr int TILE = kFwdBN * D * 2;  // one swizzled K or V block
    static constexpr int OFF_V = 2 * TILE;       // two K stages, then two V stages
    static constexpr int TOTAL = 4 * TILE;
};

// SPLIT: the key range is cut into n_splits pieces of split_blocks key blocks; workgroup
// (query block, piece) writes the piece's normalised partial output (fp32) to OP and its
// log-sum-exp to LP, and fwd_combine_kernel merges the pieces.
template <int D, bool CAUSAL, bool SPLIT>
__global__ __launch_bounds__(64 * fwd_waves<D>(), fwd_min_blocks<D>()) void fwd_kernel(const bf16 *__restrict__ Q, const bf16 *__restrict__ K,
                                                          const bf16 *__restrict__ V, bf16 *__restrict__ O,
                                                          float *__restrict__ LSE, int Nq, int Nk, int H, int G, int n_qtiles,
                                                          float scale, float c_log2, int n_splits, int split_blocks,
                                                          float *__restrict__ OP, float *__restrict__ LP, int nx, int pair)
{
    using L = FwdSmem<D>;
    constexpr int kFwdWaves = fwd_waves<D>();
    constexpr int kFwdBM = fwd_bm<D>();
    constexpr int NKS = D / 16;          // reduction steps over d for S^T
    constexpr int NDB = D / 32;          // 32-wide column blocks of O
    // one LDS array per stage, so that reads of one stage are known not to alias the
    // direct loads into the other (no wait on those loads before the reads)
    __shared__ __attribute__((aligned(16))) char k0_raw[L::TILE], k1_raw[L::TILE], v0_raw[L::TILE], v1_raw[L::TILE];

    // Causal with `pair` set: workgroup `pos` of a head takes query blocks T-1-pos and then pos
    // (T = n_qtiles), so every workgroup but a middle one does the same T+1 blocks' worth of work.
    // Otherwise one query block per workgroup; causal blocks go longest first (T-1-pos).
    // Split: one (query block, key piece) per workgroup.
    const int n_pos = SPLIT ? n_qtiles * n_splits : (pair ? (n_qtiles + 1) / 2 : n_qtiles);
    int head, pos;
    work_item(blockIdx.x, n_pos, nx, head, pos);
    const int split = SPLIT ? pos % n_splits : 0;

    const int tid = threadIdx.x;
    const int lane = tid & 63, h = lane >> 5, c32 = lane & 31;
    const int w = wave_uniform(tid >> 6);
    const size_t hoff = (size_t)head * (size_t)Nq * D;    // Q and O of this head
    // K and V of the query head's K/V head (grouped-query attention: G query heads per K/V head)
    const int kvh = (head / H) * (H / G) + (head % H) / G;
    const size_t hoff_k = (size_t)kvh * (size_t)Nk * D;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(Q + hoff, (uint32_t)Nq * D * 2);
    // Causal mask with bottom-right alignment: query i sees keys j <= i + off.
    const int off = Nk - Nq;

    // The lane's byte offsets inside a swizzled K/V tile are computed once and kept opaque, so
    // that every LDS read of the loop is one register plus a constant (stage and row block) in the
    // instruction's offset field, and every direct load one register plus a buffer base moved by
    // scalar arithmetic; otherwise the compiler rebuilds the swizzled addresses with vector
    // arithmetic at every use (at d = 256 about 20 instructions per transposed V read).
    constexpr int kLoadNI = kFwdBN * (D / 8) / 64 / kFwdWaves;  // direct loads per wave and tile
    int ko[NKS];         // K fragment of reduction step kst: row c32, chunk 2 kst + h
    int vo[NDB][2];      // V^T fragment of column block db: rows r and r + 8 of a 16-row block
    int go[kLoadNI];     // source of direct load i within a tile
    {
#pragma unroll
        for (int kst = 0; kst < NKS; ++kst) {
            ko[kst] = swz_off<D>(c32, 2 * kst + h);
            asm volatile("" : "+v"(ko[kst]));
        }
        const int G = lane >> 4, s16 = lane & 15;
        const int vr = 4 * (G >> 1) + (s16 >> 2);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            const int byte = 2 * (32 * db + 16 * (G & 1) + 4 * (s16 & 3));
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

    for (int pass = 0; pass < ((CAUSAL && !SPLIT && pair) ? 2 : 1); ++pass) {
        const int qtile = SPLIT ? pos / n_splits : (pass == 0 ? (CAUSAL ? n_qtiles - 1 - pos : pos) : pos);
        if (pass == 1 && qtile == n_qtiles - 1 - pos) break;  // odd T: the middle block is alone
        const int q0 = qtile * kFwdBM;
        const int qw0 = q0 + 32 * w;  // wave-uniform
        const int qrow = qw0 + c32;

        // Q fragments: B operand of S^T = K Q^T, lane holds Q[qrow][16ks + 8h .. +7] (zeros past Nq).
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

        // keys that some row of this block sees (none for rows that see no key at all)
        const int kv_end = CAUSAL ? min(Nk, max(0, q0 + kFwdBM + off)) : Nk;
        // key blocks [jb, je) of this workgroup: all of them, or one piece of the split range
        const int jb = SPLIT ? split * split_blocks : 0;
        const int je = SPLIT ? min((kv_end + kFwdBN - 1) / kFwdBN, jb + split_blocks) : (kv_end + kFwdBN - 1) / kFwdBN;

        // Key / value blocks go straight from global memory into swizzled LDS tiles.
        // stage of block j is j & 1; callers pass the parity as a compile-time constant
        auto kstage = [&](auto par) __attribute__((always_inline)) { return (lds_char *)(decltype(par)::value ? k1_raw : k0_raw); };
        auto vstage = [&](auto par) __attribute__((always_inline)) { return (lds_char *)(decltype(par)::value ? v1_raw : v0_raw); };
        // key rows [j * BN, j * BN + BN) of K or V into a stage.  Rows past the last block this
        // workgroup needs read as zeros without touching memory (the pipeline's loads one and two
        // blocks past the end), as do rows past Nk.
        const int kv_lim = min(Nk, je * kFwdBN);
        auto load_blk = [&](const bf16 *src, lds_char *tile, int j) __attribute__((always_inline)) {
            const int r0 = min(j * kFwdBN, kv_lim);
            const __amdgpu_buffer_rsrc_t rj = make_rsrc(src + hoff_k + (size_t)r0 * D, (uint32_t)(kv_lim - r0) * D * 2);
#pragma unroll
            for (int i = 0; i < kLoadNI; ++i) buffer_load_lds16(rj, tile + 1024 * (w * kLoadNI + i), (uint32_t)go[i]);
        };
        auto load_part = [&](const bf16 *src, lds_char *tile, int j, int i) __attribute__((always_inline)) {
            const int r0 = min(j * kFwdBN, kv_lim);
            const __amdgpu_buffer_rsrc_t rj = make_rsrc(src + hoff_k + (size_t)r0 * D, (uint32_t)(kv_lim - r0) * D * 2);
            buffer_load_lds16(rj, tile + 1024 * (w * kLoadNI + i), (uint32_t)go[i]);
        };
        auto load_k = [&](int j, auto par) __attribute__((always_inline)) { load_blk(K, kstage(par), j); };
        auto load_v = [&](int j, auto par) __attribute__((always_inline)) { load_blk(V, vstage(par), j); };

        // S^T block (64 keys x 32 queries) of key block j
        auto scores = [&](auto par, f32x16 *s) __attribute__((always_inline)) {
            const lds_char *ks = kstage(par);
            s[0] = zero16();
            s[1] = zero16();
#pragma unroll
            for (int kst = 0; kst < NKS; ++kst) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const bf16x8 a = lds_read16(ks, swz_off<D>(32 * kb + c32, 2 * kst + h));
                    s[kb] = mfma(a, qf[kst], s[kb]);
                }
            }
        };

        // maximum over this lane's 32 keys of a score block (one half of the row's 64 keys)
        auto local_max = [&](const f32x16 *sc) __attribute__((always_inline)) {
            float m = fmaxf(sc[0][0], sc[0][1]);
#pragma unroll
            for (int r = 2; r < 16; ++r) m = fmaxf(m, sc[0][r]);
#pragma unroll
            for (int r = 0; r < 16; ++r) m = fmaxf(m, sc[1][r]);
            return m;
        };
        float mloc = -__builtin_inff();  // local maximum of the block whose scores are current

        // The wave works on key blocks [jb, ja) and only loads and waits on [ja, je): under the
        // causal mask the blocks from ja on lie wholly above its rows.  Two loops with no branch
        // on the block index inside keep the score registers out of control flow.
        const int last_key = qw0 + 31 + off;  // last key some row of the wave sees (causal)
        const int ja = (qw0 >= Nq) ? jb
                       : (!CAUSAL ? je : (last_key < 0 ? jb : max(jb, min(je, last_key / kFwdBN + 1))));

        // prologue: K0, V0 and K1 in LDS, scores of block 0 in registers
        using P0 = std::integral_constant<int, 0>;
        using P1 = std::integral_constant<int, 1>;
        load_k(jb, P0{});
        load_v(jb, P0{});
        load_k(jb + 1, P1{});
        wait_vmem();
        __syncthreads();
        f32x16 sa[2], sb[2];
        if (ja > jb) {
            scores(P0{}, sa);
            mloc = local_max(sa);
        }
        // the first step loads K of block 2 into the stage of K0: every wave must be done
        // reading K0 first (rows past the end come back as zeros almost at once)
        __syncthreads();

        // A step on a key block the wave does not see: the loads of the pipeline and the barrier.
        auto step_idle = [&](int j, auto par) __attribute__((always_inline)) {
            using PN = std::integral_constant<int, 1 - decltype(par)::value>;
            load_k(j + 2, par);
            load_v(j + 1, PN{});
            wait_vmem();
            __syncthreads();
        };
        // One pipeline step on key block j: scores of j are in `cur`, scores of j+1 go to `nxt`.
        // LAST: the wave's last block; the scores of j+1 are not needed and are not computed.
        auto step = [&](int j, auto par, f32x16 *cur, f32x16 *nxt, auto LAST) __attribute__((always_inline)) {
            constexpr bool last = decltype(LAST)::value;
            using PN = std::integral_constant<int, 1 - decltype(par)::value>;  // parity of j + 1
            {
                const int k0 = j * kFwdBN;
                if ((CAUSAL && (k0 + kFwdBN - 1 > qw0 + off)) || (k0 + kFwdBN > Nk)) {
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int key = k0 + 32 * kb + 8 * (r >> 2) + 4 * h + (r & 3);
                            if ((CAUSAL && key > qrow + off) || key >= Nk) cur[kb][r] = -__builtin_inff();
                        }
                    }
                    mloc = local_max(cur);
                }
                // Rescale check without a cross-lane exchange in the common case: each half of the
                // wave compares the maximum of its own 32 keys with the offset; only when some lane
                // outgrows it are the two halves' maxima combined and the offset moved.
                if (__builtin_amdgcn_ballot_w64(mloc > m_run + grow_thr)) {
                    const float mrow = fmaxf(mloc, __shfl_xor(mloc, 32));
                    const bool grow = mrow > m_run + grow_thr;  // identical for both halves of a row
                    const float m_new = grow ? mrow : m_run;
                    const float alpha = grow ? fast_exp2((m_run - m_new) * c_log2) : 1.f;
                    m_run = m_new;
                    msc = (m_run == -__builtin_inff()) ? 0.f : m_run * c_log2;
                    l_run *= alpha;
                    if constexpr (D >= 192) {
                        // O stays in AGPRs (a multiply there would move all of it to VGPRs and
                        // back around every step, not only in this rare branch)
                        agpr_settle();
#pragma unroll
                        for (int db = 0; db < NDB; ++db) scale_agpr(oacc[db], alpha);
                        agpr_settle();
                    } else {
#pragma unroll
                        for (int db = 0; db < NDB; ++db) {
#pragma unroll
                            for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
                        }
                    }
                }
                // One step is NC chunks, each one matrix instruction plus a slice of vector work:
                //   S1: first half of the score MFMAs of block j+1   | exponentials of keys 0..31 of block j
                //   V1: first half of the P V MFMAs (keys 0..31)     | exponentials of keys 32..63
                //   S2: second half of the score MFMAs               | exp-sum of block j
                //   V2: second half of the P V MFMAs (keys 32..63)   | maximum of block j+1
                // LDS fragments are fetched 2 chunks ahead; scheduling barriers keep each chunk whole.
                __builtin_amdgcn_s_setprio(1);
                constexpr int NS = 2 * NKS, NPV = (kFwdBN / 16) * NDB, NC = NS + NPV;
                const lds_char *ks = kstage(PN{});
                const lds_char *vs = vstage(par);
                constexpr auto is_s = [](int c) { return c < NS / 2 || (c >= NS / 2 + NPV / 2 && c < NS + NPV / 2); };
                auto fetch = [&](auto C) __attribute__((always_inline)) {
                    constexpr int c = decltype(C)::value;
                    if constexpr (is_s(c)) {
                        constexpr int s = c < NS / 2 ? c : c - NPV / 2;
                        return lds_read16(ks, ko[s >> 1] + 32 * (s & 1) * 2 * D);
                    } else {
                        constexpr int p = c < NS / 2 + NPV / 2 ? c - NS / 2 : c - NS;
                        constexpr int rb = 16 * (p / NDB) * 2 * D;
                        const bf16x4 lo = lds_read_tr(vs, vo[p % NDB][0] + rb);
                        const bf16x4 hi = lds_read_tr(vs, vo[p % NDB][1] + rb);
                        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                    }
                };
                // d >= 192 (AGPRs hold O): the score chains accumulate in VGPRs, the first instruction
                // of each from zero
                constexpr bool kVS = D >= 192;
                if constexpr (!last && !kVS) {
                    nxt[0] = zero16();
                    nxt[1] = zero16();
                }
                bf16x8 pb[kFwdBN / 16];
                float rs = 0.f, mx = -__builtin_inff();
                constexpr int PF = 2;
                bf16x8 fr[PF + 1];
                static_for<0, PF>([&](auto F) __attribute__((always_inline)) {
                    if constexpr (!(last && is_s(decltype(F)::value))) fr[decltype(F)::value] = fetch(F);
                });
                static_assert(NS / 2 == NPV / 2, "phases S1 and V1 must have equal length");
                static_assert(4 * kLoadNI <= NC, "the direct loads fit in the step's odd chunks");
                constexpr int PH = NS / 2;  // chunks per phase
                static_for<0, NC>([&](auto C) __attribute__((always_inline)) {
                    constexpr int c = decltype(C)::value;
                    if constexpr (c + PF < NC && !(last && is_s(c + PF)))
                        fr[(c + PF) % (PF + 1)] = fetch(std::integral_constant<int, c + PF>{});
                    if constexpr (is_s(c)) {
                        constexpr int s = c < NS / 2 ? c : c - NPV / 2;
                        if constexpr (!last && !kVS) {
                            nxt[s & 1] = mfma(fr[c % (PF + 1)], qf[s >> 1], nxt[s & 1]);
                        } else if constexpr (!last) {
                            if constexpr (s < 2) mfma_vgpr_zero(nxt[s & 1], fr[c % (PF + 1)], qf[s >> 1]);
                            else mfma_vgpr(nxt[s & 1], fr[c % (PF + 1)], qf[s >> 1]);
                            if constexpr (s == NS - 1) mfma_vgpr_settle(nxt[0], nxt[1]);
                        }
                    } else {
                        const bf16x8 fc = fr[c % (PF + 1)];
                        constexpr int p = c < NS / 2 + NPV / 2 ? c - NS / 2 : c - NS;
                        oacc[p % NDB] = mfma(fc, pb[p / NDB], oacc[p % NDB]);
                    }
                    // the direct loads one every second chunk from chunk 1 on, K of block j + 2 and then
                    // V of block j + 1, rather than in two bursts (at d = 256, 8 instructions each)
                    if constexpr (c % 2 == 1 && c / 2 < kLoadNI) load_part(K, kstage(par), j + 2, c / 2);
                    else if constexpr (c % 2 == 1 && c / 2 < 2 * kLoadNI) load_part(V, vstage(PN{}), j + 1, c / 2 - kLoadNI);
                    if constexpr (c < 2 * PH) {
                        // exponentials: keys 0..31 during S1, 32..63 during V1; chunk i of the phase
                        // takes elements [16 i / PH, 16 (i + 1) / PH)
                        constexpr int kb = c < PH ? 0 : 1;
                        constexpr int i = c < PH ? c : c - PH;
                        static_for<i * 16 / PH, (i + 1) * 16 / PH>([&](auto RR) __attribute__((always_inline)) {
                            constexpr int r = decltype(RR)::value;
                            cur[kb][r] = fast_exp2(fmaf(cur[kb][r], c_log2, -msc));
                            pb[2 * kb + (r >> 3)][r & 7] = (bf16)cur[kb][r];
                        });
                    } else if constexpr (c < 3 * PH) {
                        constexpr int i = c - 2 * PH;
                        static_for<i * 32 / PH, (i + 1) * 32 / PH>([&](auto RR) __attribute__((always_inline)) {
                            constexpr int r = decltype(RR)::value;
                            rs += cur[r >> 4][r & 15];
                        });
                        // keep the slice in this chunk: the sum is only read after the step, and
                        // without a use here the compiler sinks the whole chain past the barrier
                        asm volatile("" : "+v"(rs));
                    } else if constexpr (!last) {
                        constexpr int i = c - 3 * PH;
                        static_for<i * 32 / PH, (i + 1) * 32 / PH>([&](auto RR) __attribute__((always_inline)) {
                            constexpr int r = decltype(RR)::value;
                            mx = fmaxf(mx, nxt[r >> 4][r & 15]);
                        });
                        asm volatile("" : "+v"(mx));
                    }
                    __builtin_amdgcn_sched_barrier(0);
                });
                l_run += rs;
                mloc = mx;
                __builtin_amdgcn_s_setprio(0);
            }
            wait_vmem();
            __syncthreads();
        };

        // stage parity of block j is (j - jb) & 1; the wave's last block, ja - 1, runs as LAST
        using NL = std::false_type;
        using LS = std::true_type;
        int j = jb;
        for (; j + 1 < ja; j += 2) {
            step(j, P0{}, sa, sb, NL{});
            step(j + 1, P1{}, sb, sa, NL{});
        }
        if (j < ja) step(j++, P0{}, sa, sb, LS{});
        if (j < je && ((j - jb) & 1)) step_idle(j++, P1{});
        for (; j + 1 < je; j += 2) {
            step_idle(j, P0{});
            step_idle(j + 1, P1{});
        }
        if (j < je) step_idle(j, P0{});

        // epilogue: O = acc / l (bf16, nearest even), lse = m*scale + ln(l)
        const float l_tot = l_run + __shfl_xor(l_run, 32);
        if (SPLIT && qrow < Nq) {
            // this piece's O = acc / l in fp32 and its lse (-inf when it holds no visible key)
            const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
            const int n_heads = (int)gridDim.x / n_pos;  // B * H
            const size_t prow = ((size_t)split * n_heads + head) * Nq + qrow;
            float *orow = OP + prow * D;
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    f32x4 ov;
#pragma unroll
                    for (int i = 0; i < 4; ++i) ov[i] = oacc[db][4 * g + i] * inv;
                    *(f32x4 *)(orow + 32 * db + 8 * g + 4 * h) = ov;
                }
            }
            if (h == 0) LP[prow] = (l_tot > 0.f) ? fmaf(m_run, scale, __logf(l_tot)) : -__builtin_inff();
        } else if (qrow < Nq) {
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
                LSE[(size_t)head * Nq + qrow] = (l_tot > 0.f) ? fmaf(m_run, scale, __logf(l_tot)) : -__builtin_inff();
        }
    }
}

template <int D, bool CAUSAL>
hipError_t launch_fwd_t(const FwdArgs &a)
{
    constexpr int kFwdBM = fwd_bm<D>();
    constexpr int kThreads = 64 * fwd_waves<D>();
    const int n_qtiles = (a.Nq + kFwdBM - 1) / kFwdBM;
    const long long n_heads = (long long)a.B * a.H;
    const bool pair = CAUSAL && causal_pairs(n_heads, n_qtiles, (long long)a.dev.cus * fwd_min_blocks<D>());
    const long long G = n_heads * (pair ? (n_qtiles + 1) / 2 : n_qtiles);
    if (G == 0) return hipSuccess;
    const float c_log2 = a.scale * kLog2e;
    hipLaunchKernelGGL((fwd_kernel<D, CAUSAL, false>), dim3((unsigned)G), dim3(kThreads), 0, (hipStream_t)a.stream,
                       (const bf16 *)a.q, (const bf16 *)a.k, (const bf16 *)a.v, (bf16 *)a.o, a.lse, a.Nq, a.Nk,
                       a.H, a.H / a.Hk, n_qtiles, a.scale, c_log2, 1, 0, (float *)nullptr, (float *)nullptr, a.dev.nx,
                       (int)pair);
    return hipGetLastError();
}

// Merge of the split pieces of one row: lse = log sum_s exp(lse_s), O = sum_s exp(lse_s - lse) O_s
// (the merge rule of the running maxima and sums, applied to normalised pieces).  One wave per
// row; lane c holds columns c*D/64 .. c*D/64 + D/64 - 1.
template <int D>
__global__ __launch_bounds__(256) void fwd_combine_kernel(const float *__restrict__ OP, const float *__restrict__ LP,
                                                          bf16 *__restrict__ O, float *__restrict__ LSE, long long rows,
                                                          int n_splits)
{
    constexpr int E = D / 64;
    const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= rows) return;
    // the pieces' lse: lanes take pieces s = lane, lane + 64, ..., then a wave maximum
    float m = -__builtin_inff();
    for (int s = lane; s < n_splits; s += 64) m = fmaxf(m, LP[(size_t)s * rows + row]);
#pragma unroll
    for (int x = 32; x > 0; x >>= 1) m = fmaxf(m, __shfl_xor(m, x));
    float acc[E] = {};
    float wsum = 0.f;
    if (m != -__builtin_inff()) {
        // no branch on empty pieces (weight 0), so that the loads of several pieces are in flight
#pragma unroll 4
        for (int s = 0; s < n_splits; ++s) {
            const float ls = LP[(size_t)s * rows + row];
            const float wgt = (ls == -__builtin_inff()) ? 0.f : expf(ls - m);
            wsum += wgt;
            const float *op = OP + ((size_t)s * rows + row) * D + lane * E;
#pragma unroll
            for (int e = 0; e < E; ++e) acc[e] = fmaf(wgt, op[e], acc[e]);
        }
    }
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) O[row * D + lane * E + e] = (bf16)(acc[e] * inv);
    if (lane == 0) LSE[row] = wsum > 0.f ? m + logf(wsum) : -__builtin_inff();
}

// ------------------------------------------------------------ decoding (a query row or two per head)

// Split-key pieces for few query rows (Nq <= kDecRows), written in fwd_kernel<.., SPLIT>'s
// workspace layout for fwd_combine_kernel.  The G Nq rows that share a K/V head (grouped-query
// attention: the G query heads of the K/V head, Nq rows each) go to workgroups in groups of
// kDecRows, so that K and V are read once per group.  With one or two rows the score tile of the matrix instructions
// would be 1/32 or 1/16 useful, and the piece is bound by the rate at which K and V arrive; this
// kernel streams them straight into registers instead.  A key row is D/8 lanes of 16 bytes; a wave
// load covers 64 / (D/8) keys, each wave of the workgroup takes U loads of K and of V per tile,
// and the next tile's loads are in flight while a tile is worked on.  Per key: q.k over the
// lane's 8 elements with bf16 dot products in fp32, summed over the row's lanes by DPP adds;
// the running maximum and sum of the online softmax per lane (every lane of a key slot sees the
// same keys); O += p V in fp32.  At the end the key slots of a wave and then the four waves are
// merged by the same rule as the pieces ("GPU Programming and Kernel Optimization", item 57).
constexpr int kDecRows = 4;  // query rows per head up to which the decoding kernel is used; rows per workgroup
template <int D>
constexpr bool dec_supported() { return D == 64 || D == 128 || D == 256; }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// sum over the L lanes of an aligned group (L = 8, 16, 32), the result in every lane of the group
template <int L>
__device__ __forceinline__ float group_sum(float x)
{
    auto dpp_add = [](float v, auto CTRL) __attribute__((always_inline)) {
        constexpr int ctrl = decltype(CTRL)::value;
        return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), ctrl, 0xf, 0xf, false));
    };
    x = dpp_add(x, std::integral_constant<int, 0xB1>{});   // quad_perm [1,0,3,2]: lanes i ^ 1
    x = dpp_add(x, std::integral_constant<int, 0x4E>{});   // quad_perm [2,3,0,1]: lanes i ^ 2
    x = dpp_add(x, std::integral_constant<int, 0x141>{});  // row_half_mirror: quad pairs of 8
    if constexpr (L >= 16) x = dpp_add(x, std::integral_constant<int, 0x140>{});  // row_mirror: halves of 16
    if constexpr (L >= 32) x += __shfl_xor(x, 16);
    return x;
}

// unnormalised merge of (m, l, o) with another piece (m in exp2 units, -inf when empty)
__device__ __forceinline__ void merge_piece(float &m, float &l, float *o, float m2, float l2, const float *o2)
{
    const float mn = fmaxf(m, m2);
    const float a = (m == -__builtin_inff()) ? 0.f : fast_exp2(m - mn);
    const float b = (m2 == -__builtin_inff()) ? 0.f : fast_exp2(m2 - mn);
    l = l * a + l2 * b;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = o[e] * a + o2[e] * b;
    m = mn;
}

// NT: one row group per K/V head, so that every key and value is read by one workgroup alone:
// non-temporal loads (12-15% faster there; where several groups read a K/V head again from the
// caches they made that 39% slower).
template <int D, bool CAUSAL, int R, bool NT>
__global__ __launch_bounds__(256) void fwd_decode_kernel(const bf16 *__restrict__ Q, const bf16 *__restrict__ K,
                                                         const bf16 *__restrict__ V, float *__restrict__ OP,
                                                         float *__restrict__ LP, int Nq, int Nk, int H, int G,
                                                         int n_groups, int n_splits, int split_keys, float c_log2)
{
    constexpr int LPR = D / 8;       // lanes per key row
    constexpr int KPW = 64 / LPR;    // keys per wave load
    constexpr int U = 4;             // loads of K and of V per lane and tile
    constexpr int TK = 4 * U * KPW;  // keys per tile (four waves)
    const int item = (int)blockIdx.x / n_splits;  // (b * Hk + K/V head) * n_groups + row group
    const int split = (int)blockIdx.x - item * n_splits;
    const int kvh = item / n_groups;
    const int r0 = (item - kvh * n_groups) * R;  // first row of the group
    const int w = wave_uniform((int)threadIdx.x >> 6);
    const int lane = (int)threadIdx.x & 63;
    const int c = lane % LPR, slot = lane / LPR;
    const int Hk = H / G;
    const int head0 = (kvh / Hk) * H + (kvh % Hk) * G;  // b * H + first query head of the K/V head
    const size_t hoff_k = (size_t)kvh * (size_t)Nk * D;
    const int off = Nk - Nq;  // bottom-right causal alignment: row q sees keys j <= q + off
    const int nrows = G * Nq;  // row n of the K/V head: query head head0 + n / Nq, query n % Nq

    // the lane's 8 elements of each query row of the group (zeros for rows past nrows)
    bf16x2 q[R][4];
    {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const __amdgpu_buffer_rsrc_t rq = make_rsrc(Q + ((size_t)head0 * Nq + r0 + r) * D, r0 + r < nrows ? D * 2 : 0);
            const u32x4 v = buffer_load16(rq, (uint32_t)(8 * c) * 2u);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const unsigned vi = v[i];  // bit_cast of a vector element read element 0 here
                q[r][i] = __builtin_bit_cast(bf16x2, vi);
            }
        }
    }
    const long long k_lo_l = (long long)split * split_keys;
    const int k_lo = (int)(k_lo_l < Nk ? k_lo_l : Nk);
    const int k_hi = (int)(k_lo_l + split_keys < Nk ? k_lo_l + split_keys : Nk);
    const int n_tiles = (k_hi - k_lo + TK - 1) / TK;
    // last key each row sees
    int klast[R];
#pragma unroll
    for (int r = 0; r < R; ++r) klast[r] = CAUSAL ? min(k_hi - 1, (r0 + r) % Nq + off) : k_hi - 1;

    float m[R], l[R], o[R][8];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        m[r] = -__builtin_inff();
        l[r] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[r][e] = 0.f;
    }
    constexpr float thr = 8.0f;  // offset moves when a score exceeds it by 2^8 (as in fwd_kernel)

    u32x4 kb[2][U], vb[2][U];
    // tile t: keys k_lo + t TK + (w U + u) KPW + slot; keys past k_hi read as zeros and are masked
    auto load = [&](int t, auto BUF) __attribute__((always_inline)) {
        constexpr int b = decltype(BUF)::value;
        const int k0 = k_lo + t * TK;
        const uint32_t bytes = (uint32_t)min(k_hi - k0, TK) * D * 2;  // rows of this tile only
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(K + hoff_k + (size_t)k0 * D, bytes);
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(V + hoff_k + (size_t)k0 * D, bytes);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t byte = (uint32_t)(((w * U + u) * KPW + slot) * D + 8 * c) * 2u;
            kb[b][u] = __builtin_amdgcn_raw_buffer_load_b128(rk, (int)byte, 0, NT ? 2 : 0);
            vb[b][u] = __builtin_amdgcn_raw_buffer_load_b128(rv, (int)byte, 0, NT ? 2 : 0);
        }
    };
    auto work = [&](int t, auto BUF) __attribute__((always_inline)) {
        constexpr int b = decltype(BUF)::value;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int key = k_lo + t * TK + (w * U + u) * KPW + slot;
            float vf[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                vf[2 * i] = __builtin_bit_cast(float, vb[b][u][i] << 16);
                vf[2 * i + 1] = __builtin_bit_cast(float, vb[b][u][i] & 0xffff0000u);
            }
#pragma unroll
            for (int r = 0; r < R; ++r) {
                float s = 0.f;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const unsigned ki = kb[b][u][i];
                    s = __builtin_amdgcn_fdot2_f32_bf16(q[r][i], __builtin_bit_cast(bf16x2, ki), s, false);
                }
                s = group_sum<LPR>(s);
                s = (key <= klast[r]) ? s * c_log2 : -__builtin_inff();
                if (__builtin_amdgcn_ballot_w64(s > m[r] + thr)) {
                    const bool grow = s > m[r] + thr;
                    const float mn = grow ? s : m[r];
                    const float a = (grow && m[r] != -__builtin_inff()) ? fast_exp2(m[r] - mn) : (grow ? 0.f : 1.f);
                    l[r] *= a;
#pragma unroll
                    for (int e = 0; e < 8; ++e) o[r][e] *= a;
                    m[r] = mn;
                }
                const float p = fast_exp2(s - (m[r] == -__builtin_inff() ? 0.f : m[r]));
                l[r] += p;
#pragma unroll
                for (int e = 0; e < 8; ++e) o[r][e] = fmaf(p, vf[e], o[r][e]);
            }
        }
    };
    using B0 = std::integral_constant<int, 0>;
    using B1 = std::integral_constant<int, 1>;
    // two register buffers: the loads of tile t + 1 are in flight while tile t is worked on (the
    // compiler waits on each buffer's loads before their first use; loads complete in order)
    if (n_tiles > 0) load(0, B0{});
    int t = 0;
    for (; t + 1 < n_tiles; t += 2) {
        load(t + 1, B1{});
        work(t, B0{});
        if (t + 2 < n_tiles) load(t + 2, B0{});
        work(t + 1, B1{});
    }
    if (t < n_tiles) work(t, B0{});

    // merge the key slots of the wave (lanes c, c + LPR, ...), then the four waves through LDS
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
        for (int x = LPR; x < 64; x *= 2) {
            float o2[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) o2[e] = __shfl_xor(o[r][e], x);
            merge_piece(m[r], l[r], o[r], __shfl_xor(m[r], x), __shfl_xor(l[r], x), o2);
        }
    }
    __shared__ float red[4][R][D + 2];
    if (slot == 0) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
#pragma unroll
            for (int e = 0; e < 8; ++e) red[w][r][8 * c + e] = o[r][e];
            if (c == 0) {
                red[w][r][D] = m[r];
                red[w][r][D + 1] = l[r];
            }
        }
    }
    __syncthreads();
    if (w == 0 && slot == 0) {
        const int n_heads = (int)gridDim.x / (n_splits * n_groups) * G;  // B * H
#pragma unroll
        for (int r = 0; r < R; ++r) {
            if (r0 + r >= nrows) break;
            for (int ww = 1; ww < 4; ++ww) {
                float o2[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) o2[e] = red[ww][r][8 * c + e];
                merge_piece(m[r], l[r], o[r], red[ww][r][D], red[ww][r][D + 1], o2);
            }
            const size_t prow = ((size_t)split * n_heads + head0) * Nq + r0 + r;  // consecutive heads' rows are consecutive
            const float inv = l[r] > 0.f ? 1.f / l[r] : 0.f;
            f32x4 lo, hi;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                lo[e] = o[r][e] * inv;
                hi[e] = o[r][4 + e] * inv;
            }
            *(f32x4 *)(OP + prow * D + 8 * c) = lo;
            *(f32x4 *)(OP + prow * D + 8 * c + 4) = hi;
            // lse = ln(2^m l) = (m + log2 l) ln 2
            if (c == 0) LP[prow] = l[r] > 0.f ? (m[r] + __log2f(l[r])) * 0.69314718055994530942f : -__builtin_inff();
        }
    }
}

template <int D, bool CAUSAL>
hipError_t launch_fwd_split_t(const FwdArgs &a, int n_splits, float *op, float *lp)
{
    constexpr int kFwdBM = fwd_bm<D>();
    constexpr int kThreads = 64 * fwd_waves<D>();
    const int n_qtiles = (a.Nq + kFwdBM - 1) / kFwdBM;
    const long long G = (long long)a.B * a.H * n_qtiles * n_splits;
    if (G == 0) return hipSuccess;
    const int blocks = (a.Nk + kFwdBN - 1) / kFwdBN;
    const int split_blocks = (blocks + n_splits - 1) / n_splits;
    const float c_log2 = a.scale * kLog2e;
    if (dec_supported<D>() && a.Nq <= kDecRows) {
        const int rows_kv = (a.H / a.Hk) * a.Nq;  // query rows per K/V head
        const int n_groups = (rows_kv + kDecRows - 1) / kDecRows;
        const long long Gd = (long long)a.B * a.Hk * n_groups * n_splits;
        const int split_keys = split_blocks * kFwdBN;
        auto go = [&](auto RR, auto NT) {
            hipLaunchKernelGGL((fwd_decode_kernel<D, CAUSAL, decltype(RR)::value, decltype(NT)::value>), dim3((unsigned)Gd),
                               dim3(256), 0, (hipStream_t)a.stream, (const bf16 *)a.q, (const bf16 *)a.k,
                               (const bf16 *)a.v, op, lp, a.Nq, a.Nk, a.H, a.H / a.Hk, n_groups, n_splits, split_keys,
                               c_log2);
        };
        using R1 = std::integral_constant<int, 1>;
        using R2 = std::integral_constant<int, 2>;
        using R4 = std::integral_constant<int, 4>;
        static_assert(kDecRows == 4, "row counts 1, 2, 4");
        if (rows_kv == 1)
            go(R1{}, std::true_type{});
        else if (rows_kv == 2)
            go(R2{}, std::true_type{});
        else if (n_groups == 1)
            go(R4{}, std::true_type{});
        else
            go(R4{}, std::false_type{});
    } else {
        hipLaunchKernelGGL((fwd_kernel<D, CAUSAL, true>), dim3((unsigned)G), dim3(kThreads), 0, (hipStream_t)a.stream,
                           (const bf16 *)a.q, (const bf16 *)a.k, (const bf16 *)a.v, (bf16 *)a.o, a.lse, a.Nq, a.Nk,
                           a.H, a.H / a.Hk, n_qtiles, a.scale, c_log2, n_splits, split_blocks, op, lp, a.dev.nx, 0);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const long long rows = (long long)a.B * a.H * a.Nq;
    hipLaunchKernelGGL((fwd_combine_kernel<D>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, (hipStream_t)a.stream,
                       (const float *)op, (const float *)lp, (bf16 *)a.o, a.lse, rows, n_splits);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd(const FwdArgs &a)
{
    switch (a.d) {
    case 64: return a.causal ? launch_fwd_t<64, true>(a) : launch_fwd_t<64, false>(a);
    case 128: return a.causal ? launch_fwd_t<128, true>(a) : launch_fwd_t<128, false>(a);
    case 192: return a.causal ? launch_fwd_t<192, true>(a) : launch_fwd_t<192, false>(a);
    default: return a.causal ? launch_fwd_t<256, true>(a) : launch_fwd_t<256, false>(a);
    }
}

hipError_t launch_fwd_split(const FwdArgs &a, int n_splits, void *workspace)
{
    float *op = (float *)workspace;
    float *lp = op + (size_t)n_splits * a.B * a.H * a.Nq * a.d;
    switch (a.d) {
    case 64:
        return a.causal ? launch_fwd_split_t<64, true>(a, n_splits, op, lp) : launch_fwd_split_t<64, false>(a, n_splits, op, lp);
    case 128:
        return a.causal ? launch_fwd_split_t<128, true>(a, n_splits, op, lp) : launch_fwd_split_t<128, false>(a, n_splits, op, lp);
    case 192:
        return a.causal ? launch_fwd_split_t<192, true>(a, n_splits, op, lp) : launch_fwd_split_t<192, false>(a, n_splits, op, lp);
    default:
        return a.causal ? launch_fwd_split_t<256, true>(a, n_splits, op, lp) : launch_fwd_split_t<256, false>(a, n_splits, op, lp);
    }
}

long long fwd_split_workspace_bytes(int B, int H, int Nq, int d, int n_splits)
{
    // n_splits * B * H * Nq * (d + 1) * 4 bytes; -1 where that reaches 2^62
    long long r = 0;
    if (__builtin_mul_overflow((long long)B * H, (long long)Nq, &r) ||
        __builtin_mul_overflow(r, (long long)(d + 1) * 4 * n_splits, &r) || r >= (1LL << 62))
        return -1;
    return r;
}

long long fwd_split_grid_size(int B, int H, int Nq, int n_splits)
{
    return (long long)B * H * ((Nq + fwd_bm<64>() - 1) / fwd_bm<64>()) * n_splits;
}

int fwd_split_default(int B, int H, int Hk, int Nq, int Nk, int d)
{
    // Matrix-instruction pieces: about one workgroup per compute unit (one 8-wave workgroup already
    // fills a compute unit).  Decoding pieces (Nq <= kDecRows, 4-wave workgroups over row groups of
    // a K/V head): about 512 workgroups (measured flat from 256 to 1024 with one query head per K/V
    // head; grouped heads, with fewer items, needed 512).  At least two key blocks per piece.
    long long base, target;
    if ((d == 64 || d == 128 || d == 256) && Nq <= kDecRows && Hk > 0 && H % Hk == 0) {
        const long long rows_kv = (long long)(H / Hk) * Nq;
        base = (long long)B * Hk * ((rows_kv + kDecRows - 1) / kDecRows);
        target = 512;
    } else {
        const int bm = d == 128 ? fwd_bm<128>() : fwd_bm<64>();  // 128 rows for d = 64, 192 and 256
        base = (long long)B * H * ((Nq + bm - 1) / bm);
        target = 256;
    }
    const int blocks = (Nk + kFwdBN - 1) / kFwdBN;
    long long s = base > 0 ? (target + base - 1) / base : 1;
    s = s < blocks / 2 ? s : blocks / 2;
    s = s < 128 ? s : 128;
    return s < 1 ? 1 : (int)s;
}

long long fwd_grid_size(int B, int H, int Nq) { return (long long)B * H * ((Nq + fwd_bm<64>() - 1) / fwd_bm<64>()); }

}  // namespace attn
