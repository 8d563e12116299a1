// attn_fwd_fp8.hip -- fused tiled attention forward pass on 8-bit (e4m3) inputs, gfx950.
//
// Method: the same online-softmax forward as attn_fwd.hip ("digest_existing.txt", answer
// q02_flashattention, sections 1-2; "GPU Programming and Kernel Optimization", items 41,
// 57, 58, 60), on inputs stored as e4m3 codes with per-head scales.  FlashAttention v3
// takes FP8 inputs ("FlashAttention v3 (Tri Dao et al.)", section "What it is"; digest
// answer q03_fa3: about 1.2 PFLOP/s in FP8 on H100) and runs both products on 8-bit
// operands with fp32 results ("CUTLASS WGMMA Atom Skeleton", table "Atom Family Names Seen
// In CUTLASS").  A real input is scale * code value (item 33, affine quantisation with
// zero point 0).
//
// What differs from the 16-bit forward:
//   * both products use v_mfma_f32_32x32x64_f8f6f4 (e4m3 x e4m3 -> fp32, 64-deep
//     reduction, twice the 16-bit rate): S^T = K Q^T over d in steps of 64, and
//     O^T += V^T P^T over the 64 keys of a block in one instruction per 32 columns of O;
//   * the probabilities are rounded to e4m3 (nearest even) for the second product.  The
//     exponent offset keeps them at most 2^8, inside e4m3's range (largest 448); the
//     exp-sum l is accumulated from the unrounded fp32 values;
//   * the fp8 product pairs operand bytes by position: byte p of lane half h of A meets
//     byte p of lane half h of B, whatever the hardware's own order of the reduction.  So
//     S^T takes K and Q bytes in memory order, and for P V the 32 keys a lane half holds
//     in its score registers (keys 32(p/16) + 8((p%16)/4) + 4h + p%4 at byte p) are the
//     reduction order; V^T is gathered in that order with ds_read_b64_tr_b8;
//   * K and V blocks are 64 rows of d bytes in LDS with their own XOR swizzle.
//   * the scores carry the factor scale * descale_q * descale_k into the exponent, and the
//     output is multiplied by descale_v in the epilogue.
#include "attn_device.h"
#include "attn_launch.h"

#include <type_traits>

namespace attn {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

template <int D>
constexpr int f8_waves() { return D == 128 ? 8 : 4; }
template <int D>
constexpr int f8_bm() { return 32 * f8_waves<D>(); }
constexpr int kF8BN = 64;              // keys per streamed block
constexpr float kF8RescaleLog2 = 8.0f;  // probabilities stay <= 2^8 (e4m3 holds up to 448)

__device__ __forceinline__ f32x16 mfma8(i32x8 a, i32x8 b, f32x16 c)
{
    // formats 0 / 0: both operands e4m3; scale operands 0 select the unscaled instruction
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Swizzle of an LDS tile of 64 rows x D bytes: physical 16-byte chunk = chunk ^ swz8<D>(row).
// The masks (row bits 0..3) were chosen by exhaustive search on the CPU so that both reads
// of the kernel are free of bank conflicts (64 and 32 banks of 4 bytes): the 16-byte reads
// of one chunk by 32 consecutive rows (K), and the 8-byte transposing reads of 16 rows x 2
// chunks (V).
template <int D>
__device__ __forceinline__ int swz8(int r)
{
    static_assert(D == 64 || D == 128, "8-bit head dimension");
    constexpr int m0 = D == 64 ? 0 : 1, m1 = D == 64 ? 1 : 2, m2 = D == 64 ? 2 : 4, m3 = D == 64 ? 3 : 5;
    return ((r & 1) ? m0 : 0) ^ ((r & 2) ? m1 : 0) ^ ((r & 4) ? m2 : 0) ^ ((r & 8) ? m3 : 0);
}

template <int D>
__device__ __forceinline__ int swz8_off(int row, int chunk)
{
    return row * D + 16 * (chunk ^ swz8<D>(row));
}

__device__ __forceinline__ u32x4 lds_read_b128(const lds_char *base, int off)
{
    return *(const __attribute__((address_space(3))) u32x4 *)(base + off);
}

// ds_read_b64_tr_b8: within each group of 16 lanes, lane i receives byte i % 8 of the 8-byte
// chunks addressed by lanes 2e + i / 8 (e = 0..7) as its bytes e (measured on the GPU with an
// in-bounds probe).
__device__ __forceinline__ i32x2 lds_read_tr8(const lds_char *base, int off)
{
    return __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2 *)(base + off));
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(64 * f8_waves<D>(), 8 / f8_waves<D>()) void fwd_fp8_kernel(
    const uint8_t *__restrict__ Q, const uint8_t *__restrict__ K, const uint8_t *__restrict__ V,
    const float *__restrict__ DSQ, const float *__restrict__ DSK, const float *__restrict__ DSV, bf16 *__restrict__ O,
    float *__restrict__ LSE, int Nq, int Nk, int H, int G, int n_qtiles, float scale, int nx, int pair)
{
    constexpr int NW = f8_waves<D>();
    constexpr int BM = f8_bm<D>();
    constexpr int NK8 = D / 64;  // 64-deep reduction steps over d
    constexpr int NDB = D / 32;  // 32-wide column blocks of O
    constexpr int TILE = kF8BN * D;
    __shared__ __attribute__((aligned(16))) char k0_raw[TILE], k1_raw[TILE], v0_raw[TILE], v1_raw[TILE];

    // causal with `pair` set: workgroup `pos` takes query blocks T-1-pos and then pos (equal work per
    // workgroup); otherwise one query block per workgroup, causal ones longest first
    const int n_pos = pair ? (n_qtiles + 1) / 2 : n_qtiles;
    int head, pos;
    work_item(blockIdx.x, n_pos, nx, head, pos);

    const int tid = threadIdx.x;
    const int lane = tid & 63, h = lane >> 5, c32 = lane & 31;
    const int w = wave_uniform(tid >> 6);
    const int kvh = (head / H) * (H / G) + (head % H) / G;
    const size_t hoff = (size_t)head * (size_t)Nq * D;
    const size_t hoff_k = (size_t)kvh * (size_t)Nk * D;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(Q + hoff, (uint32_t)Nq * D);
    const int off = Nk - Nq;  // bottom-right causal alignment: query i sees keys j <= i + off

    // The lane's byte offsets inside a swizzled K/V tile, computed once and kept opaque: every LDS
    // read of the loop is one register plus a constant (stage, row block) in the instruction's
    // offset field, and every direct load one register plus a buffer base moved by scalar
    // arithmetic, so the step carries no address arithmetic on the vector units.
    constexpr int kLoadNI = kF8BN * (D / 16) / 64 / NW;  // direct loads per wave and tile
    int ko[NK8][2];   // K fragment of reduction step kst: row c32, chunks 4 kst + 2 h (+1)
    int vo[NDB];      // V^T fragment of column block db (key block 0 of each 16-key group)
    int go[kLoadNI];  // source of direct load i within a tile
    {
#pragma unroll
        for (int kst = 0; kst < NK8; ++kst) {
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                ko[kst][x] = swz8_off<D>(c32, 4 * kst + 2 * h + x);
                asm volatile("" : "+v"(ko[kst][x]));
            }
        }
        const int g = lane >> 4, e = (lane & 15) >> 1, o = lane & 1;
        const int klo = 8 * (e >> 2) + 4 * (g >> 1) + (e & 3);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            vo[db] = swz8_off<D>(klo, 2 * db + (g & 1)) + 8 * o;
            asm volatile("" : "+v"(vo[db]));
        }
#pragma unroll
        for (int i = 0; i < kLoadNI; ++i) {
            const int pchunk = 64 * (w * kLoadNI + i) + lane;
            const int row = pchunk / (D / 16);
            const int chunk = (pchunk - row * (D / 16)) ^ swz8<D>(row);
            go[i] = row * D + 16 * chunk;
            asm volatile("" : "+v"(go[i]));
        }
    }

    // real score per unit of the 8-bit dot product, and the exp2 factor
    const float s_raw = scale * DSQ[head] * DSK[kvh];
    const float c_log2 = s_raw * kLog2e;
    const float dsv = DSV[kvh];
    const float grow_thr = kF8RescaleLog2 / c_log2;

    for (int pass = 0; pass < ((CAUSAL && pair) ? 2 : 1); ++pass) {
        const int qtile = pass == 0 ? (CAUSAL ? n_qtiles - 1 - pos : pos) : pos;
        if (pass == 1 && qtile == n_qtiles - 1 - pos) break;  // odd T: the middle block is alone
        const int q0 = qtile * BM;
        const int qw0 = q0 + 32 * w;
        const int qrow = qw0 + c32;

        // B operand of S^T: lane (c, h) holds Q[qrow][64 kst + 32 h .. + 31] (zeros past Nq)
        i32x8 qf[NK8];
#pragma unroll
        for (int ks = 0; ks < NK8; ++ks) {
            const u32x4 lo = buffer_load16(rq, (uint32_t)(qrow * D + 64 * ks + 32 * h));
            const u32x4 hi = buffer_load16(rq, (uint32_t)(qrow * D + 64 * ks + 32 * h + 16));
            qf[ks] = __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }

        f32x16 oacc[NDB];
#pragma unroll
        for (int i = 0; i < NDB; ++i) oacc[i] = zero16();
        float m_run = -__builtin_inff();  // exponent offset (8-bit dot-product units)
        float msc = 0.f;                   // m_run * c_log2, 0 while m_run = -inf
        float l_run = 0.f;

        const int kv_end = CAUSAL ? min(Nk, max(0, q0 + BM + off)) : Nk;
        const int je = (kv_end + kF8BN - 1) / kF8BN;
        // A wave works on key blocks [0, ja) and only loads and waits on [ja, je): under the
        // causal mask the blocks past ja lie wholly above its rows.  Two loops with no branch on
        // j inside keep the score registers out of control flow.
        const int last_key = qw0 + 31 + off;  // last key some row of the wave sees (causal)
        const int ja = (qw0 >= Nq) ? 0 : (!CAUSAL ? je : (last_key < 0 ? 0 : min(je, last_key / kF8BN + 1)));

        auto kstage = [&](auto par) __attribute__((always_inline)) { return (lds_char *)(decltype(par)::value ? k1_raw : k0_raw); };
        auto vstage = [&](auto par) __attribute__((always_inline)) { return (lds_char *)(decltype(par)::value ? v1_raw : v0_raw); };
        // key rows [j * BN, j * BN + BN) of K or V into a stage.  Rows past the last block this
        // workgroup needs, and rows past Nk, read as zeros without touching memory.
        const int kv_lim = min(Nk, je * kF8BN);
        auto load_blk = [&](const uint8_t *src, lds_char *tile, int j) __attribute__((always_inline)) {
            const int r0 = min(j * kF8BN, kv_lim);
            const __amdgpu_buffer_rsrc_t rj = make_rsrc(src + hoff_k + (size_t)r0 * D, (uint32_t)(kv_lim - r0) * D);
#pragma unroll
            for (int i = 0; i < kLoadNI; ++i) buffer_load_lds16(rj, tile + 1024 * (w * kLoadNI + i), (uint32_t)go[i]);
        };
        auto load_k = [&](int j, auto par) __attribute__((always_inline)) { load_blk(K, kstage(par), j); };
        auto load_v = [&](int j, auto par) __attribute__((always_inline)) { load_blk(V, vstage(par), j); };
        // A operand of S^T = K Q^T for key rows 32 kb .. 32 kb + 31 and d bytes 64 kst .. 64 kst + 63:
        // lane (c, h) takes row 32 kb + c, bytes 64 kst + 32 h .. + 31.
        auto kfrag = [&](const lds_char *ks, int kb, int kst) __attribute__((always_inline)) {
            const u32x4 lo = lds_read_b128(ks, ko[kst][0] + 32 * kb * D);
            const u32x4 hi = lds_read_b128(ks, ko[kst][1] + 32 * kb * D);
            return __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        };
        // A operand of O^T += V^T P^T for columns 32 db .. 32 db + 31 of O: lane (c, h) takes byte
        // p = V[sigma_h(p)][32 db + c], sigma_h(p) = 32(p/16) + 8((p%16)/4) + 4h + p%4.  Read t
        // (bytes 8t .. 8t+7) is issued by source lane s = 16 g + 2 e + o at key 16 t + klo,
        // klo = 8(e/4) + 4(g/2) + e%4, bytes 32 db + 16 (g%2) + 8 o .. + 7 of that row.
        auto vfrag = [&](const lds_char *vs, int db) __attribute__((always_inline)) {
            i32x2 r[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) r[t] = lds_read_tr8(vs, vo[db] + 16 * t * D);
            return i32x8{r[0][0], r[0][1], r[1][0], r[1][1], r[2][0], r[2][1], r[3][0], r[3][1]};
        };

        auto local_max = [&](const f32x16 *sc) __attribute__((always_inline)) {
            float m = fmaxf(sc[0][0], sc[0][1]);
#pragma unroll
            for (int r = 2; r < 16; ++r) m = fmaxf(m, sc[0][r]);
#pragma unroll
            for (int r = 0; r < 16; ++r) m = fmaxf(m, sc[1][r]);
            return m;
        };
        float mloc = -__builtin_inff();

        using P0 = std::integral_constant<int, 0>;
        using P1 = std::integral_constant<int, 1>;
        load_k(0, P0{});
        load_v(0, P0{});
        load_k(1, P1{});
        wait_vmem();
        __syncthreads();
        f32x16 sa[2], sb[2];
        // P as e4m3, byte p = 16 kb + r of the lane's keys; every step rewrites all four bytes of
        // each word, so the conversions take the previous step's word as their untouched half and
        // need no cleared register
        int pw[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        if (ja > 0) {
            const lds_char *ks = kstage(P0{});
            sa[0] = zero16();
            sa[1] = zero16();
#pragma unroll
            for (int kst = 0; kst < NK8; ++kst) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) sa[kb] = mfma8(kfrag(ks, kb, kst), qf[kst], sa[kb]);
            }
            mloc = local_max(sa);
        }
        // the first step loads K of block 2 into K0's stage: every wave must be done reading it
        __syncthreads();

        auto step_idle = [&](int j, auto par) __attribute__((always_inline)) {
            using PN = std::integral_constant<int, 1 - decltype(par)::value>;
            load_k(j + 2, par);
            load_v(j + 1, PN{});
            wait_vmem();
            __syncthreads();
        };
        // LAST: the wave's last block; the scores of block j+1 are not computed.
        auto step = [&](int j, auto par, f32x16 *cur, f32x16 *nxt, auto LAST) __attribute__((always_inline)) {
            constexpr bool last = decltype(LAST)::value;
            using PN = std::integral_constant<int, 1 - decltype(par)::value>;
            {
                const int k0 = j * kF8BN;
                if ((CAUSAL && (k0 + kF8BN - 1 > qw0 + off)) || (k0 + kF8BN > Nk)) {
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
                // conditional rescaling, as in the 16-bit forward
                if (__builtin_amdgcn_ballot_w64(mloc > m_run + grow_thr)) {
                    const float mrow = fmaxf(mloc, __shfl_xor(mloc, 32));
                    const bool grow = mrow > m_run + grow_thr;
                    const float m_new = grow ? mrow : m_run;
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
                // One step is NC chunks of one matrix instruction and a slice of vector work:
                //   chunks [0, NS): scores of block j+1      | exponentials of block j -> e4m3 P
                //   chunks [NS, NC): P V of block j          | exp-sum of block j, maximum of j+1
                __builtin_amdgcn_s_setprio(1);
                constexpr int NS = 2 * NK8, NC = NS + NDB;
                const lds_char *ks = kstage(PN{});
                const lds_char *vs = vstage(par);
                auto fetch = [&](auto C) __attribute__((always_inline)) {
                    constexpr int c = decltype(C)::value;
                    if constexpr (c < NS) return kfrag(ks, c & 1, c >> 1);
                    else return vfrag(vs, c - NS);
                };
                if constexpr (!last) {
                    nxt[0] = zero16();
                    nxt[1] = zero16();
                }
                float rs = 0.f, mx = -__builtin_inff();
                constexpr int PF = 1;
                i32x8 fr[PF + 1];
                static_for<0, PF>([&](auto F) __attribute__((always_inline)) {
                    if constexpr (!(last && decltype(F)::value < NS)) fr[decltype(F)::value] = fetch(F);
                });
                static_for<0, NC>([&](auto C) __attribute__((always_inline)) {
                    constexpr int c = decltype(C)::value;
                    if constexpr (c + PF < NC && !(last && c + PF < NS))
                        fr[(c + PF) % (PF + 1)] = fetch(std::integral_constant<int, c + PF>{});
                    if constexpr (c < NS) {
                        if constexpr (!last) nxt[c & 1] = mfma8(fr[c % (PF + 1)], qf[c >> 1], nxt[c & 1]);
                    } else {
                        const i32x8 pb = i32x8{pw[0], pw[1], pw[2], pw[3], pw[4], pw[5], pw[6], pw[7]};
                        oacc[c - NS] = mfma8(fr[c % (PF + 1)], pb, oacc[c - NS]);
                    }
                    if constexpr (c == 0) load_k(j + 2, par);
                    if constexpr (c == 1) load_v(j + 1, PN{});
                    if constexpr (c < NS) {
                        // exponentials of words [8 c / NS, 8 (c + 1) / NS) of P (4 keys a word)
                        static_for<c * 8 / NS, (c + 1) * 8 / NS>([&](auto WW) __attribute__((always_inline)) {
                            constexpr int wd = decltype(WW)::value;
                            constexpr int kb = wd >> 2, r0 = 4 * (wd & 3);
                            float p[4];
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                p[i] = fast_exp2(fmaf(cur[kb][r0 + i], c_log2, -msc));
                                cur[kb][r0 + i] = p[i];
                            }
                            int x = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], pw[wd], false);
                            pw[wd] = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], x, true);
                        });
                    } else {
                        constexpr int i = c - NS;
                        static_for<i * 32 / NDB, (i + 1) * 32 / NDB>([&](auto RR) __attribute__((always_inline)) {
                            constexpr int r = decltype(RR)::value;
                            rs += cur[r >> 4][r & 15];
                        });
                        // keep each slice in its chunk: the sum and the maximum are only read after
                        // the step, and without a use here the compiler sinks them past the barrier
                        asm volatile("" : "+v"(rs));
                        if constexpr (i >= 1 && !last) {
                            // maximum of block j+1 once its scores are complete
                            static_for<(i - 1) * 32 / (NDB - 1), i * 32 / (NDB - 1)>([&](auto RR) __attribute__((always_inline)) {
                                constexpr int r = decltype(RR)::value;
                                mx = fmaxf(mx, nxt[r >> 4][r & 15]);
                            });
                            asm volatile("" : "+v"(mx));
                        }
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

        // an odd count of blocks ends with a LAST step
        int j = 0;
        for (; j + 1 < ja; j += 2) {
            step(j, P0{}, sa, sb, std::false_type{});
            step(j + 1, P1{}, sb, sa, std::false_type{});
        }
        if (j < ja) step(j++, P0{}, sa, sb, std::true_type{});
        if (j < je && (j & 1)) step_idle(j++, P1{});
        for (; j + 1 < je; j += 2) {
            step_idle(j, P0{});
            step_idle(j + 1, P1{});
        }
        if (j < je) step_idle(j, P0{});

        // epilogue: O = descale_v * acc / l (bf16, nearest even), lse = m * scale' + ln(l)
        const float l_tot = l_run + __shfl_xor(l_run, 32);
        if (qrow < Nq) {
            const float f = (l_tot > 0.f) ? dsv / l_tot : 0.f;
            bf16 *orow = O + hoff + (size_t)qrow * D;
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    bf16x4 ov;
#pragma unroll
                    for (int i = 0; i < 4; ++i) ov[i] = (bf16)(oacc[db][4 * g4 + i] * f);
                    *(bf16x4 *)(orow + 32 * db + 8 * g4 + 4 * h) = ov;
                }
            }
            if (h == 0)
                LSE[(size_t)head * Nq + qrow] = (l_tot > 0.f) ? fmaf(m_run, s_raw, __logf(l_tot)) : -__builtin_inff();
        }
    }
}

template <int D, bool CAUSAL>
hipError_t launch_fwd_fp8_t(const Fp8FwdArgs &a)
{
    constexpr int BM = f8_bm<D>();
    const int n_qtiles = (a.Nq + BM - 1) / BM;
    const long long n_heads = (long long)a.B * a.H;
    const bool pair = CAUSAL && causal_pairs(n_heads, n_qtiles, (long long)a.dev.cus * (8 / f8_waves<D>()));
    const long long G = n_heads * (pair ? (n_qtiles + 1) / 2 : n_qtiles);
    if (G == 0) return hipSuccess;
    hipLaunchKernelGGL((fwd_fp8_kernel<D, CAUSAL>), dim3((unsigned)G), dim3(64 * f8_waves<D>()), 0,
                       (hipStream_t)a.stream, (const uint8_t *)a.q, (const uint8_t *)a.k, (const uint8_t *)a.v,
                       a.descale_q, a.descale_k, a.descale_v, (bf16 *)a.o, a.lse, a.Nq, a.Nk, a.H, a.H / a.Hk,
                       n_qtiles, a.scale, a.dev.nx, (int)pair);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_fp8(const Fp8FwdArgs &a)
{
    if (a.d == 64) return a.causal ? launch_fwd_fp8_t<64, true>(a) : launch_fwd_fp8_t<64, false>(a);
    return a.causal ? launch_fwd_fp8_t<128, true>(a) : launch_fwd_fp8_t<128, false>(a);
}

}  // namespace attn
