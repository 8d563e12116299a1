// attn_device.h -- device-side building blocks shared by the gfx950 attention kernels.
//
// Matrix-core conventions (CDNA4, wave64).  All products use
// v_mfma_f32_32x32x16_bf16: C[32x32] += A[32x16] * B[16x32] with, for lane l
// (h = l / 32, c = l % 32):
//   A operand  : 8 bf16  A[c][8h + e],            e = 0..7
//   B operand  : 8 bf16  B[8h + e][c]
//   accumulator: 16 fp32 C[8(r/4) + 4h + r%4][c], r = 0..15
// A product whose reduction runs over a tile's rows (keys or queries) takes its
// reduction slot s = 8h + e to mean row 8(e/4) + 4h + e%4 of a 16-row group.
// With that choice, accumulator registers 8t'..8t'+7 (t' = 0, 1) of a 32-row
// block are exactly the B operand of the 16-row group t' of that block, so a
// probability or gradient tile computed in registers feeds the next product
// without any cross-lane movement.  The other operand of such a product is
// read from LDS with ds_read_b64_tr_b16 (a transposing LDS read), see
// lds_read_tr_rows below.
#pragma once

#include <hip/hip_runtime.h>
#include <type_traits>

#include "attn_sched.h"
#include <stdint.h>

namespace attn {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

constexpr float kLog2e = 1.44269504088896340736f;

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// The same instruction with its accumulator in VGPRs, c += a b.  In a kernel with up to 512
// registers per lane the compiler gives every matrix instruction AGPR accumulators; where the AGPRs
// all hold long-lived sums, a short chain whose result the vector units read then evicts some of
// those sums to VGPRs and back around every chain.  Written as assembly, the compiler's hazard
// recognizer does not see it, so the waits it would insert are explicit: two wait states before it
// for a vector write of a source just before (its loads are waited for by the compiler's counters,
// which do see the operands), and mfma_vgpr_settle after the chain, before any instruction reads or
// writes the accumulator.  Consecutive instructions of one chain (the same accumulator registers
// in full) need no wait states.
__device__ __forceinline__ void mfma_vgpr(f32x16 &c, bf16x8 a, bf16x8 b)
{
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
}

// c = a b (the accumulator starts from zero, an inline constant)
__device__ __forceinline__ void mfma_vgpr_zero(f32x16 &c, bf16x8 a, bf16x8 b)
{
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "v"(b));
}

// 20 wait states (the most that a 16-pass matrix instruction's VGPR result needs before a vector
// read or write), ordered after the chains that produce x and y and before any use of them
__device__ __forceinline__ void mfma_vgpr_settle(f32x16 &x, f32x16 &y)
{
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" : "+v"(x), "+v"(y));
}

// acc *= alpha for an accumulator that lives in AGPRs, element by element through one VGPR, so
// that the compiler has no reason to move the accumulator out of the AGPRs.  The reads of results
// of earlier matrix instructions and the writes before later ones are hazards the compiler cannot
// see here: agpr_settle before and after a run of these.
__device__ __forceinline__ void scale_agpr(f32x16 &acc, float alpha)
{
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        float x = acc[r], t;
        asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                     : "+a"(x), "=&v"(t)
                     : "v"(alpha));
        acc[r] = x;
    }
}

// 20 wait states
__device__ __forceinline__ void agpr_settle() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" ::: "memory"); }

__device__ __forceinline__ f32x16 zero16()
{
    f32x16 z;
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = 0.f;
    return z;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 16-byte LDS read at byte offset `off` of `base`.
__device__ __forceinline__ bf16x8 lds_read16(const lds_char *base, int off)
{
    return *(const __attribute__((address_space(3))) bf16x8 *)(base + off);
}

__device__ __forceinline__ void lds_write16(lds_char *base, int off, u32x4 v)
{
    *(__attribute__((address_space(3))) u32x4 *)(base + off) = v;
}

// ds_read_b64_tr_b16: within each group of 16 lanes, lane i receives element
// (i % 4) of the 8-byte chunks addressed by lanes 4e + i/4 (e = 0..3).
__device__ __forceinline__ bf16x4 lds_read_tr(const lds_char *base, int off)
{
    i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4 *)(base + off));
    return __builtin_bit_cast(bf16x4, r);
}

// A operand (32 columns x 16 reduction rows, transposed) for a product that
// reduces over rows r0 .. r0+15 of a row-major LDS tile of 16-bit elements with
// row stride `rs` bytes, taking columns c0 .. c0+31.  Lane l gets column
// c0 + l%32 at reduction slots 8h + e -> rows r0 + 8(e/4) + 4h + e%4.
// Each lane addresses, for its group G = l/16 and index s = l%16, row
// r0 + 4(G/2) + s/4 (and +8), columns c0 + 16(G%2) + 4(s%4) .. +3.
__device__ __forceinline__ bf16x8 lds_read_tr_rows(const lds_char *base, int rs, int r0, int c0, int lane)
{
    const int G = lane >> 4, s = lane & 15;
    const int row = r0 + 4 * (G >> 1) + (s >> 2);
    const int col = c0 + 16 * (G & 1) + 4 * (s & 3);
    const bf16x4 lo = lds_read_tr(base, row * rs + col * 2);
    const bf16x4 hi = lds_read_tr(base, (row + 8) * rs + col * 2);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Eight consecutive accumulator registers (8t' .. 8t'+7 of a 32x32 block),
// rounded to bf16 (nearest even): the B operand of a row-reduction product.
__device__ __forceinline__ bf16x8 pack_bf16(const f32x16 &acc, int half)
{
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = (bf16)acc[8 * half + e];
    return r;
}

// Calls f(std::integral_constant<int, I>{}) for I = B .. E-1 in order: loop bodies whose
// register indices must be compile-time constants.
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F &&f)
{
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// Work item of workgroup g in a grid of exactly n_heads * n_tiles workgroups, one item each, on a
// device of nx XCDs (the maps themselves are in attn_sched.h).
__device__ __forceinline__ void work_item(int g, int n_tiles, int nx, int &head, int &t)
{
    work_item_of(g, (int)gridDim.x, n_tiles, nx, head, t);
}

}  // namespace attn

namespace attn {

// Buffer resource over [base, base + bytes): loads beyond `bytes` return zeros,
// which gives ragged tiles their zero padding without branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, 0);
}

__device__ __forceinline__ int wave_uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

}  // namespace attn

namespace attn {

// Swizzled LDS tiles: rows of D bf16 (2*D bytes, no padding) whose 16-byte
// chunks are permuted per row, physical chunk = logical chunk ^ lds_swz<D>(row).
// The map XORs fixed chunk masks selected by the low four row bits; it keeps both
// access patterns of the kernels free of bank conflicts (64 banks of 4 bytes):
// 16-byte reads of one chunk column by 16 consecutive rows, and the transposing
// 8-byte reads of 4 consecutive rows x 4 consecutive chunks.  Only bits 0..3 of
// the row matter, so the map is linear over row blocks aligned to 16.  The masks
// stay below the number of chunks per row (for D = 192, 24 chunks, below 8, so
// that a chunk never leaves its group of 8).
template <int D>
__device__ __forceinline__ int lds_swz(int r)
{
    static_assert(D == 64 || D == 128 || D == 192 || D == 256, "head dimension");
    constexpr int m0 = D == 64 ? 2 : D == 128 ? 4 : D == 192 ? 0 : 4;
    constexpr int m1 = D == 64 ? 4 : D == 128 ? 10 : D == 192 ? 4 : 8;
    constexpr int m2 = 1, m3 = 2;
    return ((r & 1) ? m0 : 0) ^ ((r & 2) ? m1 : 0) ^ ((r & 4) ? m2 : 0) ^ ((r & 8) ? m3 : 0);
}

// Byte offset of logical 16-byte chunk `chunk` of row `row` in a swizzled tile.
template <int D>
__device__ __forceinline__ int swz_off(int row, int chunk)
{
    return row * (2 * D) + 16 * (chunk ^ lds_swz<D>(row));
}

// Direct global -> LDS load: every lane fetches 16 bytes at `byte_off` of the
// buffer and the wave writes its 64 x 16 bytes contiguously at `lds_dst`
// (lane i at lds_dst + 16 i).  Loads past the buffer end write zeros.
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t r, lds_char *lds_dst, uint32_t byte_off)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds_dst, 16, byte_off, 0,
                                             0, 0);
}

// Wait until this wave's vector-memory loads (including direct LDS loads) are done.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Wait until at most N of this wave's vector-memory loads (direct LDS loads included) are
// outstanding; loads complete in the order they were issued.
template <int N>
__device__ __forceinline__ void wait_vmem_upto()
{
    static_assert(N >= 0 && N < 16, "vmcnt field is 4 bits here");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier that first waits until at most N of this wave's vector-memory loads
// (direct LDS loads included) are outstanding and all its LDS accesses are done.  Unlike
// __syncthreads() it carries no release fence, which would wait for every load in flight;
// the "memory" clobber keeps the compiler from moving memory accesses across it.
template <int N>
__device__ __forceinline__ void barrier_wait_vmem_upto()
{
    static_assert(N >= 0 && N < 16, "vmcnt field is 4 bits here");
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Instruction i of the NI direct loads that wave `wave` issues to fill rows
// [row0, row0 + ROWS) of a row-major [*, D] bf16 matrix into a swizzled LDS tile.  The
// tile holds ROWS * D / 8 physical 16-byte chunks; wave instruction n = wave * NI + i
// writes physical chunks 64 n .. 64 n + 63 (1 KB, lane l at chunk 64 n + l), and each lane
// fetches the logical chunk that the swizzle puts there.
template <int D, int NW, int ROWS = 64>
__device__ __forceinline__ void load_tile_lds_part(__amdgpu_buffer_rsrc_t r, lds_char *tile, int row0, int wave,
                                                   int lane, int i)
{
    constexpr int RB = 2 * D;                   // bytes per row
    constexpr int CPR = D / 8;                  // 16-byte chunks per row
    constexpr int NI = ROWS * CPR / 64 / NW;    // instructions per wave for the tile
    static_assert(NI >= 1 && NI * 64 * NW == ROWS * CPR, "tile must split evenly over the waves");
    const int n = wave * NI + i;
    const int pchunk = 64 * n + lane;           // physical chunk of this lane
    const int row = pchunk / CPR;
    const int chunk = (pchunk - row * CPR) ^ lds_swz<D>(row);
    // byte offset in unsigned arithmetic: rows times row bytes reach 2^32 - 1 at the longest lengths
    buffer_load_lds16(r, tile + 1024 * n, (uint32_t)(row0 + row) * (uint32_t)RB + 16u * (uint32_t)chunk);
}

// Load rows [row0, row0 + ROWS) of a row-major [*, D] bf16 matrix into a swizzled
// LDS tile with direct loads; all NW waves of the workgroup take part.
template <int D, int NW, int ROWS = 64>
__device__ __forceinline__ void load_tile_lds(__amdgpu_buffer_rsrc_t r, lds_char *tile, int row0, int wave, int lane)
{
    constexpr int NI = ROWS * (D / 8) / 64 / NW;
#pragma unroll
    for (int i = 0; i < NI; ++i) load_tile_lds_part<D, NW, ROWS>(r, tile, row0, wave, lane, i);
}

// lds_read_tr_rows for a swizzled tile.
template <int D>
__device__ __forceinline__ bf16x8 lds_read_tr_rows_swz(const lds_char *base, int r0, int c0, int lane)
{
    const int G = lane >> 4, s = lane & 15;
    const int row = r0 + 4 * (G >> 1) + (s >> 2);
    const int byte = 2 * (c0 + 16 * (G & 1) + 4 * (s & 3));
    const bf16x4 lo = lds_read_tr(base, swz_off<D>(row, byte >> 4) + (byte & 15));
    const bf16x4 hi = lds_read_tr(base, swz_off<D>(row + 8, byte >> 4) + (byte & 15));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

}  // namespace attn
