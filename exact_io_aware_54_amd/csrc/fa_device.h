// Device-side building blocks for the gfx950 attention kernels: vector types,
// MFMA wrappers, wavefront reductions, conversions and the workgroup->tile map.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(_Float16)))) _Float16 f16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;
typedef __attribute__((__vector_size__(2 * sizeof(int)))) int i32x2;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Element type traits: the 8-wide operand vector of one 32x32x16 MFMA.
template <typename T> struct Vec;
template <> struct Vec<__bf16> { typedef bf16x8 x8; typedef bf16x4 x4; };
template <> struct Vec<_Float16> { typedef f16x8 x8; typedef f16x4 x4; };

// D = A * B + C on a 32x32 tile with K = 16 (bf16 / fp16 inputs, fp32 acc).
// Operand lane layout: lane l supplies row (A) or column (B) l % 32 and eight
// K values from half l / 32; the same (half, slot) pairs are contracted, so
// any K order is valid as long as A and B use the same one.
// Accumulator layout: lane l holds column l % 32, register r holds row
// 8 * (r / 4) + 4 * (l / 32) + r % 4.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(f16x8 a, f16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
// fp8 (OCP E4M3) x fp8 -> fp32, 32x32 tile, K = 64; 32 bytes per lane per
// operand. Format code 0 selects E4M3 for both operands; the E8M0 block
// scales are fixed at 127 (= 2^0).
__device__ __forceinline__ f32x16 mfma32_fp8(i32x8 a, i32x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// Row of the 32x32 accumulator held in register r by a lane of half `h`.
__device__ __forceinline__ int acc_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// Value of lane l ^ 32 (the other half of the wavefront) combined with max/+.
__device__ __forceinline__ float wave_half_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float wave_half_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Pack 8 floats from accumulator registers [base, base + 8) into one operand.
template <typename T>
__device__ __forceinline__ typename Vec<T>::x8 pack8(const f32x16& a, int base) {
    typename Vec<T>::x8 r;
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = (T)a[base + j];
    return r;
}

// Workgroups are dispatched round-robin over the 8 XCDs (each with its own
// L2). Remap the hardware id so that every XCD receives a contiguous range of
// logical ids; tiles that share K/V (same head) then share an L2.
__device__ __forceinline__ int xcd_remap(int id, int G) {
    const int per = (G + 7) >> 3;          // ids per XCD, rounded up
    const int tall = G - (per - 1) * 8;    // XCDs that receive `per` ids
    const int x = id & 7, loc = id >> 3;
    return x < tall ? x * per + loc : tall * per + (x - tall) * (per - 1) + loc;
}

// (head, query block) of causal block `id` (blockIdx.x). A causal query
// block's work grows with its index, so each XCD should run its longest
// blocks first and all XCDs should get the same total work. Block ids go to
// the eight XCDs in turn.
//  - BH a multiple of 8: xcd_remap hands every XCD BH/8 whole heads; within
//    an XCD the heads go in groups of G (at most gmax: 4, 2 or 1, dividing
//    BH/8), each group's query blocks longest first with its heads taken in
//    turn. Taking the long blocks of a few heads before the short ones leaves
//    no long block for the end of the launch, while the running blocks of an
//    XCD still read the K/V of only a few heads (fewer heads: fewer bytes
//    fetched past the XCD's L2, more imbalance at the end).
//  - otherwise the XCD ranges would split heads and one XCD would get the
//    long half of a head: the blocks are dealt instead, longest first over
//    all heads, block id k being the k-th longest, so XCD x gets every
//    eighth one.
__device__ __forceinline__ void causal_block(int id, int nqb, int BH, int& bh, int& qb,
                                             int gmax = 4) {
    if ((BH & 7) == 0) {
        const int L = xcd_remap(id, BH * nqb);
        const int hx = BH >> 3;  // heads per XCD
        const int G = ((hx & 3) == 0 && gmax >= 4) ? 4 : ((hx & 1) == 0 && gmax >= 2) ? 2 : 1;
        const int grp = L / (G * nqb), j = L - grp * G * nqb;
        bh = grp * G + j % G;
        qb = nqb - 1 - j / G;
    } else {
        bh = id % BH;
        qb = nqb - 1 - id / BH;
    }
}

// When a 32x32 accumulator is reused as an MFMA operand, registers r..r+7 of
// a lane in half h hold rows {4h..4h+3} and {8+4h..8+4h+3} of a 16-row group
// (see acc_row). The other operand, read from LDS as 8 contiguous elements at
// slot 8h, must present the same rows in the same order, so row w (0..15) of
// the group is stored at position acc_kperm16(w): groups of four rows go to
// positions 0, 8, 4, 12.
__device__ __forceinline__ int acc_kperm16(int kk) {
    const int g4 = kk >> 2, i = kk & 3;
    const int pos4 = (g4 == 1) ? 2 : (g4 == 2) ? 1 : g4;   // 0,2,1,3
    return pos4 * 4 + i;
}

// LDS layout of a row-major tile of 16-bit rows with D elements (D = 64 or
// 128) staged by global_load_lds: 16-byte chunk c of row r is stored at chunk
// position c ^ tile_swz<D>(r). The XOR pattern is chosen so that both read
// patterns used on these tiles touch every bank exactly once per pass:
//  * 16-byte row reads: 16 consecutive rows, one chunk each;
//  * ds_read_b64_tr_b16: 4 consecutive rows (first one a multiple of 4),
//    4 consecutive chunks each (chunk index a multiple of 4 first).
// D = 128 (one row per 256 bytes of banks): swap the two 2-bit halves of r%16.
// D = 256 (one row per 512 bytes): chunk c of every row falls on the banks of
// chunk c % 16, so the D = 128 pattern, applied to the low four bits of the
// chunk index, keeps both read patterns conflict-free.
// D = 64 (two rows per 256 bytes): g = (r/2)%8, rotate its 3 bits right by 1.
template <int D>
__device__ __forceinline__ int tile_swz(int r) {
    static_assert(D == 64 || D == 128 || D == 256, "head dim 64, 128 or 256");
    if constexpr (D >= 128) {
        return ((r & 3) << 2) | ((r >> 2) & 3);
    } else {
        const int g = (r >> 1) & 7;
        return ((g & 1) << 2) | (g >> 1);
    }
}

// Byte offset, inside such a tile, of element d (a multiple of 4 when used
// for transposing reads, of 8 for 16-byte reads) of row r.
template <int D>
__device__ __forceinline__ int tile_off(int r, int d) {
    return r * (2 * D) + 16 * ((d >> 3) ^ tile_swz<D>(r)) + 2 * (d & 7);
}

constexpr int kVmcntZero = 0x0F70;  // s_waitcnt vmcnt(0), expcnt/lgkmcnt untouched

// The streamed tiles (K/V in the forward passes and the dQ pass, Q/dO/LSE/D
// in the dK/dV pass) are double-buffered: the direct-to-LDS loads of tile i+1
// go into the second buffer set while tile i is computed on. A missing wait or
// barrier there would let a wave read a tile that is still landing, or let the
// next load overwrite one that a slower wave still reads. The race-guard build
// (FA_SERIAL_STAGING defined) keeps one buffer set and loads each tile only
// after every wave is done with the previous one and waits for it before any
// read: no overlap, so no race, and the same arithmetic in the same order. Its
// outputs must equal the product build's bit for bit.
#ifdef FA_SERIAL_STAGING
constexpr bool kSerialStaging = true;
#else
constexpr bool kSerialStaging = false;
#endif

}  // namespace fa
