// mfma_tile.h -- gfx950 building blocks for the attention kernels: bf16
// fragment types, the 32x32x16 bf16 MFMA, register/LDS layouts.
//
// Layout facts used throughout (v_mfma_f32_32x32x16_bf16, wave64):
//  * A operand (32 x 16): lane l supplies row  (l % 32) and 8 k-values chosen
//    by k-group kg = l / 32.
//  * B operand (16 x 32): lane l supplies column (l % 32) and the same 8
//    k-values of group kg.  Which 8 physical k's a slot holds is irrelevant as
//    long as A and B agree, so every contraction below defines its own k order.
//  * C/D (32 x 32 fp32, 16 regs): lane l holds column (l % 32); register r
//    holds row 8*(r/4) + 4*(l/32) + (r%4).
//
// Key permutation: when a 32-key tile is the A operand of S^T = K Q^T, lane
// row m loads key kperm(m) = 16*(m/16) + 8*((m/4)%2) + 4*((m/8)%2) + (m%4).
// Then C register r of lane group kg holds key 16*(r/8) + 8*kg + (r%8): the 8
// registers r = 8h..8h+7 hold 8 CONSECUTIVE keys, which is exactly a B-operand
// fragment (k = key) for the next contraction over keys.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ul {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x16 mfma32x32x16(const bf16x8 &a, const bf16x8 &b, const f32x16 &c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4 &u) { return __builtin_bit_cast(bf16x8, u); }
__device__ __forceinline__ u32x4 as_u32x4(const bf16x8 &b) { return __builtin_bit_cast(u32x4, b); }

// Row (A-operand row / C row) m -> key offset within a 32-key tile.
__device__ __forceinline__ int kperm(int m) {
    return (m & 16) | ((m & 4) << 1) | ((m & 8) >> 1) | (m & 3);
}

// C register r of lane group kg in a 32x32 tile -> row index.
__device__ __forceinline__ int crow(int r, int kg) { return ((r >> 2) << 3) | (kg << 2) | (r & 3); }

// With kperm applied on the A side: C register r of lane group kg -> key.
__device__ __forceinline__ int ckey(int r, int kg) { return ((r >> 3) << 4) | (kg << 3) | (r & 7); }

// Eight fp32 values -> one bf16x8 fragment (round to nearest even).
__device__ __forceinline__ bf16x8 pack8(float a0, float a1, float a2, float a3, float a4, float a5,
                                       float a6, float a7) {
    bf16x8 r;
    r[0] = (__bf16)a0; r[1] = (__bf16)a1; r[2] = (__bf16)a2; r[3] = (__bf16)a3;
    r[4] = (__bf16)a4; r[5] = (__bf16)a5; r[6] = (__bf16)a6; r[7] = (__bf16)a7;
    return r;
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(((uint32_t)b) << 16);
}

// ---------------------------------------------------------------------------
// LDS tiles.  Both layouts are addressed in 16-byte granules with an XOR
// swizzle so that the 16 lanes of a quarter-wave reading one granule column
// hit 16 distinct granule slots of a 256-byte bank window.
//
// Row-major tile [rows][D] bf16 (K or V rows as A operands, Q/dO rows):
//   granule G of row j lives at slot  j*(D/8) + (G ^ swz_rm(j)).
template <int D>
__device__ __forceinline__ int swz_rm(int row) {
    return D == 128 ? (row & 15) : ((row >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int rm_slot(int row, int gran) {
    return row * (D / 8) + (gran ^ swz_rm<D>(row));
}

// Transposed tile [D][KT] bf16 (V^T or K^T, KT keys per row, 16 <= KT*2/16):
// key granule KG (8 keys) of row e lives at slot  e*(KT/8) + (KG ^ swz_tr(e)).
template <int KT>
__device__ __forceinline__ int swz_tr(int e) {
    // KT = 64: 8 granules per 128-byte row, two rows per 256-byte window.
    return ((e >> 1) + (e >> 4)) & 7;
}
template <int KT>
__device__ __forceinline__ int tr_slot(int e, int kgran) {
    return e * (KT / 8) + (kgran ^ swz_tr<KT>(e));
}

}  // namespace ul
