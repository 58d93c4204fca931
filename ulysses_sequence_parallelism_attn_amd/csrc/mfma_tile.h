// mfma_tile.h -- gfx950 building blocks shared by the attention kernels:
// bf16 fragment types, the 32x32x16 bf16 MFMA, the register layouts of its
// operands, and the swizzled LDS tile with row-major and transposed reads.
//
// Layout facts used throughout (v_mfma_f32_32x32x16_bf16, wave64):
//  * A operand (32 x 16): lane l supplies row (l % 32) and 8 k-values chosen
//    by k-group kg = l / 32.
//  * B operand (16 x 32): lane l supplies column (l % 32) and the same 8
//    k-values of group kg.  Which 8 physical k's a slot holds is irrelevant as
//    long as A and B agree, so every contraction defines its own k order.
//  * C/D (32 x 32 fp32, 16 regs): lane l holds column (l % 32); register r
//    holds row 8*(r/4) + 4*(l/32) + (r%4).
//
// Row permutation: when a 32-row block is the A operand, lane row m loads
// source row kperm(m) = 16*(m/16) + 8*((m/4)%2) + 4*((m/8)%2) + (m%4).  Then C
// register r of lane group kg holds source row 16*(r/8) + 8*kg + (r%8): the 8
// registers r = 8h..8h+7 hold 8 CONSECUTIVE source rows, which is exactly a
// B-operand fragment (k = that row index) for the next contraction.
//
// LDS tiles are row-major [rows][D] bf16, addressed in 16-byte granules with
// an XOR swizzle chosen so that both access patterns below are free of bank
// conflicts on the 64 x 4-byte banks:
//  * row reads (ds_read_b128): 16 lanes read granule g of 16 distinct rows
//    that cover a full residue class mod 16;
//  * transposed reads (ds_read_b64_tr_b16): 32 lanes read 4 granules of 4
//    consecutive rows (4-aligned).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ul {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define UL_LDS __attribute__((address_space(3)))

__device__ __forceinline__ f32x16 mfma32x32x16(const bf16x8 &a, const bf16x8 &b, const f32x16 &c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 u) { return __builtin_bit_cast(bf16x8, u); }

__device__ __forceinline__ f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int r = 0; r < 16; ++r) z[r] = 0.f;
    return z;
}

// A-operand lane row m -> source row within a 32-row block.
__device__ __forceinline__ int kperm(int m) {
    return (m & 16) | ((m & 4) << 1) | ((m & 8) >> 1) | (m & 3);
}

// With kperm applied on the A side: C register r of lane group kg -> source row.
__device__ __forceinline__ int ckey(int r, int kg) { return ((r >> 3) << 4) | (kg << 3) | (r & 7); }

// Eight fp32 values -> one bf16x8 fragment (round to nearest even).
__device__ __forceinline__ bf16x8 pack8(const float *a) {
    bf16x8 r;
#pragma unroll
    for (int s = 0; s < 8; ++s) r[s] = (__bf16)a[s];
    return r;
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(((uint32_t)b) << 16);
}

// Combine a value with the one held by the lane 32 positions away (both
// halves of the wave get op(low, high)).  v_permlane32_swap exchanges the
// halves of two registers; fed the same value twice, its two results hold
// the low-half and the high-half value in every lane.
__device__ __forceinline__ float half_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ---------------------------------------------------------------- LDS tiles

// XOR applied to the granule index of row r (D = 128: 16 granules per
// 256-byte row; D = 64: 8 granules per 128-byte row, two rows per bank window).
template <int D>
__device__ __forceinline__ int swz(int r) {
    if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
    else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// Byte offset of granule g of row r.
template <int D>
__device__ __forceinline__ int tile_off(int r, int g) {
    return r * (D * 2) + ((g ^ swz<D>(r)) << 4);
}

// A/B fragment from a row: 8 consecutive elements starting at granule g of row r.
template <int D>
__device__ __forceinline__ bf16x8 row_frag(const UL_LDS unsigned char *tile, int r, int g) {
    const u32x4 v = *reinterpret_cast<const UL_LDS u32x4 *>(tile + tile_off<D>(r, g));
    return as_bf16x8(v);
}

typedef __bf16 v4bf16 __attribute__((__vector_size__(4 * sizeof(__bf16))));

// Transposed A-operand fragment: element s of lane l is
//   tile[r0 + 8*(l/32) + s][c0 + (l % 32)]       (s = 0..7)
// for r0 a multiple of 8 and c0 a multiple of 32.  Two ds_read_b64_tr_b16:
// within each 16-lane group, lane i receives element i%4 of the 4-element
// chunks addressed by lanes 4k + i/4 (k = 0..3), so lane j of the group
// addresses row 4*half + j/4 and columns 16*((l/16)%2) + 4*(j%4) .. +3.
template <int D>
struct TrAddr {
    int row_off;  // 8*kg + j/4
    int col_off;  // 16*((l/16)%2) + 4*(j%4)
    __device__ __forceinline__ explicit TrAddr(int lane) {
        const int j = lane & 15;
        row_off = ((lane >> 5) << 3) + (j >> 2);
        col_off = (((lane >> 4) & 1) << 4) + ((j & 3) << 2);
    }
};

template <int D>
__device__ __forceinline__ bf16x8 tr_frag(const UL_LDS unsigned char *tile, const TrAddr<D> &ta, int r0,
                                          int c0) {
    const int c = c0 + ta.col_off;
    const int g = c >> 3, within = (c & 7) << 1;
    const int ra = r0 + ta.row_off, rb = ra + 4;
    const v4bf16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (UL_LDS v4bf16 *)(tile + tile_off<D>(ra, g) + within));
    const v4bf16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (UL_LDS v4bf16 *)(tile + tile_off<D>(rb, g) + within));
    bf16x8 r;
    r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
    r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
    return r;
}

// ---------------------------------------------------------------- precomputed lane offsets
//
// Fragment addresses depend on the lane only through the XOR swizzle, so each
// kernel computes them once; inside the loops an address is then one of these
// registers plus a compile-time byte offset (the LDS stage, the tile within
// the stage, and a row block that is a multiple of 16 rows, which leaves the
// swizzle unchanged), which the ds_read instructions take as an immediate.

// Row read of granule g of row r (r's swizzle class is r & 15).
template <int D>
__device__ __forceinline__ uint32_t rm_off(int r, int g) { return (uint32_t)tile_off<D>(r, g); }

// The two halves of a transposed fragment at rows [8*kg + 4*half + j/4] and
// columns c0 + col_off (c0 a multiple of 32); rows advance in multiples of 16.
template <int D>
__device__ __forceinline__ uint32_t tr_off(const TrAddr<D> &ta, int c0, int half) {
    const int c = c0 + ta.col_off;
    const int r = ta.row_off + 4 * half;
    return (uint32_t)(tile_off<D>(r, c >> 3) + ((c & 7) << 1));
}

__device__ __forceinline__ bf16x8 lds_frag(const UL_LDS unsigned char *base, uint32_t off) {
    const u32x4 v = *reinterpret_cast<const UL_LDS u32x4 *>(base + off);
    return as_bf16x8(v);
}

__device__ __forceinline__ bf16x8 lds_tr_frag(const UL_LDS unsigned char *base, uint32_t off_lo,
                                              uint32_t off_hi) {
    const v4bf16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((UL_LDS v4bf16 *)(base + off_lo));
    const v4bf16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((UL_LDS v4bf16 *)(base + off_hi));
    bf16x8 r;
    r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
    r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
    return r;
}

// The same reads at absolute LDS byte addresses (a per-lane register plus a
// compile-time offset, which the ds_read takes as its immediate).
__device__ __forceinline__ bf16x8 lds_frag_at(uint32_t addr) {
    return as_bf16x8(*reinterpret_cast<const UL_LDS u32x4 *>((uintptr_t)addr));
}

__device__ __forceinline__ bf16x8 lds_tr_frag_at(uint32_t lo_addr, uint32_t hi_addr) {
    const v4bf16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((UL_LDS v4bf16 *)(uintptr_t)lo_addr);
    const v4bf16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((UL_LDS v4bf16 *)(uintptr_t)hi_addr);
    bf16x8 r;
    r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
    r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
    return r;
}

// Offsets of the two fragment kinds every attention kernel reads from a
// [rows][D] tile: row fragments of row kperm(m) (+ multiples of 32 rows) for
// k-step kk, and transposed fragments for column block eb (+ multiples of 16
// rows).
template <int D>
struct FragOffs {
    static constexpr int KK = D / 16, EB = D / 32;
    uint32_t rm[KK];
    uint32_t tr[EB][2];
    __device__ __forceinline__ explicit FragOffs(int lane) {
        const int m = lane & 31, kg = lane >> 5;
        const int prow = kperm(m);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) rm[kk] = rm_off<D>(prow, kk * 2 + kg);
        const TrAddr<D> ta(lane);
#pragma unroll
        for (int eb = 0; eb < EB; ++eb) {
            tr[eb][0] = tr_off<D>(ta, eb * 32, 0);
            tr[eb][1] = tr_off<D>(ta, eb * 32, 1);
        }
    }
};

// Cooperative tile staging: NT threads move ROWS x D bf16 between global
// memory (row stride `stride` elements) and a swizzled LDS tile, 16 bytes per
// lane per unit, consecutive lanes on consecutive granules of a row.  When the
// tile has fewer granules than threads, the surplus threads move nothing.
template <int D, int ROWS, int NT>
struct TileStage {
    static constexpr int GPR = D / 8;                          // granules per row
    static constexpr int TOTAL = ROWS * GPR;                   // granules per tile
    static constexpr int UNITS = (TOTAL + NT - 1) / NT;        // granules per thread
    static_assert(TOTAL % NT == 0 || TOTAL < NT, "tile must divide evenly among threads");
    u32x4 v[UNITS];

    // rows r0 + row >= nrows read as zeros
    __device__ __forceinline__ void load(const uint16_t *__restrict__ base, int64_t stride, int r0,
                                         int nrows, int tid) {
#pragma unroll
        for (int u = 0; u < UNITS; ++u) {
            const int idx = tid + u * NT;
            const int row = idx / GPR, g = idx % GPR;
            const int rr = r0 + row;
            v[u] = (idx < TOTAL && rr < nrows)
                       ? *reinterpret_cast<const u32x4 *>(base + (int64_t)rr * stride + g * 8)
                       : u32x4{0, 0, 0, 0};
        }
    }
    __device__ __forceinline__ void store(UL_LDS unsigned char *tile, int tid) const {
#pragma unroll
        for (int u = 0; u < UNITS; ++u) {
            const int idx = tid + u * NT;
            if (TOTAL % NT == 0 || idx < TOTAL)
                *reinterpret_cast<UL_LDS u32x4 *>(tile + tile_off<D>(idx / GPR, idx % GPR)) = v[u];
        }
    }
};

// ---------------------------------------------------------------- direct global -> LDS tiles
//
// global_load_lds_dwordx4 writes the 16 bytes of lane L at M0 + 16*L: one wave
// instruction fills 1 KB of LDS.  Wave instruction u of a tile covers bytes
// [1024u, 1024u + 1024) of the swizzled layout, so lane L fetches the granule
// the layout keeps at slot 64u + L.  Rows at or past `nrows` are read from row
// nrows - 1 instead (in bounds; the kernels mask those rows).
//
// The loads are issued from inline assembly so that the compiler does not
// treat them as LDS stores of unknown extent and wait for them before every
// LDS read; their completion is awaited explicitly (wait_vm_barrier) before
// the barrier that publishes a stage.  vmcnt retires loads in order, so the
// compiler's own waits for ordinary loads can only become more conservative.
__device__ __forceinline__ uint32_t lds_addr(const UL_LDS void *p) {
    return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)p);
}

// A pointer the whole wave agrees on, held in scalar registers.
template <typename T>
__device__ __forceinline__ const T *uniform_ptr(const T *p) {
    const uint64_t v = (uint64_t)(uintptr_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (const T *)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// Lane L copies 16 bytes from gbase + voff to LDS at M0 + 16 L, with M0 set by
// the compiler from `m0` (a wave-uniform LDS byte address); one wait state
// separates the M0 write from the load.
__device__ __forceinline__ void dma_b128_m0(const void *gbase, uint32_t voff, uint32_t m0) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(gbase), "{m0}"(m0) : "memory");
}
__device__ __forceinline__ void dma_b32_m0(const void *gbase, uint32_t voff, uint32_t m0) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(gbase), "{m0}"(m0) : "memory");
}

// Lane L copies 16 (or 4) bytes from gbase + voff to LDS at ldst + 16 L (4 L).
// gbase and ldst are wave-uniform; M0 (the LDS base of the transfer) is saved
// and restored around the instruction.
__device__ __forceinline__ void dma_b128(const void *gbase, uint32_t voff, const UL_LDS void *ldst) {
    uint32_t save;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
                 "global_load_lds_dwordx4 %2, %3\n\ts_mov_b32 m0, %0"
                 : "=&s"(save)
                 : "s"(lds_addr(ldst)), "v"(voff), "s"(uniform_ptr(gbase))
                 : "memory");
}

__device__ __forceinline__ void dma_b32(const void *gbase, uint32_t voff, const UL_LDS void *ldst) {
    uint32_t save;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
                 "global_load_lds_dword %2, %3\n\ts_mov_b32 m0, %0"
                 : "=&s"(save)
                 : "s"(lds_addr(ldst)), "v"(voff), "s"(uniform_ptr(gbase))
                 : "memory");
}

// Wave instruction u of a [ROWS][D] tile covers LDS bytes [1024u, 1024u + 1024)
// of the swizzled layout: lane L fetches the granule the layout keeps at slot
// 64u + L, i.e. row u*ROWS_PER_INSTR + L/GPR, granule (L % GPR) ^ swz(row).
template <int D, int ROWS>
struct DmaTile {
    static constexpr int ROWB = D * 2, GPR = D / 8;
    static constexpr int INSTR = ROWS * ROWB / 1024;     // wave instructions per tile
    static constexpr int ROWS_PER_INSTR = 1024 / ROWB;
    static_assert(ROWS * ROWB % 1024 == 0, "tile must be a whole number of KB");
    __device__ static __forceinline__ int row(int u, int lane) { return u * ROWS_PER_INSTR + lane / GPR; }
    __device__ static __forceinline__ uint32_t gran_bytes(int u, int lane) {
        return (uint32_t)(((lane % GPR) ^ swz<D>(row(u, lane))) * 16);
    }
};

// A workgroup barrier that the scheduler does not move work across.
__device__ __forceinline__ void fence_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// Wait until at most N of this wave's vector-memory operations are
// outstanding and all of its LDS operations are done, then meet the other
// waves (s_waitcnt encoding: vmcnt = {simm[15:14], simm[3:0]}, expcnt[6:4] = 7,
// lgkmcnt[11:8] = 0).
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 63, "vmcnt immediate (63 encodes no wait)");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70);
}

// The same wait on vector-memory operations only; LDS operations stay in
// flight (their results are waited for at their first use).
template <int N>
__device__ __forceinline__ void wait_vm_only() {
    static_assert(N >= 0 && N < 63, "vmcnt immediate (63 encodes no wait)");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xf00);
}

template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
    wait_vm<N>();
    asm volatile("s_barrier" ::: "memory");
}

}  // namespace ul
