// attn_bwd.hip -- backward of the per-rank attention (dQ, dK, dV).
//
// The pages train with this method ("Ulysses: entrenar con contextos de hasta
// 96K tokens en 4 GPUs", section "Que cambia en la practica de
// entrenamiento"), so the backward of the local attention step is on the hot
// path; they give no formula, so this is the plain gradient of L = <dO, O>:
//   p_ij = exp(s_ij - lse_i), dp_ij = dO_i . v_j, D_i = dO_i . o_i,
//   ds_ij = p_ij (dp_ij - D_i),
//   dq_i = scale sum_j ds_ij k_j,
//   dk_j = scale sum_{h in group, i} ds_ij q_i,  dv_j = sum_{h in group, i} p_ij dO_i.
//
// Three launches on the caller's stream, no atomics (bit-reproducible):
//  1. pre:   -lse/scale and -D = -rowsum(dO * O) -> workspace (fp32).  Both
//            are stored as the starting values of MFMA accumulators: S + (-lse
//            / scale) scaled by scale log2(e) is the exponent of P in base 2,
//            and dP + (-D) is what dS multiplies.
//  2. dq:    per (b, KV head, query block), like the forward: streams K/V
//            tiles, recomputes S^T = K Q^T and dP^T = V dO^T, forms dS^T and
//            accumulates dQ^T += K^T dS^T in registers.
//  3. dkdv:  per (b, KV head, key block): streams Q/dO tiles of every query
//            head of the group from the causal diagonal to N, recomputes
//            S = Q K^T and dP = dO V^T, accumulates dV^T += dO^T P and
//            dK^T += Q^T dS in registers (summed over the group's heads).
// dq and dkdv both recompute S and dP (4d extra FLOPs per visible pair over
// a fused kernel) in exchange for no dQ atomics and no shared accumulator.
//
// bf16 kernels use v_mfma_f32_32x32x16_bf16 with fp32 accumulation; P and dS
// are rounded to bf16 for the MFMA.  fp32 kernels are plain VALU loops (the
// exactness path).

#include <algorithm>
#include <utility>
#include <type_traits>

#include "mfma_tile.h"
#include "ul_internal.h"

namespace ul {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

// ============================================================================ pre kernel

// Workspace layout: for each (b, h), N floats of -lse/scale then N floats of
// -D, so both statistics of a query tile are one block apart.
struct PreParams {
    const void *o, *dout;
    const float *lse;
    float *stats;
    int64_t N;
    int64_t o_rs, do_rs;  // elements between consecutive tokens of o and of dout
    int32_t B, Hq, d;
    int32_t is_bf16;
    float scale;
};

// L lanes per (b, i, h) row, each with one 16-byte load of o and one of dout
// (8 bf16 or 4 fp32 elements): L = 16 / 8 for bf16 at d = 128 / 64, 32 / 16
// for fp32.  Rows are whole 16-byte granules (the head dim and every token
// stride are multiples of 16 bytes), so the loads are aligned.
template <bool BF16, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(PreParams p) {
    constexpr int EPL = BF16 ? 8 : 4;
    constexpr int L = D / EPL;
    constexpr int RPB = 256 / L;  // rows per workgroup
    const int64_t rows = (int64_t)p.B * p.N * p.Hq;
    const int64_t row = (int64_t)blockIdx.x * RPB + (threadIdx.x / L);
    const int sub = threadIdx.x % L;
    float acc = 0.f;
    if (row < rows) {
        // row = (b*N + i)*Hq + h
        const int64_t tok = row / p.Hq, col = (row % p.Hq) * D + sub * EPL;
        const int64_t ob = tok * p.o_rs + col, gb = tok * p.do_rs + col;
        if constexpr (BF16) {
            const u32x4 o = *reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(p.o) + ob);
            const u32x4 g = *reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(p.dout) + gb);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc = fmaf(bf16_to_f32((uint16_t)g[e]), bf16_to_f32((uint16_t)o[e]), acc);
                acc = fmaf(bf16_to_f32((uint16_t)(g[e] >> 16)), bf16_to_f32((uint16_t)(o[e] >> 16)), acc);
            }
        } else {
            const f32x4 o = *reinterpret_cast<const f32x4 *>(static_cast<const float *>(p.o) + ob);
            const f32x4 g = *reinterpret_cast<const f32x4 *>(static_cast<const float *>(p.dout) + gb);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc = fmaf(g[e], o[e], acc);
        }
    }
#pragma unroll
    for (int off = L / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, L);
    if (row < rows && sub == 0) {
        // row = (b*N + i)*Hq + h  ->  [b][h][i]
        const int64_t h = row % p.Hq;
        const int64_t bi = row / p.Hq;
        const int64_t i = bi % p.N, b = bi / p.N;
        const int64_t bh = b * p.Hq + h;
        p.stats[(2 * bh) * p.N + i] = -(p.lse[bh * p.N + i] / p.scale);
        p.stats[(2 * bh + 1) * p.N + i] = -acc;
    }
}

// ============================================================================ bf16: dQ kernel
//
// Geometry as the forward: 8 waves (2 per SIMD), 32 query rows per wave; the
// waves of a workgroup are the GQA group's query heads at the same positions,
// so each K/V tile staged in LDS serves all of them.  Per 32-key tile:
//   S^T  = K Q^T       (A = K rows, B = Q^T fragments in registers)
//   dP^T = V dO^T      (A = V rows, B = dO^T fragments in registers)
//   dS^T = P^T (dP^T - D),  P^T = exp2(S^T c - lse2)
//   dQ^T += K^T dS^T   (A = K^T by transposed LDS reads, B = dS^T fragments)
// As in the forward, the two waves of a SIMD run half a tile apart: one
// issues the 24 MFMAs of its tile (dQ of the previous tile, then S and dP of
// this one) while the other forms dS.  K/V tiles go straight from global
// memory into an 8-stage LDS ring, 6 tiles ahead of use.  (32-key tiles keep
// S and dP of a tile, the dQ accumulator and the Q^T / dO^T fragments within
// the 256 registers of a wave at 2 waves per SIMD.)

constexpr int kQWaves = 8;
constexpr int kQThreads = kQWaves * 64;
constexpr int kRowsPerWave = 32;
constexpr int kDqKT = 32;   // keys per tile
// A fragments read ahead of their MFMA: 4, and no more than the dQ steps of
// a tile, since the prefetch at the end of the softmax half covers only those.
// (6 ahead measured the same for the standalone kernel at N = 65536, but it
// left the kernel holding both backward passes at 256 registers with 49
// spilled; 4 removes the spills and took 9 % off that kernel at N = 8192.)
template <int D>
constexpr int kQAhead = 2 * (D / 32) < 4 ? 2 * (D / 32) : 4;

struct DqParams {
    const uint16_t *q, *k, *v, *dout;
    const float *stats;
    uint16_t *dq;
    int64_t q_rs, k_rs, v_rs, do_rs, dq_rs;  // elements between consecutive tokens of each tensor
    const int32_t *cu_seqlens;  // packed variable-length sequences, or nullptr
    int64_t total;              // tokens of the packed sequences
    int32_t N, B, Hq, Hkv;      // N: tokens per sequence (the longest one if packed)
    int32_t heads_per_wg, pos_blocks, head_groups, n_qblk;
    float scale_log2, scale;
    int32_t causal;
};

template <int D>
struct DqTile {
    static constexpr int kBytes = kDqKT * D * 2;      // one K or V tile
    static constexpr int kStages = 8;                 // LDS ring of tiles
    static constexpr int kAhead = kStages - 2;        // tiles loaded ahead of use
    // K tiles of every stage, then the V tiles: offsets from the start of
    // either region stay below 64 KB and fit an LDS read's immediate.
    static constexpr int kVBase = kStages * kBytes;
    static constexpr int kLds = 2 * kStages * kBytes;  // 128 KB at D = 128
    static_assert(kVBase <= 65536, "stage offsets must fit an LDS immediate");
    __device__ static constexpr int k_stage(int st) { return st * kBytes; }
};

// Absolute LDS addresses of this lane's fragments: K and V rows for S and dP,
// K^T halves for dQ (the LDS base and the V region already added).
template <int D>
struct DqOffs {
    static constexpr int KK = D / 16, EB = D / 32;
    uint32_t k[KK], v[KK], tr[EB][2];
};

// The MFMA half of a tile as one stream of A fragments from LDS:
//   DQ steps   dQ^T += K^T dS^T of the previous tile (its K tile at `pstage`,
//              B = its two dS^T fragments), 2 x EB steps;
//   SDP steps  S^T = K Q^T and dP^T = V dO^T of this tile (tiles at
//              `cstage`), alternating per k-step.
// With DQ the first kQAhead<D> fragments are already in `ring` (dq_prefetch).
// dP^T starts from `nd` (-D of the lane's query row in every register), so the
// stream leaves dP^T - D in `dp`.
template <int D, bool DQ, bool SDP>
__device__ __forceinline__ void dq_gemm(f32x16 *dqacc, const bf16x8 (&dsf)[2], f32x16 &s, f32x16 &dp, const f32x16 &nd,
                                        const bf16x8 *qf, const bf16x8 *dof, bf16x8 (&ring)[kQAhead<D>],
                                        uint32_t pstage, uint32_t cstage, const DqOffs<D> &o) {
    constexpr int EB = D / 32, KK = D / 16;
    constexpr int NDQ = DQ ? 2 * EB : 0, NSD = SDP ? 2 * KK : 0, NSTEP = NDQ + NSD;
    static_assert(!DQ || NDQ >= kQAhead<D>, "the prefetched ring holds dQ steps only");
    auto frag = [&](int st) -> bf16x8 {
        if (st < NDQ) {
            const uint32_t at = pstage + (st / EB) * 16 * D * 2;
            return lds_tr_frag_at(o.tr[st % EB][0] + at, o.tr[st % EB][1] + at);
        }
        const int x = st - NDQ, kk = x / 2;
        return lds_frag_at((x % 2 == 0 ? o.k[kk] : o.v[kk]) + cstage);
    };
    if constexpr (SDP) {
        s = zero16();
        dp = nd;
    }
    if constexpr (!DQ) {
#pragma unroll
        for (int i = 0; i < kQAhead<D>; ++i)
            if (i < NSTEP) ring[i] = frag(i);
    }
#pragma unroll
    for (int st = 0; st < NSTEP; ++st) {
        const bf16x8 a = ring[st % kQAhead<D>];
        if (st + kQAhead<D> < NSTEP) ring[st % kQAhead<D>] = frag(st + kQAhead<D>);
        if (st < NDQ) {
            const int kap = st / EB, eb = st % EB;
            dqacc[eb] = mfma32x32x16(a, dsf[kap], dqacc[eb]);
        } else {
            const int x = st - NDQ, kk = x / 2;
            if (x % 2 == 0)
                s = mfma32x32x16(a, qf[kk], s);
            else
                dp = mfma32x32x16(a, dof[kk], dp);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

// The first kQAhead<D> A fragments of the DQ steps for the K tile at `stage`.
template <int D>
__device__ __forceinline__ void dq_prefetch(bf16x8 (&ring)[kQAhead<D>], uint32_t stage, const DqOffs<D> &o) {
    constexpr int EB = D / 32;
#pragma unroll
    for (int st = 0; st < kQAhead<D>; ++st) {
        const uint32_t at = stage + (st / EB) * 16 * D * 2;
        ring[st] = lds_tr_frag_at(o.tr[st % EB][0] + at, o.tr[st % EB][1] + at);
    }
}

// dS^T = P^T (dP^T - D) with P^T = exp2(S^T c + cn), cn = -(lse/scale) c =
// -lse log2(e), as two bf16 B fragments of 16 keys; `dpd` already holds
// dP^T - D (dq_gemm).  MASK zeroes P past the causal diagonal and the ragged
// end.
template <bool MASK>
__device__ __forceinline__ void dq_ds(bf16x8 (&dsf)[2], const f32x16 &s, const f32x16 &dpd, float cn,
                                      int kg, int j0, int row, int N, int causal, float c) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        float ds[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int r = hh * 8 + q;
            float pv = __builtin_amdgcn_exp2f(fmaf(s[r], c, cn));
            if constexpr (MASK) {
                const int j = j0 + ckey(r, kg);
                if (j >= N || (causal && j > row)) pv = 0.f;
            }
            ds[q] = pv * dpd[r];
        }
        dsf[hh] = pack8(ds);
    }
    // keep the exponentials here rather than sunk into the next MFMA half
#pragma unroll
    for (int i = 0; i < 2; ++i) asm volatile("" : "+v"(dsf[i]));
}

template <int D>
__device__ __forceinline__ void dq_body(const DqParams &p, const int item) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    UL_LDS unsigned char *lds = (UL_LDS unsigned char *)smem_raw;
    using T = DqTile<D>;
    using Tile = DmaTile<D, kDqKT>;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int m = lane & 31, kg = lane >> 5;

    const int per_rank = p.B * p.Hkv * p.head_groups;
    const int rank = item / per_rank;
    int rest = item - rank * per_rank;
    const int g = rest % p.Hkv;
    rest /= p.Hkv;
    const int hg = rest % p.head_groups;
    const int b = rest / p.head_groups;
    const int qblk = p.causal ? (p.n_qblk - 1 - rank) : rank;
    const int grp = p.Hq / p.Hkv;
    const int h = g * grp + hg * p.heads_per_wg + (wave % p.heads_per_wg);
    const int wg_rows = kRowsPerWave * p.pos_blocks;
    const int wg_pos0 = qblk * wg_rows;
    const int i0 = wg_pos0 + (wave / p.heads_per_wg) * kRowsPerWave;
    const SeqRange sq = seq_range(p.cu_seqlens, b, p.N, p.Hq, p.total);
    const int N = sq.len;
    const int row = i0 + m;
    if (wg_pos0 >= N) return;  // past the end of a shorter packed sequence
    const int64_t q_rs = p.q_rs, do_rs = p.do_rs;
    const uint16_t *qb = p.q + sq.tok0 * q_rs + (int64_t)h * D;
    const uint16_t *dob = p.dout + sq.tok0 * do_rs + (int64_t)h * D;

    constexpr int KK = D / 16, EB = D / 32;
    bf16x8 qf[KK], dof[KK];
    const bool ok = row < N;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
        qf[kk] = as_bf16x8(ok ? *reinterpret_cast<const u32x4 *>(qb + row * q_rs + kk * 16 + kg * 8)
                              : u32x4{0, 0, 0, 0});
        dof[kk] = as_bf16x8(ok ? *reinterpret_cast<const u32x4 *>(dob + row * do_rs + kk * 16 + kg * 8)
                               : u32x4{0, 0, 0, 0});
    }
    const int64_t so = sq.st0 + (int64_t)h * 2 * sq.hs + (ok ? row : 0);
    const float cn = ok ? p.stats[so] * p.scale_log2 : 0.f;  // -lse log2(e)
    const float nDrow = ok ? p.stats[so + sq.hs] : 0.f;     // -D

    f32x16 dqacc[EB];
#pragma unroll
    for (int eb = 0; eb < EB; ++eb) dqacc[eb] = zero16();

    const int kend = p.causal ? min(N, wg_pos0 + wg_rows) : N;
    const int ntiles = (kend + kDqKT - 1) / kDqKT;
    const int n_full = p.causal ? min(wg_pos0, N) / kDqKT : N / kDqKT;
    const float c = p.scale_log2;

    // Absolute LDS addresses; the empty asm keeps the compiler from splitting
    // the sums again into out-of-range immediates.
    DqOffs<D> fo;
    {
        const FragOffs<D> f(lane);
        const uint32_t base = (uint32_t)(uintptr_t)lds;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            fo.k[kk] = f.rm[kk] + base;
            fo.v[kk] = f.rm[kk] + base + T::kVBase;
            asm volatile("" : "+v"(fo.k[kk]));
            asm volatile("" : "+v"(fo.v[kk]));
        }
#pragma unroll
        for (int e = 0; e < EB; ++e)
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                fo.tr[e][x] = f.tr[e][x] + base;
                asm volatile("" : "+v"(fo.tr[e][x]));
            }
    }

    // Direct loads of tile t into its LDS stage: the K and V tiles are split
    // evenly over the 8 waves.  Keys past N re-read key N-1 (their P is 0).
    constexpr int kDmaPerWave = 2 * Tile::INSTR / kQWaves;
    static_assert(2 * Tile::INSTR % kQWaves == 0 && Tile::INSTR % kDmaPerWave == 0,
                  "K and V tiles split evenly over the waves");
    static_assert((T::kAhead - 1) * kDmaPerWave < 16, "vmcnt immediate");
    const bool loads_v = wave * kDmaPerWave >= Tile::INSTR;
    const int u0 = (wave * kDmaPerWave) % Tile::INSTR;
    const int64_t t_rs = loads_v ? p.v_rs : p.k_rs;
    const uint16_t *tens = (loads_v ? p.v : p.k) + sq.tok0 * t_rs + (int64_t)g * D;
    const int tile_lds = loads_v ? T::kVBase : 0;
    const uint32_t row_bytes = (uint32_t)t_rs * 2;
    uint32_t dma_roff[kDmaPerWave], dma_gran[kDmaPerWave];
#pragma unroll
    for (int k = 0; k < kDmaPerWave; ++k) {
        dma_roff[k] = (uint32_t)Tile::row(u0 + k, lane) * row_bytes;
        dma_gran[k] = Tile::gran_bytes(u0 + k, lane);
    }
    // The tile the next loads fetch, set up by dma_prep one body ahead: the
    // address of its first key row (wave-uniform) and the byte offset of its
    // last row inside N, so that a load is a clamp, an add and the M0 write.
    // The loads run at the end of the dS half, off the MFMA stream (the dS
    // half is the shorter one): issued between the MFMAs they cost the
    // kernel 2.8 % of its time at N = 65536.
    const uint32_t dma_lds = (uint32_t)(uintptr_t)lds + tile_lds + u0 * 1024;
    const uint16_t *dma_tb = tens;
    uint32_t dma_lim = 0;
    auto dma_prep = [&](int t) {
        const int j0 = t * kDqKT;
        dma_tb = uniform_ptr(tens + (int64_t)j0 * t_rs);
        dma_lim = (uint32_t)max(min(N - 1 - j0, kDqKT), 0) * row_bytes;  // last key of the sequence
    };
    // load k of this wave's share of the prepared tile into the stage at byte offset `st`
    auto issue_k = [&](int k, uint32_t st) {
        dma_b128_m0(dma_tb, min(dma_roff[k], dma_lim) + dma_gran[k], dma_lds + st + k * 1024);
    };
    auto issue = [&](uint32_t st) {
#pragma unroll
        for (int k = 0; k < kDmaPerWave; ++k) issue_k(k, st);
    };
    auto visible = [&](int t) { return !p.causal || t * kDqKT <= i0 + kRowsPerWave - 1; };

    // The forward's schedule with a deeper ring: waves 4-7 run one barrier
    // behind waves 0-3; tile t sits in stage t % 8 from its load (in the dS
    // half of tile t-6) to the lagging group's dQ of it (MFMA half of tile
    // t+1); each wave waits for its share of tile t+1 before the barrier
    // ending its MFMA half of tile t (all but the 4 newest tiles' loads: its
    // own loads of this body come after that wait).
    const bool lagging = wave >= kQWaves / 2;
    // The Q/dO/statistics loads above stay in flight while the first tiles'
    // loads are issued: loads retire in order, so the wait for tile 0 retires
    // them too, and every later wait (at most k of the newest loads
    // outstanding) still counts only tile loads.
    for (int t = 0; t < T::kAhead; ++t)
        if (t < ntiles) {
            dma_prep(t);
            issue(T::k_stage(t));
        }
    f32x16 nd;  // the dP^T accumulator's starting value
#pragma unroll
    for (int r = 0; r < 16; ++r) nd[r] = nDrow;
    if (ntiles >= T::kAhead)
        wait_vm_barrier<(T::kAhead - 1) * kDmaPerWave>();
    else
        wait_vm_barrier<0>();
    dma_prep(T::kAhead);
    if (lagging) fence_barrier();

    f32x16 s, dp;
    bf16x8 dsf[2];
    bf16x8 ring[kQAhead<D>];
    auto body = [&](int t, auto full, auto stage, uint32_t stage_next) {  // stage_next: tile t+kAhead's
        constexpr bool FULL = decltype(full)::value;
        const bool more = t + T::kAhead < ntiles;
        // The wave feeding the MFMA pipe takes issue priority over the other
        // wave of its SIMD (busy with its dS) until its half ends.
        __builtin_amdgcn_s_setprio(2);
        if constexpr (FULL) {
            dq_gemm<D, true, true>(dqacc, dsf, s, dp, nd, qf, dof, ring, stage(t - 1), stage(t), fo);
        } else {
            if (t >= 1 && visible(t - 1))
                dq_gemm<D, true, false>(dqacc, dsf, s, dp, nd, qf, dof, ring, stage(t - 1), 0, fo);
            if (t < ntiles && visible(t))
                dq_gemm<D, false, true>(dqacc, dsf, s, dp, nd, qf, dof, ring, 0, stage(t), fo);
        }
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(0);
        if (more)
            wait_vm_barrier<(T::kAhead - 2) * kDmaPerWave>();
        else
            wait_vm_barrier<0>();
        __builtin_amdgcn_sched_barrier(0);
        if (FULL || (t < ntiles && visible(t))) {
            if constexpr (FULL)
                dq_ds<false>(dsf, s, dp, cn, kg, t * kDqKT, row, N, p.causal, c);
            else
                dq_ds<true>(dsf, s, dp, cn, kg, t * kDqKT, row, N, p.causal, c);
            dq_prefetch<D>(ring, stage(t), fo);
        }
        if (more) issue(stage_next);
        dma_prep(t + T::kAhead + 1);  // the tile the next body loads
        fence_barrier();
    };
    auto rt_stage = [](int x) { return (uint32_t)T::k_stage(x & (T::kStages - 1)); };
    body(0, std::false_type{}, rt_stage, rt_stage(T::kAhead));
    // The unmasked tiles 1 .. n_full-1 on the unrolled path: whole groups of
    // kStages in a straight loop, then one group that stops at n_full.  Every
    // group starts at a tile that is 1 modulo the stage count, so each of its
    // stage offsets is a constant.  The run-time-stage path below costs about
    // twice as much per tile (2.0 against 1.1 us at N = 65536), and a test
    // after every tile inside the main loop slows it by 1.5-3 %.
    int t0 = 1;
    for (; t0 + T::kStages <= n_full; t0 += T::kStages) {
        [&]<int... J>(std::integer_sequence<int, J...>) {
            // x - t0 + 1 folds to a constant for every tile index body derives from t0 + J
            (body(t0 + J, std::true_type{},
                  [t0](int x) { return (uint32_t)T::k_stage((x - t0 + 1) & (T::kStages - 1)); },
                  (uint32_t)T::k_stage((J + 1 + T::kAhead) & (T::kStages - 1))),
             ...);
        }(std::make_integer_sequence<int, T::kStages>{});
    }
    if (t0 < n_full) {
        [&]<int... J>(std::integer_sequence<int, J...>) {
            (void)((t0 + J < n_full &&
                    (body(t0 + J, std::true_type{},
                          [t0](int x) { return (uint32_t)T::k_stage((x - t0 + 1) & (T::kStages - 1)); },
                          (uint32_t)T::k_stage((J + 1 + T::kAhead) & (T::kStages - 1))),
                     true)) &&
                   ...);
        }(std::make_integer_sequence<int, T::kStages - 1>{});
        t0 = n_full;
    }
    for (int t = t0; t <= ntiles; ++t) body(t, std::false_type{}, rt_stage, rt_stage(t + T::kAhead));
    if (!lagging) fence_barrier();

    // dQ = scale * (dQ^T)^T, rounded to bf16: lane column = query row, registers = head dim
    if (ok) {
        uint16_t *out = p.dq + (sq.tok0 + row) * p.dq_rs + (int64_t)h * D;
#pragma unroll
        for (int eb = 0; eb < EB; ++eb)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                bf16x4 o4;
#pragma unroll
                for (int q = 0; q < 4; ++q) o4[q] = (__bf16)(dqacc[eb][r4 * 4 + q] * p.scale);
                *reinterpret_cast<u32x2 *>(out + eb * 32 + r4 * 8 + kg * 4) = __builtin_bit_cast(u32x2, o4);
            }
    }
}

template <int D>
__global__ __launch_bounds__(kQThreads) void attn_bwd_dq_bf16_kernel(DqParams p) {
    dq_body<D>(p, blockIdx.x);
}

// ============================================================================ bf16: dK/dV kernel
//
// 8 waves per workgroup, 128 keys of one KV head: waves 0-3 are producers,
// waves 4-7 consumers, and producer w shares a SIMD with consumer w+4.  The
// workgroup steps over 32-row query tiles of every query head of the group,
// from the end of the sequence down to the causal diagonal.
//   producer w, step t:  for its 32 keys, S = Q K^T and dP = dO V^T  (A = Q /
//                        dO rows from LDS, B = K / V fragments held in
//                        registers), P = exp2(S c - lse log2 e), dS = P (dP - D);
//                        the bf16 P and dS fragments go to LDS in the lane
//                        order of a B operand.
//   consumer c, step t:  for keys 64 (c/2) .. +64 and head dims 64 (c%2) ..
//                        +64, dV^T += dO^T P and dK^T += Q^T dS  (A = dO^T / Q^T
//                        by transposed LDS reads, B = the producers' P / dS),
//                        summed over the group's heads.  Each A fragment feeds
//                        the MFMAs of two 32-key blocks.
// One barrier per iteration, and in iteration t all three stages of the
// pipeline run at once, so that the matrix pipe of every SIMD always has a
// wave with MFMAs to issue:
//   * the producer issues the 16 MFMAs of step t (S and dP) and, one element
//     per MFMA, the softmax of step t-1 (whose S and dP it kept in a second
//     accumulator set), storing P / dS of step t-1; it also issues the Q/dO
//     tile loads of step t+3 and, before the barrier, the first S MFMAs of
//     step t+1;
//   * the consumer issues the 16 MFMAs of step t-2 on the P / dS that the
//     producer stored in the previous iteration (and one consumer loads the
//     rows' statistics a few steps ahead).
// The producer needs no statistics registers and no mask branch in its
// softmax: the S accumulator of a step starts from -lse/scale of its row
// (or -inf where the key is masked: past the row, past N), the dP
// accumulator from -D, so that P = exp2(c * S) and dS = P * dP.  Each role
// fits in 256 registers (2 waves per SIMD).  Q/dO tiles (and the rows'
// statistics) rotate through 6 LDS stages, P/dS through 2 buffers.

constexpr int kKvWaves = 8;
constexpr int kKvThreads = kKvWaves * 64;
constexpr int kKvPairs = 4;                          // producers (and consumers)
constexpr int kKeysPerWave = 32;                     // keys of one producer
constexpr int kKeysPerWg = kKvPairs * kKeysPerWave;  // 128
constexpr int kQT = 32;                              // query rows per step
constexpr int kKvAhead = 6;                          // A fragments read ahead of their MFMA
// LDS reads a producer issues between its last P/dS write of a step and the
// hand-over barrier: the kKvAhead first fragments of the next step.  The wait
// before the barrier lets this many stay outstanding, which retires every
// write before them.
constexpr int kReadsAfterPds = kKvAhead;
// S MFMAs of step t+1 that a producer issues at the end of iteration t, ahead
// of the barrier: step t+1's tiles and starting values are published by then,
// and the MFMAs keep the matrix pipe busy while both roles meet at the barrier.
// Two measured as well as four, six or seven at d=128; two also fits d=64,
// where the prefetch has to stay within one step.
constexpr int kEarly = 2;

struct DkvParams {
    const uint16_t *q, *k, *v, *dout;
    const float *stats;
    uint16_t *dk, *dv;
    int64_t q_rs, k_rs, v_rs, do_rs, dk_rs, dv_rs;  // elements between consecutive tokens of each tensor
    const int32_t *cu_seqlens;  // packed variable-length sequences, or nullptr
    int64_t total;              // tokens of the packed sequences
    int32_t N, B, Hq, Hkv;      // N: tokens per sequence (the longest one if packed)
    int32_t n_kblk;
    float scale_log2, scale;
    int32_t causal;
    // Head-split key blocks (shorter sequences): blocks 0 .. ksplit-1 run as
    // one workgroup per query head of the group, each writing its fp32 partial
    // dK (unscaled) and dV to part_k / part_v [ksplit][B][Hkv][grp][128][D];
    // a reduction kernel sums the heads.  0: every block is one workgroup.
    int32_t ksplit;
    float *part_k, *part_v;
};

// LDS: the Q tiles of every stage, then the dO tiles, the statistics rows and
// the two P/dS buffers.  Each region is addressed from a per-lane base
// register and every stage / step offset inside it stays below 64 KB.
template <int D>
struct DkvTile {
    static constexpr int kBytes = kQT * D * 2;                  // one Q or dO tile
    static constexpr int kStages = 6;                           // steps t-2 .. t+3
    static constexpr int kAhead = kStages - 3;                  // iterations from a load to its step
    static_assert(kStages % 2 == 0, "P/dS buffer parity follows the unrolled iteration index");
    static constexpr int kDoBase = kStages * kBytes;
    static constexpr int kStatBytes = 2 * kQT * 4;              // -lse/scale then -D, fp32
    static constexpr int kStatBase = 2 * kStages * kBytes;
    static constexpr int kPdsPair = 4 * 64 * 16;                // P[2], dS[2] fragments of one producer
    static constexpr int kPds = kKvPairs * kPdsPair;            // one buffer
    static constexpr int kPdsBase = kStatBase + kStages * kStatBytes;
    static constexpr int kLds = kPdsBase + 2 * kPds;
    static_assert(kDoBase <= 65536 && 2 * kPds <= 65536, "offsets must fit an LDS immediate");
    __device__ static constexpr int q_stage(int st) { return st * kBytes; }
    __device__ static constexpr int stat_stage(int st) { return st * kStatBytes; }
};

// ---- producer

// A fragment `st` of a step's MFMA stream: the KK fragments of S first (Q
// rows), then those of dP (dO rows), of the tile at stage offset `qst`.
template <int D>
__device__ __forceinline__ bf16x8 dkdv_sdp_frag(int st, uint32_t qst, const uint32_t *oq, const uint32_t *od) {
    constexpr int KK = D / 16;
    return lds_frag_at((st < KK ? oq[st] : od[st - KK]) + qst);
}

// The first kKvAhead fragments of a producer iteration: fragments kEarly ..
// of the step (its first kEarly S MFMAs were issued in the iteration before).
template <int D>
__device__ __forceinline__ void dkdv_sdp_prefetch(bf16x8 (&ring)[kKvAhead], uint32_t qst, const uint32_t *oq,
                                                  const uint32_t *od) {
#pragma unroll
    for (int st = 0; st < kKvAhead; ++st) ring[st] = dkdv_sdp_frag<D>(st + kEarly, qst, oq, od);
}

// The starting values of step t+1's accumulators for this lane's 16 rows
// (C register r holds row ckey(r, kg): two runs of 8 consecutive rows,
// 16*hh + 8*kg ..), read from a stage's statistics block at `stat`: -lse/scale
// into `sinit`, -D into `ninit`, both in C-register order.
__device__ __forceinline__ void dkdv_inits(f32x16 &sinit, f32x16 &ninit, uint32_t stat) {
    f32x4 l[2][2], d[2][2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int x = 0; x < 2; ++x) {
            l[hh][x] = *reinterpret_cast<const UL_LDS f32x4 *>((uintptr_t)(stat + hh * 64 + x * 16));
            d[hh][x] = *reinterpret_cast<const UL_LDS f32x4 *>((uintptr_t)(stat + kQT * 4 + hh * 64 + x * 16));
        }
    const f32x8 l0 = __builtin_shufflevector(l[0][0], l[0][1], 0, 1, 2, 3, 4, 5, 6, 7);
    const f32x8 l1 = __builtin_shufflevector(l[1][0], l[1][1], 0, 1, 2, 3, 4, 5, 6, 7);
    sinit = __builtin_shufflevector(l0, l1, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
    const f32x8 d0 = __builtin_shufflevector(d[0][0], d[0][1], 0, 1, 2, 3, 4, 5, 6, 7);
    const f32x8 d1 = __builtin_shufflevector(d[1][0], d[1][1], 0, 1, 2, 3, 4, 5, 6, 7);
    ninit = __builtin_shufflevector(d0, d1, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
}

// Masked step (rows r0 .. r0+31 against this lane's key): the S accumulator
// starts at -inf where the key is not visible to the row or either lies past
// N, so P = exp2(-inf) = 0 there.
__device__ __forceinline__ void dkdv_mask_init(f32x16 &sinit, int kg, int r0, int key, int N, int causal) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int i = r0 + ckey(r, kg);
        sinit[r] = (i >= N || key >= N || (causal && key > i)) ? -INFINITY : sinit[r];
    }
}

// One producer iteration: the MFMA stream of step t into (sa, dpa), whose
// starting values (-lse/scale or -inf, and -D) they already hold, with A
// fragments from the tile at stage offset `qst` (the first kKvAhead already in
// `ring`).  Between the MFMAs runs the softmax of step t-1 from (sb, dpb),
// software-pipelined so that the VALU work after each MFMA has no dependency
// inside it: element e's exponent argument c * s, two elements' worth of the
// exp2 and of the product dS = p * dp trail by one MFMA each (at D = 64 two
// elements per MFMA).  P and dS go to `pds` as bf16 B fragments (P of the
// lane's rows 0-7 / 8-15, then dS) as soon as 8 of them are done.  `mid()` runs
// halfway through the stream (it loads the next step's starting values);
// `side(k)`, k < NSIDE, runs after MFMA k+1, early in the stream, so that the
// tile loads it issues have most of two iterations to land.
template <int D, int NSIDE, typename Mid, typename Side>
__device__ __forceinline__ void dkdv_producer_iter(f32x16 &sa, f32x16 &dpa, const f32x16 &sb, const f32x16 &dpb,
                                                   f32x16 &sn, const bf16x8 *kf, const bf16x8 *vf,
                                                   bf16x8 (&ring)[kKvAhead], uint32_t qst, uint32_t qst_next,
                                                   const uint32_t *oq, const uint32_t *od,
                                                   uint32_t pds, float c, Mid &&mid, Side &&side) {
    constexpr int KK = D / 16, NSTEP = 2 * KK, EPB = 16 / NSTEP;
    static_assert(NSIDE < NSTEP, "side work goes to distinct MFMA slots");
    static_assert(16 % NSTEP == 0, "softmax elements spread evenly over the MFMAs");
    float arg[16], pv[16], ds[16];
    auto write_half = [&](int hh) {
        *reinterpret_cast<UL_LDS u32x4 *>((uintptr_t)(pds + hh * 64 * 16)) =
            __builtin_bit_cast(u32x4, pack8(pv + 8 * hh));
        *reinterpret_cast<UL_LDS u32x4 *>((uintptr_t)(pds + (2 + hh) * 64 * 16)) =
            __builtin_bit_cast(u32x4, pack8(ds + 8 * hh));
    };
#pragma unroll
    for (int e = 0; e < EPB; ++e) arg[e] = c * sb[e];
#pragma unroll
    for (int st = 0; st <= NSTEP; ++st) {
        if (st < NSTEP) {
            // slot st: MFMA j = st + kEarly of step t, or S MFMA j - NSTEP of step t+1
            const bf16x8 a = ring[st % kKvAhead];
            if (st + kKvAhead < NSTEP) {
                const int f = st + kKvAhead + kEarly;
                ring[st % kKvAhead] = f < NSTEP ? dkdv_sdp_frag<D>(f, qst, oq, od)
                                                : dkdv_sdp_frag<D>(f - NSTEP, qst_next, oq, od);
            }
            const int j = st + kEarly;
            if (j < KK)
                sa = mfma32x32x16(a, kf[j], sa);
            else if (j < NSTEP)
                dpa = mfma32x32x16(a, vf[j - KK], dpa);
            else
                sn = mfma32x32x16(a, kf[j - NSTEP], sn);
        }
#pragma unroll
        for (int e = 0; e < EPB; ++e) {
            const int r = st * EPB + e;  // this block: arg of r + EPB, exp of r, dS of r - EPB
            if (r + EPB < 16) arg[r + EPB] = c * sb[r + EPB];
            if (r < 16) pv[r] = __builtin_amdgcn_exp2f(arg[r]);
            if (r >= EPB) ds[r - EPB] = pv[r - EPB] * dpb[r - EPB];
        }
        if (st >= 1 && (st * EPB) % 8 == 0) write_half(st * EPB / 8 - 1);
#pragma unroll
        for (int k = 0; k < NSIDE; ++k)
            if (k + 1 == st) side(k);
        if (st == KK) mid();
        __builtin_amdgcn_sched_barrier(0);
    }
}

// ---- consumer

// The consumer's MFMAs of a step: for k-step ks (16 rows), head-dim block e2
// of its half (EBC = D/64 blocks of 32) and dV / dK, one transposed A
// fragment (dO^T / Q^T of the tile at `qst`) times the P / dS fragments of
// its two 32-key blocks.
template <int D>
struct DkdvCons {
    static constexpr int EBC = D / 64;                 // head-dim blocks per half
    static constexpr int NA = 2 * EBC * 2;             // A fragments per step: ks x e2 x {dO^T, Q^T}
    static constexpr int AH = NA < kKvAhead ? NA : kKvAhead;
    uint32_t tq[EBC][2], td[EBC][2];                   // transposed Q / dO halves of the half's blocks
    __device__ __forceinline__ bf16x8 frag(int st, uint32_t qst) const {
        const int ks = st / (2 * EBC), e2 = (st / 2) % EBC;
        const uint32_t at = qst + ks * 16 * D * 2;
        const uint32_t *t = st % 2 == 0 ? td[e2] : tq[e2];
        return lds_tr_frag_at(t[0] + at, t[1] + at);
    }
    __device__ __forceinline__ void prefetch(bf16x8 (&ring)[AH], uint32_t qst) const {
#pragma unroll
        for (int st = 0; st < AH; ++st) ring[st] = frag(st, qst);
    }
    // pb / db[kb2][ks]: P / dS B fragments of key block kb2, k-step ks;
    // `side(k)`, k < NSIDE, runs between MFMAs spread over the stream
    template <int NSIDE, typename Side>
    __device__ __forceinline__ void run(f32x16 (&dvacc)[EBC][2], f32x16 (&dkacc)[EBC][2],
                                        const bf16x8 (&pb)[2][2], const bf16x8 (&db)[2][2],
                                        bf16x8 (&ring)[AH], uint32_t qst, Side &&side) const {
        static_assert(NSIDE <= NA, "at most one load per MFMA step");
#pragma unroll
        for (int st = 0; st < NA; ++st) {
            const bf16x8 a = ring[st % AH];
            if (st + AH < NA) ring[st % AH] = frag(st + AH, qst);
            const int ks = st / (2 * EBC), e2 = (st / 2) % EBC;
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2) {
                if (st % 2 == 0)
                    dvacc[e2][kb2] = mfma32x32x16(a, pb[kb2][ks], dvacc[e2][kb2]);
                else
                    dkacc[e2][kb2] = mfma32x32x16(a, db[kb2][ks], dkacc[e2][kb2]);
            }
            if constexpr (NSIDE > 0) {
#pragma unroll
                for (int k = 0; k < NSIDE; ++k)
                    if (k * NA / NSIDE == st) side(k);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
};

template <int D>
__device__ __forceinline__ void dkdv_body(const DkvParams &p, const int item) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    UL_LDS unsigned char *lds = (UL_LDS unsigned char *)smem_raw;
    using T = DkvTile<D>;
    using Tile = DmaTile<D, kQT>;
    constexpr int KK = D / 16;
    static_assert(D == 128 || D == 64, "head_dim");
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int m = lane & 31, kg = lane >> 5;
    const bool producer = wave < kKvPairs;
    const int pair = producer ? wave : wave - kKvPairs;

    // Items: first the head-split blocks, ((kblk * B + b) * Hkv + g) * grp +
    // head, then the whole blocks, kblk * (B*Hkv) + (b*Hkv + g), each part
    // with key block 0 (the most work) first.
    const int per_rank = p.B * p.Hkv;
    const int grp = p.Hq / p.Hkv;
    const int n_split = p.ksplit * per_rank * grp;
    int kblk, bg, hsel;
    if (item < n_split) {
        kblk = item / (per_rank * grp);
        const int rest = item - kblk * per_rank * grp;
        bg = rest / grp;
        hsel = rest - bg * grp;
    } else {
        const int it = item - n_split;
        kblk = p.ksplit + it / per_rank;
        bg = it - (kblk - p.ksplit) * per_rank;
        hsel = -1;
    }
    const int b = bg / p.Hkv, g = bg % p.Hkv;
    const bool split = hsel >= 0;
    const int gsteps = split ? 1 : grp;  // query heads this workgroup walks
    const int h0 = split ? hsel : 0;     // the first of them within the group
    const SeqRange sq = seq_range(p.cu_seqlens, b, p.N, p.Hq, p.total);
    const int N = sq.len;
    const int kb0 = kblk * kKeysPerWg;
    if (kb0 >= N) return;  // past the end of a shorter packed sequence
    const uint32_t lbase = (uint32_t)(uintptr_t)lds;

    // Steps: 32-row tiles from the end of the sequence down to the causal
    // diagonal, the group's query heads innermost.  Every workgroup walks the
    // rows in the same order, so workgroups resident at the same time stream
    // the same Q/dO tiles and share them through L2.  A cursor (step, head
    // within the group, first row) advances one step at a time.
    const int qt_first = p.causal ? kb0 / kQT : 0;
    const int nqt = (N + kQT - 1) / kQT;
    const int per_head = nqt - qt_first;
    const int nsteps = per_head * gsteps;
    struct Cur {
        int s, hi, r0;
    };
    auto advance = [&](Cur &cu) {  // stays on the last step once there
        if (cu.s + 1 < nsteps) {
            ++cu.s;
            if (++cu.hi == gsteps) {
                cu.hi = 0;
                cu.r0 -= kQT;
            }
        }
    };
    const Cur first{0, 0, (nqt - 1) * kQT};

    // Zero the LDS: the first two iterations' consumers read never-written
    // stage and P/dS memory, which must hold zeros (P = dS = 0 contribute
    // nothing).
    for (int x = tid; x < T::kLds / 16; x += kKvThreads)
        *reinterpret_cast<UL_LDS u32x4 *>(lds + x * 16) = u32x4{0, 0, 0, 0};
    __builtin_amdgcn_s_waitcnt(0xc07f);
    fence_barrier();

    // Iterations t = 0 .. nsteps+1, unrolled by the stage count so that every
    // stage offset and buffer parity is a constant: step t's tiles and
    // statistics sit in stage t % 6, its P/dS in buffer t % 2.  Past the last
    // step the producer works on re-reads of the last step's tiles, and what
    // it computes from them is dropped or stored where no consumer reads.
    const int niter = nsteps + 2;
    // Whole groups in a straight loop, then the rest in a loop whose
    // iterations each test the count (a test per iteration inside the main
    // loop costs ~1 %).  The rest is a loop although it runs at most once:
    // its back edge keeps the reads that follow each P/dS hand-over live in
    // the compiled code, which the hand-over wait counts on.
    auto run = [&](auto iter) {
        int i0 = 0;
        for (; i0 + T::kStages <= niter; i0 += T::kStages) {
            [&]<int... J>(std::integer_sequence<int, J...>) {
                (iter(std::integral_constant<int, J>{}), ...);
            }(std::make_integer_sequence<int, T::kStages>{});
        }
        for (; i0 < niter; i0 += T::kStages) {
            [&]<int... J>(std::integer_sequence<int, J...>) {
                ((i0 + J < niter ? iter(std::integral_constant<int, J>{}) : void()), ...);
            }(std::make_integer_sequence<int, T::kStages>{});
        }
    };

    // Direct loads of a step into its LDS stage.  The Q and dO tiles are split
    // evenly over the 4 waves of a role: the consumers load the first kAhead
    // steps before the loop, and from then on the producers load step t+3 in
    // iteration t, between their MFMAs.  Consumer 3 loads the 32 rows'
    // -lse/scale (lanes 0-31) and -D (lanes 32-63, one statistics block
    // later), one dword per lane in one instruction, kStatAhead steps ahead.
    // Rows past N re-read row N-1 (masked by the producers); past the last
    // step the loads re-read it into a free stage.
    constexpr int kDmaPerWave = 2 * Tile::INSTR / kKvPairs;
    static_assert(2 * Tile::INSTR % kKvPairs == 0 && Tile::INSTR % kDmaPerWave == 0,
                  "Q and dO tiles split evenly over the waves of a role");
    const bool loads_do = pair * kDmaPerWave >= Tile::INSTR;
    const int u0 = (pair * kDmaPerWave) % Tile::INSTR;
    const uint16_t *tens = loads_do ? p.dout : p.q;
    const int64_t t_rs = loads_do ? p.do_rs : p.q_rs;
    const int tile_lds = loads_do ? T::kDoBase : 0;
    const uint32_t row_bytes = (uint32_t)t_rs * 2;
    uint32_t dma_roff[kDmaPerWave], dma_gran[kDmaPerWave];
#pragma unroll
    for (int k = 0; k < kDmaPerWave; ++k) {
        dma_roff[k] = (uint32_t)Tile::row(u0 + k, lane) * row_bytes;
        dma_gran[k] = Tile::gran_bytes(u0 + k, lane);
    }
    // The cursor of a step to load, with its row pointers: at the group's
    // first head (tb / sb) and at the step's head (tr / sr), so that no load
    // multiplies by the head index.  The -D half's offset, hs * 4 bytes, fits
    // the 32-bit lane offset: the launcher rejects statistics strides of 2^30.
    struct LoadCur {
        Cur cu;
        const uint16_t *tb, *tr;
        const float *sb, *sr;
    };
    const int64_t head_stride_st = 2 * sq.hs;
    const uint32_t stat_off = lane < kQT ? 0u : (uint32_t)sq.hs * 4u;
    const int64_t trow_step = (int64_t)kQT * t_rs;
    const uint16_t *tb0 = tens + (sq.tok0 + first.r0) * t_rs + (int64_t)(g * grp + h0) * D;
    const float *sb0 = p.stats + sq.st0 + (int64_t)(g * grp + h0) * head_stride_st + first.r0;
    const LoadCur load_first{first, tb0, tb0, sb0, sb0};
    auto advance_load = [&](LoadCur &l) {
        const int r0 = l.cu.r0, hi = l.cu.hi;
        advance(l.cu);
        if (l.cu.r0 != r0) {
            l.tb -= trow_step;
            l.sb -= kQT;
            l.tr = l.tb;
            l.sr = l.sb;
        } else if (l.cu.hi != hi) {
            l.tr += D;
            l.sr += head_stride_st;
        }
    };
    // load k of this wave's share of the step's Q or dO tile into stage st
    auto tile_k = [&](const LoadCur &l, int st, int k) {
        const int lim = min(N - 1 - l.cu.r0, kQT);  // last valid row within the tile
        dma_b128_m0(l.tr, min(dma_roff[k], (uint32_t)lim * row_bytes) + dma_gran[k],
                    lbase + tile_lds + T::q_stage(st) + (u0 + k) * 1024);
    };
    auto stat_load = [&](const LoadCur &l, int st) {
        const int r = min(lane & (kQT - 1), min(N - 1 - l.cu.r0, kQT));
        dma_b32_m0(l.sr, (uint32_t)r * 4 + stat_off, lbase + T::kStatBase + T::stat_stage(st));
    };

    if (producer) {
        const int key = kb0 + pair * kKeysPerWave + m;  // this lane's key (C column)
        // K and V rows of the producer's 32 keys as B fragments (column = key, k = head dim)
        bf16x8 kf[KK], vf[KK];
        {
            const bool ok = key < N;
            const int64_t tok = sq.tok0 + (ok ? key : 0);
            const uint16_t *kr = p.k + tok * p.k_rs + (int64_t)g * D;
            const uint16_t *vr = p.v + tok * p.v_rs + (int64_t)g * D;
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                kf[kk] = as_bf16x8(ok ? *reinterpret_cast<const u32x4 *>(kr + kk * 16 + kg * 8) : u32x4{0, 0, 0, 0});
                vf[kk] = as_bf16x8(ok ? *reinterpret_cast<const u32x4 *>(vr + kk * 16 + kg * 8) : u32x4{0, 0, 0, 0});
            }
        }
        __builtin_amdgcn_s_waitcnt(0x70);
        // absolute LDS addresses: Q / dO row fragments (stage 0), statistics
        // of this lane group's rows (stage 0), this lane's P/dS slot (buffer 0)
        uint32_t oq[KK], od[KK];
        {
            const int qrow = kperm(m);
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                oq[kk] = lbase + rm_off<D>(qrow, kk * 2 + kg);
                od[kk] = oq[kk] + T::kDoBase;
                asm volatile("" : "+v"(oq[kk]));
                asm volatile("" : "+v"(od[kk]));
            }
        }
        uint32_t stat = lbase + T::kStatBase + kg * 8 * 4;
        uint32_t pds = lbase + T::kPdsBase + pair * T::kPdsPair + lane * 16;
        asm volatile("" : "+v"(stat));
        asm volatile("" : "+v"(pds));
        const float c = p.scale_log2;

        // A step is masked when its rows reach below mlo (the causal diagonal)
        // or above mhi (the ragged end), or when the key block runs past N.
        // The producer needs only each step's first row: it drops by a tile
        // every grp steps.  The two steps past the last one need no mask:
        // their S and dP are dropped, and the P / dS stored from the first of
        // them goes to a buffer that no consumer reads again.
        const int mlo = kb0 + kKeysPerWg > N ? INT_MAX : (p.causal ? kb0 + kKeysPerWg : INT_MIN);
        const int mhi = N - kQT;
        int r0 = first.r0, hc = gsteps;
        auto prepare = [&](f32x16 &sinit) {  // mask the S starting values of the step at r0
            if (r0 < mlo || r0 > mhi) dkdv_mask_init(sinit, kg, r0, key, N, p.causal);
        };
        auto next_step = [&]() {
            if (--hc == 0) {
                hc = gsteps;
                r0 -= kQT;
            }
        };

        LoadCur lc = load_first;  // the consumers loaded steps 0 .. kAhead-1
#pragma unroll
        for (int i = 0; i < T::kAhead; ++i) advance_load(lc);
        fence_barrier();  // the consumers' first loads have landed
        // Three register sets rotate: step t accumulates in set t % 3, the
        // softmax of step t-1 reads set (t-1) % 3, and the starting values of
        // step t+1 are loaded straight into set (t+1) % 3, whose step t-2 is
        // done, so no copy is needed (the stage count, 6, keeps every index a
        // constant).  Set 0 starts as step 0; set 2 holds "step -1":
        // P = exp2(-inf) = 0, dS = 0.
        static_assert(T::kStages % 3 == 0, "register sets rotate with the stages");
        f32x16 s[3], dp[3];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            s[2][r] = -INFINITY;
            dp[2][r] = 0.f;
        }
        bf16x8 ring[kKvAhead];
        dkdv_inits(s[0], dp[0], stat + T::stat_stage(0));
        prepare(s[0]);
        // the early MFMAs come after the starting values are loaded (slot KK of the stream)
        static_assert(kEarly < KK && kEarly + kKvAhead <= 2 * KK, "early MFMAs follow the loads");
#pragma unroll
        for (int j = 0; j < kEarly; ++j)  // step 0's first S MFMAs, as iteration -1 would have
            s[0] = mfma32x32x16(dkdv_sdp_frag<D>(j, T::q_stage(0), oq, od), kf[j], s[0]);
        dkdv_sdp_prefetch<D>(ring, T::q_stage(0), oq, od);
        run([&](auto J) {
            constexpr int ST = decltype(J)::value;          // stage of step t
            constexpr int A = ST % 3, Pv = (ST + 2) % 3;    // register sets of steps t and t-1
            constexpr int X = (ST + 1) % 3;                 // set of step t+1 (step t-2's, done)
            constexpr int NX = (ST + 1) % T::kStages;       // stage of step t+1
            constexpr int PB = (ST + 1) % 2;                // P/dS buffer of step t-1
            constexpr int NN = (ST + T::kAhead) % T::kStages;  // stage of step t+3
            // the starting values of step t+1 are loaded (and masked) halfway
            // through the stream, before its first S MFMAs at the end of it;
            // the tile loads of step t+3 run between the MFMAs
            dkdv_producer_iter<D, kDmaPerWave>(
                s[A], dp[A], s[Pv], dp[Pv], s[X], kf, vf, ring, T::q_stage(ST), T::q_stage(NX), oq, od,
                pds + PB * T::kPds, c,
                [&]() {
                    dkdv_inits(s[X], dp[X], stat + T::stat_stage(NX));
                    next_step();
                    prepare(s[X]);
                },
                [&](int k) { tile_k(lc, NN, k); });
            advance_load(lc);
            dkdv_sdp_prefetch<D>(ring, T::q_stage(NX), oq, od);
            // P / dS of step t-1 stored before the barrier; the next step's
            // operand reads may stay in flight across it (they are waited for
            // at their first use).  LDS operations retire in order, the loop
            // issues no scalar memory operation, and after the last P / dS
            // write only LDS reads follow (16-byte reads of distinct addresses,
            // which the compiler cannot merge): the kKvAhead first fragments
            // of step t+1.  Waiting until at most that many are outstanding
            // retires the writes.  The same wait lets only this iteration's
            // tile loads stay in flight: step t+2's, which the producers read
            // from the next iteration on, have landed.
            static_assert(kDmaPerWave < 16, "vmcnt immediate");
            __builtin_amdgcn_s_waitcnt(kDmaPerWave | 0x70 | (kReadsAfterPds << 8));
            fence_barrier();
        });
        // no load may still be writing this workgroup's LDS when it exits
        __builtin_amdgcn_s_waitcnt(0x70);
        return;
    }

    // ---- consumers: for keys 64 kh .. +64 and head dims 64 eh .. +64
    const int kh = pair >> 1, eh = pair & 1;
    // Statistics run kStatAhead = 5 steps ahead: step t+5's go to the stage of
    // step t-1, whose statistics the producers read in iteration t-2.  Before
    // the barrier ending iteration t, step t+2's must have landed (the
    // producers read them in iteration t+1): all but the 3 newest loads.
    constexpr int kStatAhead = T::kStages - 1;
    const bool stats_wave = pair == kKvPairs - 1;
    LoadCur lt = load_first, ls = load_first;
    [&]<int... J>(std::integer_sequence<int, J...>) {
        (([&] {
#pragma unroll
             for (int k = 0; k < kDmaPerWave; ++k) tile_k(lt, J, k);
             advance_load(lt);
         }()),
         ...);
    }(std::make_integer_sequence<int, T::kAhead>{});
    if (stats_wave) {
        [&]<int... J>(std::integer_sequence<int, J...>) {
            ((stat_load(ls, J), advance_load(ls)), ...);
        }(std::make_integer_sequence<int, kStatAhead>{});
    }
    wait_vm<0>();  // the first steps have landed
    fence_barrier();

    // absolute LDS addresses: transposed Q / dO halves of the head-dim
    // blocks, and this lane's slot in the P/dS blocks of the key half
    using Cons = DkdvCons<D>;
    constexpr int EBC = Cons::EBC;
    Cons cons;
    {
        const TrAddr<D> ta(lane);
#pragma unroll
        for (int e2 = 0; e2 < EBC; ++e2)
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                cons.tq[e2][x] = lbase + tr_off<D>(ta, (eh * EBC + e2) * 32, x);
                cons.td[e2][x] = cons.tq[e2][x] + T::kDoBase;
                asm volatile("" : "+v"(cons.tq[e2][x]));
                asm volatile("" : "+v"(cons.td[e2][x]));
            }
    }
    uint32_t pds = lbase + T::kPdsBase + 2 * kh * T::kPdsPair + lane * 16;
    asm volatile("" : "+v"(pds));
    f32x16 dvacc[EBC][2], dkacc[EBC][2];
#pragma unroll
    for (int e2 = 0; e2 < EBC; ++e2)
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
            dvacc[e2][k2] = zero16();
            dkacc[e2][k2] = zero16();
        }
    bf16x8 ring[Cons::AH], pb[2][2], db[2][2];
    cons.prefetch(ring, T::q_stage(T::kStages - 2));  // step -2 (zeros)
    run([&](auto J) {
        constexpr int ST = decltype(J)::value;
        constexpr int PV = (ST + T::kStages - 2) % T::kStages;  // stage of step t-2
        constexpr int NX = (ST + T::kStages - 1) % T::kStages;  // stage of step t-1
        constexpr int NS = (ST + kStatAhead) % T::kStages;      // statistics stage of step t+5
        const uint32_t buf = pds + (ST % 2) * T::kPds;          // P/dS of step t-2
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                pb[k2][ks] = lds_frag_at(buf + k2 * T::kPdsPair + ks * 64 * 16);
                db[k2][ks] = lds_frag_at(buf + k2 * T::kPdsPair + (2 + ks) * 64 * 16);
            }
        cons.template run<1>(dvacc, dkacc, pb, db, ring, T::q_stage(PV), [&](int) {
            if (stats_wave) stat_load(ls, NS);
        });
        if (stats_wave) advance_load(ls);
        cons.prefetch(ring, T::q_stage(NX));
        if (stats_wave) wait_vm_only<kStatAhead - 2>();
        fence_barrier();
    });
    // no load may still be writing this workgroup's LDS when it exits
    __builtin_amdgcn_s_waitcnt(0x70);

    if (split) {  // fp32 partials of this head; the reduction scales and rounds
        const int64_t blk = (((int64_t)kblk * p.B + b) * p.Hkv + g) * grp + hsel;
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
            const int kl = (2 * kh + k2) * kKeysPerWave + m;  // key within the block
            float *pk = p.part_k + (blk * kKeysPerWg + kl) * D;
            float *pv = p.part_v + (blk * kKeysPerWg + kl) * D;
#pragma unroll
            for (int e2 = 0; e2 < EBC; ++e2)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const int e = (eh * EBC + e2) * 32 + r4 * 8 + kg * 4;
                    f32x4 k4, v4;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        k4[q] = dkacc[e2][k2][r4 * 4 + q];
                        v4[q] = dvacc[e2][k2][r4 * 4 + q];
                    }
                    *reinterpret_cast<f32x4 *>(pk + e) = k4;
                    *reinterpret_cast<f32x4 *>(pv + e) = v4;
                }
        }
        return;
    }
    // dK = scale * acc, dV = acc (bf16): lane column = key, registers = head dim
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
        const int key = kb0 + (2 * kh + k2) * kKeysPerWave + m;
        if (key < N) {
            uint16_t *dkr = p.dk + (sq.tok0 + key) * p.dk_rs + (int64_t)g * D;
            uint16_t *dvr = p.dv + (sq.tok0 + key) * p.dv_rs + (int64_t)g * D;
#pragma unroll
            for (int e2 = 0; e2 < EBC; ++e2)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    bf16x4 k4, v4;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        k4[q] = (__bf16)(dkacc[e2][k2][r4 * 4 + q] * p.scale);
                        v4[q] = (__bf16)(dvacc[e2][k2][r4 * 4 + q]);
                    }
                    const int e = (eh * EBC + e2) * 32 + r4 * 8 + kg * 4;
                    *reinterpret_cast<u32x2 *>(dkr + e) = __builtin_bit_cast(u32x2, k4);
                    *reinterpret_cast<u32x2 *>(dvr + e) = __builtin_bit_cast(u32x2, v4);
                }
        }
    }
}

template <int D>
__global__ __launch_bounds__(kKvThreads) void attn_bwd_dkdv_bf16_kernel(DkvParams p) {
    dkdv_body<D>(p, blockIdx.x);
}

// Sum of the head-split partials: for key j of a split block, dK = scale *
// sum over the group's query heads of part_k, dV = sum of part_v, rounded to
// bf16.  One thread per 4 head dims of one key, heads summed in order.
template <int D>
__global__ __launch_bounds__(256) void dkdv_reduce_kernel(DkvParams p) {
    const int grp = p.Hq / p.Hkv;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t total = (int64_t)p.ksplit * p.B * p.Hkv * kKeysPerWg * (D / 4);
    if (idx >= total) return;
    const int d4 = (int)(idx % (D / 4));
    int64_t r = idx / (D / 4);
    const int kl = (int)(r % kKeysPerWg);
    r /= kKeysPerWg;
    const int g = (int)(r % p.Hkv);
    r /= p.Hkv;
    const int b = (int)(r % p.B);
    const int kblk = (int)(r / p.B);
    const int key = kblk * kKeysPerWg + kl;
    if (key >= p.N) return;
    const int64_t blk0 = (((int64_t)kblk * p.B + b) * p.Hkv + g) * grp;
    f32x4 sk = {0.f, 0.f, 0.f, 0.f}, sv = {0.f, 0.f, 0.f, 0.f};
    for (int h = 0; h < grp; ++h) {
        const int64_t off = ((blk0 + h) * kKeysPerWg + kl) * D + d4 * 4;
        const f32x4 a = *reinterpret_cast<const f32x4 *>(p.part_k + off);
        const f32x4 c = *reinterpret_cast<const f32x4 *>(p.part_v + off);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            sk[q] += a[q];
            sv[q] += c[q];
        }
    }
    bf16x4 k4, v4;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        k4[q] = (__bf16)(sk[q] * p.scale);
        v4[q] = (__bf16)sv[q];
    }
    const int64_t tok = (int64_t)b * p.N + key;
    *reinterpret_cast<u32x2 *>(p.dk + tok * p.dk_rs + (int64_t)g * D + d4 * 4) = __builtin_bit_cast(u32x2, k4);
    *reinterpret_cast<u32x2 *>(p.dv + tok * p.dv_rs + (int64_t)g * D + d4 * 4) = __builtin_bit_cast(u32x2, v4);
}

// Both backward passes in one launch, for grids too small to fill the chip
// on their own (short sequences), so the two passes share the compute units
// instead of each leaving part of them idle.  Each workgroup runs exactly the
// body of the standalone kernel for its item.  The items run in the order
// `order` gives, longest first over both families (the host estimates each
// item's length, see merged_order); without it (use_order = 0) the dK/dV
// items run first, then the dQ items.
static_assert(kQThreads == kKvThreads, "one block size for both passes");
constexpr int kMergedMaxItems = 1024;
constexpr uint16_t kMergedDq = 0x8000;  // item code: dQ item (low bits: its index), else dK/dV
struct MergedOrder {
    uint16_t item[kMergedMaxItems];
};
template <int D>
__global__ __launch_bounds__(kKvThreads) void attn_bwd_dq_dkdv_bf16_kernel(DqParams dp, DkvParams kp,
                                                                           int kv_items, MergedOrder order,
                                                                           int use_order) {
    int code;
    if (use_order)
        code = order.item[blockIdx.x];
    else
        code = (int)blockIdx.x < kv_items ? (int)blockIdx.x : (kMergedDq | ((int)blockIdx.x - kv_items));
    if (!(code & kMergedDq))
        dkdv_body<D>(kp, code);
    else
        dq_body<D>(dp, code & ~kMergedDq);
}

// Longest first over both families of the merged launch: each item's length
// estimated from its steps (32 query rows of a 128-key block for one head,
// dK/dV) or tiles (32 keys for all rows of a dQ block), weighted 3 : 4, their
// measured costs at N = 65536 (0.89 and 1.20 us).  The head-split dK/dV
// items, the whole dK/dV items and the dQ items are each already in
// decreasing order of that estimate, so the order is their merge, taking the
// earlier family on ties (the result of a stable sort of the three in that
// order); no allocation.  Causal, equal-length sequences only (packed ones
// have lengths only the device knows); false when the grid is too large for
// the table.
bool merged_order(const DqParams &dp, const DkvParams &kp, int kv_items, int dq_items, MergedOrder *out) {
    if (!kp.causal || kp.cu_seqlens || kv_items + dq_items > kMergedMaxItems) return false;
    const int64_t nqt = ((int64_t)kp.N + kQT - 1) / kQT;
    const int grp = kp.Hq / kp.Hkv;
    const int kv_lanes = kp.B * kp.Hkv;
    const int n_split = kp.ksplit * kv_lanes * grp;
    const int dq_lanes = dp.B * dp.Hkv * dp.head_groups;
    const int64_t wg_rows = (int64_t)kRowsPerWave * dp.pos_blocks;
    auto kv_cost = [&](int i) {  // i < kv_items
        const bool split = i < n_split;
        const int kblk = split ? i / (kv_lanes * grp) : kp.ksplit + (i - n_split) / kv_lanes;
        return 3 * (nqt - (int64_t)kblk * (kKeysPerWg / kQT)) * (split ? 1 : grp);
    };
    auto dq_cost = [&](int i) {  // i < dq_items
        const int qblk = dp.n_qblk - 1 - i / dq_lanes;
        const int64_t keys = std::min<int64_t>(dp.N, (qblk + 1) * wg_rows);
        return 4 * ((keys + kDqKT - 1) / kDqKT);
    };
    // cursors: head-split dK/dV items [0, n_split), whole ones [n_split, kv_items), dQ items
    int a = 0, w = std::min(n_split, kv_items), q = 0;
    for (int r = 0; r < kv_items + dq_items; ++r) {
        const int64_t ca = a < std::min(n_split, kv_items) ? kv_cost(a) : -1;
        const int64_t cw = w < kv_items ? kv_cost(w) : -1;
        const int64_t cq = q < dq_items ? dq_cost(q) : -1;
        if (ca >= cw && ca >= cq)
            out->item[r] = (uint16_t)a++;
        else if (cw >= cq)
            out->item[r] = (uint16_t)w++;
        else
            out->item[r] = (uint16_t)(kMergedDq | q++);
    }
    return true;
}

// ============================================================================ fp32 kernels

constexpr int kF32Rows = 64;
constexpr int kF32Keys = 32;

struct BwdF32Params {
    const float *q, *k, *v, *dout;
    const float *lse;    // natural-log units
    const float *stats;  // the workspace statistics (D is read from it)
    float *dq, *dk, *dv;
    int64_t N;
    int64_t q_rs, k_rs, v_rs, do_rs, dq_rs, dk_rs, dv_rs;  // token strides in elements
    const int32_t *cu_seqlens;  // packed variable-length sequences, or nullptr
    int64_t total;
    int32_t B, Hq, Hkv;
    float scale;
    int32_t causal;
    int32_t n_blk;
};

// one thread per query row: dq_i = scale sum_j p_ij (dp_ij - D_i) k_j
template <int D>
__global__ __launch_bounds__(kF32Rows) void attn_bwd_dq_f32_kernel(BwdF32Params p) {
    __shared__ float ks[kF32Keys][D];
    __shared__ float vs[kF32Keys][D];
    const int tid = threadIdx.x;
    const int bh = blockIdx.x % (p.B * p.Hq);
    const int rank = blockIdx.x / (p.B * p.Hq);
    const int rblk = p.causal ? (p.n_blk - 1 - rank) : rank;
    const int b = bh / p.Hq, h = bh % p.Hq;
    const int g = h / (p.Hq / p.Hkv);
    const SeqRange sq = seq_range(p.cu_seqlens, b, p.N, p.Hq, p.total);
    const int64_t N = sq.len;
    if ((int64_t)rblk * kF32Rows >= N) return;  // past the end of a shorter packed sequence
    const int64_t i = (int64_t)rblk * kF32Rows + tid;
    const bool valid = i < N;
    const int64_t ri = valid ? i : 0;
    float qv[D], dov[D], acc[D];
    const float *qrow = p.q + (sq.tok0 + ri) * p.q_rs + (int64_t)h * D;
    const float *drow = p.dout + (sq.tok0 + ri) * p.do_rs + (int64_t)h * D;
#pragma unroll
    for (int e = 0; e < D; ++e) {
        qv[e] = valid ? qrow[e] : 0.f;
        dov[e] = valid ? drow[e] : 0.f;
        acc[e] = 0.f;
    }
    const float lse = valid ? p.lse[sq.lse0 + (int64_t)h * sq.hs + ri] : 0.f;
    const float nDi = valid ? p.stats[sq.st0 + (2 * (int64_t)h + 1) * sq.hs + ri] : 0.f;  // -D
    const int64_t blk_last = (int64_t)rblk * kF32Rows + kF32Rows - 1;
    const int64_t kend = p.causal ? (blk_last + 1 < N ? blk_last + 1 : N) : N;
    for (int64_t j0 = 0; j0 < kend; j0 += kF32Keys) {
        __syncthreads();
        for (int idx = tid; idx < kF32Keys * D; idx += kF32Rows) {
            const int jj = idx / D, e = idx % D;
            const int64_t j = j0 + jj;
            const int64_t tok = sq.tok0 + j, col = (int64_t)g * D + e;
            ks[jj][e] = j < N ? p.k[tok * p.k_rs + col] : 0.f;
            vs[jj][e] = j < N ? p.v[tok * p.v_rs + col] : 0.f;
        }
        __syncthreads();
        for (int jj = 0; jj < kF32Keys; ++jj) {
            const int64_t j = j0 + jj;
            if (j >= N || (p.causal && j > i)) continue;
            float s = 0.f, dp = 0.f;
#pragma unroll
            for (int e = 0; e < D; ++e) {
                s = fmaf(qv[e], ks[jj][e], s);
                dp = fmaf(dov[e], vs[jj][e], dp);
            }
            const float pr = expf(s * p.scale - lse);
            const float ds = pr * (dp + nDi);
#pragma unroll
            for (int e = 0; e < D; ++e) acc[e] = fmaf(ds, ks[jj][e], acc[e]);
        }
    }
    if (valid) {
        float *out = p.dq + (sq.tok0 + i) * p.dq_rs + (int64_t)h * D;
#pragma unroll
        for (int e = 0; e < D; ++e) out[e] = acc[e] * p.scale;
    }
}

// one thread per key row of a KV head: loops over the group's query heads and rows
constexpr int kF32KvKeys = 32;
constexpr int kF32KvRows = 16;

template <int D>
__global__ __launch_bounds__(kF32KvKeys) void attn_bwd_dkdv_f32_kernel(BwdF32Params p) {
    __shared__ float qs[kF32KvRows][D];
    __shared__ float ds_[kF32KvRows][D];
    __shared__ float kown[kF32KvKeys][D + 1];
    __shared__ float vown[kF32KvKeys][D + 1];
    __shared__ float ls[kF32KvRows], nDs[kF32KvRows];  // lse, -D
    const int tid = threadIdx.x;
    const int bg = blockIdx.x % (p.B * p.Hkv);
    const int kblk = blockIdx.x / (p.B * p.Hkv);
    const int b = bg / p.Hkv, g = bg % p.Hkv;
    const int grp = p.Hq / p.Hkv;
    const SeqRange sq = seq_range(p.cu_seqlens, b, p.N, p.Hq, p.total);
    const int64_t N = sq.len;
    if ((int64_t)kblk * kF32KvKeys >= N) return;  // past the end of a shorter packed sequence
    const int64_t j = (int64_t)kblk * kF32KvKeys + tid;
    const bool valid = j < N;
    const int64_t rj = valid ? j : 0;
    for (int e = 0; e < D; ++e) {
        kown[tid][e] = valid ? p.k[(sq.tok0 + rj) * p.k_rs + (int64_t)g * D + e] : 0.f;
        vown[tid][e] = valid ? p.v[(sq.tok0 + rj) * p.v_rs + (int64_t)g * D + e] : 0.f;
    }
    float dk[D], dv[D];
#pragma unroll
    for (int e = 0; e < D; ++e) { dk[e] = 0.f; dv[e] = 0.f; }
    const int64_t blk_first = (int64_t)kblk * kF32KvKeys;
    const int64_t i_start = p.causal ? (blk_first / kF32KvRows) * kF32KvRows : 0;
    for (int hh = 0; hh < grp; ++hh) {
        const int h = g * grp + hh;
        for (int64_t i0 = i_start; i0 < N; i0 += kF32KvRows) {
            __syncthreads();
            for (int idx = tid; idx < kF32KvRows * D; idx += kF32KvKeys) {
                const int ii = idx / D, e = idx % D;
                const int64_t i = i0 + ii;
                const int64_t tok = sq.tok0 + i, col = (int64_t)h * D + e;
                qs[ii][e] = i < N ? p.q[tok * p.q_rs + col] : 0.f;
                ds_[ii][e] = i < N ? p.dout[tok * p.do_rs + col] : 0.f;
            }
            if (tid < kF32KvRows) {
                const int64_t i = i0 + tid;
                ls[tid] = i < N ? p.lse[sq.lse0 + (int64_t)h * sq.hs + i] : 0.f;
                nDs[tid] = i < N ? p.stats[sq.st0 + (2 * (int64_t)h + 1) * sq.hs + i] : 0.f;
            }
            __syncthreads();
            for (int ii = 0; ii < kF32KvRows; ++ii) {
                const int64_t i = i0 + ii;
                if (i >= N || !valid || (p.causal && j > i)) continue;
                float s = 0.f, dp = 0.f;
                for (int e = 0; e < D; ++e) {
                    s = fmaf(qs[ii][e], kown[tid][e], s);
                    dp = fmaf(ds_[ii][e], vown[tid][e], dp);
                }
                const float pr = expf(s * p.scale - ls[ii]);
                const float dsv = pr * (dp + nDs[ii]);
#pragma unroll
                for (int e = 0; e < D; ++e) {
                    dk[e] = fmaf(dsv, qs[ii][e], dk[e]);
                    dv[e] = fmaf(pr, ds_[ii][e], dv[e]);
                }
            }
        }
    }
    if (valid) {
        float *dkr = p.dk + (sq.tok0 + j) * p.dk_rs + (int64_t)g * D;
        float *dvr = p.dv + (sq.tok0 + j) * p.dv_rs + (int64_t)g * D;
#pragma unroll
        for (int e = 0; e < D; ++e) {
            dkr[e] = dk[e] * p.scale;
            dvr[e] = dv[e];
        }
    }
}

size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

// Head-split dK/dV for shorter sequences.  When the dK/dV grid is at most
// half a round of the 256 compute units, the longest work item (key block 0:
// every query row of every head of the group) is far longer than the average
// work per compute unit, and it alone sets the backward's time.  Key blocks
// whose whole item would exceed the longest single-head item then run as one
// workgroup per query head (fp32 partials, summed by dkdv_reduce_kernel).
// Measured (8q/2kv, d = 128, whole backward): N = 4096 0.37 -> 0.19 ms, 8192
// 0.76 -> 0.54 ms; at 16384 (256 items) neutral, so the split stops there.
// The plan depends on the sizes only (not on the mask or the device), so the
// workspace size does too.
constexpr int64_t kSplitMaxItems = 128;
constexpr size_t kSplitMaxBytes = size_t(192) << 20;

struct BwdPlan {
    int32_t ksplit;       // key blocks run head by head
    size_t stats_bytes;   // -lse/scale and -D per query row and head
    size_t part_bytes;    // fp32 partials of dK and dV of the split blocks
};

BwdPlan bwd_plan(const AttnShape &s, int32_t dtype) {
    BwdPlan pl{0, 0, 0};
    const size_t rows = s.cu ? (size_t)s.Hq * (size_t)s.total : (size_t)s.B * (size_t)s.Hq * (size_t)s.N;
    pl.stats_bytes = round256(2 * rows * sizeof(float));
    const int64_t grp = s.Hq / s.Hkv;
    const int64_t n_kblk = (s.N + kKeysPerWg - 1) / kKeysPerWg;
    if (dtype != UL_BF16 || s.cu || grp < 2 || n_kblk * s.B * s.Hkv > kSplitMaxItems) return pl;
    const int64_t nqt = (s.N + kQT - 1) / kQT;
    int64_t ks = 0;
    // the causal rule for both masks: the workspace size takes no mask argument
    while (ks < n_kblk && grp * (nqt - ks * (kKeysPerWg / kQT)) > nqt) ++ks;
    const size_t per_block = (size_t)s.B * s.Hkv * grp * kKeysPerWg * s.d * sizeof(float) * 2;
    ks = std::min<int64_t>(ks, (int64_t)(kSplitMaxBytes / per_block));
    pl.ksplit = (int32_t)ks;
    pl.part_bytes = (size_t)ks * per_block;
    return pl;
}

}  // namespace

size_t attn_bwd_workspace_bytes(const AttnShape &s, int32_t dtype) {
    const BwdPlan pl = bwd_plan(s, dtype);
    return pl.stats_bytes + pl.part_bytes;
}

static hipError_t launch_pre(const void *o, const void *dout, const float *lse, float *stats,
                             const AttnShape &s, bool bf16, hipStream_t stream) {
    // Packed sequences lay lse and the statistics out as one sequence of
    // `total` tokens, so the pre-pass runs over all of them at once.
    const int64_t Bp = s.cu ? 1 : s.B, Np = s.cu ? s.total : s.N;
    PreParams pp{o, dout, lse, stats, Np, s.o_rs, s.do_rs, (int32_t)Bp, s.Hq, s.d, bf16 ? 1 : 0,
                 s.scale};
    const int64_t rows = Bp * Np * s.Hq;
    const int lanes = s.d / (bf16 ? 8 : 4);  // lanes per row, as the kernel takes them
    const int64_t per_block = 256 / lanes;
    const int64_t blocks = (rows + per_block - 1) / per_block;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    const dim3 grid((uint32_t)blocks), block(256);
    if (bf16 && s.d == 128)
        hipLaunchKernelGGL((bwd_pre_kernel<true, 128>), grid, block, 0, stream, pp);
    else if (bf16)
        hipLaunchKernelGGL((bwd_pre_kernel<true, 64>), grid, block, 0, stream, pp);
    else if (s.d == 128)
        hipLaunchKernelGGL((bwd_pre_kernel<false, 128>), grid, block, 0, stream, pp);
    else
        hipLaunchKernelGGL((bwd_pre_kernel<false, 64>), grid, block, 0, stream, pp);
    return hipGetLastError();
}

hipError_t launch_attn_bwd_bf16(const void *q, const void *k, const void *v, const void *o,
                                const void *dout, const float *lse, void *dq, void *dk, void *dv,
                                void *ws, const AttnShape &s, int stages, hipStream_t stream) {
    float *stats = static_cast<float *>(ws);
    hipError_t err = hipSuccess;
    if (stages & UL_BWD_PREP) {
        err = launch_pre(o, dout, lse, stats, s, true, stream);
        if (err != hipSuccess) return err;
    }

    DqParams dp;
    dp.q = static_cast<const uint16_t *>(q);
    dp.k = static_cast<const uint16_t *>(k);
    dp.v = static_cast<const uint16_t *>(v);
    dp.dout = static_cast<const uint16_t *>(dout);
    dp.stats = stats;
    dp.dq = static_cast<uint16_t *>(dq);
    dp.N = (int32_t)s.N;
    dp.B = (int32_t)s.B;
    dp.Hq = s.Hq;
    dp.Hkv = s.Hkv;
    dp.q_rs = s.q_rs;
    dp.k_rs = s.k_rs;
    dp.v_rs = s.v_rs;
    dp.do_rs = s.do_rs;
    dp.dq_rs = s.dq_rs;
    dp.cu_seqlens = s.cu;
    dp.total = s.total;
    const int grp = s.Hq / s.Hkv;
    dp.heads_per_wg = (grp % 4 == 0) ? 4 : (grp % 2 == 0) ? 2 : 1;
    dp.pos_blocks = kQWaves / dp.heads_per_wg;
    dp.head_groups = grp / dp.heads_per_wg;
    const int64_t pos_per_wg = (int64_t)kRowsPerWave * dp.pos_blocks;
    dp.n_qblk = (int32_t)((s.N + pos_per_wg - 1) / pos_per_wg);
    dp.scale_log2 = s.scale * kLog2e;
    dp.scale = s.scale;
    dp.causal = s.causal;
    const int64_t dq_items = (int64_t)dp.n_qblk * dp.B * dp.Hkv * dp.head_groups;
    if (dq_items > 0x7fffffff) return hipErrorInvalidConfiguration;

    DkvParams kp;
    kp.q = dp.q;
    kp.k = dp.k;
    kp.v = dp.v;
    kp.dout = dp.dout;
    kp.stats = stats;
    kp.dk = static_cast<uint16_t *>(dk);
    kp.dv = static_cast<uint16_t *>(dv);
    kp.N = (int32_t)s.N;
    kp.B = (int32_t)s.B;
    kp.Hq = s.Hq;
    kp.Hkv = s.Hkv;
    kp.q_rs = s.q_rs;
    kp.k_rs = s.k_rs;
    kp.v_rs = s.v_rs;
    kp.do_rs = s.do_rs;
    kp.dk_rs = s.dk_rs;
    kp.dv_rs = s.dv_rs;
    kp.cu_seqlens = s.cu;
    kp.total = s.total;
    kp.n_kblk = (int32_t)((s.N + kKeysPerWg - 1) / kKeysPerWg);
    kp.scale_log2 = dp.scale_log2;
    kp.scale = s.scale;
    kp.causal = s.causal;
    const BwdPlan plan = bwd_plan(s, UL_BF16);
    kp.ksplit = plan.ksplit;
    kp.part_k = reinterpret_cast<float *>(static_cast<unsigned char *>(ws) + plan.stats_bytes);
    kp.part_v = kp.part_k + plan.part_bytes / sizeof(float) / 2;
    const int64_t kv_items = (int64_t)kp.n_kblk * kp.B * kp.Hkv + (int64_t)plan.ksplit * kp.B * kp.Hkv * (grp - 1);
    if (kv_items > 0x7fffffff) return hipErrorInvalidConfiguration;
    // the reduction of the head-split partials, after the dK/dV work items
    auto reduce = [&]() -> hipError_t {
        if (plan.ksplit == 0) return hipSuccess;
        const int64_t n = (int64_t)plan.ksplit * kp.B * kp.Hkv * kKeysPerWg * (s.d / 4);
        const dim3 grid((uint32_t)((n + 255) / 256)), block(256);
        if (s.d == 128)
            hipLaunchKernelGGL(dkdv_reduce_kernel<128>, grid, block, 0, stream, kp);
        else
            hipLaunchKernelGGL(dkdv_reduce_kernel<64>, grid, block, 0, stream, kp);
        return hipGetLastError();
    };

    // Shorter sequences: when the dK/dV grid covers fewer than four rounds of
    // the compute units, run both passes in one launch so they fill the chip
    // together (both stages requested only).  Measured on MI355X for 8q/2kv,
    // d = 128: -20 % backward time at N = 8192 and 16384, -2.5 % at 49152,
    // neutral at 32768; at 65536 (four rounds) separate launches are as fast.
    if ((stages & UL_BWD_DQ) && (stages & UL_BWD_DKDV) && kv_items + dq_items <= 0x7fffffff) {
        int dev = 0, cus = 0;
        if ((err = hipGetDevice(&dev)) != hipSuccess) return err;
        if ((err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess)
            return err;
        if ((int64_t)kp.n_kblk * kp.B * kp.Hkv < 4 * (int64_t)cus) {
            const dim3 grid((uint32_t)(kv_items + dq_items)), block(kKvThreads);
            MergedOrder order;
            const int use_order = merged_order(dp, kp, (int)kv_items, (int)dq_items, &order) ? 1 : 0;
            if (s.d == 128) {
                constexpr size_t lds = DqTile<128>::kLds > DkvTile<128>::kLds ? DqTile<128>::kLds
                                                                              : DkvTile<128>::kLds;
                if ((err = allow_lds(attn_bwd_dq_dkdv_bf16_kernel<128>, lds)) != hipSuccess) return err;
                hipLaunchKernelGGL(attn_bwd_dq_dkdv_bf16_kernel<128>, grid, block, lds, stream, dp, kp,
                                   (int)kv_items, order, use_order);
            } else {
                constexpr size_t lds = DqTile<64>::kLds > DkvTile<64>::kLds ? DqTile<64>::kLds
                                                                            : DkvTile<64>::kLds;
                if ((err = allow_lds(attn_bwd_dq_dkdv_bf16_kernel<64>, lds)) != hipSuccess) return err;
                hipLaunchKernelGGL(attn_bwd_dq_dkdv_bf16_kernel<64>, grid, block, lds, stream, dp, kp,
                                   (int)kv_items, order, use_order);
            }
            if ((err = hipGetLastError()) != hipSuccess) return err;
            return reduce();
        }
    }

    if (s.d == 128) {
        if (stages & UL_BWD_DQ) {
            if ((err = allow_lds(attn_bwd_dq_bf16_kernel<128>, DqTile<128>::kLds)) != hipSuccess) return err;
            hipLaunchKernelGGL(attn_bwd_dq_bf16_kernel<128>, dim3((uint32_t)dq_items), dim3(kQThreads),
                               DqTile<128>::kLds, stream, dp);
            if ((err = hipGetLastError()) != hipSuccess) return err;
        }
        if (stages & UL_BWD_DKDV) {
            if ((err = allow_lds(attn_bwd_dkdv_bf16_kernel<128>, DkvTile<128>::kLds)) != hipSuccess) return err;
            hipLaunchKernelGGL(attn_bwd_dkdv_bf16_kernel<128>, dim3((uint32_t)kv_items), dim3(kKvThreads),
                               DkvTile<128>::kLds, stream, kp);
            if ((err = hipGetLastError()) != hipSuccess) return err;
            if ((err = reduce()) != hipSuccess) return err;
        }
    } else {
        if (stages & UL_BWD_DQ) {
            if ((err = allow_lds(attn_bwd_dq_bf16_kernel<64>, DqTile<64>::kLds)) != hipSuccess) return err;
            hipLaunchKernelGGL(attn_bwd_dq_bf16_kernel<64>, dim3((uint32_t)dq_items), dim3(kQThreads),
                               DqTile<64>::kLds, stream, dp);
            if ((err = hipGetLastError()) != hipSuccess) return err;
        }
        if (stages & UL_BWD_DKDV) {
            if ((err = allow_lds(attn_bwd_dkdv_bf16_kernel<64>, DkvTile<64>::kLds)) != hipSuccess) return err;
            hipLaunchKernelGGL(attn_bwd_dkdv_bf16_kernel<64>, dim3((uint32_t)kv_items), dim3(kKvThreads),
                               DkvTile<64>::kLds, stream, kp);
            if ((err = hipGetLastError()) != hipSuccess) return err;
            if ((err = reduce()) != hipSuccess) return err;
        }
    }
    return hipGetLastError();
}

hipError_t launch_attn_bwd_f32(const float *q, const float *k, const float *v, const float *o,
                               const float *dout, const float *lse, float *dq, float *dk,
                               float *dv, void *ws, const AttnShape &s, int stages, hipStream_t stream) {
    float *stats = static_cast<float *>(ws);
    hipError_t err = hipSuccess;
    if (stages & UL_BWD_PREP) {
        err = launch_pre(o, dout, lse, stats, s, false, stream);
        if (err != hipSuccess) return err;
    }
    BwdF32Params p{q, k, v, dout, lse, stats, dq, dk, dv, s.N, s.q_rs, s.k_rs, s.v_rs, s.do_rs,
                   s.dq_rs, s.dk_rs, s.dv_rs, s.cu, s.total, (int32_t)s.B, s.Hq, s.Hkv,
                   s.scale, s.causal, 0};
    p.n_blk = (int32_t)((s.N + kF32Rows - 1) / kF32Rows);
    const int64_t dq_items = (int64_t)p.n_blk * p.B * p.Hq;
    const int64_t kv_items = ((s.N + kF32KvKeys - 1) / kF32KvKeys) * p.B * p.Hkv;
    if (dq_items > 0x7fffffff || kv_items > 0x7fffffff) return hipErrorInvalidConfiguration;
    if (s.d == 128) {
        if (stages & UL_BWD_DQ) {
            hipLaunchKernelGGL(attn_bwd_dq_f32_kernel<128>, dim3((uint32_t)dq_items), dim3(kF32Rows), 0, stream, p);
            if ((err = hipGetLastError()) != hipSuccess) return err;
        }
        if (stages & UL_BWD_DKDV)
            hipLaunchKernelGGL(attn_bwd_dkdv_f32_kernel<128>, dim3((uint32_t)kv_items), dim3(kF32KvKeys), 0, stream, p);
    } else {
        if (stages & UL_BWD_DQ) {
            hipLaunchKernelGGL(attn_bwd_dq_f32_kernel<64>, dim3((uint32_t)dq_items), dim3(kF32Rows), 0, stream, p);
            if ((err = hipGetLastError()) != hipSuccess) return err;
        }
        if (stages & UL_BWD_DKDV)
            hipLaunchKernelGGL(attn_bwd_dkdv_f32_kernel<64>, dim3((uint32_t)kv_items), dim3(kF32KvKeys), 0, stream, p);
    }
    return hipGetLastError();
}

}  // namespace ul
