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
//  1. pre:   D = rowsum(dO * O) and lse in log2 units -> workspace (fp32).
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

#include <type_traits>
#include <utility>

#include "mfma_tile.h"
#include "ul_internal.h"

namespace ul {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

// ============================================================================ pre kernel

struct PreParams {
    const void *o, *dout;
    const float *lse;
    float *lse2, *Dv;
    int64_t N;
    int32_t B, Hq, d;
    int32_t is_bf16;
};

// 16 lanes per (b, i, h) row; each lane reduces d/16 elements.
__global__ __launch_bounds__(256) void bwd_pre_kernel(PreParams p) {
    const int64_t rows = (int64_t)p.B * p.N * p.Hq;
    const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
    const int sub = threadIdx.x & 15;
    float acc = 0.f;
    if (row < rows) {
        const int per = p.d / 16;
        const int64_t base = row * p.d + sub * per;
        if (p.is_bf16) {
            const uint16_t *o = static_cast<const uint16_t *>(p.o) + base;
            const uint16_t *g = static_cast<const uint16_t *>(p.dout) + base;
            for (int e = 0; e < per; ++e) acc = fmaf(bf16_to_f32(g[e]), bf16_to_f32(o[e]), acc);
        } else {
            const float *o = static_cast<const float *>(p.o) + base;
            const float *g = static_cast<const float *>(p.dout) + base;
            for (int e = 0; e < per; ++e) acc = fmaf(g[e], o[e], acc);
        }
    }
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 16);
    if (row < rows && sub == 0) {
        // row = (b*N + i)*Hq + h  ->  [b][h][i]
        const int64_t h = row % p.Hq;
        const int64_t bi = row / p.Hq;
        const int64_t i = bi % p.N, b = bi / p.N;
        const int64_t o = (b * p.Hq + h) * p.N + i;
        p.Dv[o] = acc;
        p.lse2[o] = p.lse[o] * kLog2e;
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
// A fragments read ahead of their MFMA: 6, but no more than the dQ steps of
// a tile, since the prefetch at the end of the softmax half covers only those.
template <int D>
constexpr int kQAhead = 2 * (D / 32) < 6 ? 2 * (D / 32) : 6;

struct DqParams {
    const uint16_t *q, *k, *v, *dout;
    const float *lse2, *Dv;
    uint16_t *dq;
    int32_t N, B, Hq, Hkv;
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
// `side(k)`, k < NSIDE, runs between MFMAs spread over the stream.
template <int D, bool DQ, bool SDP, int NSIDE, typename Side>
__device__ __forceinline__ void dq_gemm(f32x16 *dqacc, const bf16x8 (&dsf)[2], f32x16 &s, f32x16 &dp,
                                        const bf16x8 *qf, const bf16x8 *dof, bf16x8 (&ring)[kQAhead<D>],
                                        uint32_t pstage, uint32_t cstage, const DqOffs<D> &o, Side &&side) {
    constexpr int EB = D / 32, KK = D / 16;
    constexpr int NDQ = DQ ? 2 * EB : 0, NSD = SDP ? 2 * KK : 0, NSTEP = NDQ + NSD;
    static_assert(!DQ || NDQ >= kQAhead<D>, "the prefetched ring holds dQ steps only");
    constexpr int EVERY = NSIDE > 0 ? NSTEP / NSIDE : 1;
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
        dp = zero16();
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
        if constexpr (NSIDE > 0)
            if (st % EVERY == 1 && st / EVERY < NSIDE) side(st / EVERY);
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

// dS^T = P^T (dP^T - D) with P^T = exp2(S^T c - lse2), as two bf16 B
// fragments of 16 keys.  MASK zeroes P past the causal diagonal and the
// ragged end.
template <bool MASK>
__device__ __forceinline__ void dq_ds(bf16x8 (&dsf)[2], const f32x16 &s, const f32x16 &dp, float lse2, float Drow,
                                      int kg, int j0, int row, int N, int causal, float c) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        float ds[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int r = hh * 8 + q;
            float pv = __builtin_amdgcn_exp2f(fmaf(s[r], c, -lse2));
            if constexpr (MASK) {
                const int j = j0 + ckey(r, kg);
                if (j >= N || (causal && j > row)) pv = 0.f;
            }
            ds[q] = pv * (dp[r] - Drow);
        }
        dsf[hh] = pack8(ds);
    }
    // keep the exponentials here rather than sunk into the next MFMA half
#pragma unroll
    for (int i = 0; i < 2; ++i) asm volatile("" : "+v"(dsf[i]));
}

template <int D>
__global__ __launch_bounds__(kQThreads) void attn_bwd_dq_bf16_kernel(DqParams p) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    UL_LDS unsigned char *lds = (UL_LDS unsigned char *)smem_raw;
    using T = DqTile<D>;
    using Tile = DmaTile<D, kDqKT>;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int m = lane & 31, kg = lane >> 5;

    const int per_rank = p.B * p.Hkv * p.head_groups;
    const int rank = blockIdx.x / per_rank;
    int rest = blockIdx.x - rank * per_rank;
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
    const int N = p.N;
    const int row = i0 + m;
    const int64_t q_rs = (int64_t)p.Hq * D, kv_rs = (int64_t)p.Hkv * D;
    const uint16_t *qb = p.q + ((int64_t)b * N * p.Hq + h) * D;
    const uint16_t *dob = p.dout + ((int64_t)b * N * p.Hq + h) * D;

    constexpr int KK = D / 16, EB = D / 32;
    bf16x8 qf[KK], dof[KK];
    const bool ok = row < N;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
        qf[kk] = as_bf16x8(ok ? *reinterpret_cast<const u32x4 *>(qb + row * q_rs + kk * 16 + kg * 8)
                              : u32x4{0, 0, 0, 0});
        dof[kk] = as_bf16x8(ok ? *reinterpret_cast<const u32x4 *>(dob + row * q_rs + kk * 16 + kg * 8)
                               : u32x4{0, 0, 0, 0});
    }
    const int64_t so = ((int64_t)b * p.Hq + h) * N + (ok ? row : 0);
    const float lse2 = ok ? p.lse2[so] : 0.f;
    const float Drow = ok ? p.Dv[so] : 0.f;
    // Retire these loads: inside the loop vmcnt counts only the tile loads.
    __builtin_amdgcn_s_waitcnt(0x70);

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
    const uint16_t *tens = (loads_v ? p.v : p.k) + ((int64_t)b * N * p.Hkv + g) * D;
    const int tile_lds = loads_v ? T::kVBase : 0;
    const uint32_t row_bytes = (uint32_t)kv_rs * 2;
    uint32_t dma_roff[kDmaPerWave], dma_gran[kDmaPerWave];
#pragma unroll
    for (int k = 0; k < kDmaPerWave; ++k) {
        dma_roff[k] = (uint32_t)Tile::row(u0 + k, lane) * row_bytes;
        dma_gran[k] = Tile::gran_bytes(u0 + k, lane);
    }
    auto issue_k = [&](int t, int k, UL_LDS unsigned char *base) {
        const int j0 = t * kDqKT;
        const uint32_t lim = (uint32_t)(N - 1 - j0) * row_bytes;
        dma_b128(tens + (int64_t)j0 * kv_rs, min(dma_roff[k], lim) + dma_gran[k],
                 base + tile_lds + (u0 + k) * 1024);
    };
    auto issue = [&](int t, UL_LDS unsigned char *base) {
#pragma unroll
        for (int k = 0; k < kDmaPerWave; ++k) issue_k(t, k, base);
    };
    auto visible = [&](int t) { return !p.causal || t * kDqKT <= i0 + kRowsPerWave - 1; };

    // The forward's schedule with a deeper ring: waves 4-7 run one barrier
    // behind waves 0-3; tile t sits in stage t % 8 from its load (in the MFMA
    // half of tile t-6) to the lagging group's dQ of it (MFMA half of tile
    // t+1); each wave waits for its share of tile t+1 before the barrier
    // ending its MFMA half of tile t (all but the 5 newest tiles' loads).
    const bool lagging = wave >= kQWaves / 2;
    for (int t = 0; t < T::kAhead; ++t)
        if (t < ntiles) issue(t, lds + T::k_stage(t));
    if (ntiles >= T::kAhead)
        wait_vm_barrier<(T::kAhead - 1) * kDmaPerWave>();
    else
        wait_vm_barrier<0>();
    if (lagging) fence_barrier();

    f32x16 s, dp;
    bf16x8 dsf[2];
    bf16x8 ring[kQAhead<D>];
    auto body = [&](int t, auto full, auto stage) {
        constexpr bool FULL = decltype(full)::value;
        const bool more = t + T::kAhead < ntiles;
        UL_LDS unsigned char *nx = lds + stage(t + T::kAhead);
        if constexpr (FULL) {
            dq_gemm<D, true, true, kDmaPerWave>(dqacc, dsf, s, dp, qf, dof, ring, stage(t - 1), stage(t), fo,
                                                [&](int k) {
                                                    if (more) issue_k(t + T::kAhead, k, nx);
                                                });
        } else {
            if (more) issue(t + T::kAhead, nx);
            auto none = [](int) {};
            if (t >= 1 && visible(t - 1))
                dq_gemm<D, true, false, 0>(dqacc, dsf, s, dp, qf, dof, ring, stage(t - 1), 0, fo, none);
            if (t < ntiles && visible(t))
                dq_gemm<D, false, true, 0>(dqacc, dsf, s, dp, qf, dof, ring, 0, stage(t), fo, none);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (more)
            wait_vm_barrier<(T::kAhead - 1) * kDmaPerWave>();
        else
            wait_vm_barrier<0>();
        __builtin_amdgcn_sched_barrier(0);
        if (FULL || (t < ntiles && visible(t))) {
            if constexpr (FULL)
                dq_ds<false>(dsf, s, dp, lse2, Drow, kg, t * kDqKT, row, N, p.causal, c);
            else
                dq_ds<true>(dsf, s, dp, lse2, Drow, kg, t * kDqKT, row, N, p.causal, c);
            dq_prefetch<D>(ring, stage(t), fo);
        }
        fence_barrier();
    };
    auto rt_stage = [](int x) { return (uint32_t)T::k_stage(x & (T::kStages - 1)); };
    body(0, std::false_type{}, rt_stage);
    int t0 = 1;
    for (; t0 + T::kStages <= n_full; t0 += T::kStages) {
        [&]<int... J>(std::integer_sequence<int, J...>) {
            // x - t0 + 1 folds to a constant for every tile index body derives from t0 + J
            (body(t0 + J, std::true_type{},
                  [t0](int x) { return (uint32_t)T::k_stage((x - t0 + 1) & (T::kStages - 1)); }),
             ...);
        }(std::make_integer_sequence<int, T::kStages>{});
    }
    for (int t = t0; t <= ntiles; ++t) body(t, std::false_type{}, rt_stage);
    if (!lagging) fence_barrier();

    // dQ = scale * (dQ^T)^T, rounded to bf16: lane column = query row, registers = head dim
    if (ok) {
        uint16_t *out = p.dq + ((int64_t)b * N + row) * q_rs + (int64_t)h * D;
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

// ============================================================================ bf16: dK/dV kernel
//
// 8 waves per workgroup, 128 keys of one KV head: waves 0-3 are producers and
// waves 4-7 consumers; producer w and consumer w+4 share a SIMD and own the
// same 32 keys.  The workgroup steps over 32-row query tiles of every query
// head of the group, from the causal diagonal to N.
//   producer, step s:  S = Q K^T, dP = dO V^T   (A = Q / dO rows from LDS,
//                      B = K / V fragments held in registers), P = exp2(S c - lse2),
//                      dS = P (dP - D); the bf16 P and dS fragments go to LDS
//                      in the lane order of the consumer's B operand.
//   consumer, step s-1: dV^T += dO^T P, dK^T += Q^T dS  (A = dO^T / Q^T by
//                      transposed LDS reads), summed over the group's heads.
// The producer's softmax VALU work overlaps the consumer's MFMAs on the same
// SIMD, and each role stays inside a 256-register budget (2 waves per SIMD).
// Q/dO tiles rotate through 3 LDS stages (being filled / produced / consumed);
// P/dS through 2.

constexpr int kKvWaves = 8;
constexpr int kKvThreads = kKvWaves * 64;
constexpr int kKvPairs = 4;                          // producer/consumer pairs
constexpr int kKeysPerWave = 32;
constexpr int kKeysPerWg = kKvPairs * kKeysPerWave;  // 128
constexpr int kQT = 32;                              // query rows per step

struct DkvParams {
    const uint16_t *q, *k, *v, *dout;
    const float *lse2, *Dv;
    uint16_t *dk, *dv;
    int32_t N, B, Hq, Hkv;
    int32_t n_kblk;
    float scale_log2, scale;
    int32_t causal;
};

template <int D>
struct DkvTile {
    static constexpr int kBytes = kQT * D * 2;          // one Q or dO tile
    static constexpr int kStats = 2 * kQT * 4;          // lse2 then D, fp32
    static constexpr int kStage = 2 * kBytes + kStats;  // Q, dO, stats
    static constexpr int kPds = kKvPairs * 4 * 64 * 16; // P[2], dS[2] fragments per pair, per lane
    static constexpr int kAhead = 4;                    // steps of loads in flight
    static constexpr int kStages = kAhead + 2;          // + produced + consumed
    static constexpr int kPdsStages = 2;
    static constexpr int kPds0 = kStages * kStage;
    static constexpr int kLds = kPds0 + kPdsStages * kPds;
    __device__ static constexpr int stage(int st) { return st * kStage; }
    __device__ static constexpr int pds(int st) { return kPds0 + st * kPds; }
};

// Per-lane LDS offsets used inside the step loop (see precomputed lane offsets).
template <int D>
struct DkvOffs {
    static constexpr int KK = D / 16, EB = D / 32;
    uint32_t rm[KK];      // producer: Q / dO row fragment of k-step kk (row kperm(m))
    uint32_t stat;        // producer: first of the 8 statistics rows of this lane group
    uint32_t pds;         // both: this lane's P/dS fragment slot in its pair's block
    uint32_t tr[EB][2];   // consumer: transposed Q / dO fragment halves, rows 0..15
    __device__ __forceinline__ DkvOffs(int lane, int pair) {
        const int m = lane & 31, kg = lane >> 5;
        const int qrow = kperm(m);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) rm[kk] = rm_off<D>(qrow, kk * 2 + kg);
        stat = 2 * DkvTile<D>::kBytes + kg * 8 * 4;
        pds = (uint32_t)(pair * 4 * 64 + lane) * 16;
        const TrAddr<D> ta(lane);
#pragma unroll
        for (int eb = 0; eb < EB; ++eb) {
            tr[eb][0] = tr_off<D>(ta, eb * 32, 0);
            tr[eb][1] = tr_off<D>(ta, eb * 32, 1);
        }
    }
};

// Producer step on the Q/dO tile at `tile` (stage base): S, dP -> P, dS
// fragments -> the P/dS block at `pdsb`.  `masked` applies the causal diagonal
// and the ragged ends (only the softmax block is duplicated for it).
template <int D>
__device__ __forceinline__ void dkdv_produce(const bf16x8 *kf, const bf16x8 *vf,
                                             const UL_LDS unsigned char *tile, UL_LDS unsigned char *pdsb,
                                             const DkvOffs<D> &o, int kg, bool masked, int r0, int key,
                                             int N, int causal, float c) {
    using T = DkvTile<D>;
    constexpr int KK = D / 16;
    f32x16 s = zero16(), dp = zero16();
    bf16x8 aq = lds_frag(tile, o.rm[0]), ad = lds_frag(tile + T::kBytes, o.rm[0]);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
        bf16x8 nq = aq, nd = ad;
        if (kk + 1 < KK) {
            nq = lds_frag(tile, o.rm[kk + 1]);
            nd = lds_frag(tile + T::kBytes, o.rm[kk + 1]);
        }
        s = mfma32x32x16(aq, kf[kk], s);
        dp = mfma32x32x16(ad, vf[kk], dp);
        aq = nq;
        ad = nd;
        __builtin_amdgcn_sched_barrier(0);
    }
    // C register r of lane group kg holds query row ckey(r, kg): two runs of 8
    // consecutive rows (16*hh + 8*kg ..), so the row statistics load as float4s.
    float pv[16], dsv[16];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        const UL_LDS unsigned char *st = tile + o.stat + hh * 16 * 4;
        const f32x4 l0 = *reinterpret_cast<const UL_LDS f32x4 *>(st);
        const f32x4 l1 = *reinterpret_cast<const UL_LDS f32x4 *>(st + 16);
        const f32x4 d0 = *reinterpret_cast<const UL_LDS f32x4 *>(st + kQT * 4);
        const f32x4 d1 = *reinterpret_cast<const UL_LDS f32x4 *>(st + kQT * 4 + 16);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int r = hh * 8 + q;
            const float lz = q < 4 ? l0[q] : l1[q - 4];
            const float dz = q < 4 ? d0[q] : d1[q - 4];
            pv[r] = __builtin_amdgcn_exp2f(fmaf(s[r], c, -lz));
            dsv[r] = dp[r] - dz;
        }
    }
    if (masked) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int i = r0 + ckey(r, kg);
            if (i >= N || key >= N || (causal && key > i)) pv[r] = 0.f;
        }
    }
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        float ds8[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) ds8[q] = pv[hh * 8 + q] * dsv[hh * 8 + q];
        *reinterpret_cast<UL_LDS u32x4 *>(pdsb + o.pds + hh * 64 * 16) = __builtin_bit_cast(u32x4, pack8(pv + hh * 8));
        *reinterpret_cast<UL_LDS u32x4 *>(pdsb + o.pds + (2 + hh) * 64 * 16) = __builtin_bit_cast(u32x4, pack8(ds8));
    }
}

// Consumer step: dV^T += dO^T P ; dK^T += Q^T dS  (k = query rows, 2 steps of 16)
template <int D>
__device__ __forceinline__ void dkdv_consume(f32x16 *dkacc, f32x16 *dvacc, const UL_LDS unsigned char *tile,
                                             const UL_LDS unsigned char *pdsb, const DkvOffs<D> &o) {
    using T = DkvTile<D>;
    constexpr int EB = D / 32;
    bf16x8 pf[2], dsf[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        pf[hh] = lds_frag(pdsb, o.pds + hh * 64 * 16);
        dsf[hh] = lds_frag(pdsb, o.pds + (2 + hh) * 64 * 16);
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
        for (int eb = 0; eb < EB; ++eb) {
            const int rofs = ks * 16 * D * 2;
            const bf16x8 ado = lds_tr_frag(tile + T::kBytes + rofs, o.tr[eb][0], o.tr[eb][1]);
            const bf16x8 aq = lds_tr_frag(tile + rofs, o.tr[eb][0], o.tr[eb][1]);
            dvacc[eb] = mfma32x32x16(ado, pf[ks], dvacc[eb]);
            dkacc[eb] = mfma32x32x16(aq, dsf[ks], dkacc[eb]);
        }
    }
}

template <int D>
__global__ __launch_bounds__(kKvThreads) void attn_bwd_dkdv_bf16_kernel(DkvParams p) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    UL_LDS unsigned char *lds = (UL_LDS unsigned char *)smem_raw;
    using T = DkvTile<D>;
    using Tile = DmaTile<D, kQT>;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int m = lane & 31, kg = lane >> 5;
    const bool producer = wave < kKvPairs;
    const int pair = producer ? wave : wave - kKvPairs;

    // item = kblk * (B*Hkv) + (b*Hkv + g): key block 0 (the most work) first
    const int per_rank = p.B * p.Hkv;
    const int kblk = blockIdx.x / per_rank;
    const int bg = blockIdx.x - kblk * per_rank;
    const int b = bg / p.Hkv, g = bg % p.Hkv;
    const int grp = p.Hq / p.Hkv;
    const int N = p.N;
    const int64_t q_rs = (int64_t)p.Hq * D;
    const int kb0 = kblk * kKeysPerWg;
    const int jw0 = kb0 + pair * kKeysPerWave;  // the pair's first key
    const int key = jw0 + m;                    // this lane's key (C column)

    // Steps: 32-row tiles from the end of the sequence down to the causal
    // diagonal, the group's query heads innermost.  Every workgroup walks the
    // rows in the same order, so workgroups resident at the same time stream
    // the same Q/dO tiles and share them through L2.  A cursor (step, head
    // within the group, first row) advances one step at a time.
    const int qt_first = p.causal ? kb0 / kQT : 0;
    const int nqt = (N + kQT - 1) / kQT;
    const int per_head = nqt - qt_first;
    const int nsteps = per_head * grp;
    struct Cur {
        int s, hi, r0;
    };
    auto advance = [&](Cur &cu) {  // stays on the last step once there
        if (cu.s + 1 < nsteps) {
            ++cu.s;
            if (++cu.hi == grp) {
                cu.hi = 0;
                cu.r0 -= kQT;
            }
        }
    };
    const Cur first{0, 0, (nqt - 1) * kQT};
    const float c = p.scale_log2;
    const DkvOffs<D> o(lane, pair);

    // Direct loads of a step into its LDS stage: the Q and dO tiles are split
    // evenly over the 8 waves (each wave's share lies in one of the two), and
    // the last wave also fetches the 32 lse2 and D values, one dword per lane.
    // Rows past N re-read row N-1 (masked by the producer).
    constexpr int kDmaPerWave = 2 * Tile::INSTR / kKvWaves;  // per step; the last wave has one more
    static_assert(2 * Tile::INSTR % kKvWaves == 0 && Tile::INSTR % kDmaPerWave == 0,
                  "Q and dO tiles split evenly over the waves");
    const bool loads_do = wave * kDmaPerWave >= Tile::INSTR;
    const int u0 = (wave * kDmaPerWave) % Tile::INSTR;
    const uint16_t *tens = loads_do ? p.dout : p.q;
    const int tile_lds = loads_do ? T::kBytes : 0;
    const uint32_t row_bytes = (uint32_t)q_rs * 2;
    int dma_row[kDmaPerWave];
    uint32_t dma_gran[kDmaPerWave];
#pragma unroll
    for (int k = 0; k < kDmaPerWave; ++k) {
        dma_row[k] = Tile::row(u0 + k, lane);
        dma_gran[k] = Tile::gran_bytes(u0 + k, lane);
    }
    const int64_t dv_delta = (const char *)p.Dv - (const char *)p.lse2;
    const bool stats_wave = wave == kKvWaves - 1;
    auto issue = [&](const Cur &cu, UL_LDS unsigned char *base) {
        const int lim = N - 1 - cu.r0;  // last valid row within the tile
        const int h = g * grp + cu.hi;
        const uint16_t *tb = tens + (((int64_t)b * N + cu.r0) * p.Hq + h) * D;
#pragma unroll
        for (int k = 0; k < kDmaPerWave; ++k)
            dma_b128(tb, (uint32_t)min(dma_row[k], lim) * row_bytes + dma_gran[k],
                     base + tile_lds + (u0 + k) * 1024);
        if (stats_wave) {
            const char *sb = (const char *)(p.lse2 + ((int64_t)b * p.Hq + h) * N + cu.r0);
            const int r = min(lane & (kQT - 1), lim);
            // lanes 0..31 read lse2, lanes 32..63 read D (a fixed distance away)
            if (lane < kQT)
                dma_b32(sb, (uint32_t)r * 4, base + 2 * T::kBytes);
            else
                dma_b32(sb + dv_delta, (uint32_t)r * 4, base + 2 * T::kBytes);
        }
    };
    // the pair's keys see at least one row of a step starting at row r0
    auto visible = [&](int r0) { return (!p.causal || jw0 <= r0 + kQT - 1) && jw0 < N; };

    // Loads always run kAhead steps ahead (past the last step they re-read it
    // into a free stage), so every wave has the same number in flight at each
    // barrier: waiting for all but the newest (kAhead-1) steps' worth leaves
    // the oldest one landed.
    Cur iss = first;
    [&]<int... J>(std::integer_sequence<int, J...>) {
        ((issue(iss, lds + T::stage(J)), advance(iss)), ...);
    }(std::make_integer_sequence<int, T::kAhead>{});
    wait_vm_barrier<(T::kAhead - 1) * kDmaPerWave>();

    // Iteration i (LDS stage i % 6, unrolled by 6 so stages are immediates):
    // issue step i+4, producers handle step i, consumers step i-1; the
    // barrier at the end waits for step i+1, the oldest load still in flight.
    auto run = [&](auto body) {
        for (int i0 = 0; i0 <= nsteps; i0 += T::kStages) {
            [&]<int... J>(std::integer_sequence<int, J...>) {
                ((i0 + J <= nsteps ? body(i0 + J, std::integral_constant<int, J>{}) : void()), ...);
            }(std::make_integer_sequence<int, T::kStages>{});
        }
        // no load may still be writing this workgroup's LDS when it exits
        __builtin_amdgcn_s_waitcnt(0x70);
    };

    if (producer) {
        // K and V rows of the pair's 32 keys as B fragments (column = key, k = head dim)
        constexpr int KK = D / 16;
        bf16x8 kf[KK], vf[KK];
        {
            const bool ok = key < N;
            const uint16_t *kr = p.k + (((int64_t)b * N + (ok ? key : 0)) * p.Hkv + g) * D;
            const uint16_t *vr = p.v + (((int64_t)b * N + (ok ? key : 0)) * p.Hkv + g) * D;
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                kf[kk] = as_bf16x8(ok ? *reinterpret_cast<const u32x4 *>(kr + kk * 16 + kg * 8) : u32x4{0, 0, 0, 0});
                vf[kk] = as_bf16x8(ok ? *reinterpret_cast<const u32x4 *>(vr + kk * 16 + kg * 8) : u32x4{0, 0, 0, 0});
            }
        }
        // Retire these loads here: inside the loop vmcnt must count only the
        // stage loads, or a wait for a fragment would also wait for the
        // newest stage.
        __builtin_amdgcn_s_waitcnt(0x70);
        Cur cmp = first;
        run([&](int i, auto stage) {
            constexpr int ST = decltype(stage)::value, NN = (ST + T::kAhead) % T::kStages, PD = ST % 2;
            issue(iss, lds + T::stage(NN));
            advance(iss);
            if (i < nsteps && visible(cmp.r0)) {
                const int r0 = cmp.r0;
                const bool masked = (p.causal && r0 < kb0 + kKeysPerWg) || r0 + kQT > N ||
                                    kb0 + kKeysPerWg > N;
                dkdv_produce<D>(kf, vf, lds + T::stage(ST), lds + T::pds(PD), o, kg, masked, r0, key, N,
                                p.causal, c);
            }
            advance(cmp);
            wait_vm_barrier<(T::kAhead - 1) * kDmaPerWave>();
        });
        return;
    }

    constexpr int EB = D / 32;
    f32x16 dkacc[EB], dvacc[EB];
#pragma unroll
    for (int eb = 0; eb < EB; ++eb) {
        dkacc[eb] = zero16();
        dvacc[eb] = zero16();
    }
    Cur cmp = first;
    run([&](int i, auto stage) {
        constexpr int ST = decltype(stage)::value, NN = (ST + T::kAhead) % T::kStages;
        constexpr int PV = (ST + T::kStages - 1) % T::kStages, PD = (ST + 1) % 2;
        issue(iss, lds + T::stage(NN));
        advance(iss);
        if (i >= 1) {
            if (visible(cmp.r0)) dkdv_consume<D>(dkacc, dvacc, lds + T::stage(PV), lds + T::pds(PD), o);
            advance(cmp);
        }
        wait_vm_barrier<(T::kAhead - 1) * kDmaPerWave>();
    });

    // dK = scale * acc, dV = acc (bf16); lane column = key, registers = head dim
    if (key < N) {
        uint16_t *dkr = p.dk + (((int64_t)b * N + key) * p.Hkv + g) * D;
        uint16_t *dvr = p.dv + (((int64_t)b * N + key) * p.Hkv + g) * D;
#pragma unroll
        for (int eb = 0; eb < EB; ++eb)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                bf16x4 k4, v4;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    k4[q] = (__bf16)(dkacc[eb][r4 * 4 + q] * p.scale);
                    v4[q] = (__bf16)(dvacc[eb][r4 * 4 + q]);
                }
                const int e = eb * 32 + r4 * 8 + kg * 4;
                *reinterpret_cast<u32x2 *>(dkr + e) = __builtin_bit_cast(u32x2, k4);
                *reinterpret_cast<u32x2 *>(dvr + e) = __builtin_bit_cast(u32x2, v4);
            }
    }
}

// ============================================================================ fp32 kernels

constexpr int kF32Rows = 64;
constexpr int kF32Keys = 32;

struct BwdF32Params {
    const float *q, *k, *v, *dout;
    const float *lse, *Dv;  // lse in natural-log units
    float *dq, *dk, *dv;
    int64_t N;
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
    const int64_t N = p.N;
    const int64_t i = (int64_t)rblk * kF32Rows + tid;
    const bool valid = i < N;
    const int64_t ri = valid ? i : 0;
    float qv[D], dov[D], acc[D];
    const float *qrow = p.q + (((int64_t)b * N + ri) * p.Hq + h) * D;
    const float *drow = p.dout + (((int64_t)b * N + ri) * p.Hq + h) * D;
#pragma unroll
    for (int e = 0; e < D; ++e) {
        qv[e] = valid ? qrow[e] : 0.f;
        dov[e] = valid ? drow[e] : 0.f;
        acc[e] = 0.f;
    }
    const int64_t so = ((int64_t)b * p.Hq + h) * N + ri;
    const float lse = valid ? p.lse[so] : 0.f;
    const float Di = valid ? p.Dv[so] : 0.f;
    const int64_t blk_last = (int64_t)rblk * kF32Rows + kF32Rows - 1;
    const int64_t kend = p.causal ? (blk_last + 1 < N ? blk_last + 1 : N) : N;
    for (int64_t j0 = 0; j0 < kend; j0 += kF32Keys) {
        __syncthreads();
        for (int idx = tid; idx < kF32Keys * D; idx += kF32Rows) {
            const int jj = idx / D, e = idx % D;
            const int64_t j = j0 + jj;
            const int64_t off = (((int64_t)b * N + j) * p.Hkv + g) * D + e;
            ks[jj][e] = j < N ? p.k[off] : 0.f;
            vs[jj][e] = j < N ? p.v[off] : 0.f;
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
            const float ds = pr * (dp - Di);
#pragma unroll
            for (int e = 0; e < D; ++e) acc[e] = fmaf(ds, ks[jj][e], acc[e]);
        }
    }
    if (valid) {
        float *out = p.dq + (((int64_t)b * N + i) * p.Hq + h) * D;
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
    __shared__ float ls[kF32KvRows], Ds[kF32KvRows];
    const int tid = threadIdx.x;
    const int bg = blockIdx.x % (p.B * p.Hkv);
    const int kblk = blockIdx.x / (p.B * p.Hkv);
    const int b = bg / p.Hkv, g = bg % p.Hkv;
    const int grp = p.Hq / p.Hkv;
    const int64_t N = p.N;
    const int64_t j = (int64_t)kblk * kF32KvKeys + tid;
    const bool valid = j < N;
    const int64_t rj = valid ? j : 0;
    for (int e = 0; e < D; ++e) {
        kown[tid][e] = valid ? p.k[(((int64_t)b * N + rj) * p.Hkv + g) * D + e] : 0.f;
        vown[tid][e] = valid ? p.v[(((int64_t)b * N + rj) * p.Hkv + g) * D + e] : 0.f;
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
                const int64_t off = (((int64_t)b * N + i) * p.Hq + h) * D + e;
                qs[ii][e] = i < N ? p.q[off] : 0.f;
                ds_[ii][e] = i < N ? p.dout[off] : 0.f;
            }
            if (tid < kF32KvRows) {
                const int64_t i = i0 + tid;
                const int64_t so = ((int64_t)b * p.Hq + h) * N + i;
                ls[tid] = i < N ? p.lse[so] : 0.f;
                Ds[tid] = i < N ? p.Dv[so] : 0.f;
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
                const float dsv = pr * (dp - Ds[ii]);
#pragma unroll
                for (int e = 0; e < D; ++e) {
                    dk[e] = fmaf(dsv, qs[ii][e], dk[e]);
                    dv[e] = fmaf(pr, ds_[ii][e], dv[e]);
                }
            }
        }
    }
    if (valid) {
        float *dkr = p.dk + (((int64_t)b * N + j) * p.Hkv + g) * D;
        float *dvr = p.dv + (((int64_t)b * N + j) * p.Hkv + g) * D;
#pragma unroll
        for (int e = 0; e < D; ++e) {
            dkr[e] = dk[e] * p.scale;
            dvr[e] = dv[e];
        }
    }
}

size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

size_t attn_bwd_workspace_bytes(const AttnShape &s, int32_t /*dtype*/) {
    const size_t rows = (size_t)s.B * (size_t)s.Hq * (size_t)s.N;
    return 2 * round256(rows * sizeof(float));
}

static hipError_t launch_pre(const void *o, const void *dout, const float *lse, float *lse2,
                             float *Dv, const AttnShape &s, bool bf16, hipStream_t stream) {
    PreParams pp{o, dout, lse, lse2, Dv, s.N, (int32_t)s.B, s.Hq, s.d, bf16 ? 1 : 0};
    const int64_t rows = s.B * s.N * s.Hq;
    const int64_t blocks = (rows + 15) / 16;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(bwd_pre_kernel, dim3((uint32_t)blocks), dim3(256), 0, stream, pp);
    return hipGetLastError();
}

hipError_t launch_attn_bwd_bf16(const void *q, const void *k, const void *v, const void *o,
                                const void *dout, const float *lse, void *dq, void *dk, void *dv,
                                void *ws, const AttnShape &s, int stages, hipStream_t stream) {
    const size_t rows = (size_t)s.B * (size_t)s.Hq * (size_t)s.N;
    float *lse2 = static_cast<float *>(ws);
    float *Dv = reinterpret_cast<float *>(static_cast<char *>(ws) + round256(rows * sizeof(float)));
    hipError_t err = hipSuccess;
    if (stages & UL_BWD_PREP) {
        err = launch_pre(o, dout, lse, lse2, Dv, s, true, stream);
        if (err != hipSuccess) return err;
    }

    DqParams dp;
    dp.q = static_cast<const uint16_t *>(q);
    dp.k = static_cast<const uint16_t *>(k);
    dp.v = static_cast<const uint16_t *>(v);
    dp.dout = static_cast<const uint16_t *>(dout);
    dp.lse2 = lse2;
    dp.Dv = Dv;
    dp.dq = static_cast<uint16_t *>(dq);
    dp.N = (int32_t)s.N;
    dp.B = (int32_t)s.B;
    dp.Hq = s.Hq;
    dp.Hkv = s.Hkv;
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
    kp.lse2 = lse2;
    kp.Dv = Dv;
    kp.dk = static_cast<uint16_t *>(dk);
    kp.dv = static_cast<uint16_t *>(dv);
    kp.N = (int32_t)s.N;
    kp.B = (int32_t)s.B;
    kp.Hq = s.Hq;
    kp.Hkv = s.Hkv;
    kp.n_kblk = (int32_t)((s.N + kKeysPerWg - 1) / kKeysPerWg);
    kp.scale_log2 = dp.scale_log2;
    kp.scale = s.scale;
    kp.causal = s.causal;
    const int64_t kv_items = (int64_t)kp.n_kblk * kp.B * kp.Hkv;
    if (kv_items > 0x7fffffff) return hipErrorInvalidConfiguration;

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
        }
    }
    return hipGetLastError();
}

hipError_t launch_attn_bwd_f32(const float *q, const float *k, const float *v, const float *o,
                               const float *dout, const float *lse, float *dq, float *dk,
                               float *dv, void *ws, const AttnShape &s, int stages, hipStream_t stream) {
    const size_t rows = (size_t)s.B * (size_t)s.Hq * (size_t)s.N;
    float *lse2 = static_cast<float *>(ws);
    float *Dv = reinterpret_cast<float *>(static_cast<char *>(ws) + round256(rows * sizeof(float)));
    hipError_t err = hipSuccess;
    if (stages & UL_BWD_PREP) {
        err = launch_pre(o, dout, lse, lse2, Dv, s, false, stream);
        if (err != hipSuccess) return err;
    }
    BwdF32Params p{q, k, v, dout, lse, Dv, dq, dk, dv, s.N, (int32_t)s.B, s.Hq, s.Hkv,
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
