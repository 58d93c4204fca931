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

constexpr int kWaves = 4;
constexpr int kRowsPerWave = 64;
constexpr int kKT = 64;

struct DqParams {
    const uint16_t *q, *k, *v, *dout;
    const float *lse2, *Dv;
    uint16_t *dq;
    int64_t N;
    int32_t B, Hq, Hkv;
    int32_t heads_per_wg, pos_blocks, head_groups, n_qblk;
    float scale_log2, scale;
    int32_t causal;
};

template <int D>
struct DqSmem {
    u32x4 kt[2][kKT * D / 8];   // K rows (row-major, swizzled)
    u32x4 vt[2][kKT * D / 8];   // V rows
    u32x4 ktt[2][D * kKT / 8];  // K^T
};

template <int D>
struct DqTileRegs {
    static constexpr int kRowUnits = kKT * (D / 8) / (kWaves * 64);
    static constexpr int kPairUnits = (kKT / 2) * (D / 8) / (kWaves * 64);
    u32x4 k[kRowUnits], v[kRowUnits];
    u32x4 t0[kPairUnits], t1[kPairUnits];
};

template <int D>
__device__ __forceinline__ void load_rows(u32x4 *dst, const uint16_t *__restrict__ base,
                                          int64_t row_stride, int64_t r0, int64_t N, int tid,
                                          int units) {
    constexpr int GPR = D / 8;
    for (int u = 0; u < units; ++u) {
        const int idx = tid + u * kWaves * 64;
        const int row = idx / GPR, gran = idx % GPR;
        const int64_t r = r0 + row;
        dst[u] = (r < N) ? *reinterpret_cast<const u32x4 *>(base + r * row_stride + gran * 8)
                         : u32x4{0, 0, 0, 0};
    }
}

template <int D>
__device__ __forceinline__ void load_pairs(u32x4 *d0, u32x4 *d1, const uint16_t *__restrict__ base,
                                           int64_t row_stride, int64_t r0, int64_t N, int tid,
                                           int units) {
    constexpr int GPR = D / 8;
    for (int u = 0; u < units; ++u) {
        const int idx = tid + u * kWaves * 64;
        const int kp = idx / GPR, gran = idx % GPR;
        const int64_t r = r0 + 2 * kp;
        d0[u] = (r < N) ? *reinterpret_cast<const u32x4 *>(base + r * row_stride + gran * 8)
                        : u32x4{0, 0, 0, 0};
        d1[u] = (r + 1 < N) ? *reinterpret_cast<const u32x4 *>(base + (r + 1) * row_stride + gran * 8)
                            : u32x4{0, 0, 0, 0};
    }
}

template <int D>
__device__ __forceinline__ void store_rows(u32x4 *tile, const u32x4 *src, int tid, int units) {
    constexpr int GPR = D / 8;
    for (int u = 0; u < units; ++u) {
        const int idx = tid + u * kWaves * 64;
        tile[rm_slot<D>(idx / GPR, idx % GPR)] = src[u];
    }
}

// Transposed store: rows (2kp, 2kp+1) x d-granule -> 8 packed words of the
// [D][64] transposed tile.
template <int D>
__device__ __forceinline__ void store_pairs_t(u32x4 *tile, const u32x4 *s0, const u32x4 *s1, int tid,
                                              int units) {
    constexpr int GPR = D / 8;
    uint32_t *t32 = reinterpret_cast<uint32_t *>(tile);
    for (int u = 0; u < units; ++u) {
        const int idx = tid + u * kWaves * 64;
        const int kp = idx / GPR, gran = idx % GPR;
        const int kgran = kp >> 2, within = kp & 3;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const uint32_t a = s0[u][s >> 1], b = s1[u][s >> 1];
            const uint32_t lo = (s & 1) ? (a >> 16) : (a & 0xffffu);
            const uint32_t hi = (s & 1) ? (b & 0xffff0000u) : (b << 16);
            t32[tr_slot<64>(gran * 8 + s, kgran) * 4 + within] = lo | hi;
        }
    }
}

template <int D>
__global__ __launch_bounds__(kWaves * 64, 1) void attn_bwd_dq_bf16_kernel(DqParams p) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    DqSmem<D> &sm = *reinterpret_cast<DqSmem<D> *>(smem_raw);
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
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
    const int64_t wg_pos0 = (int64_t)qblk * kRowsPerWave * p.pos_blocks;
    const int64_t i0 = wg_pos0 + (int64_t)(wave / p.heads_per_wg) * kRowsPerWave;
    const int64_t N = p.N;
    const int64_t q_rs = (int64_t)p.Hq * D, kv_rs = (int64_t)p.Hkv * D;
    const uint16_t *qb = p.q + ((int64_t)b * N * p.Hq + h) * D;
    const uint16_t *dob = p.dout + ((int64_t)b * N * p.Hq + h) * D;
    const uint16_t *kb = p.k + ((int64_t)b * N * p.Hkv + g) * D;
    const uint16_t *vb = p.v + ((int64_t)b * N * p.Hkv + g) * D;

    constexpr int KK = D / 16, EB = D / 32;
    bf16x8 qf[2][KK], dof[2][KK];
    float lse2[2], Drow[2];
#pragma unroll
    for (int ib = 0; ib < 2; ++ib) {
        const int64_t i = i0 + ib * 32 + m;
        const bool ok = i < N;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            qf[ib][kk] = as_bf16x8(ok ? *reinterpret_cast<const u32x4 *>(qb + i * q_rs + kk * 16 + kg * 8)
                                      : u32x4{0, 0, 0, 0});
            dof[ib][kk] = as_bf16x8(ok ? *reinterpret_cast<const u32x4 *>(dob + i * q_rs + kk * 16 + kg * 8)
                                       : u32x4{0, 0, 0, 0});
        }
        const int64_t so = ((int64_t)b * p.Hq + h) * N + (ok ? i : 0);
        lse2[ib] = ok ? p.lse2[so] : 0.f;
        Drow[ib] = ok ? p.Dv[so] : 0.f;
    }

    f32x16 dqacc[EB][2];
#pragma unroll
    for (int eb = 0; eb < EB; ++eb)
#pragma unroll
        for (int ib = 0; ib < 2; ++ib)
#pragma unroll
            for (int r = 0; r < 16; ++r) dqacc[eb][ib][r] = 0.f;

    const int64_t wg_end = wg_pos0 + kRowsPerWave * p.pos_blocks;
    const int64_t kend = p.causal ? (N < wg_end ? N : wg_end) : N;
    const int ntiles = (int)((kend + kKT - 1) / kKT);
    const int64_t wave_last_row = i0 + kRowsPerWave - 1;

    DqTileRegs<D> tr;
    load_rows<D>(tr.k, kb, kv_rs, 0, N, tid, DqTileRegs<D>::kRowUnits);
    load_rows<D>(tr.v, vb, kv_rs, 0, N, tid, DqTileRegs<D>::kRowUnits);
    load_pairs<D>(tr.t0, tr.t1, kb, kv_rs, 0, N, tid, DqTileRegs<D>::kPairUnits);
    store_rows<D>(sm.kt[0], tr.k, tid, DqTileRegs<D>::kRowUnits);
    store_rows<D>(sm.vt[0], tr.v, tid, DqTileRegs<D>::kRowUnits);
    store_pairs_t<D>(sm.ktt[0], tr.t0, tr.t1, tid, DqTileRegs<D>::kPairUnits);
    __syncthreads();

    for (int t = 0; t < ntiles; ++t) {
        const int st = t & 1;
        const int64_t j0 = (int64_t)t * kKT;
        if (t + 1 < ntiles) {
            load_rows<D>(tr.k, kb, kv_rs, j0 + kKT, N, tid, DqTileRegs<D>::kRowUnits);
            load_rows<D>(tr.v, vb, kv_rs, j0 + kKT, N, tid, DqTileRegs<D>::kRowUnits);
            load_pairs<D>(tr.t0, tr.t1, kb, kv_rs, j0 + kKT, N, tid, DqTileRegs<D>::kPairUnits);
        }
        const bool active = !p.causal || j0 <= wave_last_row;
        if (active) {
            const bool need_mask = (p.causal && j0 + kKT - 1 > i0) || j0 + kKT > N;
#pragma unroll
            for (int js = 0; js < 2; ++js) {
                f32x16 sacc[2], pacc[2];
#pragma unroll
                for (int ib = 0; ib < 2; ++ib)
#pragma unroll
                    for (int r = 0; r < 16; ++r) { sacc[ib][r] = 0.f; pacc[ib][r] = 0.f; }
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) {
                    const int row = js * 32 + kperm(m);
                    const bf16x8 ak = as_bf16x8(sm.kt[st][rm_slot<D>(row, kk * 2 + kg)]);
                    const bf16x8 av = as_bf16x8(sm.vt[st][rm_slot<D>(row, kk * 2 + kg)]);
#pragma unroll
                    for (int ib = 0; ib < 2; ++ib) {
                        sacc[ib] = mfma32x32x16(ak, qf[ib][kk], sacc[ib]);
                        pacc[ib] = mfma32x32x16(av, dof[ib][kk], pacc[ib]);
                    }
                }
                // dS^T = P^T (dP^T - D), P^T = exp2(S^T * c - lse2)
                bf16x8 dsf[2][2];
#pragma unroll
                for (int ib = 0; ib < 2; ++ib) {
                    const int64_t i = i0 + ib * 32 + m;
                    float ds[16];
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        float pv = __builtin_amdgcn_exp2f(fmaf(sacc[ib][r], p.scale_log2, -lse2[ib]));
                        if (need_mask) {
                            const int64_t j = j0 + js * 32 + ckey(r, kg);
                            if (j >= N || (p.causal && j > i)) pv = 0.f;
                        }
                        ds[r] = pv * (pacc[ib][r] - Drow[ib]);
                    }
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh)
                        dsf[hh][ib] = pack8(ds[hh * 8 + 0], ds[hh * 8 + 1], ds[hh * 8 + 2], ds[hh * 8 + 3],
                                            ds[hh * 8 + 4], ds[hh * 8 + 5], ds[hh * 8 + 6], ds[hh * 8 + 7]);
                }
                // dQ^T += K^T dS^T over this subtile's 32 keys (2 k-steps of 16)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
                    for (int eb = 0; eb < EB; ++eb) {
                        const bf16x8 a = as_bf16x8(sm.ktt[st][tr_slot<64>(eb * 32 + m, (js * 2 + hh) * 2 + kg)]);
#pragma unroll
                        for (int ib = 0; ib < 2; ++ib) dqacc[eb][ib] = mfma32x32x16(a, dsf[hh][ib], dqacc[eb][ib]);
                    }
                }
            }
        }
        if (t + 1 < ntiles) {
            store_rows<D>(sm.kt[st ^ 1], tr.k, tid, DqTileRegs<D>::kRowUnits);
            store_rows<D>(sm.vt[st ^ 1], tr.v, tid, DqTileRegs<D>::kRowUnits);
            store_pairs_t<D>(sm.ktt[st ^ 1], tr.t0, tr.t1, tid, DqTileRegs<D>::kPairUnits);
        }
        __syncthreads();
    }

    // dQ = scale * dQ^T^T, rounded to bf16
#pragma unroll
    for (int ib = 0; ib < 2; ++ib) {
        const int64_t i = i0 + ib * 32 + m;
        if (i >= N) continue;
        uint16_t *row = p.dq + ((int64_t)b * N + i) * q_rs + (int64_t)h * D;
#pragma unroll
        for (int eb = 0; eb < EB; ++eb)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                bf16x4 o4;
#pragma unroll
                for (int s = 0; s < 4; ++s) o4[s] = (__bf16)(dqacc[eb][ib][r4 * 4 + s] * p.scale);
                *reinterpret_cast<u32x2 *>(row + eb * 32 + r4 * 8 + kg * 4) = __builtin_bit_cast(u32x2, o4);
            }
    }
}

// ============================================================================ bf16: dK/dV kernel

constexpr int kKeysPerWave = 32;
constexpr int kKeysPerWg = kWaves * kKeysPerWave;  // 128
constexpr int kQT = 64;                            // query rows per step

struct DkvParams {
    const uint16_t *q, *k, *v, *dout;
    const float *lse2, *Dv;
    uint16_t *dk, *dv;
    int64_t N;
    int32_t B, Hq, Hkv;
    int32_t n_kblk;
    float scale_log2, scale;
    int32_t causal;
};

template <int D>
struct DkvSmem {
    u32x4 qt[2][kQT * D / 8];    // Q rows
    u32x4 dot[2][kQT * D / 8];   // dO rows
    u32x4 qtt[2][D * kQT / 8];   // Q^T
    u32x4 dott[2][D * kQT / 8];  // dO^T
    float lse2[2][kQT];
    float Dv[2][kQT];
};

template <int D>
struct DkvTileRegs {
    static constexpr int kRowUnits = kQT * (D / 8) / (kWaves * 64);
    static constexpr int kPairUnits = (kQT / 2) * (D / 8) / (kWaves * 64);
    u32x4 q[kRowUnits], d[kRowUnits];
    u32x4 q0[kPairUnits], q1[kPairUnits], d0[kPairUnits], d1[kPairUnits];
    float st;  // lse2 (tid < 64) or D (64 <= tid < 128)
};

template <int D>
__global__ __launch_bounds__(kWaves * 64, 1) void attn_bwd_dkdv_bf16_kernel(DkvParams p) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    DkvSmem<D> &sm = *reinterpret_cast<DkvSmem<D> *>(smem_raw);
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int m = lane & 31, kg = lane >> 5;

    // item = kblk * (B*Hkv) + (b*Hkv + g): key block 0 (the most work) first
    const int per_rank = p.B * p.Hkv;
    const int kblk = blockIdx.x / per_rank;
    const int bg = blockIdx.x - kblk * per_rank;
    const int b = bg / p.Hkv, g = bg % p.Hkv;
    const int grp = p.Hq / p.Hkv;
    const int64_t N = p.N;
    const int64_t q_rs = (int64_t)p.Hq * D, kv_rs = (int64_t)p.Hkv * D;
    const int64_t kb0 = (int64_t)kblk * kKeysPerWg;
    const int64_t jw0 = kb0 + wave * kKeysPerWave;  // this wave's first key

    constexpr int KK = D / 16, EB = D / 32;
    // K and V fragments of this wave's 32 keys: B operand (column = key, k = head dim)
    bf16x8 kf[KK], vf[KK];
    {
        const int64_t j = jw0 + m;
        const bool ok = j < N;
        const uint16_t *kr = p.k + (((int64_t)b * N + (ok ? j : 0)) * p.Hkv + g) * D;
        const uint16_t *vr = p.v + (((int64_t)b * N + (ok ? j : 0)) * p.Hkv + g) * D;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            kf[kk] = as_bf16x8(ok ? *reinterpret_cast<const u32x4 *>(kr + kk * 16 + kg * 8) : u32x4{0, 0, 0, 0});
            vf[kk] = as_bf16x8(ok ? *reinterpret_cast<const u32x4 *>(vr + kk * 16 + kg * 8) : u32x4{0, 0, 0, 0});
        }
    }
    f32x16 dkacc[EB], dvacc[EB];
#pragma unroll
    for (int eb = 0; eb < EB; ++eb)
#pragma unroll
        for (int r = 0; r < 16; ++r) { dkacc[eb][r] = 0.f; dvacc[eb][r] = 0.f; }

    // Steps: every query head of the group x query tiles from the diagonal.
    const int64_t qt_first = p.causal ? kb0 / kQT : 0;
    const int64_t nqt = (N + kQT - 1) / kQT;
    const int64_t per_head = nqt - qt_first;
    const int64_t nsteps = per_head * grp;

    auto step_rows = [&](int64_t s, int &h, int64_t &r0) {
        h = g * grp + (int)(s / per_head);
        r0 = (qt_first + s % per_head) * kQT;
    };
    auto load_step = [&](DkvTileRegs<D> &tr, int64_t s) {
        int h;
        int64_t r0;
        step_rows(s, h, r0);
        const uint16_t *qb = p.q + ((int64_t)b * N * p.Hq + h) * D;
        const uint16_t *db = p.dout + ((int64_t)b * N * p.Hq + h) * D;
        load_rows<D>(tr.q, qb, q_rs, r0, N, tid, DkvTileRegs<D>::kRowUnits);
        load_rows<D>(tr.d, db, q_rs, r0, N, tid, DkvTileRegs<D>::kRowUnits);
        load_pairs<D>(tr.q0, tr.q1, qb, q_rs, r0, N, tid, DkvTileRegs<D>::kPairUnits);
        load_pairs<D>(tr.d0, tr.d1, db, q_rs, r0, N, tid, DkvTileRegs<D>::kPairUnits);
        if (tid < 2 * kQT) {
            const int64_t i = r0 + (tid & (kQT - 1));
            const int64_t so = ((int64_t)b * p.Hq + h) * N + i;
            tr.st = (i < N) ? ((tid < kQT) ? p.lse2[so] : p.Dv[so]) : 0.f;
        }
    };
    auto store_step = [&](const DkvTileRegs<D> &tr, int stage) {
        store_rows<D>(sm.qt[stage], tr.q, tid, DkvTileRegs<D>::kRowUnits);
        store_rows<D>(sm.dot[stage], tr.d, tid, DkvTileRegs<D>::kRowUnits);
        store_pairs_t<D>(sm.qtt[stage], tr.q0, tr.q1, tid, DkvTileRegs<D>::kPairUnits);
        store_pairs_t<D>(sm.dott[stage], tr.d0, tr.d1, tid, DkvTileRegs<D>::kPairUnits);
        if (tid < kQT) sm.lse2[stage][tid] = tr.st;
        else if (tid < 2 * kQT) sm.Dv[stage][tid - kQT] = tr.st;
    };

    DkvTileRegs<D> tr;
    if (nsteps > 0) {
        load_step(tr, 0);
        store_step(tr, 0);
    }
    __syncthreads();

    for (int64_t s = 0; s < nsteps; ++s) {
        const int st = (int)(s & 1);
        int h_unused;
        int64_t r0;
        step_rows(s, h_unused, r0);
        if (s + 1 < nsteps) load_step(tr, s + 1);

        // this wave's keys [jw0, jw0+32) vs rows [r0, r0+64)
        const bool active = (!p.causal || jw0 <= r0 + kQT - 1) && jw0 < N;
        if (active) {
            const bool need_mask = (p.causal && jw0 + kKeysPerWave - 1 > r0) || r0 + kQT > N ||
                                   jw0 + kKeysPerWave > N;
            f32x16 sacc[2], pacc[2];
#pragma unroll
            for (int ib = 0; ib < 2; ++ib)
#pragma unroll
                for (int r = 0; r < 16; ++r) { sacc[ib][r] = 0.f; pacc[ib][r] = 0.f; }
            // S = Q K^T, dP = dO V^T: A = rows (permuted by kperm), B = key fragments
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
                for (int ib = 0; ib < 2; ++ib) {
                    const int row = ib * 32 + kperm(m);
                    const bf16x8 aq = as_bf16x8(sm.qt[st][rm_slot<D>(row, kk * 2 + kg)]);
                    const bf16x8 ad = as_bf16x8(sm.dot[st][rm_slot<D>(row, kk * 2 + kg)]);
                    sacc[ib] = mfma32x32x16(aq, kf[kk], sacc[ib]);
                    pacc[ib] = mfma32x32x16(ad, vf[kk], pacc[ib]);
                }
            }
            // P = exp2(S c - lse2_i); dS = P (dP - D_i); lane column = key, registers = rows
            const int64_t j = jw0 + m;
            bf16x8 pf[2][2], dsf[2][2];
#pragma unroll
            for (int ib = 0; ib < 2; ++ib) {
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int rbase = ib * 32 + hh * 16 + kg * 8;  // 8 consecutive rows
                    const f32x4 l0 = *reinterpret_cast<const f32x4 *>(&sm.lse2[st][rbase]);
                    const f32x4 l1 = *reinterpret_cast<const f32x4 *>(&sm.lse2[st][rbase + 4]);
                    const f32x4 d0 = *reinterpret_cast<const f32x4 *>(&sm.Dv[st][rbase]);
                    const f32x4 d1 = *reinterpret_cast<const f32x4 *>(&sm.Dv[st][rbase + 4]);
                    float pv[8], dsv[8];
#pragma unroll
                    for (int s8 = 0; s8 < 8; ++s8) {
                        const int r = hh * 8 + s8;
                        const float lz = s8 < 4 ? l0[s8] : l1[s8 - 4];
                        const float dz = s8 < 4 ? d0[s8] : d1[s8 - 4];
                        float pz = __builtin_amdgcn_exp2f(fmaf(sacc[ib][r], p.scale_log2, -lz));
                        if (need_mask) {
                            const int64_t i = r0 + rbase + s8;
                            if (i >= N || j >= N || (p.causal && j > i)) pz = 0.f;
                        }
                        pv[s8] = pz;
                        dsv[s8] = pz * (pacc[ib][r] - dz);
                    }
                    pf[ib][hh] = pack8(pv[0], pv[1], pv[2], pv[3], pv[4], pv[5], pv[6], pv[7]);
                    dsf[ib][hh] = pack8(dsv[0], dsv[1], dsv[2], dsv[3], dsv[4], dsv[5], dsv[6], dsv[7]);
                }
            }
            // dV^T += dO^T P ; dK^T += Q^T dS   (k = query row, 4 steps of 16)
#pragma unroll
            for (int ib = 0; ib < 2; ++ib)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int kgran = (ib * 2 + hh) * 2 + kg;
#pragma unroll
                    for (int eb = 0; eb < EB; ++eb) {
                        const bf16x8 ado = as_bf16x8(sm.dott[st][tr_slot<64>(eb * 32 + m, kgran)]);
                        const bf16x8 aq = as_bf16x8(sm.qtt[st][tr_slot<64>(eb * 32 + m, kgran)]);
                        dvacc[eb] = mfma32x32x16(ado, pf[ib][hh], dvacc[eb]);
                        dkacc[eb] = mfma32x32x16(aq, dsf[ib][hh], dkacc[eb]);
                    }
                }
        }
        if (s + 1 < nsteps) store_step(tr, st ^ 1);
        __syncthreads();
    }

    // write dK = scale * acc, dV = acc (bf16); lane column = key, registers = head-dim rows
    const int64_t j = jw0 + m;
    if (j < N) {
        uint16_t *dkr = p.dk + (((int64_t)b * N + j) * p.Hkv + g) * D;
        uint16_t *dvr = p.dv + (((int64_t)b * N + j) * p.Hkv + g) * D;
#pragma unroll
        for (int eb = 0; eb < EB; ++eb)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                bf16x4 k4, v4;
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    k4[s] = (__bf16)(dkacc[eb][r4 * 4 + s] * p.scale);
                    v4[s] = (__bf16)(dvacc[eb][r4 * 4 + s]);
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

template <typename KernelT>
static hipError_t allow_lds(KernelT kernel, size_t bytes) {
    if (bytes <= 64 * 1024) return hipSuccess;
    return hipFuncSetAttribute(reinterpret_cast<const void *>(kernel),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

hipError_t launch_attn_bwd_bf16(const void *q, const void *k, const void *v, const void *o,
                                const void *dout, const float *lse, void *dq, void *dk, void *dv,
                                void *ws, const AttnShape &s, hipStream_t stream) {
    const size_t rows = (size_t)s.B * (size_t)s.Hq * (size_t)s.N;
    float *lse2 = static_cast<float *>(ws);
    float *Dv = reinterpret_cast<float *>(static_cast<char *>(ws) + round256(rows * sizeof(float)));
    hipError_t err = launch_pre(o, dout, lse, lse2, Dv, s, true, stream);
    if (err != hipSuccess) return err;

    // dQ
    DqParams dp;
    dp.q = static_cast<const uint16_t *>(q);
    dp.k = static_cast<const uint16_t *>(k);
    dp.v = static_cast<const uint16_t *>(v);
    dp.dout = static_cast<const uint16_t *>(dout);
    dp.lse2 = lse2;
    dp.Dv = Dv;
    dp.dq = static_cast<uint16_t *>(dq);
    dp.N = s.N;
    dp.B = (int32_t)s.B;
    dp.Hq = s.Hq;
    dp.Hkv = s.Hkv;
    const int grp = s.Hq / s.Hkv;
    dp.heads_per_wg = (grp % 4 == 0) ? 4 : (grp % 2 == 0) ? 2 : 1;
    dp.pos_blocks = kWaves / dp.heads_per_wg;
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
    kp.N = s.N;
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
        if ((err = allow_lds(attn_bwd_dq_bf16_kernel<128>, sizeof(DqSmem<128>))) != hipSuccess) return err;
        if ((err = allow_lds(attn_bwd_dkdv_bf16_kernel<128>, sizeof(DkvSmem<128>))) != hipSuccess) return err;
        hipLaunchKernelGGL(attn_bwd_dq_bf16_kernel<128>, dim3((uint32_t)dq_items), dim3(kWaves * 64),
                           sizeof(DqSmem<128>), stream, dp);
        if ((err = hipGetLastError()) != hipSuccess) return err;
        hipLaunchKernelGGL(attn_bwd_dkdv_bf16_kernel<128>, dim3((uint32_t)kv_items), dim3(kWaves * 64),
                           sizeof(DkvSmem<128>), stream, kp);
    } else {
        if ((err = allow_lds(attn_bwd_dq_bf16_kernel<64>, sizeof(DqSmem<64>))) != hipSuccess) return err;
        if ((err = allow_lds(attn_bwd_dkdv_bf16_kernel<64>, sizeof(DkvSmem<64>))) != hipSuccess) return err;
        hipLaunchKernelGGL(attn_bwd_dq_bf16_kernel<64>, dim3((uint32_t)dq_items), dim3(kWaves * 64),
                           sizeof(DqSmem<64>), stream, dp);
        if ((err = hipGetLastError()) != hipSuccess) return err;
        hipLaunchKernelGGL(attn_bwd_dkdv_bf16_kernel<64>, dim3((uint32_t)kv_items), dim3(kWaves * 64),
                           sizeof(DkvSmem<64>), stream, kp);
    }
    return hipGetLastError();
}

hipError_t launch_attn_bwd_f32(const float *q, const float *k, const float *v, const float *o,
                               const float *dout, const float *lse, float *dq, float *dk,
                               float *dv, void *ws, const AttnShape &s, hipStream_t stream) {
    const size_t rows = (size_t)s.B * (size_t)s.Hq * (size_t)s.N;
    float *lse2 = static_cast<float *>(ws);
    float *Dv = reinterpret_cast<float *>(static_cast<char *>(ws) + round256(rows * sizeof(float)));
    hipError_t err = launch_pre(o, dout, lse, lse2, Dv, s, false, stream);
    if (err != hipSuccess) return err;
    BwdF32Params p{q, k, v, dout, lse, Dv, dq, dk, dv, s.N, (int32_t)s.B, s.Hq, s.Hkv,
                   s.scale, s.causal, 0};
    p.n_blk = (int32_t)((s.N + kF32Rows - 1) / kF32Rows);
    const int64_t dq_items = (int64_t)p.n_blk * p.B * p.Hq;
    const int64_t kv_items = ((s.N + kF32KvKeys - 1) / kF32KvKeys) * p.B * p.Hkv;
    if (dq_items > 0x7fffffff || kv_items > 0x7fffffff) return hipErrorInvalidConfiguration;
    if (s.d == 128) {
        hipLaunchKernelGGL(attn_bwd_dq_f32_kernel<128>, dim3((uint32_t)dq_items), dim3(kF32Rows), 0, stream, p);
        if ((err = hipGetLastError()) != hipSuccess) return err;
        hipLaunchKernelGGL(attn_bwd_dkdv_f32_kernel<128>, dim3((uint32_t)kv_items), dim3(kF32KvKeys), 0, stream, p);
    } else {
        hipLaunchKernelGGL(attn_bwd_dq_f32_kernel<64>, dim3((uint32_t)dq_items), dim3(kF32Rows), 0, stream, p);
        if ((err = hipGetLastError()) != hipSuccess) return err;
        hipLaunchKernelGGL(attn_bwd_dkdv_f32_kernel<64>, dim3((uint32_t)kv_items), dim3(kF32KvKeys), 0, stream, p);
    }
    return hipGetLastError();
}

}  // namespace ul
