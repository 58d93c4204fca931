// attn_fwd.hip -- forward attention for one Ulysses rank's heads over the full
// sequence, with per-row logsumexp.
//
// "Ulysses Sequence Parallelism: Training with Million-Token Contexts",
// section "How Does Ulysses Sequence Parallelism Actually Work?": after the
// sequence-to-head all-to-all a GPU holds all N positions of H/P heads and
// computes attention for them locally; section "Why Train Million-Token
// Contexts Anyway?": at long N the N x N score matrix must be tiled away.
// So the kernel streams K/V tiles past a block of query rows and keeps the
// softmax in online form (running max m, running sum l, rescaled
// accumulator), never materialising scores beyond one tile.
//
// bf16 path (gfx950 MFMA):
//  * workgroup = 4 waves; a work item is (batch b, KV head g, a block of query
//    positions); each wave owns 64 query rows of one query head.  When the
//    GQA group has >= 4 query heads the 4 waves are 4 heads of the group at
//    the same 64 positions, so every K/V tile staged in LDS serves 4 x 64 rows.
//  * per 64-key tile:  S^T = K Q^T  (A = K rows from LDS, B = Q^T fragments
//    held in registers), so a lane owns one query row and the row max/sum
//    are in-lane plus one cross-half exchange; P^T (bf16) feeds O^T += V^T P^T
//    directly from registers (A = V^T from a transposed LDS tile).
//  * K/V tiles are double-buffered in LDS; the next tile's global loads are
//    in flight while the current one is computed.
//  * tiles entirely above a wave's causal diagonal are skipped; the running
//    max is only raised when a tile's max exceeds it by more than 2^8, which
//    keeps O and l exact (both use the same reference) and skips most
//    rescales of the accumulator.
//  * work items are issued longest-first (late query blocks first) for load
//    balance across the 256 CUs; items sharing a KV head stay on one XCD.
//
// fp32 path: one thread per query row, K/V tiles in LDS, fp32 FMA and
// online softmax; it is the exactness path (max-abs 1e-5), not a fast one.

#include "mfma_tile.h"
#include "ul_internal.h"

namespace ul {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleSlack = 8.0f;  // log2 units: p <= 2^8 between rescales

// ============================================================================ bf16 MFMA kernel

constexpr int kWaves = 4;
constexpr int kRowsPerWave = 64;
constexpr int kKT = 64;  // keys per tile

struct FwdParams {
    const uint16_t *q, *k, *v;
    uint16_t *o;
    float *lse;
    int64_t N;
    int32_t B, Hq, Hkv;
    int32_t heads_per_wg;   // query heads of one group handled by one workgroup (1, 2 or 4)
    int32_t pos_blocks;     // 64-position blocks per workgroup = 4 / heads_per_wg
    int32_t head_groups;    // (Hq/Hkv) / heads_per_wg
    int32_t n_qblk;         // ceil(N / (64 * pos_blocks))
    float scale_log2;       // softmax_scale * log2(e)
    int32_t causal;
};

template <int D>
struct FwdSmem {
    u32x4 kt[2][kKT * D / 8];  // K tile, row-major swizzled
    u32x4 vt[2][D * kKT / 8];  // V^T tile, swizzled
};

// Stage one 64-key tile of K (row-major) and V (transposed) from registers.
template <int D>
struct TileRegs {
    static constexpr int kKUnits = kKT * (D / 8) / (kWaves * 64);       // 16-byte K granules per lane
    static constexpr int kVUnits = (kKT / 2) * (D / 8) / (kWaves * 64); // (key pair, granule) per lane
    u32x4 kg[kKUnits];
    u32x4 v0[kVUnits], v1[kVUnits];
};

template <int D>
__device__ __forceinline__ void load_tile(TileRegs<D> &r, const uint16_t *__restrict__ kbase,
                                          const uint16_t *__restrict__ vbase, int64_t row_stride,
                                          int j0, int64_t N, int tid) {
    constexpr int GPR = D / 8;  // granules per row
#pragma unroll
    for (int u = 0; u < TileRegs<D>::kKUnits; ++u) {
        const int idx = tid + u * kWaves * 64;
        const int row = idx / GPR, gran = idx % GPR;
        const int64_t j = j0 + row;
        r.kg[u] = (j < N) ? *reinterpret_cast<const u32x4 *>(kbase + j * row_stride + gran * 8)
                          : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < TileRegs<D>::kVUnits; ++u) {
        const int idx = tid + u * kWaves * 64;
        const int kp = idx / GPR, gran = idx % GPR;
        const int64_t j = j0 + 2 * kp;
        r.v0[u] = (j < N) ? *reinterpret_cast<const u32x4 *>(vbase + j * row_stride + gran * 8)
                          : u32x4{0, 0, 0, 0};
        r.v1[u] = (j + 1 < N)
                      ? *reinterpret_cast<const u32x4 *>(vbase + (j + 1) * row_stride + gran * 8)
                      : u32x4{0, 0, 0, 0};
    }
}

template <int D>
__device__ __forceinline__ void store_tile(const TileRegs<D> &r, u32x4 *kt, u32x4 *vt, int tid) {
    constexpr int GPR = D / 8;
#pragma unroll
    for (int u = 0; u < TileRegs<D>::kKUnits; ++u) {
        const int idx = tid + u * kWaves * 64;
        const int row = idx / GPR, gran = idx % GPR;
        kt[rm_slot<D>(row, gran)] = r.kg[u];
    }
    // V^T: the lane holds keys (2kp, 2kp+1) x d-values (8*gran .. 8*gran+7);
    // it writes 8 packed key pairs, one 32-bit word per d row e.
    uint32_t *vt32 = reinterpret_cast<uint32_t *>(vt);
#pragma unroll
    for (int u = 0; u < TileRegs<D>::kVUnits; ++u) {
        const int idx = tid + u * kWaves * 64;
        const int kp = idx / GPR, gran = idx % GPR;
        const int kgran = kp >> 2, within = kp & 3;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const uint32_t a = r.v0[u][s >> 1], b = r.v1[u][s >> 1];
            // element s of each row: low half for even s, high half for odd s
            const uint32_t lo = (s & 1) ? (a >> 16) : (a & 0xffffu);
            const uint32_t hi = (s & 1) ? (b & 0xffff0000u) : (b << 16);
            const int e = gran * 8 + s;
            vt32[tr_slot<kKT>(e, kgran) * 4 + within] = lo | hi;
        }
    }
}

template <int D>
__global__ __launch_bounds__(kWaves * 64, 1) void attn_fwd_bf16_kernel(FwdParams p) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    FwdSmem<D> &sm = *reinterpret_cast<FwdSmem<D> *>(smem_raw);

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int m = lane & 31, kg = lane >> 5;

    // ---- work item (longest first): item = rank * (B*Hkv*head_groups) + rest
    const int per_rank = p.B * p.Hkv * p.head_groups;
    const int item = blockIdx.x;
    const int rank = item / per_rank;
    int rest = item - rank * per_rank;
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

    const int64_t q_rs = (int64_t)p.Hq * D;   // row stride of q / o
    const int64_t kv_rs = (int64_t)p.Hkv * D; // row stride of k / v
    const uint16_t *qb = p.q + ((int64_t)b * N * p.Hq + h) * D;
    const uint16_t *kb = p.k + ((int64_t)b * N * p.Hkv + g) * D;
    const uint16_t *vb = p.v + ((int64_t)b * N * p.Hkv + g) * D;

    // ---- Q^T fragments: B operand, column = query row, k = head dim
    constexpr int KK = D / 16;
    bf16x8 qf[2][KK];
#pragma unroll
    for (int ib = 0; ib < 2; ++ib) {
        const int64_t i = i0 + ib * 32 + m;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
            qf[ib][kk] = as_bf16x8(i < N ? *reinterpret_cast<const u32x4 *>(qb + i * q_rs + kk * 16 + kg * 8)
                                         : u32x4{0, 0, 0, 0});
    }

    constexpr int EB = D / 32;
    f32x16 oacc[EB][2];
#pragma unroll
    for (int eb = 0; eb < EB; ++eb)
#pragma unroll
        for (int ib = 0; ib < 2; ++ib)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[eb][ib][r] = 0.f;
    float mrow[2] = {-INFINITY, -INFINITY};
    float lrow[2] = {0.f, 0.f};

    const int64_t kend = p.causal ? (N < wg_pos0 + kRowsPerWave * p.pos_blocks ? N : wg_pos0 + kRowsPerWave * p.pos_blocks) : N;
    const int ntiles = (int)((kend + kKT - 1) / kKT);
    const int64_t wave_last_row = i0 + kRowsPerWave - 1;

    TileRegs<D> tr;
    load_tile<D>(tr, kb, vb, kv_rs, 0, N, tid);
    store_tile<D>(tr, sm.kt[0], sm.vt[0], tid);
    __syncthreads();

    for (int t = 0; t < ntiles; ++t) {
        const int st = t & 1;
        const int j0 = t * kKT;
        if (t + 1 < ntiles) load_tile<D>(tr, kb, vb, kv_rs, j0 + kKT, N, tid);

        const bool active = !p.causal || (int64_t)j0 <= wave_last_row;
        if (active) {
            // ---- S^T = K Q^T for 2 key subtiles x 2 row blocks
            f32x16 sacc[2][2];
#pragma unroll
            for (int js = 0; js < 2; ++js)
#pragma unroll
                for (int ib = 0; ib < 2; ++ib)
#pragma unroll
                    for (int r = 0; r < 16; ++r) sacc[js][ib][r] = 0.f;
            const u32x4 *kt = sm.kt[st];
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
                for (int js = 0; js < 2; ++js) {
                    const bf16x8 a = as_bf16x8(kt[rm_slot<D>(js * 32 + kperm(m), kk * 2 + kg)]);
#pragma unroll
                    for (int ib = 0; ib < 2; ++ib) sacc[js][ib] = mfma32x32x16(a, qf[ib][kk], sacc[js][ib]);
                }
            }

            // ---- mask (causal diagonal / ragged tail), scale to log2 units, row max
            const bool need_mask = (p.causal && (int64_t)j0 + kKT - 1 > i0) || (int64_t)j0 + kKT > N;
            float tmax[2];
#pragma unroll
            for (int ib = 0; ib < 2; ++ib) {
                const int64_t i = i0 + ib * 32 + m;
                float mx = -INFINITY;
#pragma unroll
                for (int js = 0; js < 2; ++js)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        float sv = sacc[js][ib][r] * p.scale_log2;
                        if (need_mask) {
                            const int64_t j = j0 + js * 32 + ckey(r, kg);
                            if (j >= N || (p.causal && j > i)) sv = -INFINITY;
                        }
                        sacc[js][ib][r] = sv;
                        mx = fmaxf(mx, sv);
                    }
                tmax[ib] = fmaxf(mx, __shfl_xor(mx, 32));
            }

            // ---- raise the running max only when a tile exceeds it by the slack
#pragma unroll
            for (int ib = 0; ib < 2; ++ib) {
                const bool raise = tmax[ib] > mrow[ib] + kRescaleSlack;
                if (__any(raise)) {
                    const float mnew = raise ? tmax[ib] : mrow[ib];
                    const float alpha = (mrow[ib] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mrow[ib] - mnew);
                    lrow[ib] *= alpha;
#pragma unroll
                    for (int eb = 0; eb < EB; ++eb)
#pragma unroll
                        for (int r = 0; r < 16; ++r) oacc[eb][ib][r] *= alpha;
                    mrow[ib] = mnew;
                }
            }

            // ---- P^T = exp2(S^T - m), row sums, bf16 fragments
            bf16x8 pf[4][2];
#pragma unroll
            for (int ib = 0; ib < 2; ++ib) {
                float ls = 0.f;
#pragma unroll
                for (int js = 0; js < 2; ++js)
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        float e[8];
#pragma unroll
                        for (int s = 0; s < 8; ++s) {
                            e[s] = __builtin_amdgcn_exp2f(sacc[js][ib][hh * 8 + s] - mrow[ib]);
                            ls += e[s];
                        }
                        pf[js * 2 + hh][ib] = pack8(e[0], e[1], e[2], e[3], e[4], e[5], e[6], e[7]);
                    }
                lrow[ib] += ls;
            }

            // ---- O^T += V^T P^T
            const u32x4 *vt = sm.vt[st];
#pragma unroll
            for (int kap = 0; kap < 4; ++kap) {
#pragma unroll
                for (int eb = 0; eb < EB; ++eb) {
                    const bf16x8 a = as_bf16x8(vt[tr_slot<kKT>(eb * 32 + m, kap * 2 + kg)]);
#pragma unroll
                    for (int ib = 0; ib < 2; ++ib) oacc[eb][ib] = mfma32x32x16(a, pf[kap][ib], oacc[eb][ib]);
                }
            }
        }

        if (t + 1 < ntiles) store_tile<D>(tr, sm.kt[st ^ 1], sm.vt[st ^ 1], tid);
        __syncthreads();
    }

    // ---- epilogue: normalise, round to bf16, write O and lse
#pragma unroll
    for (int ib = 0; ib < 2; ++ib) {
        const float ltot = lrow[ib] + __shfl_xor(lrow[ib], 32);
        const float inv = 1.f / ltot;
        const int64_t i = i0 + ib * 32 + m;
        if (i < N) {
            uint16_t *orow = p.o + ((int64_t)b * N + i) * q_rs + (int64_t)h * D;
#pragma unroll
            for (int eb = 0; eb < EB; ++eb)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const int e = eb * 32 + r4 * 8 + kg * 4;
                    bf16x4 ov;
                    ov[0] = (__bf16)(oacc[eb][ib][r4 * 4 + 0] * inv);
                    ov[1] = (__bf16)(oacc[eb][ib][r4 * 4 + 1] * inv);
                    ov[2] = (__bf16)(oacc[eb][ib][r4 * 4 + 2] * inv);
                    ov[3] = (__bf16)(oacc[eb][ib][r4 * 4 + 3] * inv);
                    *reinterpret_cast<u32x2 *>(orow + e) = __builtin_bit_cast(u32x2, ov);
                }
            if (kg == 0) p.lse[((int64_t)b * p.Hq + h) * N + i] = (mrow[ib] + log2f(ltot)) * kLn2;
        }
    }
}

// ============================================================================ fp32 kernel

constexpr int kF32Rows = 64;  // rows (threads) per workgroup
constexpr int kF32Keys = 32;  // keys per LDS tile

struct FwdF32Params {
    const float *q, *k, *v;
    float *o, *lse;
    int64_t N;
    int32_t B, Hq, Hkv;
    float scale;
    int32_t causal;
    int32_t n_rblk;
};

template <int D>
__global__ __launch_bounds__(kF32Rows) void attn_fwd_f32_kernel(FwdF32Params p) {
    __shared__ float ks[kF32Keys][D];
    __shared__ float vs[kF32Keys][D];
    const int tid = threadIdx.x;
    // item = rank * (B*Hq) + bh, longest first
    const int bh = blockIdx.x % (p.B * p.Hq);
    const int rank = blockIdx.x / (p.B * p.Hq);
    const int rblk = p.causal ? (p.n_rblk - 1 - rank) : rank;
    const int b = bh / p.Hq, h = bh % p.Hq;
    const int g = h / (p.Hq / p.Hkv);
    const int64_t N = p.N;
    const int64_t i = (int64_t)rblk * kF32Rows + tid;
    const bool valid = i < N;

    float qv[D], acc[D];
    const float *qrow = p.q + (((int64_t)b * N + (valid ? i : 0)) * p.Hq + h) * D;
#pragma unroll
    for (int e = 0; e < D; ++e) {
        qv[e] = valid ? qrow[e] : 0.f;
        acc[e] = 0.f;
    }
    float mrow = -INFINITY, lrow = 0.f;
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
            float s = 0.f;
#pragma unroll
            for (int e = 0; e < D; ++e) s = fmaf(qv[e], ks[jj][e], s);
            s *= p.scale;
            if (s > mrow) {
                const float alpha = expf(mrow - s);  // 0 when mrow = -inf
                lrow *= alpha;
#pragma unroll
                for (int e = 0; e < D; ++e) acc[e] *= alpha;
                mrow = s;
            }
            const float w = expf(s - mrow);
            lrow += w;
#pragma unroll
            for (int e = 0; e < D; ++e) acc[e] = fmaf(w, vs[jj][e], acc[e]);
        }
    }
    if (valid) {
        float *orow = p.o + (((int64_t)b * N + i) * p.Hq + h) * D;
        const float inv = 1.f / lrow;
#pragma unroll
        for (int e = 0; e < D; ++e) orow[e] = acc[e] * inv;
        p.lse[((int64_t)b * p.Hq + h) * N + i] = mrow + logf(lrow);
    }
}

}  // namespace

hipError_t launch_attn_fwd_bf16(const void *q, const void *k, const void *v, void *o, float *lse,
                                const AttnShape &s, hipStream_t stream) {
    FwdParams p;
    p.q = static_cast<const uint16_t *>(q);
    p.k = static_cast<const uint16_t *>(k);
    p.v = static_cast<const uint16_t *>(v);
    p.o = static_cast<uint16_t *>(o);
    p.lse = lse;
    p.N = s.N;
    p.B = (int32_t)s.B;
    p.Hq = s.Hq;
    p.Hkv = s.Hkv;
    const int grp = s.Hq / s.Hkv;
    p.heads_per_wg = (grp % 4 == 0) ? 4 : (grp % 2 == 0) ? 2 : 1;
    p.pos_blocks = kWaves / p.heads_per_wg;
    p.head_groups = grp / p.heads_per_wg;
    const int64_t pos_per_wg = (int64_t)kRowsPerWave * p.pos_blocks;
    p.n_qblk = (int32_t)((s.N + pos_per_wg - 1) / pos_per_wg);
    p.scale_log2 = s.scale * kLog2e;
    p.causal = s.causal;
    const int64_t items = (int64_t)p.n_qblk * p.B * p.Hkv * p.head_groups;
    if (items <= 0) return hipSuccess;
    if (items > 0x7fffffff) return hipErrorInvalidConfiguration;
    const dim3 grid((uint32_t)items), block(kWaves * 64);
    if (s.d == 128) {
        hipLaunchKernelGGL(attn_fwd_bf16_kernel<128>, grid, block, sizeof(FwdSmem<128>), stream, p);
    } else {
        hipLaunchKernelGGL(attn_fwd_bf16_kernel<64>, grid, block, sizeof(FwdSmem<64>), stream, p);
    }
    return hipGetLastError();
}

hipError_t launch_attn_fwd_f32(const float *q, const float *k, const float *v, float *o,
                               float *lse, const AttnShape &s, hipStream_t stream) {
    FwdF32Params p{q, k, v, o, lse, s.N, (int32_t)s.B, s.Hq, s.Hkv, s.scale, s.causal, 0};
    p.n_rblk = (int32_t)((s.N + kF32Rows - 1) / kF32Rows);
    const int64_t items = (int64_t)p.n_rblk * p.B * p.Hq;
    if (items <= 0) return hipSuccess;
    if (items > 0x7fffffff) return hipErrorInvalidConfiguration;
    if (s.d == 128)
        hipLaunchKernelGGL(attn_fwd_f32_kernel<128>, dim3((uint32_t)items), dim3(kF32Rows), 0, stream, p);
    else
        hipLaunchKernelGGL(attn_fwd_f32_kernel<64>, dim3((uint32_t)items), dim3(kF32Rows), 0, stream, p);
    return hipGetLastError();
}

}  // namespace ul
