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

#include <type_traits>

#include "mfma_tile.h"
#include "ul_internal.h"

namespace ul {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleSlack = 8.0f;  // log2 units: p <= 2^8 between rescales

// ============================================================================ bf16 MFMA kernel

constexpr int kWaves = 8;                // 2 waves per SIMD
constexpr int kThreads = kWaves * 64;
constexpr int kRowsPerWave = 32;         // query rows per wave (one MFMA column block)
constexpr int kKT = 64;                  // keys per tile

struct FwdParams {
    const uint16_t *q, *k, *v;
    uint16_t *o;
    float *lse;
    int32_t N, B, Hq, Hkv;
    int32_t heads_per_wg;   // query heads of one KV group handled by one workgroup (1, 2 or 4)
    int32_t pos_blocks;     // 32-position row blocks per workgroup = 8 / heads_per_wg
    int32_t head_groups;    // (Hq/Hkv) / heads_per_wg
    int32_t n_qblk;         // ceil(N / (32 * pos_blocks))
    float scale_log2;       // softmax_scale * log2(e)
    int32_t causal;
};

template <int D>
struct FwdTile {
    static constexpr int kBytes = kKT * D * 2;  // one K or V tile
    static constexpr int kStage = 2 * kBytes;   // K then V
    static constexpr int kLds = 2 * kStage;     // double-buffered
};

// Per-wave state carried across key tiles.
template <int D>
struct FwdAcc {
    static constexpr int EB = D / 32;
    f32x16 o[EB];   // O^T: rows = head-dim, columns = this wave's 32 query rows
    float m;        // running max of scaled scores, log2 units
    float l;        // this lane's partial running sum (the other half holds the rest)
};

// One 64-key tile for one wave: S^T = K Q^T, online softmax, O^T += V^T P^T.
// MASK applies the causal diagonal and the ragged end of the sequence.
template <int D, bool MASK>
__device__ __forceinline__ void fwd_tile(FwdAcc<D> &acc, const bf16x8 *qf,
                                         const UL_LDS unsigned char *kt,
                                         const UL_LDS unsigned char *vt, const FragOffs<D> &o,
                                         int kg, int j0, int row, int N, int causal, float c) {
    constexpr int KK = D / 16, EB = D / 32, HALF = 32 * D * 2;
    // S^T: one k-step of fragments in flight ahead of the MFMAs that use them
    // (the barrier stops the scheduler from hoisting every LDS read of the
    // tile, which would not fit in the register budget of 2 waves per SIMD).
    f32x16 s[2] = {zero16(), zero16()};
    bf16x8 a0 = lds_frag(kt, o.rm[0]), a1 = lds_frag(kt + HALF, o.rm[0]);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
        bf16x8 n0 = a0, n1 = a1;
        if (kk + 1 < KK) {
            n0 = lds_frag(kt, o.rm[kk + 1]);
            n1 = lds_frag(kt + HALF, o.rm[kk + 1]);
        }
        s[0] = mfma32x32x16(a0, qf[kk], s[0]);
        s[1] = mfma32x32x16(a1, qf[kk], s[1]);
        a0 = n0;
        a1 = n1;
        __builtin_amdgcn_sched_barrier(0);
    }

    float mx = -INFINITY;
#pragma unroll
    for (int js = 0; js < 2; ++js)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            if constexpr (MASK) {
                const int j = j0 + js * 32 + ckey(r, kg);
                if (j >= N || (causal && j > row)) s[js][r] = -INFINITY;
            }
            mx = fmaxf(mx, s[js][r]);
        }
    const float tmax = half_max(mx) * c;

    // Raise the running max only when the tile exceeds it by 2^8: O and l
    // share the reference, so the result is exact either way.
    const bool raise = tmax > acc.m + 8.0f;
    if (__builtin_amdgcn_ballot_w64(raise)) {
        const float mnew = raise ? tmax : acc.m;
        const float alpha = acc.m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(acc.m - mnew);
        acc.l *= alpha;
#pragma unroll
        for (int eb = 0; eb < EB; ++eb)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc.o[eb][r] *= alpha;
        acc.m = mnew;
    }

    bf16x8 pf[4];
    float ls = 0.f;
#pragma unroll
    for (int js = 0; js < 2; ++js)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            float e[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                e[q] = __builtin_amdgcn_exp2f(fmaf(s[js][hh * 8 + q], c, -acc.m));
                ls += e[q];
            }
            pf[js * 2 + hh] = pack8(e);
        }
    acc.l += ls;

    // O^T += V^T P^T, same one-step lookahead
    bf16x8 va = lds_tr_frag(vt, o.tr[0][0], o.tr[0][1]);
#pragma unroll
    for (int step = 0; step < 4 * EB; ++step) {
        const int kap = step / EB, eb = step % EB;
        bf16x8 vn = va;
        if (step + 1 < 4 * EB) {
            const int nk = (step + 1) / EB, ne = (step + 1) % EB;
            vn = lds_tr_frag(vt + nk * 16 * D * 2, o.tr[ne][0], o.tr[ne][1]);
        }
        acc.o[eb] = mfma32x32x16(va, pf[kap], acc.o[eb]);
        va = vn;
        __builtin_amdgcn_sched_barrier(0);
    }
}

template <int D>
__global__ __launch_bounds__(kThreads) void attn_fwd_bf16_kernel(FwdParams p) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    UL_LDS unsigned char *lds = (UL_LDS unsigned char *)smem_raw;
    using T = FwdTile<D>;

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int m = lane & 31, kg = lane >> 5;

    // ---- work item, longest first: item = rank * (B*Hkv*head_groups) + rest
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
    const uint16_t *kb = p.k + ((int64_t)b * N * p.Hkv + g) * D;
    const uint16_t *vb = p.v + ((int64_t)b * N * p.Hkv + g) * D;

    // ---- Q^T fragments (B operand: column = query row, k = head dim)
    constexpr int KK = D / 16, EB = D / 32;
    bf16x8 qf[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
        qf[kk] = as_bf16x8(row < N ? *reinterpret_cast<const u32x4 *>(qb + row * q_rs + kk * 16 + kg * 8)
                                   : u32x4{0, 0, 0, 0});

    FwdAcc<D> acc;
#pragma unroll
    for (int eb = 0; eb < EB; ++eb) acc.o[eb] = zero16();
    acc.m = -INFINITY;
    acc.l = 0.f;

    // tiles [0, n_full) are visible to every row of the workgroup and inside N
    const int kend = p.causal ? min(N, wg_pos0 + wg_rows) : N;
    const int ntiles = (kend + kKT - 1) / kKT;
    const int n_full = p.causal ? min(wg_pos0, N) / kKT : N / kKT;
    const float c = p.scale_log2;
    const FragOffs<D> fo(lane);

    TileStage<D, kKT, kThreads> sk, sv;
    sk.load(kb, kv_rs, 0, N, tid);
    sv.load(vb, kv_rs, 0, N, tid);
    sk.store(lds, tid);
    sv.store(lds + T::kBytes, tid);
    __syncthreads();

    // One pipeline step: fetch tile t+1 into registers, compute tile t from
    // LDS, park tile t+1 in the other LDS stage.  The unmasked and masked
    // tiles run in separate loops so each loop keeps only its own invariants.
    auto step = [&](int t, auto masked, auto stage) {
        constexpr int st = decltype(stage)::value;
        const int j0 = t * kKT;
        if (t + 1 < ntiles) {
            sk.load(kb, kv_rs, j0 + kKT, N, tid);
            sv.load(vb, kv_rs, j0 + kKT, N, tid);
        }
        const UL_LDS unsigned char *kt = lds + st * T::kStage;
        const UL_LDS unsigned char *vt = kt + T::kBytes;
        if constexpr (decltype(masked)::value) {
            if (!p.causal || j0 <= i0 + kRowsPerWave - 1)
                fwd_tile<D, true>(acc, qf, kt, vt, fo, kg, j0, row, N, p.causal, c);
        } else {
            fwd_tile<D, false>(acc, qf, kt, vt, fo, kg, j0, row, N, p.causal, c);
        }
        if (t + 1 < ntiles) {
            UL_LDS unsigned char *nk = lds + (st ^ 1) * T::kStage;
            sk.store(nk, tid);
            sv.store(nk + T::kBytes, tid);
        }
        __syncthreads();
    };
    // Tiles go in pairs so that the LDS stage is a compile-time offset.
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    int t = 0;
    for (; t + 1 < n_full; t += 2) {
        step(t, std::false_type{}, S0{});
        step(t + 1, std::false_type{}, S1{});
    }
    if (t < n_full) {
        step(t, std::false_type{}, S0{});
        ++t;
        if (t < ntiles) step(t, std::true_type{}, S1{});
        ++t;
    }
    for (; t + 1 < ntiles; t += 2) {
        step(t, std::true_type{}, S0{});
        step(t + 1, std::true_type{}, S1{});
    }
    if (t < ntiles) step(t, std::true_type{}, S0{});

    // ---- epilogue: normalise, round to bf16, write O and lse
    const float ltot = half_sum(acc.l);
    if (row < N) {
        const float inv = 1.f / ltot;
        uint16_t *orow = p.o + ((int64_t)b * N + row) * q_rs + (int64_t)h * D;
#pragma unroll
        for (int eb = 0; eb < EB; ++eb)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                bf16x4 ov;
#pragma unroll
                for (int q = 0; q < 4; ++q) ov[q] = (__bf16)(acc.o[eb][r4 * 4 + q] * inv);
                *reinterpret_cast<u32x2 *>(orow + eb * 32 + r4 * 8 + kg * 4) = __builtin_bit_cast(u32x2, ov);
            }
        if (kg == 0) p.lse[((int64_t)b * p.Hq + h) * N + row] = (acc.m + __log2f(ltot)) * kLn2;
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
    p.N = (int32_t)s.N;
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
    const dim3 grid((uint32_t)items), block(kThreads);
    if (s.d == 128)
        hipLaunchKernelGGL(attn_fwd_bf16_kernel<128>, grid, block, FwdTile<128>::kLds, stream, p);
    else
        hipLaunchKernelGGL(attn_fwd_bf16_kernel<64>, grid, block, FwdTile<64>::kLds, stream, p);
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
