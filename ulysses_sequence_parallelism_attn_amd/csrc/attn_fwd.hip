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
//  * workgroup = 8 waves, two per SIMD; a work item is (batch b, KV head g,
//    a block of query positions) and each wave owns 32 query rows of one
//    query head.  When the GQA group has >= 4 query heads, waves w and w+4
//    are heads w of the group at two consecutive 32-row blocks, so every K/V
//    tile staged in LDS serves 4 heads x 64 rows.
//  * per 64-key tile:  S^T = K Q^T  (A = K rows from LDS, B = Q^T fragments
//    held in registers), so a lane owns one query row and the row max/sum
//    are in-lane plus one cross-half exchange; P^T (bf16) feeds O^T += V^T P^T
//    directly from registers (A = V^T by transposed LDS reads).
//  * the two waves of a SIMD run half a tile apart (waves 4-7 one barrier
//    behind waves 0-3): while one issues its 32 MFMAs (PV of the previous
//    tile, then S of this one) the other does the softmax VALU work of its
//    own tile, and the barrier between the halves swaps the roles.
//  * K/V tiles go straight from global memory into a 4-stage LDS ring
//    (global_load_lds, no register staging), two tiles ahead of use, the
//    loads spread between the MFMAs.
//  * tiles entirely above a wave's causal diagonal are skipped; the running
//    max is only raised when a tile's max exceeds it by more than 2^8, which
//    keeps O and l exact (both use the same reference) and skips most
//    rescales of the accumulator.
//  * work items are issued longest-first (late query blocks first) for load
//    balance across the 256 CUs.
//
// fp32 path: one thread per query row, K/V tiles in LDS, fp32 FMA and
// online softmax; it is the exactness path (max-abs 1e-5), not a fast one.

#include <type_traits>
#include <utility>

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
    int64_t q_rs, k_rs, v_rs, o_rs;  // elements between consecutive tokens of each tensor
    const int32_t *cu_seqlens;       // packed variable-length sequences, or nullptr
    int64_t total;                   // tokens of the packed sequences
    int32_t N, B, Hq, Hkv;           // N: tokens per sequence (the longest one if packed)
    int32_t heads_per_wg;   // query heads of one KV group handled by one workgroup (1, 2 or 4)
    int32_t pos_blocks;     // 32-position row blocks per workgroup = 8 / heads_per_wg
    int32_t head_groups;    // (Hq/Hkv) / heads_per_wg
    int32_t n_qblk;         // ceil(N / (32 * pos_blocks))
    float scale_log2;       // softmax_scale * log2(e)
    int32_t causal;
    // Split key range (shorter causal sequences): query blocks split_from ..
    // n_qblk-1 run as two work items, one over the first half of their key
    // tiles and one over the rest, each writing its unnormalised fp32 O and
    // (running max, sum) to part_o / part_ml; fwd_merge_kernel combines them.
    // split_from = n_qblk: no split.
    int32_t split_from;
    float *part_o, *part_ml;
};

// The work items of one lane (b, KV head, head group) when the upper query
// blocks are split: cycles of the two halves of two split blocks followed by
// one whole block, all taken from the longest down, so that the dispatch
// order stays close to longest-first (a split half of block i has about
// (i+1)/2 tiles, a whole block j has j+1, and the cycle keeps the two in
// step); then the last split block if their count is odd, then the remaining
// whole blocks.  Returns the query block; `chunk` is 0 / 1 for the halves and
// -1 for a whole block.
__device__ __forceinline__ int fwd_split_item(int u, int n, int K, int &chunk) {
    const int S = n - K, C = S / 2, odd = S % 2;
    if (u < 5 * C) {
        const int c = u / 5, r = u % 5;
        if (r < 4) {
            chunk = r % 2;
            return n - 1 - 2 * c - r / 2;
        }
        chunk = -1;
        return K - 1 - c;
    }
    u -= 5 * C;
    if (odd && u < 2) {
        chunk = u;
        return K;
    }
    chunk = -1;
    return K - 1 - C - (u - 2 * odd);
}

template <int D>
struct FwdTile {
    static constexpr int kBytes = kKT * D * 2;          // one K or V tile
    static constexpr int kStages = 4;                   // tiles t .. t+3 in LDS
    // K tiles of the 4 stages first, then the V tiles: every offset from the
    // start of either region stays below 64 KB, so stage and step offsets fit
    // the immediate offset of an LDS read (the V region's base is folded into
    // the per-lane V fragment offsets once).
    static constexpr int kVBase = kStages * kBytes;
    static constexpr int kLds = 2 * kStages * kBytes;   // 128 KB at D = 128
    static_assert(kVBase <= 65536, "stage offsets must fit an LDS immediate");
    __device__ static constexpr int k_stage(int st) { return st * kBytes; }
};

// Per-wave state carried across key tiles.
template <int D>
struct FwdAcc {
    static constexpr int EB = D / 32;
    f32x16 o[EB];   // O^T: rows = head-dim, columns = this wave's 32 query rows
    float m;        // running max of scaled scores, log2 units
    float l;        // this lane's partial running sum (the other half holds the rest)
};

constexpr int kAhead = 6;  // A fragments read ahead of their MFMA

// The MFMA half of a tile as one stream of 32 MFMAs, each with one A
// fragment from LDS:
//   PV steps  O^T += V^T P^T of the previous tile (A = V^T by transposed reads
//             of the V tile at `vstage`, B = its P^T fragments in `pf`),
//             4 x EB steps;
//   S steps   S^T = K Q^T of this tile (A = K rows of the K tile at `kstage`,
//             B = the wave's Q^T fragments), alternating the 32-key halves.
// Addresses are absolute: `o` holds the lane's offsets with the LDS base (and
// for V the V region) already added, the stage offsets are constants.  The A
// fragments are read kAhead steps before their MFMA, enough to cover the LDS
// latency while the other wave of the SIMD is not issuing MFMAs; with PV the
// first kAhead of them are already in `ring` (fwd_prefetch).  `side(k)`, k <
// NSIDE, runs between MFMAs spread over the stream (the tile loads).  The
// scheduling barriers keep this order, and the register budget, intact.
template <int D, bool PV, bool S, int NSIDE, typename Side>
__device__ __forceinline__ void fwd_gemm(FwdAcc<D> &acc, const bf16x8 (&pf)[4], f32x16 (&s)[2],
                                         const bf16x8 *qf, bf16x8 (&ring)[kAhead], uint32_t vstage,
                                         uint32_t kstage, const FragOffs<D> &o, Side &&side) {
    constexpr int EB = D / 32, KK = D / 16, HALF = 32 * D * 2;
    constexpr int NPV = PV ? 4 * EB : 0, NS = S ? 2 * KK : 0, NSTEP = NPV + NS;
    static_assert(!PV || NPV >= kAhead, "the prefetched ring holds PV steps only");
    constexpr int EVERY = NSIDE > 0 ? NSTEP / NSIDE : 1;
    auto frag = [&](int st) -> bf16x8 {
        if (st < NPV) {
            const uint32_t at = vstage + (st / EB) * 16 * D * 2;
            return lds_tr_frag_at(o.tr[st % EB][0] + at, o.tr[st % EB][1] + at);
        }
        const int x = st - NPV;
        return lds_frag_at(o.rm[x / 2] + kstage + (x % 2) * HALF);
    };
    if constexpr (S) {
        s[0] = zero16();
        s[1] = zero16();
    }
    if constexpr (!PV) {
#pragma unroll
        for (int i = 0; i < kAhead; ++i)
            if (i < NSTEP) ring[i] = frag(i);
    }
#pragma unroll
    for (int st = 0; st < NSTEP; ++st) {
        const bf16x8 a = ring[st % kAhead];
        if (st + kAhead < NSTEP) ring[st % kAhead] = frag(st + kAhead);
        if (st < NPV) {
            const int kap = st / EB, eb = st % EB;
            acc.o[eb] = mfma32x32x16(a, pf[kap], acc.o[eb]);
        } else {
            const int x = st - NPV, kk = x / 2, js = x % 2;
            s[js] = mfma32x32x16(a, qf[kk], s[js]);
        }
        if constexpr (NSIDE > 0)
            if (st % EVERY == 1 && st / EVERY < NSIDE) side(st / EVERY);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// The first kAhead A fragments of the PV steps for the V tile at `vstage`.
template <int D>
__device__ __forceinline__ void fwd_prefetch(bf16x8 (&ring)[kAhead], uint32_t vstage, const FragOffs<D> &o) {
    constexpr int EB = D / 32;
#pragma unroll
    for (int st = 0; st < kAhead; ++st) {
        const uint32_t at = vstage + (st / EB) * 16 * D * 2;
        ring[st] = lds_tr_frag_at(o.tr[st % EB][0] + at, o.tr[st % EB][1] + at);
    }
}

// Online softmax of one tile: new running max, rescale of O and l when it
// moves, P = exp2(S c - m) packed to bf16 B fragments.  MASK applies the
// causal diagonal and the ragged end of the sequence.
template <int D, bool MASK>
__device__ __forceinline__ void fwd_softmax(FwdAcc<D> &acc, f32x16 (&s)[2], bf16x8 (&pf)[4], int kg, int j0,
                                            int row, int N, int causal, float c) {
    constexpr int EB = D / 32;
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
    const bool raise = tmax > acc.m + kRescaleSlack;
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
    // Pin P and l here: otherwise the compiler sinks the exponentials to their
    // use, into the next MFMA half, which is the other wave's softmax time.
#pragma unroll
    for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(pf[i]));
    asm volatile("" : "+v"(acc.l));
}

template <int D>
__global__ __launch_bounds__(kThreads) void attn_fwd_bf16_kernel(FwdParams p) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    UL_LDS unsigned char *lds = (UL_LDS unsigned char *)smem_raw;
    using T = FwdTile<D>;
    using Tile = DmaTile<D, kKT>;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int m = lane & 31, kg = lane >> 5;

    // ---- work item, longest first: item = rank * (B*Hkv*head_groups) + rest
    const int per_rank = p.B * p.Hkv * p.head_groups;
    const int rank = blockIdx.x / per_rank;
    const int lane_id = blockIdx.x - rank * per_rank;
    int rest = lane_id;
    const int g = rest % p.Hkv;
    rest /= p.Hkv;
    const int hg = rest % p.head_groups;
    const int b = rest / p.head_groups;
    int chunk = -1;
    const int qblk = p.split_from < p.n_qblk ? fwd_split_item(rank, p.n_qblk, p.split_from, chunk)
                                             : (p.causal ? (p.n_qblk - 1 - rank) : rank);
    const SeqRange sq = seq_range(p.cu_seqlens, b, p.N, p.Hq, p.total);

    const int grp = p.Hq / p.Hkv;
    const int h = g * grp + hg * p.heads_per_wg + (wave % p.heads_per_wg);
    const int wg_rows = kRowsPerWave * p.pos_blocks;
    const int wg_pos0 = qblk * wg_rows;
    const int i0 = wg_pos0 + (wave / p.heads_per_wg) * kRowsPerWave;
    const int N = sq.len;
    const int row = i0 + m;
    if (wg_pos0 >= N) return;  // past the end of a shorter packed sequence

    const int64_t q_rs = p.q_rs;
    const uint16_t *qb = p.q + sq.tok0 * q_rs + (int64_t)h * D;

    // ---- Q^T fragments (B operand: column = query row, k = head dim)
    constexpr int KK = D / 16, EB = D / 32;
    bf16x8 qf[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
        qf[kk] = as_bf16x8(row < N ? *reinterpret_cast<const u32x4 *>(qb + row * q_rs + kk * 16 + kg * 8)
                                   : u32x4{0, 0, 0, 0});
    // Retire these loads: inside the loop vmcnt counts only the tile loads.
    __builtin_amdgcn_s_waitcnt(0x70);

    FwdAcc<D> acc;
#pragma unroll
    for (int eb = 0; eb < EB; ++eb) acc.o[eb] = zero16();
    acc.m = -INFINITY;
    acc.l = 0.f;

    // tiles [0, n_full) are visible to every row of the workgroup and inside N;
    // this item takes tiles [ta, tb): all of them, or one half of a split
    // block's (the first half lies inside [0, n_full))
    const int kend = p.causal ? min(N, wg_pos0 + wg_rows) : N;
    const int ntiles_all = (kend + kKT - 1) / kKT;
    const int n_full_all = p.causal ? min(wg_pos0, N) / kKT : N / kKT;
    const int half = ntiles_all / 2;
    const int ta = chunk == 1 ? half : 0;
    const int ntiles = chunk == 0 ? half : ntiles_all;
    const int n_full = chunk == 0 ? min(half, n_full_all) : n_full_all;
    const float c = p.scale_log2;
    // Absolute LDS addresses: the lane's fragment offsets plus the LDS base
    // (and, for V, the V region); the empty asm keeps the compiler from
    // splitting the sums again into out-of-range immediates.
    FragOffs<D> fo(lane);
    {
        const uint32_t base = (uint32_t)(uintptr_t)lds;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            fo.rm[kk] += base;
            asm volatile("" : "+v"(fo.rm[kk]));
        }
#pragma unroll
        for (int e = 0; e < EB; ++e)
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                fo.tr[e][x] += base + T::kVBase;
                asm volatile("" : "+v"(fo.tr[e][x]));
            }
    }

    // Direct loads of tile t into its LDS stage: the K and V tiles are split
    // evenly over the 8 waves, each wave's share inside one of the two.  Keys
    // past N re-read key N-1 (their scores are masked, so P is 0 there).
    constexpr int kDmaPerWave = 2 * Tile::INSTR / kWaves;
    static_assert(2 * Tile::INSTR % kWaves == 0 && Tile::INSTR % kDmaPerWave == 0,
                  "K and V tiles split evenly over the waves");
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
    // The tile the next loads fetch, set up by dma_prep one body ahead (at
    // the end of the softmax half, off the MFMA stream): the address of its
    // first key row (wave-uniform) and the byte offset of its last row inside
    // N.  A load in the MFMA stream is then a clamp, an add and the M0 write;
    // computing the address there took ~17 scalar instructions per load,
    // which held back the MFMAs behind them.
    const uint32_t dma_lds = (uint32_t)(uintptr_t)lds + tile_lds + u0 * 1024;
    const uint16_t *dma_tb = tens;
    uint32_t dma_lim = 0;
    auto dma_prep = [&](int t) {
        const int j0 = t * kKT;
        dma_tb = uniform_ptr(tens + (int64_t)j0 * t_rs);
        dma_lim = (uint32_t)max(min(N - 1 - j0, kKT), 0) * row_bytes;  // last key of the sequence
    };
    // load k of this wave's share of the prepared tile into the stage at byte offset `st`
    auto issue_k = [&](int k, uint32_t st) {
        dma_b128_m0(dma_tb, min(dma_roff[k], dma_lim) + dma_gran[k], dma_lds + st + k * 1024);
    };
    auto issue = [&](uint32_t st) {
#pragma unroll
        for (int k = 0; k < kDmaPerWave; ++k) issue_k(k, st);
    };
    // tile t holds keys this wave's rows can see
    auto visible = [&](int t) { return !p.causal || t * kKT <= i0 + kRowsPerWave - 1; };

    // Two groups of 4 waves, one wave of each per SIMD, run half a tile apart:
    // while one wave of a SIMD issues its MFMAs (PV of tile t-1, S of tile t)
    // the other runs the softmax VALU work of its own tile, and the barrier
    // between the halves swaps the roles.  Both groups run the same sequence
    // of (MFMA half, barrier, softmax half, barrier) per tile; the second group
    // enters it one barrier later and the first leaves it with one extra
    // barrier, so every wave meets the same number of barriers.
    //
    // Tile t sits in stage t % 4 from its load (issued at the start of the MFMA
    // half of tile t-2) to the second group's PV of it (the MFMA half of tile
    // t+1); each wave waits for its share of tile t+1 before the barrier that
    // ends its MFMA half of tile t, which is before anyone reads it.
    const bool lagging = wave >= kWaves / 2;
    // stages follow the tile index relative to the item's first tile
    dma_prep(ta);
    issue(T::k_stage(0));
    if (ntiles - ta > 1) {
        dma_prep(ta + 1);
        issue(T::k_stage(1));
        wait_vm_barrier<kDmaPerWave>();
    } else {
        wait_vm_barrier<0>();
    }
    dma_prep(ta + 2);
    if (lagging) fence_barrier();

    f32x16 s[2];
    bf16x8 pf[4];
    bf16x8 ring[kAhead];
    // One tile: the MFMA half (PV of tile t-1, S of tile t, the loads of tile
    // t+2 between the MFMAs), then the softmax half, which ends by reading the
    // first V fragments of the next MFMA half.  `stage(x)` is tile x's stage
    // offset.  FULL: both tiles take part and tile t is unmasked (the steady
    // state, one straight block); otherwise each part is checked on its own.
    auto body = [&](int t, auto full, auto stage, uint32_t stage2) {  // stage2: tile t+2's
        constexpr bool FULL = decltype(full)::value;
        const bool more = t + 2 < ntiles;
        // The wave feeding the MFMA pipe takes issue priority over the other
        // wave of its SIMD (busy with its softmax) until its half ends.
        __builtin_amdgcn_s_setprio(2);
        if constexpr (FULL) {
            fwd_gemm<D, true, true, kDmaPerWave>(acc, pf, s, qf, ring, stage(t - 1), stage(t), fo,
                                                 [&](int k) {
                                                     if (more) issue_k(k, stage2);
                                                 });
        } else {
            if (more) issue(stage2);
            auto none = [](int) {};
            if (t >= ta + 1 && visible(t - 1))
                fwd_gemm<D, true, false, 0>(acc, pf, s, qf, ring, stage(t - 1), 0, fo, none);
            if (t < ntiles && visible(t)) fwd_gemm<D, false, true, 0>(acc, pf, s, qf, ring, 0, stage(t), fo, none);
        }
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(0);
        if (more)
            wait_vm_barrier<kDmaPerWave>();
        else
            wait_vm_barrier<0>();
        __builtin_amdgcn_sched_barrier(0);
        if (FULL || (t < ntiles && visible(t))) {
            if constexpr (FULL)
                fwd_softmax<D, false>(acc, s, pf, kg, t * kKT, row, N, p.causal, c);
            else
                fwd_softmax<D, true>(acc, s, pf, kg, t * kKT, row, N, p.causal, c);
            fwd_prefetch<D>(ring, stage(t), fo);
        }
        dma_prep(t + 3);  // the tile the next body loads
        fence_barrier();
    };
    // Tile 0 (no PV yet), then the whole unmasked tiles 1 .. n_full-1 in
    // fours so that every stage offset is a constant, then the rest (at most
    // three unmasked tiles, the masked ones and the last PV) with computed
    // stages and the masking softmax, which is exact on unmasked tiles too.
    auto rt_stage = [ta](int x) { return (uint32_t)T::k_stage((x - ta) & (T::kStages - 1)); };
    body(ta, std::false_type{}, rt_stage, rt_stage(ta + 2));
    int t0 = ta + 1;
    for (; t0 + T::kStages <= n_full; t0 += T::kStages) {
        [&]<int... J>(std::integer_sequence<int, J...>) {
            // x - t0 + 1 folds to a constant for every tile index body derives from t0 + J
            // (t0 - ta is 1 modulo the stage count, as the run-time stages assume)
            (body(t0 + J, std::true_type{},
                  [t0](int x) { return (uint32_t)T::k_stage((x - t0 + 1) & (T::kStages - 1)); },
                  (uint32_t)T::k_stage((J + 3) & (T::kStages - 1))),
             ...);
        }(std::make_integer_sequence<int, T::kStages>{});
    }
    for (int t = t0; t <= ntiles; ++t) body(t, std::false_type{}, rt_stage, rt_stage(t + 2));
    if (!lagging) fence_barrier();

    // ---- epilogue: normalise, round to bf16, write O and lse
    const float ltot = half_sum(acc.l);
    if (chunk >= 0) {  // half of a split block: unnormalised O and (m, l), fp32
        const int64_t slot = ((int64_t)lane_id * (p.n_qblk - p.split_from) + (qblk - p.split_from)) * 2 + chunk;
        const int64_t rw = (slot * kWaves + wave) * kRowsPerWave + m;
        float *po = p.part_o + rw * D;
#pragma unroll
        for (int eb = 0; eb < EB; ++eb)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                f32x4 ov;
#pragma unroll
                for (int q = 0; q < 4; ++q) ov[q] = acc.o[eb][r4 * 4 + q];
                *reinterpret_cast<f32x4 *>(po + eb * 32 + r4 * 8 + kg * 4) = ov;
            }
        if (kg == 0) {
            p.part_ml[rw * 2] = acc.m;
            p.part_ml[rw * 2 + 1] = ltot;
        }
        return;
    }
    if (row < N) {
        const float inv = 1.f / ltot;
        uint16_t *orow = p.o + (sq.tok0 + row) * p.o_rs + (int64_t)h * D;
#pragma unroll
        for (int eb = 0; eb < EB; ++eb)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                bf16x4 ov;
#pragma unroll
                for (int q = 0; q < 4; ++q) ov[q] = (__bf16)(acc.o[eb][r4 * 4 + q] * inv);
                *reinterpret_cast<u32x2 *>(orow + eb * 32 + r4 * 8 + kg * 4) = __builtin_bit_cast(u32x2, ov);
            }
        if (kg == 0) p.lse[sq.lse0 + (int64_t)h * sq.hs + row] = (acc.m + __log2f(ltot)) * kLn2;
    }
}

// Combines the two halves of each split query block (the key ranges [0, h)
// and [h, end) of every row): with m_c, l_c and the unnormalised O_c of half
// c, all relative to 2^m_c,
//   M = max(m_0, m_1),  a_c = 2^(m_c - M),
//   o = (a_0 O_0 + a_1 O_1) / (a_0 l_0 + a_1 l_1),  lse = (M + log2 l) ln 2,
// the same online-softmax update the kernel applies between key tiles.  One
// thread per 4 dimensions of a row; rows past N are skipped.
template <int D>
__global__ __launch_bounds__(256) void fwd_merge_kernel(FwdParams p, int64_t n_threads) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= n_threads) return;
    constexpr int Q = D / 4;
    const int dq = (int)(t % Q);
    const int64_t r = t / Q;  // (pair, wave, m)
    const int m = (int)(r % kRowsPerWave);
    const int wave = (int)((r / kRowsPerWave) % kWaves);
    const int64_t pair = r / (kRowsPerWave * kWaves);  // lane_id * S + split block
    const int S = p.n_qblk - p.split_from;
    const int lane_id = (int)(pair / S);
    const int qblk = p.split_from + (int)(pair % S);
    const int g = lane_id % p.Hkv;
    const int hg = (lane_id / p.Hkv) % p.head_groups;
    const int b = lane_id / (p.Hkv * p.head_groups);
    const int h = g * (p.Hq / p.Hkv) + hg * p.heads_per_wg + wave % p.heads_per_wg;
    const int row = qblk * kRowsPerWave * p.pos_blocks + (wave / p.heads_per_wg) * kRowsPerWave + m;
    if (row >= p.N) return;
    const int64_t rw0 = ((pair * 2) * kWaves + wave) * kRowsPerWave + m;
    const int64_t rw1 = rw0 + kWaves * kRowsPerWave;
    const float m0 = p.part_ml[rw0 * 2], l0 = p.part_ml[rw0 * 2 + 1];
    const float m1 = p.part_ml[rw1 * 2], l1 = p.part_ml[rw1 * 2 + 1];
    const float mm = fmaxf(m0, m1);
    const float a0 = exp2f(m0 - mm), a1 = exp2f(m1 - mm);  // one of them is 1
    const float l = a0 * l0 + a1 * l1;
    const float inv = 1.f / l;
    const f32x4 o0 = *reinterpret_cast<const f32x4 *>(p.part_o + rw0 * D + dq * 4);
    const f32x4 o1 = *reinterpret_cast<const f32x4 *>(p.part_o + rw1 * D + dq * 4);
    bf16x4 ov;
#pragma unroll
    for (int e = 0; e < 4; ++e) ov[e] = (__bf16)(fmaf(a0, o0[e], a1 * o1[e]) * inv);
    const int64_t tok = (int64_t)b * p.N + row;
    *reinterpret_cast<u32x2 *>(p.o + tok * p.o_rs + (int64_t)h * D + dq * 4) = __builtin_bit_cast(u32x2, ov);
    if (dq == 0) p.lse[((int64_t)b * p.Hq + h) * p.N + row] = (mm + __log2f(l)) * kLn2;
}

// ============================================================================ fp32 kernel

constexpr int kF32Rows = 64;  // rows (threads) per workgroup
constexpr int kF32Keys = 32;  // keys per LDS tile

struct FwdF32Params {
    const float *q, *k, *v;
    float *o, *lse;
    int64_t N;
    int64_t q_rs, k_rs, v_rs, o_rs;  // token strides in elements
    const int32_t *cu_seqlens;       // packed variable-length sequences, or nullptr
    int64_t total;
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
    const SeqRange sq = seq_range(p.cu_seqlens, b, p.N, p.Hq, p.total);
    const int64_t N = sq.len;
    if ((int64_t)rblk * kF32Rows >= N) return;  // past the end of a shorter packed sequence
    const int64_t i = (int64_t)rblk * kF32Rows + tid;
    const bool valid = i < N;

    float qv[D], acc[D];
    const float *qrow = p.q + (sq.tok0 + (valid ? i : 0)) * p.q_rs + (int64_t)h * D;
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
            const int64_t tok = sq.tok0 + j, col = (int64_t)g * D + e;
            ks[jj][e] = j < N ? p.k[tok * p.k_rs + col] : 0.f;
            vs[jj][e] = j < N ? p.v[tok * p.v_rs + col] : 0.f;
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
        float *orow = p.o + (sq.tok0 + i) * p.o_rs + (int64_t)h * D;
        const float inv = 1.f / lrow;
#pragma unroll
        for (int e = 0; e < D; ++e) orow[e] = acc[e] * inv;
        p.lse[sq.lse0 + (int64_t)h * sq.hs + i] = mrow + logf(lrow);
    }
}

// Work decomposition of one bf16 call.  The key range of the upper half of
// the query blocks is split in two when the call has at most kSplitMaxItems
// work items (one per query block of each lane): with about one item per CU
// the longest-first order cannot balance the CUs, since the last block holds
// twice the mean work, and halving the longest items fixes most of that.
// With more items the order balances by itself and the partials' round trip
// costs more than it gains (measured: N=8192 with 8 query / 2 KV heads, 256
// items, forward 203 -> 174 us; with 32 / 8 heads, 1024 items, 502 -> 558 us).
// The partials take at most kSplitMaxItems x 2 x 256 rows x (4 d + 8) bytes,
// 34 MB at d = 128.
constexpr int64_t kSplitMaxItems = 256;
constexpr int kSplitMinBlocks = 16;  // a split block keeps >= 8 key tiles, its first half unmasked

struct FwdPlan {
    int32_t heads_per_wg, pos_blocks, head_groups, n_qblk, split_from;
    int64_t lanes;
    size_t part_o_bytes, part_ml_bytes;
};

FwdPlan fwd_plan(const AttnShape &s, int32_t dtype) {
    FwdPlan pl{};
    const int grp = s.Hq / s.Hkv;
    pl.heads_per_wg = (grp % 4 == 0) ? 4 : (grp % 2 == 0) ? 2 : 1;
    pl.pos_blocks = kWaves / pl.heads_per_wg;
    pl.head_groups = grp / pl.heads_per_wg;
    const int64_t pos_per_wg = (int64_t)kRowsPerWave * pl.pos_blocks;
    pl.n_qblk = (int32_t)((s.N + pos_per_wg - 1) / pos_per_wg);
    pl.split_from = pl.n_qblk;
    pl.lanes = s.B * s.Hkv * pl.head_groups;
    if (dtype != 1 || !s.causal || s.cu || pl.n_qblk < kSplitMinBlocks ||
        pl.lanes * pl.n_qblk > kSplitMaxItems)
        return pl;
    const int32_t K = (pl.n_qblk + 1) / 2;
    const int64_t slots = pl.lanes * (pl.n_qblk - K) * 2;
    const size_t rows = (size_t)slots * kWaves * kRowsPerWave;
    const size_t ob = rows * s.d * 4, mb = rows * 2 * 4;
    pl.split_from = K;
    pl.part_o_bytes = ob;
    pl.part_ml_bytes = mb;
    return pl;
}

}  // namespace

size_t attn_fwd_workspace_bytes(const AttnShape &s, int32_t dtype) {
    const FwdPlan pl = fwd_plan(s, dtype);
    return pl.part_o_bytes + pl.part_ml_bytes;
}

hipError_t launch_attn_fwd_bf16(const void *q, const void *k, const void *v, void *o, float *lse,
                                void *ws, const AttnShape &s, hipStream_t stream) {
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
    p.q_rs = s.q_rs;
    p.k_rs = s.k_rs;
    p.v_rs = s.v_rs;
    p.o_rs = s.o_rs;
    p.cu_seqlens = s.cu;
    p.total = s.total;
    // a null workspace runs the call unsplit
    const FwdPlan pl = fwd_plan(s, 1);
    p.heads_per_wg = pl.heads_per_wg;
    p.pos_blocks = pl.pos_blocks;
    p.head_groups = pl.head_groups;
    p.n_qblk = pl.n_qblk;
    p.scale_log2 = s.scale * kLog2e;
    p.causal = s.causal;
    const bool split = ws && pl.split_from < pl.n_qblk;
    p.split_from = split ? pl.split_from : pl.n_qblk;
    p.part_o = split ? static_cast<float *>(ws) : nullptr;
    p.part_ml = split ? reinterpret_cast<float *>(static_cast<unsigned char *>(ws) + pl.part_o_bytes) : nullptr;
    // items per lane: every query block once, the split ones twice
    const int64_t per_lane = (int64_t)p.n_qblk + (p.n_qblk - p.split_from);
    const int64_t items = per_lane * pl.lanes;
    if (items <= 0) return hipSuccess;
    if (items > 0x7fffffff) return hipErrorInvalidConfiguration;
    const dim3 grid((uint32_t)items), block(kThreads);
    const int64_t merge_threads = pl.lanes * (p.n_qblk - p.split_from) * kWaves * kRowsPerWave * (s.d / 4);
    const dim3 mgrid((uint32_t)((merge_threads + 255) / 256));
    hipError_t err;
    if (s.d == 128) {
        if ((err = allow_lds(attn_fwd_bf16_kernel<128>, FwdTile<128>::kLds)) != hipSuccess) return err;
        hipLaunchKernelGGL(attn_fwd_bf16_kernel<128>, grid, block, FwdTile<128>::kLds, stream, p);
        if (split) hipLaunchKernelGGL(fwd_merge_kernel<128>, mgrid, dim3(256), 0, stream, p, merge_threads);
    } else {
        if ((err = allow_lds(attn_fwd_bf16_kernel<64>, FwdTile<64>::kLds)) != hipSuccess) return err;
        hipLaunchKernelGGL(attn_fwd_bf16_kernel<64>, grid, block, FwdTile<64>::kLds, stream, p);
        if (split) hipLaunchKernelGGL(fwd_merge_kernel<64>, mgrid, dim3(256), 0, stream, p, merge_threads);
    }
    return hipGetLastError();
}

hipError_t launch_attn_fwd_f32(const float *q, const float *k, const float *v, float *o,
                               float *lse, const AttnShape &s, hipStream_t stream) {
    FwdF32Params p{q,      k,      v,    o,       lse,          s.N,  s.q_rs, s.k_rs,
                   s.v_rs, s.o_rs, s.cu, s.total, (int32_t)s.B, s.Hq, s.Hkv,  s.scale,
                   s.causal, 0};
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
