// relayout.hip -- sequence-sharded <-> head-sharded permutation on one GPU.
//
// "Ulysses Sequence Parallelism: Training with Million-Token Contexts",
// section "How Does Ulysses Sequence Parallelism Actually Work?": each GPU
// starts with a contiguous chunk of N/P tokens for all H heads; after the
// all-to-all it holds all N tokens for a contiguous slice of H/P heads, and
// the reversed shuffle undoes that.  In the world view of one buffer:
//
//   s2h:  out[c][r][t][hh][e] = in[c][t][r*Hs + hh][e]        (Hs = H/P)
//   h2s:  out[c][t][h][e]     = in[c][h/Hs][t][h%Hs][e]
//
// Both sides consist of contiguous "segments" of Hs*d elements: segment
// (c, r, t) of the head-sharded tensor is the r-th slice of token row (c, t)
// of the sequence-sharded one.  The kernel walks the OUTPUT in order, one
// 16-byte unit per lane per step, so stores are fully coalesced and loads are
// coalesced within each segment (2 KiB for 8 heads x 128 x bf16).  The data
// is touched once, so loads and stores are non-temporal.  No arithmetic is
// done on the payload: it moves as opaque integers, which keeps every bit
// pattern (NaN payloads included).
//
// HBM bound: 2 * C*N*H*d*elt bytes of algorithmic traffic per call.

#include "ul_internal.h"

namespace ul {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;  // units per lane per block step, all loads issued before stores

// Index maps are evaluated in 32-bit with FastDiv32 when every index fits;
// the host picks the 64-bit instantiation otherwise.
struct Geo32 {
    FastDiv32 ups;  // units per segment
    FastDiv32 n;    // N
    FastDiv32 p;    // P
    uint32_t total; // total units
};

struct Geo64 {
    uint64_t ups, n, p, total;
};

template <bool kToHead>
__device__ __forceinline__ uint32_t src_unit32(uint32_t u, const Geo32 &g) {
    const uint32_t seg = g.ups.div(u);
    const uint32_t w = u - seg * g.ups.d;
    uint32_t src_seg;
    if (kToHead) {
        // output segment seg = (c*P + r)*N + t  ->  input segment (c*N + t)*P + r
        const uint32_t cr = g.n.div(seg);
        const uint32_t t = seg - cr * g.n.d;
        const uint32_t c = g.p.div(cr);
        const uint32_t r = cr - c * g.p.d;
        src_seg = (c * g.n.d + t) * g.p.d + r;
    } else {
        // output segment seg = (c*N + t)*P + r  ->  input segment (c*P + r)*N + t
        const uint32_t ct = g.p.div(seg);
        const uint32_t r = seg - ct * g.p.d;
        const uint32_t c = g.n.div(ct);
        const uint32_t t = ct - c * g.n.d;
        src_seg = (c * g.p.d + r) * g.n.d + t;
    }
    return src_seg * g.ups.d + w;
}

template <bool kToHead>
__device__ __forceinline__ uint64_t src_unit64(uint64_t u, const Geo64 &g) {
    const uint64_t seg = u / g.ups, w = u % g.ups;
    uint64_t src_seg;
    if (kToHead) {
        const uint64_t t = seg % g.n, cr = seg / g.n, r = cr % g.p, c = cr / g.p;
        src_seg = (c * g.n + t) * g.p + r;
    } else {
        const uint64_t r = seg % g.p, ct = seg / g.p, t = ct % g.n, c = ct / g.n;
        src_seg = (c * g.p + r) * g.n + t;
    }
    return src_seg * g.ups + w;
}

template <typename Unit, bool kToHead>
__global__ __launch_bounds__(kThreads) void relayout32_kernel(const Unit *__restrict__ in,
                                                              Unit *__restrict__ out, Geo32 g) {
    const uint32_t base = blockIdx.x * (uint32_t)(kThreads * kUnroll) + threadIdx.x;
    Unit buf[kUnroll];
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) {
        const uint32_t u = base + k * kThreads;
        if (u < g.total) buf[k] = __builtin_nontemporal_load(in + src_unit32<kToHead>(u, g));
    }
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) {
        const uint32_t u = base + k * kThreads;
        if (u < g.total) __builtin_nontemporal_store(buf[k], out + u);
    }
}

template <typename Unit, bool kToHead>
__global__ __launch_bounds__(kThreads) void relayout64_kernel(const Unit *__restrict__ in,
                                                              Unit *__restrict__ out, Geo64 g) {
    const uint64_t base = (uint64_t)blockIdx.x * (kThreads * kUnroll) + threadIdx.x;
    Unit buf[kUnroll];
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) {
        const uint64_t u = base + (uint64_t)k * kThreads;
        if (u < g.total) buf[k] = __builtin_nontemporal_load(in + src_unit64<kToHead>(u, g));
    }
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) {
        const uint64_t u = base + (uint64_t)k * kThreads;
        if (u < g.total) __builtin_nontemporal_store(buf[k], out + u);
    }
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <typename Unit>
hipError_t launch_typed(const void *in, void *out, uint64_t seg_units, uint64_t n, uint64_t p,
                        uint64_t total, bool to_head, hipStream_t stream) {
    const uint64_t per_block = (uint64_t)kThreads * kUnroll;
    const uint64_t blocks = (total + per_block - 1) / per_block;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7fffffffull) return hipErrorInvalidConfiguration;
    const dim3 grid((uint32_t)blocks), block(kThreads);
    const Unit *src = static_cast<const Unit *>(in);
    Unit *dst = static_cast<Unit *>(out);
    // 32-bit path: every unit index, and base + unroll span, below 2^32.
    if (total + per_block < (1ull << 32)) {
        Geo32 g{FastDiv32((uint32_t)seg_units), FastDiv32((uint32_t)n), FastDiv32((uint32_t)p),
                (uint32_t)total};
        if (to_head)
            hipLaunchKernelGGL((relayout32_kernel<Unit, true>), grid, block, 0, stream, src, dst, g);
        else
            hipLaunchKernelGGL((relayout32_kernel<Unit, false>), grid, block, 0, stream, src, dst, g);
    } else {
        Geo64 g{seg_units, n, p, total};
        if (to_head)
            hipLaunchKernelGGL((relayout64_kernel<Unit, true>), grid, block, 0, stream, src, dst, g);
        else
            hipLaunchKernelGGL((relayout64_kernel<Unit, false>), grid, block, 0, stream, src, dst, g);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------- head chunks
//
// The same exchange for Hc heads starting h0 heads into every rank's slice:
//
//   s2h:  out[c][r][t][hh][e] = in[c][t][r*Hs + h0 + hh][e]     hh < Hc
//   h2s:  the inverse, writing only those heads of the sequence-sharded side
//
// A rank that works through its heads a few at a time exchanges one chunk
// per call, so its head-sharded buffers hold Hc heads instead of Hs.  A
// segment is now the chunk's Hc*d elements of one (c, r, t); on the
// sequence-sharded side it starts at  (c*N + t)*row + r*rank + off  units,
// with row = H*d, rank = Hs*d and off = h0*d (in units).  Each kernel walks
// its OUTPUT in order, as the full exchange does: the head-sharded side for
// s2h, the chunk's units of each token row for h2s.

struct ChunkGeo32 {
    FastDiv32 ups;  // units per segment
    FastDiv32 n;    // N
    FastDiv32 p;    // P
    uint32_t total; // units moved: C*P*N*ups
    uint32_t row, rank, off;
};

struct ChunkGeo64 {
    uint64_t ups, n, p, total, row, rank, off;
};

// Head-sharded and sequence-sharded unit of the u-th unit in output order.
template <bool kToHead>
__device__ __forceinline__ void chunk_units32(uint32_t u, const ChunkGeo32 &g, uint32_t &head,
                                              uint32_t &seq) {
    const uint32_t s = g.ups.div(u);
    const uint32_t w = u - s * g.ups.d;
    uint32_t c, r, t;
    if (kToHead) {  // s = (c*P + r)*N + t
        const uint32_t cr = g.n.div(s);
        t = s - cr * g.n.d;
        c = g.p.div(cr);
        r = cr - c * g.p.d;
    } else {        // s = (c*N + t)*P + r
        const uint32_t ct = g.p.div(s);
        r = s - ct * g.p.d;
        c = g.n.div(ct);
        t = ct - c * g.n.d;
    }
    head = ((c * g.p.d + r) * g.n.d + t) * g.ups.d + w;
    seq = (c * g.n.d + t) * g.row + r * g.rank + g.off + w;
}

template <bool kToHead>
__device__ __forceinline__ void chunk_units64(uint64_t u, const ChunkGeo64 &g, uint64_t &head,
                                              uint64_t &seq) {
    const uint64_t s = u / g.ups, w = u % g.ups;
    uint64_t c, r, t;
    if (kToHead) {
        t = s % g.n;
        r = (s / g.n) % g.p;
        c = s / g.n / g.p;
    } else {
        r = s % g.p;
        t = (s / g.p) % g.n;
        c = s / g.p / g.n;
    }
    head = ((c * g.p + r) * g.n + t) * g.ups + w;
    seq = (c * g.n + t) * g.row + r * g.rank + g.off + w;
}

template <typename Unit, bool kToHead>
__global__ __launch_bounds__(kThreads) void relayout_heads32_kernel(const Unit *__restrict__ in,
                                                                    Unit *__restrict__ out,
                                                                    ChunkGeo32 g) {
    const uint32_t base = blockIdx.x * (uint32_t)(kThreads * kUnroll) + threadIdx.x;
    Unit buf[kUnroll];
    uint32_t dst[kUnroll];
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) {
        const uint32_t u = base + k * kThreads;
        if (u < g.total) {
            uint32_t head, seq;
            chunk_units32<kToHead>(u, g, head, seq);
            buf[k] = __builtin_nontemporal_load(in + (kToHead ? seq : head));
            dst[k] = kToHead ? head : seq;
        }
    }
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) {
        const uint32_t u = base + k * kThreads;
        if (u < g.total) __builtin_nontemporal_store(buf[k], out + dst[k]);
    }
}

template <typename Unit, bool kToHead>
__global__ __launch_bounds__(kThreads) void relayout_heads64_kernel(const Unit *__restrict__ in,
                                                                    Unit *__restrict__ out,
                                                                    ChunkGeo64 g) {
    const uint64_t base = (uint64_t)blockIdx.x * (kThreads * kUnroll) + threadIdx.x;
    Unit buf[kUnroll];
    uint64_t dst[kUnroll];
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) {
        const uint64_t u = base + (uint64_t)k * kThreads;
        if (u < g.total) {
            uint64_t head, seq;
            chunk_units64<kToHead>(u, g, head, seq);
            buf[k] = __builtin_nontemporal_load(in + (kToHead ? seq : head));
            dst[k] = kToHead ? head : seq;
        }
    }
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) {
        const uint64_t u = base + (uint64_t)k * kThreads;
        if (u < g.total) __builtin_nontemporal_store(buf[k], out + dst[k]);
    }
}

template <typename Unit>
hipError_t launch_heads_typed(const void *in, void *out, uint64_t C, uint64_t N, uint64_t P,
                              uint64_t ups, uint64_t row, uint64_t rank, uint64_t off,
                              bool to_head, hipStream_t stream) {
    const uint64_t total = C * P * N * ups;
    const uint64_t per_block = (uint64_t)kThreads * kUnroll;
    const uint64_t blocks = (total + per_block - 1) / per_block;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7fffffffull) return hipErrorInvalidConfiguration;
    const dim3 grid((uint32_t)blocks), block(kThreads);
    const Unit *src = static_cast<const Unit *>(in);
    Unit *dst = static_cast<Unit *>(out);
    // 32-bit path: every unit index on both sides (the sequence-sharded side
    // spans C*N*row units), and base + unroll span, below 2^32.
    if (total + per_block < (1ull << 32) && C * N * row < (1ull << 32)) {
        ChunkGeo32 g{FastDiv32((uint32_t)ups), FastDiv32((uint32_t)N), FastDiv32((uint32_t)P),
                     (uint32_t)total, (uint32_t)row, (uint32_t)rank, (uint32_t)off};
        if (to_head)
            hipLaunchKernelGGL((relayout_heads32_kernel<Unit, true>), grid, block, 0, stream, src, dst, g);
        else
            hipLaunchKernelGGL((relayout_heads32_kernel<Unit, false>), grid, block, 0, stream, src, dst, g);
    } else {
        ChunkGeo64 g{ups, N, P, total, row, rank, off};
        if (to_head)
            hipLaunchKernelGGL((relayout_heads64_kernel<Unit, true>), grid, block, 0, stream, src, dst, g);
        else
            hipLaunchKernelGGL((relayout_heads64_kernel<Unit, false>), grid, block, 0, stream, src, dst, g);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_relayout_heads(const void *in, void *out, int64_t C, int64_t N, int64_t H,
                                 int64_t d, int64_t P, int64_t h0, int64_t Hc, int64_t elt,
                                 bool to_head, hipStream_t stream) {
    const uint64_t row_b = (uint64_t)H * d * elt, rank_b = (uint64_t)(H / P) * d * elt;
    const uint64_t off_b = (uint64_t)h0 * d * elt, seg_b = (uint64_t)Hc * d * elt;
    // the widest unit that divides every extent and offset and both pointers
    const uint64_t all = row_b | rank_b | off_b | seg_b | (uint64_t)(uintptr_t)in |
                         (uint64_t)(uintptr_t)out;
    const uint64_t U = (all % 16 == 0) ? 16 : (all % 4 == 0) ? 4 : (all % 2 == 0) ? 2 : 1;
    const uint64_t c = (uint64_t)C, n = (uint64_t)N, p = (uint64_t)P;
    if (U == 16)
        return launch_heads_typed<u32x4>(in, out, c, n, p, seg_b / 16, row_b / 16, rank_b / 16,
                                         off_b / 16, to_head, stream);
    if (U == 4)
        return launch_heads_typed<uint32_t>(in, out, c, n, p, seg_b / 4, row_b / 4, rank_b / 4,
                                            off_b / 4, to_head, stream);
    if (U == 2)
        return launch_heads_typed<uint16_t>(in, out, c, n, p, seg_b / 2, row_b / 2, rank_b / 2,
                                            off_b / 2, to_head, stream);
    return launch_heads_typed<uint8_t>(in, out, c, n, p, seg_b, row_b, rank_b, off_b, to_head,
                                       stream);
}

hipError_t launch_relayout(const void *in, void *out, int64_t C, int64_t N, int64_t H, int64_t d,
                           int64_t P, int64_t elt, bool to_head, hipStream_t stream) {
    const uint64_t seg_bytes = (uint64_t)(H / P) * (uint64_t)d * (uint64_t)elt;
    const uint64_t nseg = (uint64_t)C * (uint64_t)P * (uint64_t)N;
    const bool aligned16 = ((uintptr_t)in % 16 == 0) && ((uintptr_t)out % 16 == 0);
    if (seg_bytes % 16 == 0 && aligned16)
        return launch_typed<u32x4>(in, out, seg_bytes / 16, N, P, nseg * (seg_bytes / 16), to_head,
                                   stream);
    if (seg_bytes % 4 == 0 && (uintptr_t)in % 4 == 0 && (uintptr_t)out % 4 == 0)
        return launch_typed<uint32_t>(in, out, seg_bytes / 4, N, P, nseg * (seg_bytes / 4),
                                      to_head, stream);
    if (seg_bytes % 2 == 0 && (uintptr_t)in % 2 == 0 && (uintptr_t)out % 2 == 0)
        return launch_typed<uint16_t>(in, out, seg_bytes / 2, N, P, nseg * (seg_bytes / 2),
                                      to_head, stream);
    return launch_typed<uint8_t>(in, out, seg_bytes, N, P, nseg * seg_bytes, to_head, stream);
}

}  // namespace ul
