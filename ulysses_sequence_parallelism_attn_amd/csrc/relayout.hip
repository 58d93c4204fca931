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
// of the sequence-sharded one.  Both directions walk the SEQUENCE-SHARDED
// side in order, one 16-byte unit per lane, 64 lanes per workgroup: s2h reads
// it in order and h2s writes it in order.  A wave's 64 units are then 1 KiB
// contiguous on that side, and the head-sharded side's addresses form P
// contiguous streams (one per rank slice).  Walking the head-sharded side
// instead leaves the sequence side strided (one segment out of every H*d
// elements); measured on MI355X for [3, 65536, 32, 128] bf16 with P = 4,
// walking the sequence side moves 6.6 (s2h) and 6.8 (h2s) TB/s against 5.4
// and 6.0 TB/s, and more units per lane or larger workgroups only lose.
// The data is touched once, so loads and stores are non-temporal.  No
// arithmetic is done on the payload: it moves as opaque integers, which
// keeps every bit pattern (NaN payloads included).
//
// HBM bound: 2 * C*N*H*d*elt bytes of algorithmic traffic per call.

#include "ul_internal.h"

namespace ul {
namespace {

constexpr int kThreads = 64;  // one wave per workgroup, one unit per lane

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

// Head-sharded unit of sequence-sharded unit u: segment (c*N + t)*P + r of
// the sequence side is segment (c*P + r)*N + t of the head side.
__device__ __forceinline__ uint32_t head_unit32(uint32_t u, const Geo32 &g) {
    const uint32_t seg = g.ups.div(u);
    const uint32_t w = u - seg * g.ups.d;
    const uint32_t ct = g.p.div(seg);
    const uint32_t r = seg - ct * g.p.d;
    const uint32_t c = g.n.div(ct);
    const uint32_t t = ct - c * g.n.d;
    return ((c * g.p.d + r) * g.n.d + t) * g.ups.d + w;
}

__device__ __forceinline__ uint64_t head_unit64(uint64_t u, const Geo64 &g) {
    const uint64_t seg = u / g.ups, w = u % g.ups;
    const uint64_t r = seg % g.p, ct = seg / g.p, t = ct % g.n, c = ct / g.n;
    return ((c * g.p + r) * g.n + t) * g.ups + w;
}

// kToHead (s2h): out[head_unit(u)] = in[u];  h2s: out[u] = in[head_unit(u)].
template <typename Unit, bool kToHead>
__global__ __launch_bounds__(kThreads) void relayout32_kernel(const Unit *__restrict__ in,
                                                              Unit *__restrict__ out, Geo32 g) {
    const uint32_t u = blockIdx.x * (uint32_t)kThreads + threadIdx.x;
    if (u >= g.total) return;
    const uint32_t h = head_unit32(u, g);
    const Unit x = __builtin_nontemporal_load(in + (kToHead ? u : h));
    __builtin_nontemporal_store(x, out + (kToHead ? h : u));
}

// Above 2^32 units: the same map in 64-bit, grid-stride so that any size fits
// the grid.
template <typename Unit, bool kToHead>
__global__ __launch_bounds__(kThreads) void relayout64_kernel(const Unit *__restrict__ in,
                                                              Unit *__restrict__ out, Geo64 g) {
    const uint64_t stride = (uint64_t)gridDim.x * kThreads;
    for (uint64_t u = (uint64_t)blockIdx.x * kThreads + threadIdx.x; u < g.total; u += stride) {
        const uint64_t h = head_unit64(u, g);
        const Unit x = __builtin_nontemporal_load(in + (kToHead ? u : h));
        __builtin_nontemporal_store(x, out + (kToHead ? h : u));
    }
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr uint64_t kMaxBlocks = 1ull << 24;  // grid cap of the 64-bit kernels (2^30 lanes)

template <typename Unit>
hipError_t launch_typed(const void *in, void *out, uint64_t seg_units, uint64_t n, uint64_t p,
                        uint64_t total, bool to_head, hipStream_t stream) {
    const uint64_t blocks = (total + kThreads - 1) / kThreads;
    if (blocks == 0) return hipSuccess;
    const dim3 block(kThreads);
    const Unit *src = static_cast<const Unit *>(in);
    Unit *dst = static_cast<Unit *>(out);
    // 32-bit path: every unit index, and the grid's last lane, below 2^32.
    if (total + kThreads < (1ull << 32)) {
        const dim3 grid((uint32_t)blocks);
        Geo32 g{FastDiv32((uint32_t)seg_units), FastDiv32((uint32_t)n), FastDiv32((uint32_t)p),
                (uint32_t)total};
        if (to_head)
            hipLaunchKernelGGL((relayout32_kernel<Unit, true>), grid, block, 0, stream, src, dst, g);
        else
            hipLaunchKernelGGL((relayout32_kernel<Unit, false>), grid, block, 0, stream, src, dst, g);
    } else {
        const dim3 grid((uint32_t)(blocks < kMaxBlocks ? blocks : kMaxBlocks));
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
// with row = H*d, rank = Hs*d and off = h0*d (in units).  As in the full
// exchange, both directions walk the sequence-sharded side's units in order
// (token rows, then ranks, then the chunk's units), one unit per lane.

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

// Head-sharded and sequence-sharded unit of the u-th moved unit, u walking
// segments s = (c*N + t)*P + r.
__device__ __forceinline__ void chunk_units32(uint32_t u, const ChunkGeo32 &g, uint32_t &head,
                                              uint32_t &seq) {
    const uint32_t s = g.ups.div(u);
    const uint32_t w = u - s * g.ups.d;
    const uint32_t ct = g.p.div(s);
    const uint32_t r = s - ct * g.p.d;
    const uint32_t c = g.n.div(ct);
    const uint32_t t = ct - c * g.n.d;
    head = ((c * g.p.d + r) * g.n.d + t) * g.ups.d + w;
    seq = (c * g.n.d + t) * g.row + r * g.rank + g.off + w;
}

__device__ __forceinline__ void chunk_units64(uint64_t u, const ChunkGeo64 &g, uint64_t &head,
                                              uint64_t &seq) {
    const uint64_t s = u / g.ups, w = u % g.ups;
    const uint64_t r = s % g.p, t = (s / g.p) % g.n, c = s / g.p / g.n;
    head = ((c * g.p + r) * g.n + t) * g.ups + w;
    seq = (c * g.n + t) * g.row + r * g.rank + g.off + w;
}

template <typename Unit, bool kToHead>
__global__ __launch_bounds__(kThreads) void relayout_heads32_kernel(const Unit *__restrict__ in,
                                                                    Unit *__restrict__ out,
                                                                    ChunkGeo32 g) {
    const uint32_t u = blockIdx.x * (uint32_t)kThreads + threadIdx.x;
    if (u >= g.total) return;
    uint32_t head, seq;
    chunk_units32(u, g, head, seq);
    const Unit x = __builtin_nontemporal_load(in + (kToHead ? seq : head));
    __builtin_nontemporal_store(x, out + (kToHead ? head : seq));
}

template <typename Unit, bool kToHead>
__global__ __launch_bounds__(kThreads) void relayout_heads64_kernel(const Unit *__restrict__ in,
                                                                    Unit *__restrict__ out,
                                                                    ChunkGeo64 g) {
    const uint64_t stride = (uint64_t)gridDim.x * kThreads;
    for (uint64_t u = (uint64_t)blockIdx.x * kThreads + threadIdx.x; u < g.total; u += stride) {
        uint64_t head, seq;
        chunk_units64(u, g, head, seq);
        const Unit x = __builtin_nontemporal_load(in + (kToHead ? seq : head));
        __builtin_nontemporal_store(x, out + (kToHead ? head : seq));
    }
}

template <typename Unit>
hipError_t launch_heads_typed(const void *in, void *out, uint64_t C, uint64_t N, uint64_t P,
                              uint64_t ups, uint64_t row, uint64_t rank, uint64_t off,
                              bool to_head, hipStream_t stream) {
    const uint64_t total = C * P * N * ups;
    const uint64_t blocks = (total + kThreads - 1) / kThreads;
    if (blocks == 0) return hipSuccess;
    const dim3 block(kThreads);
    const Unit *src = static_cast<const Unit *>(in);
    Unit *dst = static_cast<Unit *>(out);
    // 32-bit path: every unit index on both sides (the sequence-sharded side
    // spans C*N*row units), and the grid's last lane, below 2^32.
    if (total + kThreads < (1ull << 32) && C * N * row < (1ull << 32)) {
        const dim3 grid((uint32_t)blocks);
        ChunkGeo32 g{FastDiv32((uint32_t)ups), FastDiv32((uint32_t)N), FastDiv32((uint32_t)P),
                     (uint32_t)total, (uint32_t)row, (uint32_t)rank, (uint32_t)off};
        if (to_head)
            hipLaunchKernelGGL((relayout_heads32_kernel<Unit, true>), grid, block, 0, stream, src, dst, g);
        else
            hipLaunchKernelGGL((relayout_heads32_kernel<Unit, false>), grid, block, 0, stream, src, dst, g);
    } else {
        const dim3 grid((uint32_t)(blocks < kMaxBlocks ? blocks : kMaxBlocks));
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
