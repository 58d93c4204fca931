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

}  // namespace

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
