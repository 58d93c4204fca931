// ul_internal.h -- internal declarations shared by the host API and the HIP
// kernel files of libulattn.so (not installed, not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/ul_attn.h"

namespace ul {

// Unsigned 32-bit division by a runtime-invariant divisor d >= 1 with one
// multiply-high, an add and two shifts (Granlund and Montgomery, "Division by
// invariant integers using multiplication", 1994, unsigned case): with
// l = ceil(log2 d) and m = floor(2^32 (2^l - d) / d) + 1,
//   t = mulhi(m, n),  n / d = (t + ((n - t) >> min(l,1))) >> max(l-1,0).
struct FastDiv32 {
    uint32_t d = 1, m = 1, sh1 = 0, sh2 = 0;
    FastDiv32() = default;
    explicit FastDiv32(uint32_t div) : d(div) {
        uint32_t l = 0;
        while ((1ull << l) < div) ++l;
        m = (uint32_t)((((1ull << l) - div) << 32) / div + 1);
        sh1 = l < 1 ? l : 1;
        sh2 = l > 1 ? l - 1 : 0;
    }
    __host__ __device__ __forceinline__ uint32_t div(uint32_t n) const {
#if defined(__HIP_DEVICE_COMPILE__)
        const uint32_t t = __umulhi(n, m);
#else
        const uint32_t t = (uint32_t)(((uint64_t)n * m) >> 32);
#endif
        return (t + ((n - t) >> sh1)) >> sh2;
    }
};

// The tokens of sequence b of a call and where its statistics live.  With
// no table (cu == nullptr) the call holds B sequences of N tokens each, lse
// is [B][Hq][N] and the backward statistics are [B][Hq][2][N].  With a table
// the call holds packed variable-length sequences: sequence b is tokens
// [cu[b], cu[b+1]) of `total`, lse is [Hq][total] and the statistics are
// [Hq][2][total].  Table entries are clamped into [0, total] and a length to
// at most N (the caller's maximum), so a malformed table can give wrong
// values but never an access outside the tensors.
struct SeqRange {
    int64_t tok0;  // first token of the sequence
    int32_t len;   // its number of tokens
    int64_t lse0;  // lse index of (head 0, row 0); head h adds h * hs
    int64_t st0;   // statistics index of (head 0, row 0); head h adds 2h * hs, D is hs further
    int64_t hs;
};

__host__ __device__ __forceinline__ SeqRange seq_range(const int32_t *cu, int b, int64_t N, int32_t Hq,
                                              int64_t total) {
    SeqRange r;
    if (cu) {
        int64_t a = cu[b], e = cu[b + 1];
        a = a < 0 ? 0 : (a > total ? total : a);
        e = e < a ? a : (e > total ? total : e);
        r.tok0 = a;
        r.len = (int32_t)(e - a < N ? e - a : N);
        r.lse0 = a;
        r.st0 = a;
        r.hs = total;
    } else {
        r.tok0 = (int64_t)b * N;
        r.len = (int32_t)N;
        r.lse0 = (int64_t)b * Hq * N;
        r.st0 = 2 * r.lse0;
        r.hs = N;
    }
    return r;
}

// Lets `kernel` take `bytes` of dynamic LDS (the default limit is 64 KB).
template <typename KernelT>
inline hipError_t allow_lds(KernelT kernel, size_t bytes) {
    if (bytes <= 64 * 1024) return hipSuccess;
    return hipFuncSetAttribute(reinterpret_cast<const void *>(kernel),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

// ---------------------------------------------------------------- launchers
// Each returns hipSuccess or the launch error; arguments are already
// validated by the host API.

hipError_t launch_relayout(const void *in, void *out, int64_t C, int64_t N, int64_t H, int64_t d,
                           int64_t P, int64_t elt, bool to_head, hipStream_t stream);
// The exchange of heads h0 .. h0+Hc-1 of every rank's slice (h0 + Hc <= H/P).
hipError_t launch_relayout_heads(const void *in, void *out, int64_t C, int64_t N, int64_t H,
                                 int64_t d, int64_t P, int64_t h0, int64_t Hc, int64_t elt,
                                 bool to_head, hipStream_t stream);

// Sizes of one attention call.  Token t of batch b of a tensor starts
// (b*N + t) * its token stride elements from the tensor's base pointer; head
// h of that token starts h*d elements later.
struct AttnShape {
    int64_t B, N;
    int32_t Hq, Hkv, d;
    float scale;
    int32_t causal;
    int64_t q_rs, k_rs, v_rs, o_rs, do_rs, dq_rs, dk_rs, dv_rs;  // token strides, elements
    // Packed variable-length sequences: B sequences given by the device table
    // cu (B + 1 entries) over `total` tokens, N the longest; nullptr for B
    // sequences of N tokens.
    const int32_t *cu = nullptr;
    int64_t total = 0;
};

hipError_t launch_attn_fwd_f32(const float *q, const float *k, const float *v, float *o,
                               float *lse, const AttnShape &s, hipStream_t stream);
// Device workspace of the bf16 forward's split key range (0 when these sizes
// run unsplit); launch_attn_fwd_bf16 with a null `ws` runs unsplit.
size_t attn_fwd_workspace_bytes(const AttnShape &s, int32_t dtype);
hipError_t launch_attn_fwd_bf16(const void *q, const void *k, const void *v, void *o, float *lse,
                                void *ws, const AttnShape &s, hipStream_t stream);

size_t attn_bwd_workspace_bytes(const AttnShape &s, int32_t dtype);
hipError_t launch_attn_bwd_f32(const float *q, const float *k, const float *v, const float *o,
                               const float *dout, const float *lse, float *dq, float *dk,
                               float *dv, void *ws, const AttnShape &s, int stages, hipStream_t stream);
hipError_t launch_attn_bwd_bf16(const void *q, const void *k, const void *v, const void *o,
                                const void *dout, const float *lse, void *dq, void *dk, void *dv,
                                void *ws, const AttnShape &s, int stages, hipStream_t stream);

}  // namespace ul
