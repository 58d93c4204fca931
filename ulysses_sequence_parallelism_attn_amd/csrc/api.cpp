// api.cpp -- the extern "C" entry points of libulattn.so: argument
// validation (entirely on the host, before any HIP call) and dispatch to the
// kernel launchers.  The contract of each function is documented in
// include/ul_attn.h.

#include <math.h>
#include <stdint.h>

#include "ul_internal.h"

namespace {

using ul::AttnShape;

bool mul_ok(int64_t a, int64_t b, int64_t *out) {
    if (a < 0 || b < 0) return false;
    if (a != 0 && b > INT64_MAX / a) return false;
    *out = a * b;
    return true;
}

// Product of all factors, false on overflow.
bool elems(int64_t *out, std::initializer_list<int64_t> f) {
    int64_t acc = 1;
    for (int64_t x : f)
        if (!mul_ok(acc, x, &acc)) return false;
    *out = acc;
    return true;
}

int64_t elt_size(int32_t dtype) { return dtype == UL_F32 ? 4 : 2; }

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

Range range(const void *p, int64_t bytes) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Range{lo, lo + (uintptr_t)bytes};
}

bool aligned16(const void *p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; }

struct AttnSizes {
    int64_t q_bytes, kv_bytes, lse_bytes;
};

ul_status check_attn(int64_t B, int64_t N, int32_t Hq, int32_t Hkv, int32_t head_dim, float scale,
                     int32_t causal, int32_t dtype, AttnSizes *sz) {
    if (B < 1 || N < 1 || Hq < 1 || Hkv < 1 || head_dim < 1) return UL_ERR_SHAPE;
    if (!isfinite(scale) || !(scale > 0.f)) return UL_ERR_SHAPE;
    if (causal != 0 && causal != 1) return UL_ERR_SHAPE;
    if (Hq % Hkv != 0) return UL_ERR_DIVISIBILITY;
    if (dtype != UL_F32 && dtype != UL_BF16) return UL_ERR_UNSUPPORTED;
    if (head_dim != 64 && head_dim != 128) return UL_ERR_UNSUPPORTED;
    const int64_t es = elt_size(dtype);
    int64_t qe, kve, le;
    if (!elems(&qe, {B, N, Hq, head_dim, es}) || !elems(&kve, {B, N, Hkv, head_dim, es}) ||
        !elems(&le, {B, N, Hq, 4}))
        return UL_ERR_SHAPE;
    // kernel index arithmetic: per-launch work-item counts fit in 31 bits and
    // row indices in int64; B and N individually fit in 32 bits.
    if (B > INT32_MAX || N > INT32_MAX) return UL_ERR_SHAPE;
    sz->q_bytes = qe;
    sz->kv_bytes = kve;
    sz->lse_bytes = le;
    return UL_OK;
}

ul_status check_relayout(const void *in, const void *out, int64_t C, int64_t N, int32_t H,
                         int32_t head_dim, int32_t P, int32_t dtype, int64_t *bytes) {
    if (!in || !out) return UL_ERR_NULL;
    if (C < 1 || N < 1 || H < 1 || head_dim < 1) return UL_ERR_SHAPE;
    if (P < 1 || H % P != 0 || N % P != 0) return UL_ERR_DIVISIBILITY;
    if (dtype != UL_F32 && dtype != UL_BF16) return UL_ERR_UNSUPPORTED;
    if (!elems(bytes, {C, N, H, head_dim, elt_size(dtype)})) return UL_ERR_SHAPE;
    if (overlap(range(in, *bytes), range(out, *bytes))) return UL_ERR_OVERLAP;
    return UL_OK;
}

ul_status from_hip(hipError_t e) { return e == hipSuccess ? UL_OK : UL_ERR_HIP; }

}  // namespace

extern "C" {

const char *ul_status_str(ul_status s) {
    switch (s) {
        case UL_OK: return "UL_OK";
        case UL_ERR_NULL: return "UL_ERR_NULL";
        case UL_ERR_SHAPE: return "UL_ERR_SHAPE";
        case UL_ERR_DIVISIBILITY: return "UL_ERR_DIVISIBILITY";
        case UL_ERR_UNSUPPORTED: return "UL_ERR_UNSUPPORTED";
        case UL_ERR_ALIGNMENT: return "UL_ERR_ALIGNMENT";
        case UL_ERR_WORKSPACE: return "UL_ERR_WORKSPACE";
        case UL_ERR_OVERLAP: return "UL_ERR_OVERLAP";
        case UL_ERR_HIP: return "UL_ERR_HIP";
    }
    return "UL_ERR_UNKNOWN";
}

ul_status ul_relayout_s2h(const void *in, void *out, int64_t C, int64_t N, int32_t H,
                          int32_t head_dim, int32_t P, int32_t dtype, void *stream) {
    int64_t bytes;
    const ul_status st = check_relayout(in, out, C, N, H, head_dim, P, dtype, &bytes);
    if (st != UL_OK) return st;
    return from_hip(ul::launch_relayout(in, out, C, N, H, head_dim, P, elt_size(dtype), true,
                                        static_cast<hipStream_t>(stream)));
}

ul_status ul_relayout_h2s(const void *in, void *out, int64_t C, int64_t N, int32_t H,
                          int32_t head_dim, int32_t P, int32_t dtype, void *stream) {
    int64_t bytes;
    const ul_status st = check_relayout(in, out, C, N, H, head_dim, P, dtype, &bytes);
    if (st != UL_OK) return st;
    return from_hip(ul::launch_relayout(in, out, C, N, H, head_dim, P, elt_size(dtype), false,
                                        static_cast<hipStream_t>(stream)));
}

ul_status ul_attn_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
                      int64_t B, int64_t N, int32_t Hq, int32_t Hkv, int32_t head_dim,
                      float softmax_scale, int32_t causal, int32_t dtype, void *stream) {
    if (!q || !k || !v || !o || !lse) return UL_ERR_NULL;
    AttnSizes sz;
    const ul_status st = check_attn(B, N, Hq, Hkv, head_dim, softmax_scale, causal, dtype, &sz);
    if (st != UL_OK) return st;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
        return UL_ERR_ALIGNMENT;
    const Range rq = range(q, sz.q_bytes), rk = range(k, sz.kv_bytes), rv = range(v, sz.kv_bytes);
    const Range ro = range(o, sz.q_bytes), rl = range(lse, sz.lse_bytes);
    for (Range out : {ro, rl})
        for (Range in : {rq, rk, rv})
            if (overlap(out, in)) return UL_ERR_OVERLAP;
    if (overlap(ro, rl)) return UL_ERR_OVERLAP;
    const AttnShape s{B, N, Hq, Hkv, head_dim, softmax_scale, causal};
    hipStream_t hs = static_cast<hipStream_t>(stream);
    if (dtype == UL_F32)
        return from_hip(ul::launch_attn_fwd_f32(static_cast<const float *>(q),
                                                static_cast<const float *>(k),
                                                static_cast<const float *>(v),
                                                static_cast<float *>(o), lse, s, hs));
    return from_hip(ul::launch_attn_fwd_bf16(q, k, v, o, lse, s, hs));
}

size_t ul_attn_bwd_workspace_bytes(int64_t B, int64_t N, int32_t Hq, int32_t Hkv,
                                   int32_t head_dim, int32_t dtype) {
    AttnSizes sz;
    if (check_attn(B, N, Hq, Hkv, head_dim, 1.0f, 1, dtype, &sz) != UL_OK) return 0;
    const AttnShape s{B, N, Hq, Hkv, head_dim, 1.0f, 1};
    return ul::attn_bwd_workspace_bytes(s, dtype);
}

ul_status ul_attn_bwd_stages(int32_t stages, const void *q, const void *k, const void *v,
                             const void *o, const void *dout, const float *lse, void *dq, void *dk,
                             void *dv, void *workspace, size_t workspace_bytes, int64_t B,
                             int64_t N, int32_t Hq, int32_t Hkv, int32_t head_dim,
                             float softmax_scale, int32_t causal, int32_t dtype, void *stream) {
    if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return UL_ERR_NULL;
    AttnSizes sz;
    const ul_status st = check_attn(B, N, Hq, Hkv, head_dim, softmax_scale, causal, dtype, &sz);
    if (st != UL_OK) return st;
    if (stages < 1 || (stages & ~UL_BWD_ALL) != 0) return UL_ERR_UNSUPPORTED;
    const AttnShape s{B, N, Hq, Hkv, head_dim, softmax_scale, causal};
    const size_t need = ul::attn_bwd_workspace_bytes(s, dtype);
    if (!workspace || workspace_bytes < need) return UL_ERR_WORKSPACE;
    for (const void *ptr : {q, k, v, o, dout, (const void *)lse, (const void *)dq, (const void *)dk,
                            (const void *)dv, (const void *)workspace})
        if (!aligned16(ptr)) return UL_ERR_ALIGNMENT;
    const Range ins[] = {range(q, sz.q_bytes),  range(k, sz.kv_bytes),  range(v, sz.kv_bytes),
                         range(o, sz.q_bytes),  range(dout, sz.q_bytes), range(lse, sz.lse_bytes)};
    const Range outs[] = {range(dq, sz.q_bytes), range(dk, sz.kv_bytes), range(dv, sz.kv_bytes),
                          range(workspace, (int64_t)need)};
    for (int a = 0; a < 4; ++a) {
        for (const Range &in : ins)
            if (overlap(outs[a], in)) return UL_ERR_OVERLAP;
        for (int c = a + 1; c < 4; ++c)
            if (overlap(outs[a], outs[c])) return UL_ERR_OVERLAP;
    }
    hipStream_t hs = static_cast<hipStream_t>(stream);
    if (dtype == UL_F32)
        return from_hip(ul::launch_attn_bwd_f32(
            static_cast<const float *>(q), static_cast<const float *>(k),
            static_cast<const float *>(v), static_cast<const float *>(o),
            static_cast<const float *>(dout), lse, static_cast<float *>(dq),
            static_cast<float *>(dk), static_cast<float *>(dv), workspace, s, stages, hs));
    return from_hip(ul::launch_attn_bwd_bf16(q, k, v, o, dout, lse, dq, dk, dv, workspace, s, stages, hs));
}

ul_status ul_attn_bwd(const void *q, const void *k, const void *v, const void *o,
                      const void *dout, const float *lse, void *dq, void *dk, void *dv,
                      void *workspace, size_t workspace_bytes, int64_t B, int64_t N, int32_t Hq,
                      int32_t Hkv, int32_t head_dim, float softmax_scale, int32_t causal,
                      int32_t dtype, void *stream) {
    return ul_attn_bwd_stages(UL_BWD_ALL, q, k, v, o, dout, lse, dq, dk, dv, workspace,
                              workspace_bytes, B, N, Hq, Hkv, head_dim, softmax_scale, causal, dtype,
                              stream);
}

}  // extern "C"
