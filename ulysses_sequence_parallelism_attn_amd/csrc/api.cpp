// api.cpp -- the extern "C" entry points of libulattn.so: argument
// validation (entirely on the host, before any HIP call) and dispatch to the
// kernel launchers.  The contract of each function is documented in
// include/ul_attn.h.

#include <math.h>
#include <stdint.h>

#include <mutex>

#include "ul_internal.h"

// Scratch of ul_attn_bwd_noalloc: a file-scope device array, one copy per GPU
// the library runs on, held until the process ends.  Host code never passes
// `scratch` itself to a kernel (its host-side name is not a device address):
// the device address comes from hipGetSymbolAddress, once per device.
__device__ __align__(256) unsigned char scratch[UL_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_addr[kMaxDevices] = {};

// The device address of `scratch` on the device `stream` belongs to (the
// current device for the null stream), looked up on the first call there
// with that device current.
hipError_t scratch_address(hipStream_t stream, void **out) {
    int cur = 0, dev = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    dev = cur;
    if (stream && (e = hipStreamGetDevice(stream, &dev)) != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_addr[dev]) {
        if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != cur) {
            const hipError_t r = hipSetDevice(cur);
            if (e == hipSuccess) e = r;
        }
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_addr[dev] = p;
    }
    *out = g_scratch_addr[dev];
    return hipSuccess;
}

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

// The kernels address a tile's rows with 32-bit byte offsets (up to 64 rows).
constexpr int64_t kMaxTokenStrideBytes = int64_t(1) << 24;

bool aligned16(const void *p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; }

int64_t floor_div(int64_t a, int64_t b) {  // b > 0
    const int64_t q = a / b;
    return (a % b != 0 && a < 0) ? q - 1 : q;
}

// The bytes of a tensor: `count` rows of `width` bytes, `stride` bytes apart.
struct Rows {
    uintptr_t base;
    int64_t stride, width, count;
};

Range span(const Rows &t) { return range(reinterpret_cast<const void *>(t.base), (t.count - 1) * t.stride + t.width); }

// Whether two tensors share a byte.  Rows with the same stride (head slices
// of one token-major buffer, e.g. q, k and v inside a packed QKV tensor) are
// compared exactly: row t of a meets row s of b iff, with u = t - s and
// delta = b.base - a.base,  delta - a.width < u * stride < delta + b.width.
// Otherwise any intersection of the two spans counts.
bool intersects(const Rows &a, const Rows &b) {
    if (!overlap(span(a), span(b))) return false;
    if (a.stride != b.stride || a.count == 1 || b.count == 1) return true;
    const int64_t S = a.stride;
    const int64_t delta = (int64_t)(b.base - a.base);
    const int64_t u_lo = floor_div(delta - a.width, S) + 1;       // least u: u S > delta - a.width
    const int64_t u_hi = -floor_div(-(delta + b.width), S) - 1;   // greatest u: u S < delta + b.width
    const int64_t lo = u_lo > -(b.count - 1) ? u_lo : -(b.count - 1);
    const int64_t hi = u_hi < a.count - 1 ? u_hi : a.count - 1;
    return lo <= hi;
}

// A token-strided attention tensor: B*N tokens of `heads` heads of head_dim
// elements, `ts` elements from one token to the next.  Fills `rows`.
ul_status check_tensor(const void *p, int64_t ts, int64_t tokens, int64_t heads, int32_t head_dim,
                       int64_t es, Rows *rows) {
    const int64_t width = heads * head_dim;  // elements; both factors validated >= 1
    if (ts < width || ts > kMaxTokenStrideBytes / es) return UL_ERR_SHAPE;
    if ((ts * es) % 16 != 0 || !aligned16(p)) return UL_ERR_ALIGNMENT;
    int64_t last;
    if (!elems(&last, {tokens - 1, ts, es})) return UL_ERR_SHAPE;
    if (last > INT64_MAX - width * es) return UL_ERR_SHAPE;
    *rows = Rows{reinterpret_cast<uintptr_t>(p), ts * es, width * es, tokens};
    return UL_OK;
}

Rows dense(const void *p, int64_t bytes) { return Rows{reinterpret_cast<uintptr_t>(p), bytes, bytes, 1}; }

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

// A head chunk of the exchange: the world side is [C][N][H][d], the chunk side
// [C][P][N][Hc][d] with 0 <= h0 and h0 + Hc <= H/P.
ul_status check_relayout_heads(const void *in, const void *out, int64_t C, int64_t N, int32_t H,
                               int32_t head_dim, int32_t P, int32_t h0, int32_t Hc, int32_t dtype,
                               bool to_head) {
    if (!in || !out) return UL_ERR_NULL;
    if (C < 1 || N < 1 || H < 1 || head_dim < 1) return UL_ERR_SHAPE;
    if (P < 1 || H % P != 0 || N % P != 0) return UL_ERR_DIVISIBILITY;
    if (h0 < 0 || Hc < 1 || (int64_t)h0 + Hc > H / P) return UL_ERR_SHAPE;
    if (dtype != UL_F32 && dtype != UL_BF16) return UL_ERR_UNSUPPORTED;
    int64_t world, chunk;
    if (!elems(&world, {C, N, H, head_dim, elt_size(dtype)}) ||
        !elems(&chunk, {C, P, N, Hc, head_dim, elt_size(dtype)}))
        return UL_ERR_SHAPE;
    const Range w = range(to_head ? in : out, world), c = range(to_head ? out : in, chunk);
    if (overlap(w, c)) return UL_ERR_OVERLAP;
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
        case UL_ERR_SCRATCH: return "UL_ERR_SCRATCH";
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

}  // extern "C"

namespace {

// Packed variable-length sequences (cu == nullptr: fixed-length batches).
struct Seqs {
    const int32_t *cu = nullptr;  // device table of n + 1 token offsets
    int32_t n = 0, max_len = 0;
};

// The table is on the device, so only its size and placement are checked
// here; the kernels clamp its entries (see seq_range).
ul_status check_seqs(const Seqs &sq, int64_t total) {
    if (!sq.cu) return UL_ERR_NULL;
    if (sq.n < 1 || sq.max_len < 1 || sq.max_len > total || total > INT32_MAX) return UL_ERR_SHAPE;
    if (reinterpret_cast<uintptr_t>(sq.cu) % 4 != 0) return UL_ERR_ALIGNMENT;
    return UL_OK;
}

// Tensor extents follow (B, N) and the token strides; with packed sequences
// B = 1 and N = the total token count.
ul_status fwd_impl(const void *q, const void *k, const void *v, void *o, float *lse, int64_t B,
                   int64_t N, int32_t Hq, int32_t Hkv, int32_t head_dim, const int64_t ts[4],
                   float softmax_scale, int32_t causal, int32_t dtype, void *stream,
                   const Seqs *seqs, bool with_ws = false, void *workspace = nullptr,
                   size_t workspace_bytes = 0) {
    if (!q || !k || !v || !o || !lse) return UL_ERR_NULL;
    AttnSizes sz;
    ul_status st = check_attn(B, N, Hq, Hkv, head_dim, softmax_scale, causal, dtype, &sz);
    if (st != UL_OK) return st;
    if (seqs && (st = check_seqs(*seqs, N)) != UL_OK) return st;
    const int64_t es = elt_size(dtype), T = B * N;
    Rows rq, rk, rv, ro;
    if ((st = check_tensor(q, ts[0], T, Hq, head_dim, es, &rq)) != UL_OK ||
        (st = check_tensor(k, ts[1], T, Hkv, head_dim, es, &rk)) != UL_OK ||
        (st = check_tensor(v, ts[2], T, Hkv, head_dim, es, &rv)) != UL_OK ||
        (st = check_tensor(o, ts[3], T, Hq, head_dim, es, &ro)) != UL_OK)
        return st;
    if (!aligned16(lse)) return UL_ERR_ALIGNMENT;
    AttnShape s{B, N, Hq, Hkv, head_dim, softmax_scale, causal};
    // the workspace is needed only where the sizes split the key range
    const size_t need = with_ws ? ul::attn_fwd_workspace_bytes(s, dtype) : 0;
    if (need > 0 && (!workspace || workspace_bytes < need)) return UL_ERR_WORKSPACE;
    if (need > 0 && !aligned16(workspace)) return UL_ERR_ALIGNMENT;
    const Rows rl = dense(lse, sz.lse_bytes);
    const Rows rw = dense(need > 0 ? workspace : nullptr, (int64_t)need);
    const Rows rc = seqs ? dense(seqs->cu, ((int64_t)seqs->n + 1) * 4) : dense(nullptr, 0);
    for (const Rows &out : {ro, rl, rw})
        for (const Rows &in : {rq, rk, rv, rc})
            if (intersects(out, in)) return UL_ERR_OVERLAP;
    if (intersects(ro, rl) || intersects(ro, rw) || intersects(rl, rw)) return UL_ERR_OVERLAP;
    s.q_rs = ts[0];
    s.k_rs = ts[1];
    s.v_rs = ts[2];
    s.o_rs = ts[3];
    if (seqs) {
        s.B = seqs->n;
        s.N = seqs->max_len;
        s.cu = seqs->cu;
        s.total = N;
    }
    hipStream_t hs = static_cast<hipStream_t>(stream);
    if (dtype == UL_F32)
        return from_hip(ul::launch_attn_fwd_f32(static_cast<const float *>(q),
                                                static_cast<const float *>(k),
                                                static_cast<const float *>(v),
                                                static_cast<float *>(o), lse, s, hs));
    return from_hip(ul::launch_attn_fwd_bf16(q, k, v, o, lse, need > 0 ? workspace : nullptr, s, hs));
}

struct BwdStrides {
    int64_t q, k, v, o, dout, dq, dk, dv;
};

BwdStrides dense_strides(int32_t Hq, int32_t Hkv, int32_t head_dim) {
    const int64_t qs = (int64_t)Hq * head_dim, kvs = (int64_t)Hkv * head_dim;
    return BwdStrides{qs, kvs, kvs, qs, qs, qs, kvs, kvs};
}

ul_status bwd_impl(int32_t stages, const void *q, const void *k, const void *v, const void *o,
                   const void *dout, const float *lse, void *dq, void *dk, void *dv,
                   void *workspace, size_t workspace_bytes, int64_t B, int64_t N, int32_t Hq,
                   int32_t Hkv, int32_t head_dim, const BwdStrides &ts, float softmax_scale,
                   int32_t causal, int32_t dtype, void *stream, const Seqs *seqs,
                   bool use_scratch = false) {
    if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return UL_ERR_NULL;
    AttnSizes sz;
    ul_status st = check_attn(B, N, Hq, Hkv, head_dim, softmax_scale, causal, dtype, &sz);
    if (st != UL_OK) return st;
    // the bf16 dK/dV kernel addresses the -D half of its statistics (N floats,
    // or total for packed sequences, past the -lse half) with a 32-bit offset
    if (dtype == UL_BF16 && N >= (int64_t(1) << 30)) return UL_ERR_SHAPE;
    if (seqs && (st = check_seqs(*seqs, N)) != UL_OK) return st;
    if (stages < 1 || (stages & ~UL_BWD_ALL) != 0) return UL_ERR_UNSUPPORTED;
    AttnShape s{B, N, Hq, Hkv, head_dim, softmax_scale, causal};
    const size_t need = ul::attn_bwd_workspace_bytes(s, dtype);  // packed: B = 1, N = total
    if (use_scratch) {
        // the library's own array stands in for the workspace: it must hold the
        // call, and it cannot overlap a caller's tensor
        if (need > (size_t)UL_NOALLOC_SCRATCH_BYTES) return UL_ERR_SCRATCH;
        workspace = nullptr;
    } else if (!workspace || workspace_bytes < need) {
        return UL_ERR_WORKSPACE;
    }
    const int64_t es = elt_size(dtype), T = B * N;
    Rows r[8];
    if ((st = check_tensor(q, ts.q, T, Hq, head_dim, es, &r[0])) != UL_OK ||
        (st = check_tensor(k, ts.k, T, Hkv, head_dim, es, &r[1])) != UL_OK ||
        (st = check_tensor(v, ts.v, T, Hkv, head_dim, es, &r[2])) != UL_OK ||
        (st = check_tensor(o, ts.o, T, Hq, head_dim, es, &r[3])) != UL_OK ||
        (st = check_tensor(dout, ts.dout, T, Hq, head_dim, es, &r[4])) != UL_OK ||
        (st = check_tensor(dq, ts.dq, T, Hq, head_dim, es, &r[5])) != UL_OK ||
        (st = check_tensor(dk, ts.dk, T, Hkv, head_dim, es, &r[6])) != UL_OK ||
        (st = check_tensor(dv, ts.dv, T, Hkv, head_dim, es, &r[7])) != UL_OK)
        return st;
    if (!aligned16(lse) || !aligned16(workspace)) return UL_ERR_ALIGNMENT;
    const Rows ins[] = {r[0], r[1], r[2], r[3], r[4], dense(lse, sz.lse_bytes),
                        seqs ? dense(seqs->cu, ((int64_t)seqs->n + 1) * 4) : dense(nullptr, 0)};
    const Rows outs[] = {r[5], r[6], r[7], dense(workspace, (int64_t)need)};
    const int n_outs = use_scratch ? 3 : 4;
    for (int a = 0; a < n_outs; ++a) {
        for (const Rows &in : ins)
            if (intersects(outs[a], in)) return UL_ERR_OVERLAP;
        for (int c = a + 1; c < n_outs; ++c)
            if (intersects(outs[a], outs[c])) return UL_ERR_OVERLAP;
    }
    if (use_scratch) {  // every check above is done: only now touch the runtime
        const hipError_t e = scratch_address(static_cast<hipStream_t>(stream), &workspace);
        if (e != hipSuccess) return UL_ERR_HIP;
    }
    s.q_rs = ts.q;
    s.k_rs = ts.k;
    s.v_rs = ts.v;
    s.o_rs = ts.o;
    s.do_rs = ts.dout;
    s.dq_rs = ts.dq;
    s.dk_rs = ts.dk;
    s.dv_rs = ts.dv;
    if (seqs) {
        s.B = seqs->n;
        s.N = seqs->max_len;
        s.cu = seqs->cu;
        s.total = N;
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

}  // namespace

extern "C" {

ul_status ul_relayout_s2h_heads(const void *in, void *out, int64_t C, int64_t N, int32_t H,
                                int32_t head_dim, int32_t P, int32_t h0, int32_t Hc, int32_t dtype,
                                void *stream) {
    const ul_status st =
        check_relayout_heads(in, out, C, N, H, head_dim, P, h0, Hc, dtype, true);
    if (st != UL_OK) return st;
    return from_hip(ul::launch_relayout_heads(in, out, C, N, H, head_dim, P, h0, Hc,
                                              elt_size(dtype), true,
                                              static_cast<hipStream_t>(stream)));
}

ul_status ul_relayout_h2s_heads(const void *in, void *out, int64_t C, int64_t N, int32_t H,
                                int32_t head_dim, int32_t P, int32_t h0, int32_t Hc, int32_t dtype,
                                void *stream) {
    const ul_status st =
        check_relayout_heads(in, out, C, N, H, head_dim, P, h0, Hc, dtype, false);
    if (st != UL_OK) return st;
    return from_hip(ul::launch_relayout_heads(in, out, C, N, H, head_dim, P, h0, Hc,
                                              elt_size(dtype), false,
                                              static_cast<hipStream_t>(stream)));
}

ul_status ul_attn_fwd_strided(const void *q, const void *k, const void *v, void *o, float *lse,
                              int64_t B, int64_t N, int32_t Hq, int32_t Hkv, int32_t head_dim,
                              int64_t q_tok_stride, int64_t k_tok_stride, int64_t v_tok_stride,
                              int64_t o_tok_stride, float softmax_scale, int32_t causal,
                              int32_t dtype, void *stream) {
    const int64_t ts[4] = {q_tok_stride, k_tok_stride, v_tok_stride, o_tok_stride};
    return fwd_impl(q, k, v, o, lse, B, N, Hq, Hkv, head_dim, ts, softmax_scale, causal, dtype,
                    stream, nullptr);
}

ul_status ul_attn_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
                      int64_t B, int64_t N, int32_t Hq, int32_t Hkv, int32_t head_dim,
                      float softmax_scale, int32_t causal, int32_t dtype, void *stream) {
    const int64_t qs = (int64_t)Hq * head_dim, kvs = (int64_t)Hkv * head_dim;
    const int64_t ts[4] = {qs, kvs, kvs, qs};
    return fwd_impl(q, k, v, o, lse, B, N, Hq, Hkv, head_dim, ts, softmax_scale, causal, dtype,
                    stream, nullptr);
}

size_t ul_attn_fwd_workspace_bytes(int64_t B, int64_t N, int32_t Hq, int32_t Hkv,
                                   int32_t head_dim, int32_t dtype) {
    AttnSizes sz;
    if (check_attn(B, N, Hq, Hkv, head_dim, 1.0f, 1, dtype, &sz) != UL_OK) return 0;
    const AttnShape s{B, N, Hq, Hkv, head_dim, 1.0f, 1};
    return ul::attn_fwd_workspace_bytes(s, dtype);
}

ul_status ul_attn_fwd_ws(const void *q, const void *k, const void *v, void *o, float *lse,
                         void *workspace, size_t workspace_bytes, int64_t B, int64_t N, int32_t Hq,
                         int32_t Hkv, int32_t head_dim, float softmax_scale, int32_t causal,
                         int32_t dtype, void *stream) {
    const int64_t qs = (int64_t)Hq * head_dim, kvs = (int64_t)Hkv * head_dim;
    const int64_t ts[4] = {qs, kvs, kvs, qs};
    return fwd_impl(q, k, v, o, lse, B, N, Hq, Hkv, head_dim, ts, softmax_scale, causal, dtype,
                    stream, nullptr, true, workspace, workspace_bytes);
}

ul_status ul_attn_fwd_varlen(const void *q, const void *k, const void *v, void *o, float *lse,
                             const int32_t *cu_seqlens, int32_t n_seqs, int64_t total_tokens,
                             int32_t max_seqlen, int32_t Hq, int32_t Hkv, int32_t head_dim,
                             float softmax_scale, int32_t causal, int32_t dtype, void *stream) {
    const int64_t qs = (int64_t)Hq * head_dim, kvs = (int64_t)Hkv * head_dim;
    const int64_t ts[4] = {qs, kvs, kvs, qs};
    Seqs sq;
    sq.cu = cu_seqlens;
    sq.n = n_seqs;
    sq.max_len = max_seqlen;
    return fwd_impl(q, k, v, o, lse, 1, total_tokens, Hq, Hkv, head_dim, ts, softmax_scale, causal,
                    dtype, stream, &sq);
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
    return bwd_impl(stages, q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B, N,
                    Hq, Hkv, head_dim, dense_strides(Hq, Hkv, head_dim), softmax_scale, causal,
                    dtype, stream, nullptr);
}

ul_status ul_attn_bwd(const void *q, const void *k, const void *v, const void *o,
                      const void *dout, const float *lse, void *dq, void *dk, void *dv,
                      void *workspace, size_t workspace_bytes, int64_t B, int64_t N, int32_t Hq,
                      int32_t Hkv, int32_t head_dim, float softmax_scale, int32_t causal,
                      int32_t dtype, void *stream) {
    return bwd_impl(UL_BWD_ALL, q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B,
                    N, Hq, Hkv, head_dim, dense_strides(Hq, Hkv, head_dim), softmax_scale, causal,
                    dtype, stream, nullptr);
}

ul_status ul_attn_bwd_strided(const void *q, const void *k, const void *v, const void *o,
                              const void *dout, const float *lse, void *dq, void *dk, void *dv,
                              void *workspace, size_t workspace_bytes, int64_t B, int64_t N,
                              int32_t Hq, int32_t Hkv, int32_t head_dim, int64_t q_tok_stride,
                              int64_t k_tok_stride, int64_t v_tok_stride, int64_t o_tok_stride,
                              int64_t dout_tok_stride, int64_t dq_tok_stride,
                              int64_t dk_tok_stride, int64_t dv_tok_stride, float softmax_scale,
                              int32_t causal, int32_t dtype, void *stream) {
    const BwdStrides ts{q_tok_stride,    k_tok_stride,  v_tok_stride,  o_tok_stride,
                        dout_tok_stride, dq_tok_stride, dk_tok_stride, dv_tok_stride};
    return bwd_impl(UL_BWD_ALL, q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B,
                    N, Hq, Hkv, head_dim, ts, softmax_scale, causal, dtype, stream, nullptr);
}

ul_status ul_attn_bwd_varlen(const void *q, const void *k, const void *v, const void *o,
                             const void *dout, const float *lse, void *dq, void *dk, void *dv,
                             void *workspace, size_t workspace_bytes, const int32_t *cu_seqlens,
                             int32_t n_seqs, int64_t total_tokens, int32_t max_seqlen, int32_t Hq,
                             int32_t Hkv, int32_t head_dim, float softmax_scale, int32_t causal,
                             int32_t dtype, void *stream) {
    Seqs sq;
    sq.cu = cu_seqlens;
    sq.n = n_seqs;
    sq.max_len = max_seqlen;
    return bwd_impl(UL_BWD_ALL, q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, 1,
                    total_tokens, Hq, Hkv, head_dim, dense_strides(Hq, Hkv, head_dim),
                    softmax_scale, causal, dtype, stream, &sq);
}

ul_status ul_attn_bwd_noalloc(const void *q, const void *k, const void *v, const void *o,
                              const void *dout, const float *lse, void *dq, void *dk, void *dv,
                              int64_t B, int64_t N, int32_t Hq, int32_t Hkv, int32_t head_dim,
                              float softmax_scale, int32_t causal, int32_t dtype, void *stream) {
    return bwd_impl(UL_BWD_ALL, q, k, v, o, dout, lse, dq, dk, dv, nullptr, 0, B, N, Hq, Hkv,
                    head_dim, dense_strides(Hq, Hkv, head_dim), softmax_scale, causal, dtype,
                    stream, nullptr, true);
}

}  // extern "C"
