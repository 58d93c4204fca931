/*
 * ul_attn.h -- C ABI of libulattn.so: the per-rank hot path of Ulysses
 * sequence parallelism on one MI355X (gfx950).
 *
 * The method ("Ulysses Sequence Parallelism: Training with Million-Token
 * Contexts", section "How Does Ulysses Sequence Parallelism Actually Work?"):
 * every GPU holds a chunk of N/P tokens; an all-to-all leaves each GPU with
 * all N positions but only a slice of H/P heads; each GPU runs exact
 * attention locally on its heads; a second all-to-all reverses the shuffle.
 * This library provides the local pieces of that step:
 *
 *   ul_relayout_s2h   the sequence-sharded -> head-sharded permutation that the
 *                     first all-to-all performs, done inside one GPU's memory;
 *   ul_relayout_h2s   its inverse (the reversed shuffle);
 *   ul_attn_fwd       causal (or full) softmax attention over the full N for a
 *                     slice of query heads with grouped KV heads, also
 *                     returning the per-row logsumexp;
 *   ul_attn_fwd_ws    the same with a workspace, which lets shorter causal
 *                     sequences split the key range of their longest rows;
 *   ul_attn_bwd       its gradient (dQ, dK, dV);
 *   ul_attn_*_strided the same on token-strided views, so that a rank's head
 *                     slice is read from and written to sequence-sharded
 *                     buffers in place (no relayout pass around attention);
 *   ul_attn_*_varlen  the same over packed variable-length sequences;
 *   ul_relayout_*_heads  the exchange for a chunk of each rank's heads.
 *
 * Conventions shared by every entry point:
 *  - Tensor pointers are DEVICE pointers owned by the caller.  No call
 *    allocates device memory, synchronises the device, or keeps state between
 *    calls; every call validates its arguments on the host, enqueues its
 *    kernels on `stream` (a hipStream_t passed as void*, NULL = the null
 *    stream) and returns.  Results are ready when the stream reaches that
 *    point.  Calls are thread-safe.
 *  - All tensors are row-major (C order) and dense, except the token-strided
 *    views that the *_strided calls take.
 *  - Outputs are fully overwritten, never accumulated into.
 *  - Errors are reported only through the returned status.  Validation runs
 *    before any HIP call, so an invalid call enqueues nothing.
 *    UL_ERR_HIP means a launch failed (hipGetLastError after the launch);
 *    the output contents are then unspecified.
 */
#ifndef UL_ATTN_H
#define UL_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    UL_OK = 0,
    UL_ERR_NULL = 1,         /* a required pointer is NULL */
    UL_ERR_SHAPE = 2,        /* a size < 1, a non-finite or non-positive scale, or int64 overflow */
    UL_ERR_DIVISIBILITY = 3, /* Hq % Hkv, H % P or N % P is non-zero, or P < 1 */
    UL_ERR_UNSUPPORTED = 4,  /* head_dim or dtype outside what the kernels implement */
    UL_ERR_ALIGNMENT = 5,    /* an attention tensor is not 16-byte aligned */
    UL_ERR_WORKSPACE = 6,    /* workspace NULL or smaller than ul_attn_*_workspace_bytes */
    UL_ERR_OVERLAP = 7,      /* an output's byte range overlaps an input or another output */
    UL_ERR_HIP = 8,          /* the HIP runtime reported an error at launch */
    UL_ERR_SCRATCH = 9       /* the problem needs more than the fixed scratch of
                                ul_attn_bwd_noalloc (UL_NOALLOC_SCRATCH_BYTES) */
} ul_status;

typedef enum {
    UL_F32 = 0,  /* IEEE binary32 inputs and outputs; fp32 arithmetic throughout */
    UL_BF16 = 1  /* bfloat16 inputs and outputs; bf16 MFMA with fp32 accumulation */
} ul_dtype;

/*
 * Forward attention for one rank's heads (section "How Does Ulysses Sequence
 * Parallelism Actually Work?": attention over all N positions of a slice of
 * heads, computed locally; "Ulysses: entrenar con contextos de hasta 96K
 * tokens en 4 GPUs", section "Conclusion rapida": the attention mathematics
 * itself is unchanged).
 *
 * For every batch b, query head h (KV head g = h / (Hq/Hkv), contiguous
 * groups) and query row i:
 *   s_ij   = softmax_scale * sum_e q[b,i,h,e] k[b,j,g,e]   for j <= i if causal
 *                                                           (every j otherwise)
 *   o[b,i,h,:] = sum_j softmax_j(s_ij) v[b,j,g,:]
 *   lse[b,h,i] = ln sum_j exp(s_ij)                         (natural log)
 *
 *   q, o        [B][N][Hq][head_dim]   dtype
 *   k, v        [B][N][Hkv][head_dim]  dtype
 *   lse         [B][Hq][N]             fp32 (for either dtype)
 *   head_dim    64 or 128
 *   causal      1 = key j visible to query i iff j <= i; 0 = all keys visible
 *   dtype       ul_dtype
 * bf16 outputs are rounded to nearest-even from fp32 accumulators.
 * Deterministic: identical inputs give bit-identical outputs.
 * Errors: NULL, SHAPE, DIVISIBILITY (Hq % Hkv), UNSUPPORTED, ALIGNMENT,
 * OVERLAP (o or lse overlapping q, k, v or each other), HIP.
 */
ul_status ul_attn_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
                      int64_t B, int64_t N, int32_t Hq, int32_t Hkv, int32_t head_dim,
                      float softmax_scale, int32_t causal, int32_t dtype, void *stream);

/*
 * Device workspace bytes that ul_attn_fwd_ws needs for these sizes (causal
 * assumed; a multiple of 16).  0 where the sizes run the key range unsplit:
 * the fp32 dtype, and bf16 calls with too many work items for the split to
 * pay (B x Hkv x query blocks above 256, the CU count of the part) or too few
 * query blocks (N of a few hundred).  At most 34 MB.  0 for invalid sizes.
 */
size_t ul_attn_fwd_workspace_bytes(int64_t B, int64_t N, int32_t Hq, int32_t Hkv,
                                   int32_t head_dim, int32_t dtype);

/*
 * ul_attn_fwd with a workspace.  Same result definition, layouts and
 * determinism; on bf16 causal calls where ul_attn_fwd_workspace_bytes is
 * non-zero, the upper half of the query blocks is computed as two halves of
 * its key range whose partial softmax sums (running max m, sum l and the
 * unnormalised output, fp32) are combined afterwards by the same rescaling
 * that the online softmax applies between key tiles ("Why Train Million-Token
 * Contexts Anyway?": attention over long N is computed in tiles of keys, the
 * softmax kept in running form).  The result differs from ul_attn_fwd only in
 * rounding: the order of the fp32 sums changes for those rows.  Whether a
 * call splits depends on its sizes (B, N, Hq, Hkv), so the same head may
 * round differently in calls of different sizes; a given call is
 * deterministic.
 *   workspace        device buffer of at least ul_attn_fwd_workspace_bytes(
 *                    B, N, Hq, Hkv, head_dim, dtype) bytes, 16-byte aligned;
 *                    may be NULL when that is 0.  Its contents on entry are
 *                    ignored and on return unspecified.
 * Errors: as ul_attn_fwd, plus WORKSPACE, and OVERLAP when the workspace
 * overlaps an input or an output.
 */
ul_status ul_attn_fwd_ws(const void *q, const void *k, const void *v, void *o, float *lse,
                         void *workspace, size_t workspace_bytes, int64_t B, int64_t N, int32_t Hq,
                         int32_t Hkv, int32_t head_dim, float softmax_scale, int32_t causal,
                         int32_t dtype, void *stream);

/*
 * ul_attn_fwd on token-strided tensors: the head slice of one rank read from,
 * and written to, token-major buffers that hold more heads than the rank's,
 * so that no separate relayout pass runs on either side of the attention.
 * (The first all-to-all of "How Does Ulysses Sequence Parallelism Actually
 * Work?" hands each GPU all positions of a slice of heads, and the second
 * reverses it; in the world view of one memory that slice is a strided view.)
 *
 * Element (b, t, h, e) of q and o is at
 *     q[(b*N + t) * q_tok_stride + h*head_dim + e]    (o likewise with o_tok_stride)
 * and element (b, t, g, e) of k and v at
 *     k[(b*N + t) * k_tok_stride + g*head_dim + e]    (v likewise with v_tok_stride).
 * The pointers are the addresses of element (0, 0, 0, 0), i.e. already offset
 * to the first head of the slice.  Example: rank r of P reading its Hq query
 * heads out of a sequence-sharded world tensor x[N][P*Hq][head_dim] passes
 * q = x + r*Hq*head_dim and q_tok_stride = P*Hq*head_dim.
 *
 * Strides are in elements, at least (heads of that tensor) * head_dim, a
 * multiple of 16 bytes, and at most 16 MiB; otherwise SHAPE (too small or too
 * large) or ALIGNMENT (not a 16-byte multiple).  lse stays dense [B][Hq][N].
 * OVERLAP: an output shares a byte with an input or another output (tensors
 * with equal strides are compared row by row, so disjoint head slices of one
 * buffer are accepted).  Everything else is as ul_attn_fwd, which is this
 * call with q/o strides Hq*head_dim and k/v strides Hkv*head_dim.
 */
ul_status ul_attn_fwd_strided(const void *q, const void *k, const void *v, void *o, float *lse,
                              int64_t B, int64_t N, int32_t Hq, int32_t Hkv, int32_t head_dim,
                              int64_t q_tok_stride, int64_t k_tok_stride, int64_t v_tok_stride,
                              int64_t o_tok_stride, float softmax_scale, int32_t causal,
                              int32_t dtype, void *stream);

/*
 * ul_attn_fwd over packed variable-length sequences: n_seqs independent
 * sequences (documents) concatenated along the token axis, each attending
 * only within itself (causally if `causal`), with no padding between them.
 * ("Ulysses Sequence Parallelism: Training with Million-Token Contexts":
 * section "Ulysses vs. Ring Attention: Who's Faster?" makes variable lengths a
 * mode that has to be switched on; section "Can You Integrate Ulysses with
 * Hugging Face Today?" asks for bucketed variable-length batches and no
 * padding.)
 *
 *   q, o          [total_tokens][Hq][head_dim]    dtype, dense
 *   k, v          [total_tokens][Hkv][head_dim]   dtype, dense
 *   lse           [Hq][total_tokens]              fp32
 *   cu_seqlens    DEVICE int32 table of n_seqs + 1 token offsets, read by the
 *                 kernels: sequence s is tokens [cu_seqlens[s], cu_seqlens[s+1]).
 *                 It must start at 0, be non-decreasing and end at
 *                 total_tokens, with no sequence longer than max_seqlen.  The
 *                 host cannot read it without synchronising, so it is not
 *                 checked: the kernels clamp every entry into [0, total_tokens]
 *                 and every length to max_seqlen, so a malformed table gives
 *                 unspecified values but never an access outside the tensors.
 *                 Tokens that no sequence covers are left unwritten.  Empty
 *                 sequences are allowed.
 *   max_seqlen    the longest sequence (sizes the launch), 1..total_tokens
 * For each sequence the result is exactly ul_attn_fwd with B = 1 on that
 * sequence's tokens.  Errors: as ul_attn_fwd (tensor sizes taken with B = 1,
 * N = total_tokens), plus NULL for cu_seqlens, SHAPE for n_seqs < 1,
 * max_seqlen outside 1..total_tokens or total_tokens >= 2^31, ALIGNMENT for a
 * cu_seqlens not 4-byte aligned, and OVERLAP when o or lse overlap the table.
 */
ul_status ul_attn_fwd_varlen(const void *q, const void *k, const void *v, void *o, float *lse,
                             const int32_t *cu_seqlens, int32_t n_seqs, int64_t total_tokens,
                             int32_t max_seqlen, int32_t Hq, int32_t Hkv, int32_t head_dim,
                             float softmax_scale, int32_t causal, int32_t dtype, void *stream);

/*
 * Device workspace bytes that ul_attn_bwd needs for these sizes (a multiple
 * of 256).  Returns 0 for invalid sizes.
 */
size_t ul_attn_bwd_workspace_bytes(int64_t B, int64_t N, int32_t Hq, int32_t Hkv,
                                   int32_t head_dim, int32_t dtype);

/*
 * Backward of ul_attn_fwd: the gradient of L = <dout, o> with respect to q,
 * k and v (training the method implies it; the pages give no formula, so it
 * is the plain derivative of the forward above).  With
 *   p_ij  = exp(s_ij - lse_i),  dp_ij = dout_i . v_j,  D_i = dout_i . o_i,
 *   ds_ij = p_ij (dp_ij - D_i):
 *   dq_i = softmax_scale * sum_j ds_ij k_j
 *   dk_j = softmax_scale * sum over the group's query heads and rows i of ds_ij q_i
 *   dv_j = sum over the group's query heads and rows i of p_ij dout_i
 *
 *   o, lse      outputs of ul_attn_fwd for the same q, k, v
 *   dout, dq    [B][N][Hq][head_dim]   dtype
 *   dk, dv      [B][N][Hkv][head_dim]  dtype
 *   workspace   device buffer of at least ul_attn_bwd_workspace_bytes(...)
 *               bytes, caller-owned, 16-byte aligned; its contents on entry
 *               do not matter and are scratch afterwards.
 * Deterministic: no atomics; identical inputs give bit-identical outputs.
 * Errors: as ul_attn_fwd, plus WORKSPACE, OVERLAP when dq, dk, dv or the
 * workspace overlap each other or any input, and SHAPE for BF16 with
 * N >= 2^30 (total_tokens for packed sequences: the statistics are addressed
 * with 32-bit offsets; no such problem fits one GPU's memory).
 */
ul_status ul_attn_bwd(const void *q, const void *k, const void *v, const void *o,
                      const void *dout, const float *lse, void *dq, void *dk, void *dv,
                      void *workspace, size_t workspace_bytes, int64_t B, int64_t N, int32_t Hq,
                      int32_t Hkv, int32_t head_dim, float softmax_scale, int32_t causal,
                      int32_t dtype, void *stream);

/*
 * The three stages of ul_attn_bwd, for callers that schedule them themselves.
 *
 *   UL_BWD_PREP   -D_i = -(dout_i . o_i) and lse in base-2 units, written to
 *                 the workspace (reads o, dout, lse);
 *   UL_BWD_DQ     dq from q, k, v, dout and the workspace;
 *   UL_BWD_DKDV   dk and dv from q, k, v, dout and the workspace.
 *
 * `stages` is a non-empty OR of these bits; the selected stages run in the
 * order above on `stream`.  DQ and DKDV read the workspace that PREP wrote for
 * the same inputs and sizes, and do not depend on each other: after PREP a
 * caller may run them on two streams (ordering them after PREP with events)
 * so that each fills the other's idle compute units.  Arguments, validation
 * and errors are those of ul_attn_bwd (every pointer is checked, whichever
 * stages run), plus UNSUPPORTED for an empty mask or unknown bits.
 * ul_attn_bwd(...) is ul_attn_bwd_stages(UL_BWD_ALL, ...).
 */
enum { UL_BWD_PREP = 1, UL_BWD_DQ = 2, UL_BWD_DKDV = 4, UL_BWD_ALL = 7 };

ul_status ul_attn_bwd_stages(int32_t stages, const void *q, const void *k, const void *v,
                             const void *o, const void *dout, const float *lse, void *dq, void *dk,
                             void *dv, void *workspace, size_t workspace_bytes, int64_t B,
                             int64_t N, int32_t Hq, int32_t Hkv, int32_t head_dim,
                             float softmax_scale, int32_t causal, int32_t dtype, void *stream);

/*
 * ul_attn_bwd (all three stages) on token-strided tensors, with the layout
 * rules of ul_attn_fwd_strided: q, o, dout and dq hold Hq heads per token,
 * k, v, dk and dv Hkv heads, each tensor with its own token stride in
 * elements.  dq, dk and dv may be disjoint head slices of one buffer (for
 * example a packed [N][Hq + 2*Hkv][head_dim] gradient of a fused QKV
 * projection).  lse and the workspace stay dense.  Errors as ul_attn_bwd plus
 * the stride errors of ul_attn_fwd_strided.
 */
ul_status ul_attn_bwd_strided(const void *q, const void *k, const void *v, const void *o,
                              const void *dout, const float *lse, void *dq, void *dk, void *dv,
                              void *workspace, size_t workspace_bytes, int64_t B, int64_t N,
                              int32_t Hq, int32_t Hkv, int32_t head_dim, int64_t q_tok_stride,
                              int64_t k_tok_stride, int64_t v_tok_stride, int64_t o_tok_stride,
                              int64_t dout_tok_stride, int64_t dq_tok_stride,
                              int64_t dk_tok_stride, int64_t dv_tok_stride, float softmax_scale,
                              int32_t causal, int32_t dtype, void *stream);

/*
 * Backward of ul_attn_fwd_varlen (all three stages), with its layouts and
 * table rules: dout and dq [total_tokens][Hq][head_dim], dk and dv
 * [total_tokens][Hkv][head_dim], o and lse from ul_attn_fwd_varlen for the
 * same inputs.  The workspace must hold
 * ul_attn_bwd_workspace_bytes(1, total_tokens, Hq, Hkv, head_dim, dtype)
 * bytes.  Errors as ul_attn_bwd plus those of ul_attn_fwd_varlen.
 */
ul_status ul_attn_bwd_varlen(const void *q, const void *k, const void *v, const void *o,
                             const void *dout, const float *lse, void *dq, void *dk, void *dv,
                             void *workspace, size_t workspace_bytes, const int32_t *cu_seqlens,
                             int32_t n_seqs, int64_t total_tokens, int32_t max_seqlen, int32_t Hq,
                             int32_t Hkv, int32_t head_dim, float softmax_scale, int32_t causal,
                             int32_t dtype, void *stream);

/*
 * ul_attn_bwd without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the caller passes inputs and outputs only, and the
 * call allocates nothing.  The statistics that ul_attn_bwd keeps in its
 * workspace go to a fixed array inside the library instead: a file-scope
 * device array of UL_NOALLOC_SCRATCH_BYTES (256 MiB), one copy per GPU, held
 * from the library's first use on that GPU until the process ends.  Its
 * device address is looked up once per GPU (hipGetSymbolAddress, with that
 * GPU current) on the first call there.
 *
 * Arguments, layouts, results and errors are those of ul_attn_bwd (results
 * are bit-identical to it), except:
 *   - SCRATCH when ul_attn_bwd_workspace_bytes(B, N, Hq, Hkv, head_dim, dtype)
 *     exceeds UL_NOALLOC_SCRATCH_BYTES (8 bytes per query row and head, plus
 *     the head-split partials of shorter sequences: B*Hq*N beyond about 32M
 *     rows, or less for the shorter sequences that use the partials);
 *   - HIP also when the array's address cannot be obtained.
 * Every call on one GPU uses that GPU's one array, which keeps the last
 * call's contents; each call writes all it reads before reading it.  Calls
 * that may overlap in time on one GPU (two streams, two threads) race on the
 * array: the caller must order them.
 */
#define UL_NOALLOC_SCRATCH_BYTES (256u << 20)

ul_status ul_attn_bwd_noalloc(const void *q, const void *k, const void *v, const void *o,
                              const void *dout, const float *lse, void *dq, void *dk, void *dv,
                              int64_t B, int64_t N, int32_t Hq, int32_t Hkv, int32_t head_dim,
                              float softmax_scale, int32_t causal, int32_t dtype, void *stream);

/*
 * Sequence-sharded -> head-sharded relayout (the first all-to-all of the
 * step, section "How Does Ulysses Sequence Parallelism Actually Work?": each
 * GPU takes a chunk of N/P tokens, then ends up with all positions but a
 * slice of heads), as one permutation in one GPU's memory:
 *
 *   in  [C][N][H][head_dim]       = [C][P][N/P][H][head_dim]: rank r's tokens
 *                                   are the contiguous chunk [r*N/P, (r+1)*N/P)
 *   out [C][P][N][H/P][head_dim]  rank r's contiguous head slice
 *                                   [r*H/P, (r+1)*H/P) over all N tokens
 *   out[c][r][t][hh][e] = in[c][t][r*(H/P) + hh][e]
 *
 * C is an outer batch (3 for a stacked Q/K/V tensor).  The copy moves bits:
 * the result is byte-exact for any bit patterns.  H % P == 0 (which implies
 * the method's rule that the head count be at least the parallel degree) and
 * N % P == 0 (clean chunks, no padding) are required.  Any head_dim >= 1.
 * Errors: NULL, SHAPE, DIVISIBILITY, UNSUPPORTED (dtype), OVERLAP (in and out
 * byte ranges intersect: the permutation is not in place), HIP.
 */
ul_status ul_relayout_s2h(const void *in, void *out, int64_t C, int64_t N, int32_t H,
                          int32_t head_dim, int32_t P, int32_t dtype, void *stream);

/*
 * Head-sharded -> sequence-sharded relayout (the reversed shuffle, and the
 * adjoint of ul_relayout_s2h used on gradients):
 *   in  [C][P][N][H/P][head_dim],  out [C][N][H][head_dim]
 *   out[c][t][h][e] = in[c][h / (H/P)][t][h % (H/P)][e]
 * Same requirements and errors as ul_relayout_s2h.
 */
ul_status ul_relayout_h2s(const void *in, void *out, int64_t C, int64_t N, int32_t H,
                          int32_t head_dim, int32_t P, int32_t dtype, void *stream);

/*
 * The exchange for a chunk of heads: heads h0 .. h0+Hc-1 of every rank's
 * slice.  A rank that works through its heads a few at a time (to cap the
 * activation and exchange-buffer memory of very long sequences: "Ulysses
 * Unleashed: Context Parallelism with Fragmentation by Heads" describes
 * splitting the attention work into fine-grained head fragments for that
 * purpose) exchanges one chunk per call, so its head-sharded buffers hold Hc
 * heads instead of H/P.
 *
 *   ul_relayout_s2h_heads:  in  [C][N][H][head_dim] (sequence-sharded world)
 *                           out [C][P][N][Hc][head_dim]
 *                           out[c][r][t][hh][e] = in[c][t][r*(H/P) + h0 + hh][e]
 *   ul_relayout_h2s_heads:  in  [C][P][N][Hc][head_dim]
 *                           out [C][N][H][head_dim]: writes exactly the chunk's
 *                           heads r*(H/P) + h0 + hh of every token and leaves
 *                           every other head of out untouched.
 *
 * Over a set of chunks that partition [0, H/P) these compose to
 * ul_relayout_s2h / ul_relayout_h2s.  Bits are moved, never changed.
 * Requirements and errors as ul_relayout_s2h, plus SHAPE when h0 < 0,
 * Hc < 1 or h0 + Hc > H/P.  OVERLAP compares the [C][N][H][d] side with
 * the [C][P][N][Hc][d] side.
 */
ul_status ul_relayout_s2h_heads(const void *in, void *out, int64_t C, int64_t N, int32_t H,
                                int32_t head_dim, int32_t P, int32_t h0, int32_t Hc,
                                int32_t dtype, void *stream);
ul_status ul_relayout_h2s_heads(const void *in, void *out, int64_t C, int64_t N, int32_t H,
                                int32_t head_dim, int32_t P, int32_t h0, int32_t Hc,
                                int32_t dtype, void *stream);

/* Static, NUL-terminated name of a status code ("UL_OK", ...). */
const char *ul_status_str(ul_status s);

#ifdef __cplusplus
}
#endif

#endif /* UL_ATTN_H */
