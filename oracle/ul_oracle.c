/*
 * ul_oracle.c -- plain, slow, fp64 CPU reference for the per-rank Ulysses
 * attention path and the sequence<->head relayout.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file's library: only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg use it.  It shares no code, header, table or
 * helper with the HIP library; it has its own index arithmetic throughout.
 *
 * What it follows (page titles and sections of the source pages):
 *  - "Ulysses Sequence Parallelism: Training with Million-Token Contexts",
 *    section "How Does Ulysses Sequence Parallelism Actually Work?": each GPU
 *    holds a chunk of N/P tokens, an all-to-all leaves it with every
 *    position but only a slice of the heads, attention is computed locally,
 *    and the shuffle is reversed.  Heads are independent.
 *  - "Ulysses: entrenar con contextos de hasta 96K tokens en 4 GPUs",
 *    section "Conclusion rapida": the method leaves the mathematics of
 *    attention unchanged, so the oracle is the textbook definition of
 *    causal softmax attention written out in fp64.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *  - causal mask: key j is visible to query i iff j <= i (same length N);
 *  - GQA: query head h reads KV head g = h / (Hq/Hkv) (contiguous groups);
 *  - lse is the natural log of the row sum of exp(scaled scores);
 *  - backward is the gradient of L = <dO, O> with respect to Q, K, V.
 *
 * Inputs are read in their stored precision (fp32, bf16 bit patterns, or
 * fp64) and widened exactly to double; every sum is an fp64 sum in index
 * order.  Outputs are fp64.
 *
 * Layouts (row-major): q, o, dout, dq [B][N][Hq][d]; k, v, dk, dv
 * [B][N][Hkv][d]; lse [B][Hq][N].  Row-subset outputs use [B][R][Hq][d]
 * and [B][Hq][R] for R selected rows.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_F32 0
#define OR_BF16 1
#define OR_F64 2

/* Widen one stored element to double.  bf16 is the top half of an IEEE
 * binary32, so shifting its 16 bits up by 16 gives the exact float. */
static double elem(const void *p, int64_t i, int dt)
{
    if (dt == OR_F32)
        return (double)((const float *)p)[i];
    if (dt == OR_BF16) {
        uint32_t u = ((uint32_t)((const uint16_t *)p)[i]) << 16;
        float f;
        memcpy(&f, &u, sizeof f);
        return (double)f;
    }
    return ((const double *)p)[i];
}

/* index of element (b, t, h, e) in a [B][N][H][d] tensor */
static int64_t bnhd(int64_t b, int64_t t, int64_t h, int64_t e, int64_t N, int64_t H, int64_t d)
{
    return ((b * N + t) * H + h) * d + e;
}

/* Scaled dot product s = scale * sum_e q[b,i,h,e] * k[b,j,g,e]. */
static double score(const void *q, const void *k, int dt, int64_t b, int64_t i, int64_t h,
                    int64_t j, int64_t g, int64_t N, int64_t Hq, int64_t Hkv, int64_t d,
                    double scale)
{
    double acc = 0.0;
    for (int64_t e = 0; e < d; ++e)
        acc += elem(q, bnhd(b, i, h, e, N, Hq, d), dt) * elem(k, bnhd(b, j, g, e, N, Hkv, d), dt);
    return scale * acc;
}

/* Last visible key for query row i. */
static int64_t last_key(int64_t i, int64_t N, int causal)
{
    return causal ? i : N - 1;
}

/*
 * One query row of the forward pass (definition of softmax attention):
 *   s_j  = scale * q_i . k_j           for visible j
 *   m    = max_j s_j
 *   l    = sum_j exp(s_j - m)
 *   o_i  = sum_j exp(s_j - m) v_j / l
 *   lse  = m + ln l
 * `s` is caller scratch of N doubles.
 */
static void fwd_row(const void *q, const void *k, const void *v, int dt, int64_t b, int64_t i,
                    int64_t h, int64_t N, int64_t Hq, int64_t Hkv, int64_t d, double scale,
                    int causal, double *s, double *o_row, double *lse_out)
{
    const int64_t g = h / (Hq / Hkv);
    const int64_t jmax = last_key(i, N, causal);
    double m = -INFINITY;
    for (int64_t j = 0; j <= jmax; ++j) {
        s[j] = score(q, k, dt, b, i, h, j, g, N, Hq, Hkv, d, scale);
        if (s[j] > m)
            m = s[j];
    }
    double l = 0.0;
    for (int64_t j = 0; j <= jmax; ++j)
        l += exp(s[j] - m);
    for (int64_t e = 0; e < d; ++e)
        o_row[e] = 0.0;
    for (int64_t j = 0; j <= jmax; ++j) {
        const double w = exp(s[j] - m);
        for (int64_t e = 0; e < d; ++e)
            o_row[e] += w * elem(v, bnhd(b, j, g, e, N, Hkv, d), dt);
    }
    for (int64_t e = 0; e < d; ++e)
        o_row[e] /= l;
    *lse_out = m + log(l);
}

/*
 * Forward for a set of query rows.  rows == NULL means all N rows in order.
 * o: [B][R][Hq][d] fp64, lse: [B][Hq][R] fp64.
 */
int oracle_attn_fwd_rows(const void *q, const void *k, const void *v, int dt, int64_t B,
                         int64_t N, int64_t Hq, int64_t Hkv, int64_t d, double scale, int causal,
                         const int64_t *rows, int64_t R, double *o, double *lse)
{
    if (B < 1 || N < 1 || Hq < 1 || Hkv < 1 || d < 1 || Hq % Hkv != 0 || R < 0)
        return 1;
    const int64_t nr = rows ? R : N;
    int bad = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc((size_t)N * sizeof(double));
        if (!s) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for collapse(3) schedule(dynamic, 4)
        for (int64_t b = 0; b < B; ++b)
            for (int64_t h = 0; h < Hq; ++h)
                for (int64_t r = 0; r < nr; ++r) {
                    if (!s)
                        continue;
                    const int64_t i = rows ? rows[r] : r;
                    fwd_row(q, k, v, dt, b, i, h, N, Hq, Hkv, d, scale, causal, s,
                            o + ((b * nr + r) * Hq + h) * d, lse + (b * Hq + h) * nr + r);
                }
        free(s);
    }
    return bad ? 2 : 0;
}

/*
 * dQ for a set of query rows (any N).  Row i's gradient needs only row i's
 * data: its probabilities p_ij = exp(s_ij - lse_i), dp_ij = dO_i . v_j,
 * D_i = dO_i . O_i, ds_ij = p_ij (dp_ij - D_i), dq_i = scale sum_j ds_ij k_j.
 * O_i and lse_i are recomputed here by the forward definition.
 * dq: [B][R][Hq][d] fp64.
 */
int oracle_dq_rows(const void *q, const void *k, const void *v, const void *dout, int dt,
                   int64_t B, int64_t N, int64_t Hq, int64_t Hkv, int64_t d, double scale,
                   int causal, const int64_t *rows, int64_t R, double *dq)
{
    if (B < 1 || N < 1 || Hq < 1 || Hkv < 1 || d < 1 || Hq % Hkv != 0 || R < 0)
        return 1;
    const int64_t nr = rows ? R : N;
    int bad = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc((size_t)N * sizeof(double));
        double *orow = (double *)malloc((size_t)d * sizeof(double));
        if (!s || !orow) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for collapse(3) schedule(dynamic, 4)
        for (int64_t b = 0; b < B; ++b)
            for (int64_t h = 0; h < Hq; ++h)
                for (int64_t r = 0; r < nr; ++r) {
                    if (!s || !orow)
                        continue;
                    const int64_t i = rows ? rows[r] : r;
                    const int64_t g = h / (Hq / Hkv);
                    double lse_i;
                    fwd_row(q, k, v, dt, b, i, h, N, Hq, Hkv, d, scale, causal, s, orow, &lse_i);
                    double Di = 0.0;
                    for (int64_t e = 0; e < d; ++e)
                        Di += elem(dout, bnhd(b, i, h, e, N, Hq, d), dt) * orow[e];
                    double *dqr = dq + ((b * nr + r) * Hq + h) * d;
                    for (int64_t e = 0; e < d; ++e)
                        dqr[e] = 0.0;
                    const int64_t jmax = last_key(i, N, causal);
                    for (int64_t j = 0; j <= jmax; ++j) {
                        const double p = exp(s[j] - lse_i);
                        double dp = 0.0;
                        for (int64_t e = 0; e < d; ++e)
                            dp += elem(dout, bnhd(b, i, h, e, N, Hq, d), dt) *
                                  elem(v, bnhd(b, j, g, e, N, Hkv, d), dt);
                        const double ds = p * (dp - Di);
                        for (int64_t e = 0; e < d; ++e)
                            dqr[e] += ds * elem(k, bnhd(b, j, g, e, N, Hkv, d), dt);
                    }
                    for (int64_t e = 0; e < d; ++e)
                        dqr[e] *= scale;
                }
        free(s);
        free(orow);
    }
    return bad ? 2 : 0;
}

/*
 * dK and dV for a set of key rows j of KV head g:
 *   dK_j = scale * sum_{h in group g} sum_{i : j visible to i} ds_ij q_i
 *   dV_j =         sum_{h in group g} sum_{i : j visible to i} p_ij  dO_i
 * with p_ij, ds_ij as in oracle_dq_rows; lse_i and D_i come from full
 * forward rows, recomputed for every query row that sees j (cheap for the
 * last keys of a causal sequence, quadratic otherwise).
 * kv_rows == NULL means all N key rows.  dk, dv: [B][R][Hkv][d] fp64.
 * lse_all/D_all: optional precomputed [B][Hq][N] row statistics (NULL ->
 * recompute per query row).
 */
int oracle_dkdv_rows(const void *q, const void *k, const void *v, const void *dout, int dt,
                     int64_t B, int64_t N, int64_t Hq, int64_t Hkv, int64_t d, double scale,
                     int causal, const int64_t *kv_rows, int64_t R, const double *lse_all,
                     const double *D_all, double *dk, double *dv)
{
    if (B < 1 || N < 1 || Hq < 1 || Hkv < 1 || d < 1 || Hq % Hkv != 0 || R < 0)
        return 1;
    if ((lse_all == NULL) != (D_all == NULL))
        return 1;
    const int64_t nr = kv_rows ? R : N;
    const int64_t grp = Hq / Hkv;
    int bad = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc((size_t)N * sizeof(double));
        double *orow = (double *)malloc((size_t)d * sizeof(double));
        if (!s || !orow) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for collapse(3) schedule(dynamic, 4)
        for (int64_t b = 0; b < B; ++b)
            for (int64_t g = 0; g < Hkv; ++g)
                for (int64_t r = 0; r < nr; ++r) {
                    if (!s || !orow)
                        continue;
                    const int64_t j = kv_rows ? kv_rows[r] : r;
                    double *dkr = dk + ((b * nr + r) * Hkv + g) * d;
                    double *dvr = dv + ((b * nr + r) * Hkv + g) * d;
                    for (int64_t e = 0; e < d; ++e) {
                        dkr[e] = 0.0;
                        dvr[e] = 0.0;
                    }
                    for (int64_t h = g * grp; h < (g + 1) * grp; ++h) {
                        const int64_t i0 = causal ? j : 0;
                        for (int64_t i = i0; i < N; ++i) {
                            double lse_i, Di = 0.0;
                            if (lse_all) {
                                lse_i = lse_all[(b * Hq + h) * N + i];
                                Di = D_all[(b * Hq + h) * N + i];
                            } else {
                                fwd_row(q, k, v, dt, b, i, h, N, Hq, Hkv, d, scale, causal, s,
                                        orow, &lse_i);
                                for (int64_t e = 0; e < d; ++e)
                                    Di += elem(dout, bnhd(b, i, h, e, N, Hq, d), dt) * orow[e];
                            }
                            const double p =
                                exp(score(q, k, dt, b, i, h, j, g, N, Hq, Hkv, d, scale) - lse_i);
                            double dp = 0.0;
                            for (int64_t e = 0; e < d; ++e)
                                dp += elem(dout, bnhd(b, i, h, e, N, Hq, d), dt) *
                                      elem(v, bnhd(b, j, g, e, N, Hkv, d), dt);
                            const double ds = p * (dp - Di);
                            for (int64_t e = 0; e < d; ++e) {
                                dkr[e] += ds * elem(q, bnhd(b, i, h, e, N, Hq, d), dt);
                                dvr[e] += p * elem(dout, bnhd(b, i, h, e, N, Hq, d), dt);
                            }
                        }
                    }
                    for (int64_t e = 0; e < d; ++e)
                        dkr[e] *= scale;
                }
        free(s);
        free(orow);
    }
    return bad ? 2 : 0;
}

/*
 * Row statistics for every query row: lse [B][Hq][N] and D = dO . O
 * [B][Hq][N], both from the fp64 forward definition.
 */
int oracle_row_stats(const void *q, const void *k, const void *v, const void *dout, int dt,
                     int64_t B, int64_t N, int64_t Hq, int64_t Hkv, int64_t d, double scale,
                     int causal, double *lse, double *D)
{
    if (B < 1 || N < 1 || Hq < 1 || Hkv < 1 || d < 1 || Hq % Hkv != 0)
        return 1;
    int bad = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc((size_t)N * sizeof(double));
        double *orow = (double *)malloc((size_t)d * sizeof(double));
        if (!s || !orow) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for collapse(3) schedule(dynamic, 4)
        for (int64_t b = 0; b < B; ++b)
            for (int64_t h = 0; h < Hq; ++h)
                for (int64_t i = 0; i < N; ++i) {
                    if (!s || !orow)
                        continue;
                    double lse_i, Di = 0.0;
                    fwd_row(q, k, v, dt, b, i, h, N, Hq, Hkv, d, scale, causal, s, orow, &lse_i);
                    for (int64_t e = 0; e < d; ++e)
                        Di += elem(dout, bnhd(b, i, h, e, N, Hq, d), dt) * orow[e];
                    lse[(b * Hq + h) * N + i] = lse_i;
                    D[(b * Hq + h) * N + i] = Di;
                }
        free(s);
        free(orow);
    }
    return bad ? 2 : 0;
}

/*
 * Full backward: dq [B][N][Hq][d], dk, dv [B][N][Hkv][d], all fp64.
 * Row statistics first, then every dQ row, then every dK/dV row.
 */
int oracle_attn_bwd(const void *q, const void *k, const void *v, const void *dout, int dt,
                    int64_t B, int64_t N, int64_t Hq, int64_t Hkv, int64_t d, double scale,
                    int causal, double *dq, double *dk, double *dv)
{
    if (B < 1 || N < 1 || Hq < 1 || Hkv < 1 || d < 1 || Hq % Hkv != 0)
        return 1;
    double *lse = (double *)malloc((size_t)(B * Hq * N) * sizeof(double));
    double *D = (double *)malloc((size_t)(B * Hq * N) * sizeof(double));
    int rc = (lse && D) ? 0 : 2;
    if (!rc)
        rc = oracle_row_stats(q, k, v, dout, dt, B, N, Hq, Hkv, d, scale, causal, lse, D);
    if (!rc)
        rc = oracle_dq_rows(q, k, v, dout, dt, B, N, Hq, Hkv, d, scale, causal, NULL, 0, dq);
    if (!rc)
        rc = oracle_dkdv_rows(q, k, v, dout, dt, B, N, Hq, Hkv, d, scale, causal, NULL, 0, lse, D,
                              dk, dv);
    free(lse);
    free(D);
    return rc;
}

/*
 * Sequence-to-head relayout, one element at a time.
 * in  [C][N][H][d]  (token t of rank r = t / (N/P) lives in rank r's chunk)
 * out [C][P][N][H/P][d]: rank r's head slice [r*H/P, (r+1)*H/P) over all N.
 *   out[c][r][t][hh][e] = in[c][t][r*(H/P) + hh][e]
 * elt is the element size in bytes; the copy moves bits, no arithmetic.
 */
int oracle_relayout_s2h(const uint8_t *in, uint8_t *out, int64_t C, int64_t N, int64_t H,
                        int64_t d, int64_t P, int64_t elt)
{
    if (C < 1 || N < 1 || H < 1 || d < 1 || P < 1 || H % P != 0 || N % P != 0 || elt < 1)
        return 1;
    const int64_t Hs = H / P;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t c = 0; c < C; ++c)
        for (int64_t r = 0; r < P; ++r)
            for (int64_t t = 0; t < N; ++t)
                for (int64_t hh = 0; hh < Hs; ++hh)
                    for (int64_t e = 0; e < d; ++e) {
                        const int64_t src = (((c * N + t) * H) + r * Hs + hh) * d + e;
                        const int64_t dst = ((((c * P + r) * N + t) * Hs) + hh) * d + e;
                        memcpy(out + dst * elt, in + src * elt, (size_t)elt);
                    }
    return 0;
}

/*
 * Head-to-sequence relayout (the reversed shuffle), written as its own loop
 * over the destination:
 *   out[c][t][h][e] = in[c][h / (H/P)][t][h % (H/P)][e]
 */
int oracle_relayout_h2s(const uint8_t *in, uint8_t *out, int64_t C, int64_t N, int64_t H,
                        int64_t d, int64_t P, int64_t elt)
{
    if (C < 1 || N < 1 || H < 1 || d < 1 || P < 1 || H % P != 0 || N % P != 0 || elt < 1)
        return 1;
    const int64_t Hs = H / P;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t c = 0; c < C; ++c)
        for (int64_t t = 0; t < N; ++t)
            for (int64_t h = 0; h < H; ++h)
                for (int64_t e = 0; e < d; ++e) {
                    const int64_t r = h / Hs, hh = h % Hs;
                    const int64_t src = ((((c * P + r) * N + t) * Hs) + hh) * d + e;
                    const int64_t dst = ((c * N + t) * H + h) * d + e;
                    memcpy(out + dst * elt, in + src * elt, (size_t)elt);
                }
    return 0;
}

/*
 * The same exchange for a chunk of heads: Hc heads starting h0 heads into
 * every rank's slice (a rank working through its heads a few at a time).
 *   out[c][r][t][hh][e] = in[c][t][r*(H/P) + h0 + hh][e],   hh < Hc
 * out is [C][P][N][Hc][d].
 */
int oracle_relayout_s2h_heads(const uint8_t *in, uint8_t *out, int64_t C, int64_t N, int64_t H,
                              int64_t d, int64_t P, int64_t h0, int64_t Hc, int64_t elt)
{
    if (C < 1 || N < 1 || H < 1 || d < 1 || P < 1 || H % P != 0 || N % P != 0 || elt < 1)
        return 1;
    const int64_t Hs = H / P;
    if (h0 < 0 || Hc < 1 || h0 + Hc > Hs)
        return 2;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t c = 0; c < C; ++c)
        for (int64_t r = 0; r < P; ++r)
            for (int64_t t = 0; t < N; ++t)
                for (int64_t hh = 0; hh < Hc; ++hh)
                    for (int64_t e = 0; e < d; ++e) {
                        const int64_t h = r * Hs + h0 + hh;
                        const int64_t src = ((c * N + t) * H + h) * d + e;
                        const int64_t dst = (((c * P + r) * N + t) * Hc + hh) * d + e;
                        memcpy(out + dst * elt, in + src * elt, (size_t)elt);
                    }
    return 0;
}

/*
 * Its inverse on the chunk: writes heads r*(H/P) + h0 .. + Hc - 1 of every
 * token of out [C][N][H][d] from in [C][P][N][Hc][d] and leaves the other
 * heads of out as they are.  Loops over the destination heads it owns.
 */
int oracle_relayout_h2s_heads(const uint8_t *in, uint8_t *out, int64_t C, int64_t N, int64_t H,
                              int64_t d, int64_t P, int64_t h0, int64_t Hc, int64_t elt)
{
    if (C < 1 || N < 1 || H < 1 || d < 1 || P < 1 || H % P != 0 || N % P != 0 || elt < 1)
        return 1;
    const int64_t Hs = H / P;
    if (h0 < 0 || Hc < 1 || h0 + Hc > Hs)
        return 2;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t c = 0; c < C; ++c)
        for (int64_t t = 0; t < N; ++t)
            for (int64_t h = 0; h < H; ++h) {
                const int64_t r = h / Hs, hh = h % Hs - h0;
                if (hh < 0 || hh >= Hc)
                    continue;
                for (int64_t e = 0; e < d; ++e) {
                    const int64_t src = (((c * P + r) * N + t) * Hc + hh) * d + e;
                    const int64_t dst = ((c * N + t) * H + h) * d + e;
                    memcpy(out + dst * elt, in + src * elt, (size_t)elt);
                }
            }
    return 0;
}
