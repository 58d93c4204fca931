"""fp64 CPU oracle for the per-rank Ulysses attention step (forward and backward).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code with the
HIP library or its Python binding; inputs reach it as host arrays in their
stored precision and it widens them to float64 itself.

What it follows:

* "Ulysses Sequence Parallelism: Training with Million-Token Contexts", section
  "How Does Ulysses Sequence Parallelism Actually Work?": after the all-to-all
  every GPU holds all N positions for a slice of the heads and computes attention
  locally; heads are independent, so one rank's work is plain multi-head
  attention over its heads.
* "Ulysses: entrenar con contextos de hasta 96K tokens en 4 GPUs", section
  "Conclusion rapida": the mathematics of attention is unchanged, so this module
  is the textbook definition of causal softmax attention and of its gradient,
  written out in float64 with a library matrix product for each contraction.

Readings where the pages are silent (the design notes list them all):

* softmax scale is a call argument (1/sqrt(d) in every workload);
* causal mask: key j is visible to query i iff j <= i, queries and keys share
  the length N;
* grouped KV heads: query head h reads KV head h // (Hq // Hkv);
* lse is the natural log of sum_j exp(s_ij) over the scaled scores;
* the backward is the gradient of L = <dO, O>.

Layouts: q, o, dout, dq ``[B, N, Hq, d]``; k, v, dk, dv ``[B, N, Hkv, d]``;
lse, D ``[B, Hq, N]``.  Row-subset results keep the same axes with N replaced by
the number of selected rows.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "widen",
    "attn_fwd",
    "attn_bwd",
    "row_stats",
    "dq_rows",
    "dkdv_rows",
    "probabilities",
]

# Rows of the score matrix materialised at once: at most 1024, and at most
# about 2^26 scores per block for long key ranges (bounds memory only; every
# row is computed independently by the same definition).
_ROW_CHUNK = 1024
_BLOCK_ELEMS = 1 << 26


def _chunk(n_keys: int) -> int:
    return max(1, min(_ROW_CHUNK, _BLOCK_ELEMS // max(1, n_keys)))


def widen(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of a stored tensor.

    ``dtype`` is "f32" (a float32 array), "bf16" (a uint16 array of bf16 bit
    patterns: bf16 is the upper half of an IEEE binary32, so the bits shifted
    left by 16 are that float exactly) or "f64".
    """
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        u = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return u.view(np.float32).astype(np.float64)
    if dtype == "f64":
        return np.asarray(x, dtype=np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def _check(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, N, H, d]")
    B, N, Hq, d = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[1] != N or k.shape[3] != d:
        raise ValueError("k and v must be [B, N, Hkv, d] matching q")
    Hkv = k.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    return B, N, Hq, Hkv, d


def _group(h: int, Hq: int, Hkv: int) -> int:
    """KV head read by query head h (contiguous groups of Hq/Hkv query heads)."""
    return h // (Hq // Hkv)


def _visible(rows: np.ndarray, N: int, causal: bool) -> np.ndarray:
    """Boolean [len(rows), N]: key j visible to query row i."""
    if not causal:
        return np.ones((len(rows), N), dtype=bool)
    return np.arange(N)[None, :] <= rows[:, None]


def _key_end(rows: np.ndarray, N: int, causal: bool) -> int:
    """Keys past the last row of a causal chunk are masked for every row in it."""
    return int(rows.max()) + 1 if causal else N


def _fwd_rows_one_head(qh, kg, vg, rows, scale, causal):
    """Forward for query rows `rows` of one head: (o [R, d], lse [R]).

    s = scale * q_i . k_j over visible keys; m = max_j s; l = sum_j exp(s - m);
    o_i = sum_j exp(s - m) v_j / l; lse_i = m + ln l.
    """
    o = np.empty((len(rows), qh.shape[1]))
    lse = np.empty(len(rows))
    step = _chunk(kg.shape[0])
    for c0 in range(0, len(rows), step):
        r = rows[c0 : c0 + step]
        n = _key_end(r, kg.shape[0], causal)
        s = scale * (qh[r] @ kg[:n].T)
        s = np.where(_visible(r, n, causal), s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        w = np.exp(s - m)  # exp(-inf) = 0 for masked keys
        l = w.sum(axis=1, keepdims=True)
        o[c0 : c0 + len(r)] = (w @ vg[:n]) / l
        lse[c0 : c0 + len(r)] = (m + np.log(l))[:, 0]
    return o, lse


def attn_fwd(q, k, v, scale: float, causal: bool = True, rows=None):
    """Forward attention in float64.

    q, k, v: float64 arrays ``[B, N, Hq|Hkv, d]`` (use :func:`widen` first).
    rows: optional 1-D int array of query rows; default all rows.
    Returns o ``[B, R, Hq, d]`` and lse ``[B, Hq, R]``.
    """
    B, N, Hq, Hkv, d = _check(q, k, v)
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    o = np.empty((B, len(rows), Hq, d))
    lse = np.empty((B, Hq, len(rows)))
    for b in range(B):
        for h in range(Hq):
            g = _group(h, Hq, Hkv)
            o[b, :, h], lse[b, h] = _fwd_rows_one_head(
                q[b, :, h], k[b, :, g], v[b, :, g], rows, scale, causal
            )
    return o, lse


def probabilities(q, k, scale: float, causal: bool = True):
    """The full probability matrix P ``[B, Hq, N, N]`` (tiny N only).

    P_ij = exp(s_ij - lse_i) for visible keys, 0 otherwise.
    """
    B, N, Hq, Hkv, d = _check(q, k, k)
    P = np.zeros((B, Hq, N, N))
    rows = np.arange(N)
    for b in range(B):
        for h in range(Hq):
            g = _group(h, Hq, Hkv)
            s = scale * (q[b, :, h] @ k[b, :, g].T)
            s = np.where(_visible(rows, N, causal), s, -np.inf)
            m = s.max(axis=1, keepdims=True)
            w = np.exp(s - m)
            P[b, h] = w / w.sum(axis=1, keepdims=True)
    return P


def row_stats(q, k, v, dout, scale: float, causal: bool = True, rows=None):
    """lse and D = rowsum(dO * O) for the selected query rows, ``[B, Hq, R]`` each.

    Also returns o ``[B, R, Hq, d]``.
    """
    B, N, Hq, Hkv, d = _check(q, k, v)
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    o, lse = attn_fwd(q, k, v, scale, causal, rows)
    D = np.einsum("brhe,brhe->bhr", dout[:, rows], o)
    return lse, D, o


def _p_dp_ds(qh_r, kg, vg, do_r, lse_r, D_r, rows, scale, causal):
    """p, dp and ds for query rows `rows` of one head against every key.

    p_ij = exp(s_ij - lse_i) (0 where masked), dp_ij = dO_i . v_j,
    ds_ij = p_ij (dp_ij - D_i).
    """
    N = kg.shape[0]
    s = scale * (qh_r @ kg.T)
    s = np.where(_visible(rows, N, causal), s, -np.inf)  # kg may be a prefix of the keys
    p = np.exp(s - lse_r[:, None])
    dp = do_r @ vg.T
    ds = p * (dp - D_r[:, None])
    return p, dp, ds


def dq_rows(q, k, v, dout, scale: float, causal: bool = True, rows=None):
    """dQ for the selected query rows, ``[B, R, Hq, d]``.

    dq_i = scale * sum_j ds_ij k_j; each row depends only on its own data, so
    this is exact for any subset of rows.
    """
    B, N, Hq, Hkv, d = _check(q, k, v)
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    lse, D, _ = row_stats(q, k, v, dout, scale, causal, rows)
    dq = np.empty((B, len(rows), Hq, d))
    for b in range(B):
        for h in range(Hq):
            g = _group(h, Hq, Hkv)
            step = _chunk(N)
            for c0 in range(0, len(rows), step):
                sl = slice(c0, c0 + step)
                r = rows[sl]
                n = _key_end(r, N, causal)
                _, _, ds = _p_dp_ds(
                    q[b, r, h], k[b, :n, g], v[b, :n, g], dout[b, r, h],
                    lse[b, h, sl], D[b, h, sl], r, scale, causal,
                )
                dq[b, sl, h] = scale * (ds @ k[b, :n, g])
    return dq


def dkdv_rows(q, k, v, dout, scale: float, causal: bool = True, keys=None):
    """dK and dV for the selected key rows, ``[B, R, Hkv, d]`` each.

    dk_j = scale * sum_{h in group} sum_i ds_ij q_i and
    dv_j = sum_{h in group} sum_i p_ij dO_i, summed over every query row i that
    sees key j.  Under the causal mask only rows i >= min(keys) can contribute,
    so the last keys of a long sequence are cheap.
    """
    B, N, Hq, Hkv, d = _check(q, k, v)
    keys = np.arange(N) if keys is None else np.asarray(keys, dtype=np.int64)
    i0 = int(keys.min()) if (causal and len(keys)) else 0
    qrows = np.arange(i0, N)
    lse, D, _ = row_stats(q, k, v, dout, scale, causal, qrows)
    dk = np.zeros((B, len(keys), Hkv, d))
    dv = np.zeros((B, len(keys), Hkv, d))
    for b in range(B):
        for h in range(Hq):
            g = _group(h, Hq, Hkv)
            kg, vg = k[b, keys, g], v[b, keys, g]
            step = _chunk(len(keys))
            for c0 in range(0, len(qrows), step):
                sl = slice(c0, c0 + step)
                r = qrows[sl]
                s = scale * (q[b, r, h] @ kg.T)
                vis = (keys[None, :] <= r[:, None]) if causal else np.ones(s.shape, bool)
                s = np.where(vis, s, -np.inf)
                p = np.exp(s - lse[b, h, sl][:, None])
                dp = dout[b, r, h] @ vg.T
                ds = p * (dp - D[b, h, sl][:, None])
                dk[b, :, g] += scale * (ds.T @ q[b, r, h])
                dv[b, :, g] += p.T @ dout[b, r, h]
    return dk, dv


def attn_bwd(q, k, v, dout, scale: float, causal: bool = True):
    """Full backward in float64: (dq, dk, dv, o, lse).

    P = exp(S - lse), dP = dO V^T, D = rowsum(dO * O), dS = P * (dP - D),
    dQ = scale dS K, dK = scale dS^T Q (summed over the group's query heads),
    dV = P^T dO (summed likewise).
    """
    B, N, Hq, Hkv, d = _check(q, k, v)
    rows = np.arange(N)
    lse, D, o = row_stats(q, k, v, dout, scale, causal, rows)
    dq = np.empty_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            g = _group(h, Hq, Hkv)
            step = _chunk(N)
            for c0 in range(0, N, step):
                sl = slice(c0, c0 + step)
                r = rows[sl]
                n = _key_end(r, N, causal)
                p, _, ds = _p_dp_ds(
                    q[b, r, h], k[b, :n, g], v[b, :n, g], dout[b, r, h],
                    lse[b, h, sl], D[b, h, sl], r, scale, causal,
                )
                dq[b, sl, h] = scale * (ds @ k[b, :n, g])
                dk[b, :n, g] += scale * (ds.T @ q[b, r, h])
                dv[b, :n, g] += p.T @ dout[b, r, h]
    return dq, dk, dv, o, lse
