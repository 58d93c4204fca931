"""fp64 CPU oracle for attention over packed variable-length sequences.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code with the
HIP library or its Python binding.

What it follows:

* "Ulysses Sequence Parallelism: Training with Million-Token Contexts", sections
  "Ulysses vs. Ring Attention: Who's Faster?" (variable sequence lengths are a
  mode of the method) and "Can You Integrate Ulysses with Hugging Face Today?"
  (variable-length batches are bucketed, never padded).  The pages do not spell
  out the mask; the plainest reading, taken here, is that documents packed into
  one token axis do not see each other: query token i sees key token j iff both
  lie in the same sequence and (causal) j <= i.  Within a sequence this is the
  ordinary attention of the rest of the path.

The definition is written over the whole packed axis with a block-diagonal mask,
not by slicing the sequences apart, so that the tests can compare it with the
per-sequence oracle (:mod:`oracle.attention`) as an independent formulation.

Layouts: q, o, dout, dq ``[T, Hq, d]``; k, v, dk, dv ``[T, Hkv, d]``; lse ``[Hq, T]``.
``cu`` holds the n + 1 token offsets of the n sequences (sequence s is tokens
``cu[s]:cu[s+1]``).  Tokens that no sequence covers get NaN outputs and zero
gradients.
"""

from __future__ import annotations

import numpy as np

__all__ = ["segments", "attn_varlen_fwd", "attn_varlen_bwd"]

_ROW_CHUNK = 512


def segments(cu, T: int) -> np.ndarray:
    """Sequence index of every token, -1 for tokens outside every sequence."""
    cu = np.asarray(cu, dtype=np.int64)
    seg = np.full(T, -1, dtype=np.int64)
    for s in range(len(cu) - 1):
        seg[cu[s]:cu[s + 1]] = s
    return seg


def _mask(seg, rows, causal):
    """Boolean [len(rows), T]: key j visible to query row i."""
    T = len(seg)
    same = (seg[rows][:, None] == seg[None, :]) & (seg[rows][:, None] >= 0)
    if causal:
        same &= np.arange(T)[None, :] <= rows[:, None]
    return same


def _check(q, k, v):
    T, Hq, d = q.shape
    if k.shape != v.shape or k.shape[0] != T or k.shape[2] != d or Hq % k.shape[1]:
        raise ValueError("q [T, Hq, d], k and v [T, Hkv, d] with Hkv dividing Hq")
    return T, Hq, k.shape[1], d


def _scores(qh, kg, seg, rows, scale, causal):
    s = scale * (qh[rows] @ kg.T)
    return np.where(_mask(seg, rows, causal), s, -np.inf)


def attn_varlen_fwd(q, k, v, cu, scale: float, causal: bool = True):
    """(o [T, Hq, d], lse [Hq, T]) in float64 for float64 inputs."""
    T, Hq, Hkv, d = _check(q, k, v)
    seg = segments(cu, T)
    o = np.full((T, Hq, d), np.nan)
    lse = np.full((Hq, T), np.nan)
    for h in range(Hq):
        g = h // (Hq // Hkv)
        for c0 in range(0, T, _ROW_CHUNK):
            rows = np.arange(c0, min(T, c0 + _ROW_CHUNK))
            rows = rows[seg[rows] >= 0]
            if len(rows) == 0:
                continue
            s = _scores(q[:, h], k[:, g], seg, rows, scale, causal)
            m = s.max(axis=1, keepdims=True)
            w = np.exp(s - m)
            l = w.sum(axis=1, keepdims=True)
            o[rows, h] = (w @ v[:, g]) / l
            lse[h, rows] = (m + np.log(l))[:, 0]
    return o, lse


def attn_varlen_bwd(q, k, v, dout, cu, scale: float, causal: bool = True):
    """Gradient of L = <dout, o>: (dq, dk, dv, o, lse) in float64.

    P = exp(S - lse) on visible pairs, dP = dO V^T, D = rowsum(dO * O),
    dS = P (dP - D), dQ = scale dS K, dK = scale dS^T Q and dV = P^T dO, the last
    two summed over each KV head's query heads.
    """
    T, Hq, Hkv, d = _check(q, k, v)
    seg = segments(cu, T)
    o, lse = attn_varlen_fwd(q, k, v, cu, scale, causal)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for h in range(Hq):
        g = h // (Hq // Hkv)
        for c0 in range(0, T, _ROW_CHUNK):
            rows = np.arange(c0, min(T, c0 + _ROW_CHUNK))
            rows = rows[seg[rows] >= 0]
            if len(rows) == 0:
                continue
            s = _scores(q[:, h], k[:, g], seg, rows, scale, causal)
            p = np.exp(s - lse[h, rows][:, None])
            dp = dout[rows, h] @ v[:, g].T
            D = np.sum(dout[rows, h] * o[rows, h], axis=1)
            ds = p * (dp - D[:, None])
            dq[rows, h] = scale * (ds @ k[:, g])
            dk[:, g] += scale * (ds.T @ q[rows, h])
            dv[:, g] += p.T @ dout[rows, h]
    return dq, dk, dv, o, lse
