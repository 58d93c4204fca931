"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws numbers and encodes them in the stored precision; it
holds none of the attention or relayout arithmetic, so both the HIP path and
the oracle can take their inputs from it without sharing any of the method.

Every tensor is drawn from ``numpy.random.Generator(PCG64(seed))`` as float64
standard normals, narrowed to float32, and (for bf16 workloads) rounded to the
nearest bf16 with ties to even.  The stored low-precision array *is* the input:
the oracle widens exactly these values.  Seeds are ``1000 * workload + slot``
with slot 1..8 for Q, K, V, dO, sampled rows, outlier keys, the relayout
tensor and sampled keys.

The workloads are one Ulysses rank's share of a Llama-3.1-8B-shaped layer
(32 query heads, 8 KV heads, head_dim 128) at SP = 4 or 8, plus a tiny fp32
case; the pages train that model on long documents, which are not needed:
N(0, 1) activations of the same shapes stand in for real Q/K/V.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

SLOT_Q, SLOT_K, SLOT_V, SLOT_DO, SLOT_ROWS, SLOT_OUTLIERS, SLOT_RELAYOUT, SLOT_KEYS = range(1, 9)

# Normals drawn per chunk when generating very large tensors (bounds memory).
_CHUNK = 1 << 24


@dataclass(frozen=True)
class Workload:
    """One attention workload (batch 1, causal) and its optional relayout case."""

    wid: int
    name: str
    N: int
    Hq: int
    Hkv: int
    d: int
    dtype: str  # "f32" or "bf16"
    causal: bool = True
    outlier_frac: float = 0.0  # fraction of keys per KV head shifted by +outlier_shift
    outlier_shift: float = 4.0
    relayout: tuple | None = None  # (C, N, H, d, P)
    B: int = 1

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def flops_fwd(self) -> float:
        """Counted forward FLOPs: 4d per visible (query, key) pair, N^2/2 pairs if causal."""
        pairs = self.N * self.N / 2 if self.causal else self.N * self.N
        return 4.0 * self.d * pairs * self.Hq * self.B

    def flops_bwd(self) -> float:
        """Counted backward FLOPs: 10d per visible pair (2.5x the forward)."""
        return 2.5 * self.flops_fwd()

    @property
    def exchange(self) -> tuple:
        """(C, N, H, d, P) of the QKV-stack exchange around this rank's attention: the
        workload's own relayout case, else the full 32-head stack of the layer whose rank
        share this is (P = 32 / Hq)."""
        if self.relayout is not None:
            return self.relayout
        P = max(1, 32 // self.Hq)
        return (3, self.N, self.Hq * P, self.d, P)


WORKLOADS = {
    1: Workload(1, "tiny-fp32-N256-4q4kv-d64", 256, 4, 4, 64, "f32", relayout=(3, 256, 4, 64, 2)),
    2: Workload(2, "sp4-rank-llama8b-N8192-8q2kv-d128", 8192, 8, 2, 128, "bf16"),
    3: Workload(3, "sp4-rank-llama8b-N65536-8q2kv-d128", 65536, 8, 2, 128, "bf16",
                relayout=(3, 65536, 32, 128, 4)),
    4: Workload(4, "near-oom-N98304-8q2kv-d128-outliers", 98304, 8, 2, 128, "bf16",
                outlier_frac=0.01),
    5: Workload(5, "sp8-rank-N1048576-4q1kv-d128", 1048576, 4, 1, 128, "bf16"),
}


def seed_of(wid: int, slot: int) -> int:
    return 1000 * wid + slot


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); returns uint16 bits.

    Inputs here are finite normals, so no NaN handling is needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """The float32 value of bf16 bit patterns (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_f32(shape, seed: int) -> np.ndarray:
    """float32 standard normals from PCG64(seed), drawn in float64 then narrowed."""
    rng = np.random.Generator(np.random.PCG64(seed))
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    for c0 in range(0, n, _CHUNK):
        c1 = min(n, c0 + _CHUNK)
        out[c0:c1] = rng.standard_normal(c1 - c0)
    return out.reshape(shape)


def encode(x32: np.ndarray, dtype: str) -> np.ndarray:
    """Store float32 values in the workload's precision (float32 or bf16 bits)."""
    if dtype == "f32":
        return np.ascontiguousarray(x32, dtype=np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(x32)
    raise ValueError(dtype)


def outlier_keys(wl: Workload, g: int) -> np.ndarray:
    """Sorted key positions of KV head g that get the +shift outlier (seeded)."""
    count = int(math.floor(wl.outlier_frac * wl.N))
    rng = np.random.Generator(np.random.PCG64(seed_of(wl.wid, SLOT_OUTLIERS) * 1000 + g))
    return np.sort(rng.choice(wl.N, size=count, replace=False))


def attn_inputs(wl: Workload, with_dout: bool = True) -> dict:
    """Stored q, k, v (and dout) for a workload: layouts [B, N, H, d].

    float32 workloads return float32 arrays; bf16 workloads return uint16 bf16
    bit patterns.  For outlier workloads, every component of the selected K rows
    is shifted by +outlier_shift (in float32) before rounding.
    """
    B, N, Hq, Hkv, d = wl.B, wl.N, wl.Hq, wl.Hkv, wl.d
    q = normal_f32((B, N, Hq, d), seed_of(wl.wid, SLOT_Q))
    k = normal_f32((B, N, Hkv, d), seed_of(wl.wid, SLOT_K))
    v = normal_f32((B, N, Hkv, d), seed_of(wl.wid, SLOT_V))
    if wl.outlier_frac > 0:
        for g in range(Hkv):
            k[:, outlier_keys(wl, g), g, :] += np.float32(wl.outlier_shift)
    out = {"q": encode(q, wl.dtype), "k": encode(k, wl.dtype), "v": encode(v, wl.dtype)}
    del q, k, v
    if with_dout:
        out["dout"] = encode(normal_f32((B, N, Hq, d), seed_of(wl.wid, SLOT_DO)), wl.dtype)
    return out


def custom_inputs(B, N, Hq, Hkv, d, dtype: str, seed: int, with_dout: bool = True) -> dict:
    """Stored inputs of an arbitrary shape (parity sweeps, ragged tails)."""
    out = {
        "q": encode(normal_f32((B, N, Hq, d), seed * 10 + SLOT_Q), dtype),
        "k": encode(normal_f32((B, N, Hkv, d), seed * 10 + SLOT_K), dtype),
        "v": encode(normal_f32((B, N, Hkv, d), seed * 10 + SLOT_V), dtype),
    }
    if with_dout:
        out["dout"] = encode(normal_f32((B, N, Hq, d), seed * 10 + SLOT_DO), dtype)
    return out


FIXED_ROWS = (0, 1, 63, 64, 127, 128)


def sample_rows(wl: Workload, h: int, count: int = 512) -> np.ndarray:
    """Sorted query rows checked for head h: `count` distinct rows drawn uniformly."""
    rng = np.random.Generator(np.random.PCG64(seed_of(wl.wid, SLOT_ROWS) + h))
    return np.sort(rng.choice(wl.N, size=min(count, wl.N), replace=False))


def fixed_rows(N: int) -> np.ndarray:
    """Edge rows checked in addition to the sampled ones."""
    rows = [r for r in FIXED_ROWS if r < N] + [N // 2, N - 2, N - 1]
    return np.unique(np.array([r for r in rows if 0 <= r < N], dtype=np.int64))


FIXED_KEYS = (0, 1, 127, 128)


def sample_keys(wl: Workload, g: int, count: int = 512, window: int | None = None) -> np.ndarray:
    """Sorted key positions of KV head g whose dK/dV rows are checked: `count` distinct keys
    drawn uniformly from the last `window` positions (default: the whole sequence), plus the
    fixed keys {0, 1, 127, 128, N/2} and the window's first and last keys."""
    N = wl.N
    lo = 0 if window is None else max(0, N - window)
    rng = np.random.Generator(np.random.PCG64(seed_of(wl.wid, SLOT_KEYS) * 1000 + g))
    drawn = lo + rng.choice(N - lo, size=min(count, N - lo), replace=False)
    fixed = [x for x in FIXED_KEYS + (N // 2,) if lo <= x < N] + [lo, N - 1]
    return np.unique(np.concatenate([drawn, np.array(fixed, dtype=np.int64)]))


def random_bits(shape, dtype: str, seed: int) -> np.ndarray:
    """Uniform random bit patterns in the element type (uint16 for bf16, uint32 for f32).

    Any misplaced element, or any pass through float registers that alters a
    pattern (NaN payloads, denormals), changes the bytes.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    n = int(np.prod(shape))
    if dtype == "bf16":
        return rng.integers(0, 1 << 16, size=n, dtype=np.uint16).reshape(shape)
    if dtype == "f32":
        return rng.integers(0, 1 << 32, size=n, dtype=np.uint32).reshape(shape)
    raise ValueError(dtype)


def length_mix(total: int, seed: int, lo: int = 512, hi: int = 16384) -> np.ndarray:
    """Document lengths of a packed variable-length batch of `total` tokens.

    Lengths are drawn log-uniformly in [lo, hi] (many short documents, a few long
    ones) until they cover `total`; the last one is cut to fit.  The pages give no
    length distribution; this mix only exercises ragged, unaligned boundaries and
    a wide spread of per-document work.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    out, used = [], 0
    while used < total:
        n = int(round(math.exp(rng.uniform(math.log(lo), math.log(hi)))))
        n = min(max(n, 1), total - used)
        out.append(n)
        used += n
    return np.array(out, dtype=np.int64)


def cu_seqlens(lengths) -> np.ndarray:
    """int32 token offsets [0, l0, l0 + l1, ...] of packed sequences."""
    return np.concatenate([[0], np.cumsum(np.asarray(lengths, dtype=np.int64))]).astype(np.int32)
