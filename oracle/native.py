"""ctypes wrapper for the plain C part of the oracle (``ul_oracle.c``).

TEST INFRASTRUCTURE ONLY: used by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.

The C library holds the scalar index-loop relayout (sequence-sharded to
head-sharded and back, "How Does Ulysses Sequence Parallelism Actually Work?",
"Ulysses Sequence Parallelism: Training with Million-Token Contexts") and a
scalar brute-force attention used to cross-check the float64 matrix oracle at
tiny sizes.  It is built with gcc, ``-O2 -fopenmp``, no fast-math.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "ul_oracle.c"
_LIB = _HERE / "libuloracle.so"

_DT = {"f32": 0, "bf16": 1, "f64": 2}
_lib = None


def build(force: bool = True) -> Path:
    """Compile ul_oracle.c into libuloracle.so next to it."""
    if force or not _LIB.exists() or _LIB.stat().st_mtime < _SRC.stat().st_mtime:
        tmp = _LIB.with_suffix(".so.tmp")
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall", "-Werror",
               "-o", str(tmp), str(_SRC), "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not _LIB.exists() or _LIB.stat().st_mtime < _SRC.stat().st_mtime:
            build(force=True)
        L = ctypes.CDLL(str(_LIB))
        i64, vp, dp = ctypes.c_int64, ctypes.c_void_p, ctypes.c_double
        L.oracle_attn_fwd_rows.argtypes = [vp, vp, vp, ctypes.c_int, i64, i64, i64, i64, i64, dp,
                                           ctypes.c_int, vp, i64, vp, vp]
        L.oracle_attn_bwd.argtypes = [vp, vp, vp, vp, ctypes.c_int, i64, i64, i64, i64, i64, dp,
                                      ctypes.c_int, vp, vp, vp]
        L.oracle_dq_rows.argtypes = [vp, vp, vp, vp, ctypes.c_int, i64, i64, i64, i64, i64, dp,
                                     ctypes.c_int, vp, i64, vp]
        L.oracle_dkdv_rows.argtypes = [vp, vp, vp, vp, ctypes.c_int, i64, i64, i64, i64, i64, dp,
                                       ctypes.c_int, vp, i64, vp, vp, vp, vp]
        L.oracle_row_stats.argtypes = [vp, vp, vp, vp, ctypes.c_int, i64, i64, i64, i64, i64, dp,
                                       ctypes.c_int, vp, vp]
        for name in ("oracle_relayout_s2h", "oracle_relayout_h2s"):
            getattr(L, name).argtypes = [vp, vp, i64, i64, i64, i64, i64, i64]
        for name in ("oracle_relayout_s2h_heads", "oracle_relayout_h2s_heads"):
            getattr(L, name).argtypes = [vp, vp, i64, i64, i64, i64, i64, i64, i64, i64]
        for f in (L.oracle_attn_fwd_rows, L.oracle_attn_bwd, L.oracle_dq_rows, L.oracle_dkdv_rows,
                  L.oracle_row_stats, L.oracle_relayout_s2h,
                  L.oracle_relayout_h2s, L.oracle_relayout_s2h_heads, L.oracle_relayout_h2s_heads):
            f.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def relayout_s2h(x: np.ndarray, P: int) -> np.ndarray:
    """[C, N, H, d] -> [C, P, N, H/P, d], element by element (any dtype)."""
    x = np.ascontiguousarray(x)
    C, N, H, d = x.shape
    if P < 1 or H % P or N % P:
        raise ValueError("need P >= 1, H % P == 0 and N % P == 0")
    out = np.empty((C, P, N, H // P, d), dtype=x.dtype)
    rc = lib().oracle_relayout_s2h(_ptr(x), _ptr(out), C, N, H, d, P, x.itemsize)
    if rc:
        raise RuntimeError(f"oracle_relayout_s2h failed ({rc})")
    return out


def relayout_h2s(y: np.ndarray) -> np.ndarray:
    """[C, P, N, H/P, d] -> [C, N, H, d], element by element (any dtype)."""
    y = np.ascontiguousarray(y)
    C, P, N, Hs, d = y.shape
    out = np.empty((C, N, Hs * P, d), dtype=y.dtype)
    rc = lib().oracle_relayout_h2s(_ptr(y), _ptr(out), C, N, Hs * P, d, P, y.itemsize)
    if rc:
        raise RuntimeError(f"oracle_relayout_h2s failed ({rc})")
    return out


def relayout_s2h_heads(x: np.ndarray, P: int, h0: int, Hc: int) -> np.ndarray:
    """[C, N, H, d] -> [C, P, N, Hc, d]: heads h0 .. h0+Hc-1 of every rank's slice."""
    x = np.ascontiguousarray(x)
    C, N, H, d = x.shape
    out = np.empty((C, P, N, Hc, d), dtype=x.dtype)
    rc = lib().oracle_relayout_s2h_heads(_ptr(x), _ptr(out), C, N, H, d, P, h0, Hc, x.itemsize)
    if rc:
        raise RuntimeError(f"oracle_relayout_s2h_heads failed ({rc})")
    return out


def relayout_h2s_heads(y: np.ndarray, out: np.ndarray, h0: int) -> np.ndarray:
    """Writes y [C, P, N, Hc, d] into heads h0 .. h0+Hc-1 of every rank's slice of `out`
    [C, N, H, d] (in place; the other heads are left as they are) and returns `out`."""
    y = np.ascontiguousarray(y)
    if not out.flags.c_contiguous or out.dtype != y.dtype:
        raise ValueError("out must be a C-contiguous array of y's dtype")
    C, P, N, Hc, d = y.shape
    H = out.shape[2]
    rc = lib().oracle_relayout_h2s_heads(_ptr(y), _ptr(out), C, N, H, d, P, h0, Hc, y.itemsize)
    if rc:
        raise RuntimeError(f"oracle_relayout_h2s_heads failed ({rc})")
    return out


def _stored(x: np.ndarray, dtype: str) -> np.ndarray:
    want = {"f32": np.float32, "bf16": np.uint16, "f64": np.float64}[dtype]
    return np.ascontiguousarray(x, dtype=want)


def brute_fwd(q, k, v, dtype: str, scale: float, causal: bool = True):
    """Scalar brute-force forward: (o [B,N,Hq,d], lse [B,Hq,N]) in float64."""
    q, k, v = (_stored(a, dtype) for a in (q, k, v))
    B, N, Hq, d = q.shape
    Hkv = k.shape[2]
    o = np.empty((B, N, Hq, d))
    lse = np.empty((B, Hq, N))
    rc = lib().oracle_attn_fwd_rows(_ptr(q), _ptr(k), _ptr(v), _DT[dtype], B, N, Hq, Hkv, d,
                                    scale, int(causal), None, 0, _ptr(o), _ptr(lse))
    if rc:
        raise RuntimeError(f"oracle_attn_fwd_rows failed ({rc})")
    return o, lse


def brute_bwd(q, k, v, dout, dtype: str, scale: float, causal: bool = True):
    """Scalar brute-force backward: (dq, dk, dv) in float64."""
    q, k, v, dout = (_stored(a, dtype) for a in (q, k, v, dout))
    B, N, Hq, d = q.shape
    Hkv = k.shape[2]
    dq = np.empty((B, N, Hq, d))
    dk = np.empty((B, N, Hkv, d))
    dv = np.empty((B, N, Hkv, d))
    rc = lib().oracle_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _DT[dtype], B, N, Hq, Hkv,
                               d, scale, int(causal), _ptr(dq), _ptr(dk), _ptr(dv))
    if rc:
        raise RuntimeError(f"oracle_attn_bwd failed ({rc})")
    return dq, dk, dv


def _rows_arg(rows):
    if rows is None:
        return None, 0, None
    r = np.ascontiguousarray(rows, dtype=np.int64)
    return r, len(r), _ptr(r)


def brute_fwd_rows(q, k, v, dtype: str, scale: float, causal: bool, rows):
    """Scalar forward for the query rows `rows`: (o [B,R,Hq,d], lse [B,Hq,R]) in float64."""
    q, k, v = (_stored(a, dtype) for a in (q, k, v))
    B, N, Hq, d = q.shape
    Hkv = k.shape[2]
    r, R, rp = _rows_arg(rows)
    o = np.empty((B, R, Hq, d))
    lse = np.empty((B, Hq, R))
    rc = lib().oracle_attn_fwd_rows(_ptr(q), _ptr(k), _ptr(v), _DT[dtype], B, N, Hq, Hkv, d,
                                    scale, int(causal), rp, R, _ptr(o), _ptr(lse))
    if rc:
        raise RuntimeError(f"oracle_attn_fwd_rows failed ({rc})")
    return o, lse


def brute_dq_rows(q, k, v, dout, dtype: str, scale: float, causal: bool, rows):
    """Scalar dQ for the query rows `rows`, [B,R,Hq,d] in float64."""
    q, k, v, dout = (_stored(a, dtype) for a in (q, k, v, dout))
    B, N, Hq, d = q.shape
    Hkv = k.shape[2]
    r, R, rp = _rows_arg(rows)
    dq = np.empty((B, R, Hq, d))
    rc = lib().oracle_dq_rows(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _DT[dtype], B, N, Hq, Hkv, d,
                              scale, int(causal), rp, R, _ptr(dq))
    if rc:
        raise RuntimeError(f"oracle_dq_rows failed ({rc})")
    return dq


def brute_dkdv_rows(q, k, v, dout, dtype: str, scale: float, causal: bool, keys,
                    precomputed_stats: bool = False):
    """Scalar dK, dV for the key rows `keys`, [B,R,Hkv,d] each in float64.

    With precomputed_stats the row statistics (lse, D) of every query row come from the
    scalar row-statistics loop first; otherwise they are recomputed per query row."""
    q, k, v, dout = (_stored(a, dtype) for a in (q, k, v, dout))
    B, N, Hq, d = q.shape
    Hkv = k.shape[2]
    r, R, rp = _rows_arg(keys)
    dk = np.empty((B, R, Hkv, d))
    dv = np.empty((B, R, Hkv, d))
    lse = D = None
    if precomputed_stats:
        lse = np.empty((B, Hq, N))
        D = np.empty((B, Hq, N))
        rc = lib().oracle_row_stats(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _DT[dtype], B, N, Hq,
                                    Hkv, d, scale, int(causal), _ptr(lse), _ptr(D))
        if rc:
            raise RuntimeError(f"oracle_row_stats failed ({rc})")
    rc = lib().oracle_dkdv_rows(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _DT[dtype], B, N, Hq, Hkv,
                                d, scale, int(causal), rp, R,
                                None if lse is None else _ptr(lse),
                                None if D is None else _ptr(D), _ptr(dk), _ptr(dv))
    if rc:
        raise RuntimeError(f"oracle_dkdv_rows failed ({rc})")
    return dk, dv
