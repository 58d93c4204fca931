"""Thin ctypes binding over libulattn.so (argument marshalling only).

Every computation runs in the library's HIP kernels; this module only turns
torch tensors into device pointers and sizes, passes torch's current HIP
stream, and raises :class:`UlError` on a non-zero status.  PyTorch provides
device memory and streams, nothing else.  If the library has not been built,
:func:`lib` raises instead of falling back to anything.
"""

from __future__ import annotations

import ctypes
import math
import re
from pathlib import Path

PKG = Path(__file__).resolve().parent
LIB_PATH = PKG / "libulattn.so"
HEADER = PKG.parent / "include" / "ul_attn.h"

UL_F32, UL_BF16 = 0, 1
UL_BWD_PREP, UL_BWD_DQ, UL_BWD_DKDV, UL_BWD_ALL = 1, 2, 4, 7
STATUS = {0: "UL_OK", 1: "UL_ERR_NULL", 2: "UL_ERR_SHAPE", 3: "UL_ERR_DIVISIBILITY",
          4: "UL_ERR_UNSUPPORTED", 5: "UL_ERR_ALIGNMENT", 6: "UL_ERR_WORKSPACE",
          7: "UL_ERR_OVERLAP", 8: "UL_ERR_HIP", 9: "UL_ERR_SCRATCH"}
NOALLOC_SCRATCH_BYTES = 256 << 20

_lib = None


class UlError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        self.name = STATUS.get(status, f"status {status}")
        super().__init__(f"{fn} failed: {self.name}")


def declared_functions() -> list[str]:
    """Names of the functions include/ul_attn.h declares."""
    text = HEADER.read_text()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(ul_\w+)\s*\(", text, re.M)))


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not LIB_PATH.exists():
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python -m ulysses_sequence_parallelism_attn_amd.build`"
            )
        L = ctypes.CDLL(str(LIB_PATH))
        vp, i64, i32, f32, sz = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float,
                                 ctypes.c_size_t)
        L.ul_attn_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i32, i32, i32, f32, i32, i32, vp]
        L.ul_attn_fwd.restype = ctypes.c_int
        L.ul_attn_fwd_strided.argtypes = ([vp] * 5 + [i64, i64, i32, i32, i32] + [i64] * 4 +
                                          [f32, i32, i32, vp])
        L.ul_attn_fwd_strided.restype = ctypes.c_int
        L.ul_attn_fwd_workspace_bytes.argtypes = [i64, i64, i32, i32, i32, i32]
        L.ul_attn_fwd_workspace_bytes.restype = sz
        L.ul_attn_fwd_ws.argtypes = [vp, vp, vp, vp, vp, vp, sz, i64, i64, i32, i32, i32, f32, i32,
                                     i32, vp]
        L.ul_attn_fwd_ws.restype = ctypes.c_int
        L.ul_attn_bwd_workspace_bytes.argtypes = [i64, i64, i32, i32, i32, i32]
        L.ul_attn_bwd_workspace_bytes.restype = sz
        L.ul_attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i64, i64, i32, i32,
                                  i32, f32, i32, i32, vp]
        L.ul_attn_bwd.restype = ctypes.c_int
        L.ul_attn_bwd_noalloc.argtypes = [vp] * 9 + [i64, i64, i32, i32, i32, f32, i32, i32, vp]
        L.ul_attn_bwd_noalloc.restype = ctypes.c_int
        L.ul_attn_bwd_stages.argtypes = [i32] + L.ul_attn_bwd.argtypes
        L.ul_attn_bwd_stages.restype = ctypes.c_int
        L.ul_attn_bwd_strided.argtypes = ([vp] * 10 + [sz, i64, i64, i32, i32, i32] + [i64] * 8 +
                                          [f32, i32, i32, vp])
        L.ul_attn_bwd_strided.restype = ctypes.c_int
        L.ul_attn_fwd_varlen.argtypes = ([vp] * 6 + [i32, i64, i32, i32, i32, i32, f32, i32, i32,
                                                        vp])
        L.ul_attn_fwd_varlen.restype = ctypes.c_int
        L.ul_attn_bwd_varlen.argtypes = ([vp] * 10 + [sz, vp, i32, i64, i32, i32, i32, i32, f32, i32,
                                                        i32, vp])
        L.ul_attn_bwd_varlen.restype = ctypes.c_int
        for name in ("ul_relayout_s2h", "ul_relayout_h2s"):
            f = getattr(L, name)
            f.argtypes = [vp, vp, i64, i64, i32, i32, i32, i32, vp]
            f.restype = ctypes.c_int
        for name in ("ul_relayout_s2h_heads", "ul_relayout_h2s_heads"):
            f = getattr(L, name)
            f.argtypes = [vp, vp, i64, i64, i32, i32, i32, i32, i32, i32, vp]
            f.restype = ctypes.c_int
        L.ul_status_str.argtypes = [ctypes.c_int]
        L.ul_status_str.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(fn: str, st: int) -> None:
    if st != 0:
        raise UlError(fn, st)


def _dtype_code(t) -> int:
    import torch

    if t.dtype == torch.bfloat16:
        return UL_BF16
    if t.dtype == torch.float32:
        return UL_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream(stream):
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t) -> ctypes.c_void_p:
    return ctypes.c_void_p(t.data_ptr())


# ---------------------------------------------------------------------------- validation
#
# Every public call checks, before any ctypes call, that its tensors agree with q (or with
# the relayout input) in shape, dtype and device.  A mis-shaped buffer would otherwise make
# a kernel read or write past the end of an allocation.  The checks are pure Python over
# shapes, dtypes and devices, so the CPU tests drive them with host tensors
# (device_type="cpu").


def _fail(msg: str):
    raise ValueError(msg)


def _same_place(ts, ref, names, device_type: str):
    for t, n in zip(ts, names):
        if t.device.type != device_type:
            _fail(f"{n} must be a {device_type} tensor (got {t.device})")
        if t.device != ref.device:
            _fail(f"{n} is on {t.device}, q on {ref.device}")


def _shape_is(t, shape, name: str):
    if tuple(t.shape) != tuple(shape):
        _fail(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _dtype_is(t, dtype, name: str):
    if t.dtype != dtype:
        _fail(f"{name} has dtype {t.dtype}, expected {dtype}")


def _attn_dtype(q):
    import torch

    if q.dtype not in (torch.bfloat16, torch.float32):
        _fail(f"unsupported dtype {q.dtype} (bfloat16 or float32)")
    return q.dtype


def check_attn_fwd(q, k, v, out, lse, device_type: str = "cuda"):
    """q [B,N,Hq,d]; k, v [B,N,Hkv,d]; out [B,N,Hq,d] (all one dtype); lse contiguous
    float32 [B,Hq,N]; one device."""
    import torch

    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        _fail("q, k, v must be 4-d [B, N, H, d]")
    B, N, Hq, d = q.shape
    dt = _attn_dtype(q)
    _shape_is(v, k.shape, "v")
    _shape_is(k, (B, N, k.shape[2], d), "k")
    _shape_is(out, (B, N, Hq, d), "out")
    _shape_is(lse, (B, Hq, N), "lse")
    for t, n in ((k, "k"), (v, "v"), (out, "out")):
        _dtype_is(t, dt, n)
    _dtype_is(lse, torch.float32, "lse")
    if not lse.is_contiguous():
        _fail("lse must be contiguous")
    _same_place((q, k, v, out, lse), q, ("q", "k", "v", "out", "lse"), device_type)


def check_attn_bwd(q, k, v, o, dout, lse, dq, dk, dv, device_type: str = "cuda"):
    """The forward's checks for q, k, v, o, lse, plus dout and dq [B,N,Hq,d], dk and dv
    [B,N,Hkv,d]."""
    check_attn_fwd(q, k, v, o, lse, device_type)
    dt = q.dtype
    for t, n, like in ((dout, "dout", q), (dq, "dq", q), (dk, "dk", k), (dv, "dv", k)):
        _shape_is(t, like.shape, n)
        _dtype_is(t, dt, n)
    _same_place((dout, dq, dk, dv), q, ("dout", "dq", "dk", "dv"), device_type)


def check_workspace(workspace, need: int, q, device_type: str = "cuda"):
    """A contiguous uint8 workspace of at least `need` bytes on q's device."""
    import torch

    _dtype_is(workspace, torch.uint8, "workspace")
    if not workspace.is_contiguous():
        _fail("workspace must be contiguous")
    if workspace.numel() < need:
        _fail(f"workspace holds {workspace.numel()} bytes, {need} needed")
    _same_place((workspace,), q, ("workspace",), device_type)


def check_attn_varlen(q, k, v, out, lse, cu_seqlens, device_type: str = "cuda", grads=()):
    """Packed sequences: q, out [T,Hq,d]; k, v [T,Hkv,d]; lse [Hq,T] float32; cu_seqlens a
    1-d int32 table; every tensor contiguous and on q's device.  `grads` holds (dout, dq,
    dk, dv) for the backward."""
    import torch

    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        _fail("varlen q, k, v must be 3-d [T, H, d]")
    T, Hq, d = q.shape
    dt = _attn_dtype(q)
    _shape_is(k, (T, k.shape[1], d), "k")
    _shape_is(v, k.shape, "v")
    _shape_is(out, q.shape, "out")
    _shape_is(lse, (Hq, T), "lse")
    named = [(k, "k", dt), (v, "v", dt), (out, "out", dt), (lse, "lse", torch.float32)]
    if grads:
        dout, dq, dk, dv = grads
        for t, n, like in ((dout, "dout", q), (dq, "dq", q), (dk, "dk", k), (dv, "dv", k)):
            _shape_is(t, like.shape, n)
            named.append((t, n, dt))
    for t, n, want in named:
        _dtype_is(t, want, n)
    for t, n in [(q, "q")] + [(t, n) for t, n, _ in named]:
        if not t.is_contiguous():
            _fail(f"{n} must be contiguous")
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or not cu_seqlens.is_contiguous():
        _fail("cu_seqlens must be a contiguous 1-d int32 tensor")
    if cu_seqlens.numel() < 1:
        _fail("cu_seqlens needs at least one entry")
    _same_place([q] + [t for t, _, _ in named] + [cu_seqlens], q,
                ["q"] + [n for _, n, _ in named] + ["cu_seqlens"], device_type)


def check_relayout(x, out, out_shape, device_type: str = "cuda"):
    """Relayout input and output: both contiguous, one dtype and device, out of `out_shape`."""
    if not x.is_contiguous():
        _fail("relayout input must be contiguous")
    if not out.is_contiguous():
        _fail("relayout output must be contiguous")
    _shape_is(out, out_shape, "out")
    _dtype_is(out, x.dtype, "out")
    _same_place((x, out), x, ("input", "out"), device_type)


def _tok_stride(t, name: str) -> int:
    """Token stride (elements) of a [B, N, H, d] device view whose heads and head dim are
    dense and whose batches follow each other, as the *_strided calls address it."""
    if not t.is_cuda or t.dim() != 4:
        raise ValueError(f"{name} must be a 4-d device tensor")
    Bn, N, H, d = t.shape
    if (H > 1 and t.stride(2) != d) or (d > 1 and t.stride(3) != 1):
        raise ValueError(f"{name}: heads and head dim must be dense")
    ts = t.stride(1)
    if Bn > 1 and t.stride(0) != N * ts:
        raise ValueError(f"{name}: batch stride must be N * token stride")
    return ts


def fwd_workspace_bytes(B, N, Hq, Hkv, d, dtype_code) -> int:
    return int(lib().ul_attn_fwd_workspace_bytes(B, N, Hq, Hkv, d, dtype_code))


def attn_fwd(q, k, v, scale: float | None = None, causal: bool = True, out=None, lse=None,
             stream=None, split: bool = True, workspace=None):
    """O, lse = attention(q, k, v).  q [B,N,Hq,d], k/v [B,N,Hkv,d] (bf16 or fp32).

    q, k, v and `out` may be views with a token stride (for example a rank's head slice
    of a sequence-sharded [B,N,H,d] tensor); heads and head dim must be dense.
    With `split` (dense tensors only), sizes for which fwd_workspace_bytes is non-zero run
    through ul_attn_fwd_ws, which splits the key range of the longest query blocks; the
    workspace is allocated here unless given.  split=False runs ul_attn_fwd, whose
    rounding the strided and varlen calls share.
    """
    import torch

    if q.dim() != 4:
        _fail("q must be 4-d [B, N, Hq, d]")
    B, N, Hq, d = q.shape
    Hkv = k.shape[2] if k.dim() == 4 else 0
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    o = torch.empty((B, N, Hq, d), dtype=q.dtype, device=q.device) if out is None else out
    lse_t = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device) if lse is None else lse
    check_attn_fwd(q, k, v, o, lse_t)
    ts = [_tok_stride(t, n) for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "out"))]
    head = (_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse_t), B, N, Hq, Hkv, d)
    tail = (scale, int(causal), _dtype_code(q), _stream(stream))
    dense = all(t.is_contiguous() for t in (q, k, v, o))
    need = fwd_workspace_bytes(B, N, Hq, Hkv, d, _dtype_code(q)) if split and dense else 0
    if need > 0:
        if workspace is None:
            workspace = _internal_workspace(need, q.device, stream)
        check_workspace(workspace, need, q)
        _check("ul_attn_fwd_ws", lib().ul_attn_fwd_ws(*head[:5], _ptr(workspace), workspace.numel(),
                                                      *head[5:], *tail))
    elif dense:
        _check("ul_attn_fwd", lib().ul_attn_fwd(*head, *tail))
    else:
        _check("ul_attn_fwd_strided", lib().ul_attn_fwd_strided(*head, *ts, *tail))
    return o, lse_t


def attn_bwd_noalloc(q, k, v, o, dout, lse, scale: float | None = None, causal: bool = True,
                     dq=None, dk=None, dv=None, stream=None):
    """attn_bwd through ul_attn_bwd_noalloc: no workspace argument, the library's fixed
    per-GPU scratch holds the statistics (dense tensors only).  Calls that may overlap on
    one GPU must be ordered by the caller."""
    import torch

    if q.dim() != 4 or k.dim() != 4:
        _fail("q and k must be 4-d [B, N, H, d]")
    B, N, Hq, d = q.shape
    Hkv = k.shape[2]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    dq = torch.empty((B, N, Hq, d), dtype=q.dtype, device=q.device) if dq is None else dq
    dk = torch.empty((B, N, Hkv, d), dtype=q.dtype, device=q.device) if dk is None else dk
    dv = torch.empty((B, N, Hkv, d), dtype=q.dtype, device=q.device) if dv is None else dv
    check_attn_bwd(q, k, v, o, dout, lse, dq, dk, dv)
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dout, "dout"), (dq, "dq"), (dk, "dk"),
                 (dv, "dv")):
        if not t.is_contiguous():
            _fail(f"{n} must be contiguous")
    st = lib().ul_attn_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse),
                                   _ptr(dq), _ptr(dk), _ptr(dv), B, N, Hq, Hkv, d, scale,
                                   int(causal), _dtype_code(q), _stream(stream))
    _check("ul_attn_bwd_noalloc", st)
    return dq, dk, dv


def _internal_workspace(nbytes: int, device, stream):
    """A workspace the binding allocates for one call.  When the call runs on a stream other
    than the current one, the block is recorded on that stream, so the caching allocator
    does not hand it out again before the kernels there are done with it."""
    import torch

    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
    if stream is not None and stream != torch.cuda.current_stream(device):
        ws.record_stream(stream)
    return ws


def workspace_bytes(B, N, Hq, Hkv, d, dtype_code) -> int:
    return int(lib().ul_attn_bwd_workspace_bytes(B, N, Hq, Hkv, d, dtype_code))


def attn_bwd(q, k, v, o, dout, lse, scale: float | None = None, causal: bool = True,
             workspace=None, dq=None, dk=None, dv=None, stream=None, stages: int = UL_BWD_ALL):
    """dq, dk, dv of L = <dout, attention(q, k, v)>.

    `stages` selects a subset of the backward's stages (UL_BWD_PREP, UL_BWD_DQ,
    UL_BWD_DKDV); the default runs all three.  A partial call needs the same
    `workspace` a previous PREP stage filled.
    """
    import torch

    if q.dim() != 4 or k.dim() != 4:
        _fail("q and k must be 4-d [B, N, H, d]")
    B, N, Hq, d = q.shape
    Hkv = k.shape[2]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    dq = torch.empty((B, N, Hq, d), dtype=q.dtype, device=q.device) if dq is None else dq
    dk = torch.empty((B, N, Hkv, d), dtype=q.dtype, device=q.device) if dk is None else dk
    dv = torch.empty((B, N, Hkv, d), dtype=q.dtype, device=q.device) if dv is None else dv
    check_attn_bwd(q, k, v, o, dout, lse, dq, dk, dv)
    code = _dtype_code(q)
    need = workspace_bytes(B, N, Hq, Hkv, d, code)
    if workspace is None:
        workspace = _internal_workspace(need, q.device, stream)
    check_workspace(workspace, need, q)
    tensors = ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dout, "dout"), (dq, "dq"), (dk, "dk"),
               (dv, "dv"))
    ts = [_tok_stride(t, n) for t, n in tensors]
    head = (_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk),
            _ptr(dv), _ptr(workspace), workspace.numel(), B, N, Hq, Hkv, d)
    tail = (scale, int(causal), code, _stream(stream))
    if not all(t.is_contiguous() for t, _ in tensors):
        if stages != UL_BWD_ALL:
            raise ValueError("strided tensors run all backward stages")
        _check("ul_attn_bwd_strided", lib().ul_attn_bwd_strided(*head, *ts, *tail))
    elif stages == UL_BWD_ALL:
        _check("ul_attn_bwd", lib().ul_attn_bwd(*head, *tail))
    else:
        _check("ul_attn_bwd_stages", lib().ul_attn_bwd_stages(int(stages), *head, *tail))
    return dq, dk, dv


def attn_fwd_varlen(q, k, v, cu_seqlens, max_seqlen: int, scale: float | None = None,
                    causal: bool = True, out=None, lse=None, stream=None):
    """Attention over packed variable-length sequences.

    q [T, Hq, d], k/v [T, Hkv, d] (dense); cu_seqlens: int32 device tensor of the n + 1
    token offsets; max_seqlen: the longest sequence.  Returns o [T, Hq, d], lse [Hq, T].
    """
    import torch

    if q.dim() != 3:
        _fail("varlen q must be 3-d [T, Hq, d]")
    T, Hq, d = q.shape
    Hkv = k.shape[1] if k.dim() == 3 else 0
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    o = torch.empty_like(q) if out is None else out
    lse_t = torch.empty((Hq, T), dtype=torch.float32, device=q.device) if lse is None else lse
    check_attn_varlen(q, k, v, o, lse_t, cu_seqlens)
    st = lib().ul_attn_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse_t), _ptr(cu_seqlens),
                                  cu_seqlens.numel() - 1, T, int(max_seqlen), Hq, Hkv, d, scale,
                                  int(causal), _dtype_code(q), _stream(stream))
    _check("ul_attn_fwd_varlen", st)
    return o, lse_t


def attn_bwd_varlen(q, k, v, o, dout, lse, cu_seqlens, max_seqlen: int,
                    scale: float | None = None, causal: bool = True, workspace=None, dq=None,
                    dk=None, dv=None, stream=None):
    """dq, dk, dv of L = <dout, attn_fwd_varlen(q, k, v, ...)> (layouts as attn_fwd_varlen)."""
    import torch

    if q.dim() != 3 or k.dim() != 3:
        _fail("varlen q and k must be 3-d [T, H, d]")
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    check_attn_varlen(q, k, v, o, lse, cu_seqlens, grads=(dout, dq, dk, dv))
    code = _dtype_code(q)
    need = workspace_bytes(1, T, Hq, Hkv, d, code)
    if workspace is None:
        workspace = _internal_workspace(need, q.device, stream)
    check_workspace(workspace, need, q)
    st = lib().ul_attn_bwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq),
                                  _ptr(dk), _ptr(dv), _ptr(workspace), workspace.numel(),
                                  _ptr(cu_seqlens), cu_seqlens.numel() - 1, T, int(max_seqlen), Hq,
                                  Hkv, d, scale, int(causal), code, _stream(stream))
    _check("ul_attn_bwd_varlen", st)
    return dq, dk, dv


def relayout_s2h(x, P: int, out=None, stream=None):
    """[C, N, H, d] sequence-sharded world view -> [C, P, N, H/P, d] head-sharded."""
    import torch

    if x.dim() != 4:
        _fail("relayout input must be 4-d [C, N, H, d]")
    C, N, H, d = x.shape
    if P < 1 or H % P:
        raise ValueError("H must be a multiple of P")
    y = torch.empty((C, P, N, H // P, d), dtype=x.dtype, device=x.device) if out is None else out
    check_relayout(x, y, (C, P, N, H // P, d))
    st = lib().ul_relayout_s2h(_ptr(x), _ptr(y), C, N, H, d, P, _dtype_code(x), _stream(stream))
    _check("ul_relayout_s2h", st)
    return y


def relayout_h2s(y, out=None, stream=None):
    """[C, P, N, H/P, d] head-sharded -> [C, N, H, d] sequence-sharded."""
    import torch

    if y.dim() != 5:
        _fail("relayout input must be 5-d [C, P, N, H/P, d]")
    C, P, N, Hs, d = y.shape
    x = torch.empty((C, N, Hs * P, d), dtype=y.dtype, device=y.device) if out is None else out
    check_relayout(y, x, (C, N, Hs * P, d))
    st = lib().ul_relayout_h2s(_ptr(y), _ptr(x), C, N, Hs * P, d, P, _dtype_code(y),
                               _stream(stream))
    _check("ul_relayout_h2s", st)
    return x


def relayout_s2h_heads(x, P: int, h0: int, Hc: int, out=None, stream=None):
    """[C, N, H, d] -> [C, P, N, Hc, d]: heads h0 .. h0+Hc-1 of every rank's slice."""
    import torch

    if x.dim() != 4:
        _fail("relayout input must be 4-d [C, N, H, d]")
    C, N, H, d = x.shape
    if P < 1 or H % P:
        raise ValueError("H must be a multiple of P")
    y = torch.empty((C, P, N, Hc, d), dtype=x.dtype, device=x.device) if out is None else out
    check_relayout(x, y, (C, P, N, Hc, d))
    st = lib().ul_relayout_s2h_heads(_ptr(x), _ptr(y), C, N, H, d, P, h0, Hc, _dtype_code(x),
                                     _stream(stream))
    _check("ul_relayout_s2h_heads", st)
    return y


def relayout_h2s_heads(y, out, h0: int, stream=None):
    """Writes y [C, P, N, Hc, d] into heads h0 .. h0+Hc-1 of every rank's slice of `out`
    [C, N, H, d]; the other heads of `out` are left as they are.  Returns `out`."""
    if y.dim() != 5 or out.dim() != 4:
        _fail("head-chunk exchange: y must be [C, P, N, Hc, d] and out [C, N, H, d]")
    C, P, N, Hc, d = y.shape
    H = out.shape[2]
    check_relayout(y, out, (C, N, H, d))
    st = lib().ul_relayout_h2s_heads(_ptr(y), _ptr(out), C, N, H, d, P, h0, Hc, _dtype_code(y),
                                     _stream(stream))
    _check("ul_relayout_h2s_heads", st)
    return out
