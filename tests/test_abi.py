"""The C ABI on the CPU: the library builds, loads, exports every declared symbol, and its
host-side validation returns the documented status codes before any HIP call.

These calls pass fake (never dereferenced) device addresses and invalid arguments only, so
no kernel is launched and no GPU is needed.
"""

import ctypes

import pytest

from ulysses_sequence_parallelism_attn_amd import binding as B
from ulysses_sequence_parallelism_attn_amd import build as Bld


@pytest.fixture(scope="module")
def L():
    if not B.LIB_PATH.exists():
        Bld.build()
    return B.lib()


A = 0x10000  # fake, 16-byte aligned addresses far apart
BIG = 1 << 40


def addr(i):
    return ctypes.c_void_p(A + i * BIG)


def test_exports_every_declared_symbol(L):
    names = B.declared_functions()
    assert set(names) == {"ul_attn_fwd", "ul_attn_fwd_strided", "ul_attn_fwd_varlen",
                          "ul_attn_fwd_ws", "ul_attn_fwd_workspace_bytes",
                          "ul_attn_bwd", "ul_attn_bwd_stages", "ul_attn_bwd_strided",
                          "ul_attn_bwd_varlen", "ul_attn_bwd_workspace_bytes",
                          "ul_attn_bwd_noalloc",
                          "ul_relayout_s2h", "ul_relayout_h2s", "ul_relayout_s2h_heads",
                          "ul_relayout_h2s_heads", "ul_status_str"}
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    for code, name in B.STATUS.items():
        assert L.ul_status_str(code).decode() == name
    assert L.ul_status_str(99).decode() == "UL_ERR_UNKNOWN"


def fwd(L, q=None, k=None, v=None, o=None, lse=None, Bsz=1, N=128, Hq=8, Hkv=2, d=128, scale=0.088,
        causal=1, dtype=B.UL_BF16):
    q = addr(0) if q is None else q
    k = addr(1) if k is None else k
    v = addr(2) if v is None else v
    o = addr(3) if o is None else o
    lse = addr(4) if lse is None else lse
    return L.ul_attn_fwd(q, k, v, o, lse, Bsz, N, Hq, Hkv, d, scale, causal, dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=ctypes.c_void_p(0)), 1), (dict(lse=ctypes.c_void_p(0)), 1),
    (dict(N=0), 2), (dict(Bsz=0), 2), (dict(Hq=0), 2), (dict(Hkv=0), 2), (dict(d=0), 2),
    (dict(scale=0.0), 2), (dict(scale=-1.0), 2), (dict(scale=float("inf")), 2),
    (dict(scale=float("nan")), 2), (dict(causal=2), 2),
    (dict(Hq=6, Hkv=4), 3),
    (dict(d=96), 4), (dict(d=256), 4), (dict(dtype=7), 4),
    (dict(q=ctypes.c_void_p(A + 8)), 5), (dict(lse=ctypes.c_void_p(4 * BIG + A + 4)), 5),
    (dict(o=ctypes.c_void_p(A + 64)), 7), (dict(lse=ctypes.c_void_p(A + BIG + 16)), 7),
    (dict(lse=ctypes.c_void_p(3 * BIG + A + 1024)), 7),
    (dict(N=1 << 40), 2),
])
def test_fwd_validation(L, kw, code):
    assert fwd(L, **kw) == code


def fwd_ws(L, ws=None, ws_bytes=None, **kw):
    p = dict(Bsz=1, N=8192, Hq=8, Hkv=2, d=128, scale=0.088, causal=1, dtype=B.UL_BF16)
    p.update(kw)
    need = L.ul_attn_fwd_workspace_bytes(p["Bsz"], p["N"], p["Hq"], p["Hkv"], p["d"], p["dtype"])
    ptrs = [addr(i) for i in range(5)]
    for i, n in enumerate(["q", "k", "v", "o", "lse"]):
        if n in p:
            ptrs[i] = p.pop(n)
    ws = addr(9) if ws is None else ws
    return L.ul_attn_fwd_ws(*ptrs, ws, need if ws_bytes is None else ws_bytes, p["Bsz"], p["N"],
                            p["Hq"], p["Hkv"], p["d"], p["scale"], p["causal"], p["dtype"], None)


def test_fwd_workspace_bytes(L):
    # N=8192, 8 query / 2 KV heads: 64-row query blocks, 128 per lane, the upper 64 split in
    # two; per split half 8 waves x 32 rows of d fp32 outputs plus (m, l)
    rows = 2 * 64 * 2 * 256
    assert L.ul_attn_fwd_workspace_bytes(1, 8192, 8, 2, 128, B.UL_BF16) == rows * (128 * 4 + 8)
    assert L.ul_attn_fwd_workspace_bytes(1, 8192, 8, 2, 64, B.UL_BF16) == rows * (64 * 4 + 8)
    # one KV head: 256 blocks of one lane still split
    assert L.ul_attn_fwd_workspace_bytes(1, 16384, 4, 1, 128, B.UL_BF16) == 128 * 2 * 256 * 520
    # MHA: 256-row query blocks; 4 lanes x 64 blocks split, 4 x 128 do not
    assert L.ul_attn_fwd_workspace_bytes(1, 16384, 4, 4, 128, B.UL_BF16) == 4 * 32 * 2 * 256 * 520
    assert L.ul_attn_fwd_workspace_bytes(1, 32768, 4, 4, 128, B.UL_BF16) == 0
    # more than 256 items (long N, more heads or batch), too few blocks, fp32, invalid sizes
    assert L.ul_attn_fwd_workspace_bytes(1, 65536, 8, 2, 128, B.UL_BF16) == 0
    assert L.ul_attn_fwd_workspace_bytes(1, 8193, 8, 2, 128, B.UL_BF16) == 0
    assert L.ul_attn_fwd_workspace_bytes(2, 8192, 8, 2, 128, B.UL_BF16) == 0
    assert L.ul_attn_fwd_workspace_bytes(1, 8192, 32, 8, 128, B.UL_BF16) == 0
    assert L.ul_attn_fwd_workspace_bytes(1, 960, 8, 2, 128, B.UL_BF16) == 0
    assert L.ul_attn_fwd_workspace_bytes(1, 1024, 8, 2, 128, B.UL_BF16) > 0
    assert L.ul_attn_fwd_workspace_bytes(1, 8192, 8, 2, 128, B.UL_F32) == 0
    assert L.ul_attn_fwd_workspace_bytes(1, 8192, 6, 4, 128, B.UL_BF16) == 0
    # the largest split: 256 items
    assert max(L.ul_attn_fwd_workspace_bytes(b, n, hq, hkv, 128, B.UL_BF16)
               for b in (1, 2, 4) for n in range(1024, 70000, 1024)
               for hq, hkv in ((8, 2), (4, 4), (4, 1), (2, 2))) <= 256 * 256 * 520


@pytest.mark.parametrize("kw,code", [
    (dict(q=ctypes.c_void_p(0)), 1),
    (dict(ws=ctypes.c_void_p(0)), 6), (dict(ws_bytes=16), 6),
    (dict(ws=ctypes.c_void_p(A + 9 * BIG + 8)), 5),
    (dict(ws=ctypes.c_void_p(A + 2 * BIG + 4096)), 7),   # workspace inside v
    (dict(ws=ctypes.c_void_p(A + 3 * BIG + 4096)), 7),   # workspace inside o
    (dict(ws=ctypes.c_void_p(A + 4 * BIG)), 7),          # workspace at lse
    (dict(Hq=6, Hkv=4), 3), (dict(d=80), 4), (dict(N=0), 2),
])
def test_fwd_ws_validation(L, kw, code):
    assert fwd_ws(L, **kw) == code


def bwd(L, ws_bytes=None, ws=None, stages=None, **kw):
    p = dict(Bsz=1, N=256, Hq=8, Hkv=2, d=128, scale=0.088, causal=1, dtype=B.UL_BF16)
    p.update(kw)
    need = L.ul_attn_bwd_workspace_bytes(p["Bsz"], p["N"], p["Hq"], p["Hkv"], p["d"], p["dtype"])
    ptrs = [addr(i) for i in range(9)]
    for i, n in enumerate(["q", "k", "v", "o", "dout", "lse", "dq", "dk", "dv"]):
        if n in p:
            ptrs[i] = p.pop(n)
    ws = addr(9) if ws is None else ws
    args = (*ptrs, ws, need if ws_bytes is None else ws_bytes, p["Bsz"], p["N"], p["Hq"], p["Hkv"],
            p["d"], p["scale"], p["causal"], p["dtype"], None)
    if stages is None:
        return L.ul_attn_bwd(*args)
    return L.ul_attn_bwd_stages(stages, *args)


def test_workspace_bytes(L):
    n = L.ul_attn_bwd_workspace_bytes(1, 65536, 8, 2, 128, B.UL_BF16)
    assert n >= 2 * 8 * 65536 * 4 and n % 256 == 0
    assert L.ul_attn_bwd_workspace_bytes(1, 0, 8, 2, 128, B.UL_BF16) == 0
    assert L.ul_attn_bwd_workspace_bytes(1, 8, 6, 4, 128, B.UL_BF16) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(dout=ctypes.c_void_p(0)), 1), (dict(dv=ctypes.c_void_p(0)), 1),
    (dict(ws=ctypes.c_void_p(0)), 6), (dict(ws_bytes=16), 6),
    (dict(N=-5), 2), (dict(Hq=3, Hkv=2), 3), (dict(d=80), 4),
    (dict(dk=ctypes.c_void_p(A + 7 * BIG + 8)), 5),
    (dict(dq=ctypes.c_void_p(A + 3 * BIG)), 7),   # dq aliases o
    (dict(dk=ctypes.c_void_p(A + 8 * BIG)), 7),   # dk aliases dv
    (dict(ws=ctypes.c_void_p(A + 6 * BIG + 256)), 7),  # workspace inside dq
])
def test_bwd_validation(L, kw, code):
    assert bwd(L, **kw) == code
    # every stage subset validates the same way
    for stages in (B.UL_BWD_PREP, B.UL_BWD_DQ, B.UL_BWD_DKDV, B.UL_BWD_ALL):
        assert bwd(L, stages=stages, **kw) == code


@pytest.mark.parametrize("stages", [0, 8, 9, -1])
def test_bwd_stage_mask_validation(L, stages):
    assert bwd(L, stages=stages) == 4


# ---- token-strided calls: a rank's head slice of world-layout buffers

W = 32 * 128  # token stride (elements) of a [N][32][128] world tensor


def fwd_s(L, q=None, k=None, v=None, o=None, lse=None, qs=W, ks=W, vs=W, os_=W, N=128, Hq=8,
          Hkv=2, d=128, dtype=B.UL_BF16):
    q = addr(0) if q is None else q
    k = addr(1) if k is None else k
    v = addr(2) if v is None else v
    o = addr(3) if o is None else o
    lse = addr(4) if lse is None else lse
    return L.ul_attn_fwd_strided(q, k, v, o, lse, 1, N, Hq, Hkv, d, qs, ks, vs, os_, 0.088, 1,
                                 dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=ctypes.c_void_p(0)), 1),
    (dict(N=0), 2), (dict(Hq=6, Hkv=4), 3), (dict(d=96), 4),
    (dict(qs=8 * 128 - 8), 2),            # shorter than the rank's heads
    (dict(ks=2 * 128 - 1), 2),
    (dict(os_=(1 << 23) + 8), 2),         # bf16: over 16 MiB per token
    (dict(qs=W + 4), 5),                  # 8 bytes: not a 16-byte multiple
    (dict(vs=W + 2, dtype=B.UL_F32), 5),
    (dict(q=ctypes.c_void_p(A + 8)), 5),
    # o shares q's stride and starts inside q's first row: same bytes
    (dict(o=ctypes.c_void_p(A + 64)), 7),
    # o a head slice that reaches into q's heads of the same buffer
    (dict(o=ctypes.c_void_p(A + 7 * 256)), 7),
    # o in the same buffer at a different stride whose span meets q's
    (dict(o=ctypes.c_void_p(A + 8 * 256), os_=2 * W), 7),
    # lse inside the span of q's rows
    (dict(lse=ctypes.c_void_p(A + 100 * W * 2 + 16)), 7),
])
def test_fwd_strided_validation(L, kw, code):
    assert fwd_s(L, **kw) == code


def bwd_s(L, strides=None, **kw):
    p = dict(Bsz=1, N=256, Hq=8, Hkv=2, d=128, scale=0.088, causal=1, dtype=B.UL_BF16)
    p.update(kw)
    need = L.ul_attn_bwd_workspace_bytes(p["Bsz"], p["N"], p["Hq"], p["Hkv"], p["d"], p["dtype"])
    ptrs = [addr(i) for i in range(9)]
    for i, n in enumerate(["q", "k", "v", "o", "dout", "lse", "dq", "dk", "dv"]):
        if n in p:
            ptrs[i] = p.pop(n)
    ts = [W] * 8 if strides is None else strides
    return L.ul_attn_bwd_strided(*ptrs, addr(9), need, p["Bsz"], p["N"], p["Hq"], p["Hkv"], p["d"],
                                 *ts, p["scale"], p["causal"], p["dtype"], None)


PK = (8 + 2 + 2) * 128  # packed [N][Hq + 2 Hkv][128] gradient buffer


@pytest.mark.parametrize("kw,code", [
    (dict(dv=ctypes.c_void_p(0)), 1),
    (dict(strides=[W, W, W, W, W, W, 255, W]), 2),
    (dict(strides=[W, W, W, W, W + 4, W, W, W]), 5),
    # dk's two heads overlap dq's last head inside one packed buffer
    (dict(dq=ctypes.c_void_p(A + 6 * BIG), dk=ctypes.c_void_p(A + 6 * BIG + 7 * 256),
          dv=ctypes.c_void_p(A + 6 * BIG + 10 * 256), strides=[W, W, W, W, W, PK, PK, PK]), 7),
    # dv written over o
    (dict(dv=ctypes.c_void_p(A + 3 * BIG + 256)), 7),
])
def test_bwd_strided_validation(L, kw, code):
    assert bwd_s(L, **kw) == code


# ---- packed variable-length sequences (the table lives at addr(10))


def fwd_v(L, q=None, o=None, lse=None, cu=None, n=3, T=1000, max_len=600, Hq=8, Hkv=2, d=128,
          dtype=B.UL_BF16):
    q = addr(0) if q is None else q
    o = addr(3) if o is None else o
    lse = addr(4) if lse is None else lse
    cu = addr(10) if cu is None else cu
    return L.ul_attn_fwd_varlen(q, addr(1), addr(2), o, lse, cu, n, T, max_len, Hq, Hkv, d, 0.088,
                                1, dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(cu=ctypes.c_void_p(0)), 1), (dict(q=ctypes.c_void_p(0)), 1),
    (dict(n=0), 2), (dict(max_len=0), 2), (dict(max_len=1001), 2), (dict(T=0), 2),
    (dict(T=1 << 31, max_len=5), 2),
    (dict(Hq=6, Hkv=4), 3), (dict(d=32), 4),
    (dict(cu=ctypes.c_void_p(A + 10 * BIG + 2)), 5),
    (dict(lse=ctypes.c_void_p(A + 10 * BIG)), 7),       # lse over the table
    (dict(o=ctypes.c_void_p(A + 10 * BIG - 256)), 7),   # o's last row reaches the table
])
def test_fwd_varlen_validation(L, kw, code):
    assert fwd_v(L, **kw) == code


def bwd_v(L, ws_bytes=None, n=3, T=1000, max_len=600, **kw):
    need = L.ul_attn_bwd_workspace_bytes(1, T, 8, 2, 128, B.UL_BF16)
    ptrs = [addr(i) for i in range(9)]
    for i, nm in enumerate(["q", "k", "v", "o", "dout", "lse", "dq", "dk", "dv"]):
        if nm in kw:
            ptrs[i] = kw.pop(nm)
    cu = kw.pop("cu", addr(10))
    return L.ul_attn_bwd_varlen(*ptrs, addr(9), need if ws_bytes is None else ws_bytes, cu, n, T,
                                max_len, 8, 2, 128, 0.088, 1, B.UL_BF16, None)


@pytest.mark.parametrize("kw,code", [
    (dict(cu=ctypes.c_void_p(0)), 1), (dict(dv=ctypes.c_void_p(0)), 1),
    (dict(n=-1), 2), (dict(max_len=2000), 2),
    (dict(ws_bytes=16), 6),
    (dict(cu=ctypes.c_void_p(A + 10 * BIG + 1)), 5),
    (dict(dq=ctypes.c_void_p(A + 10 * BIG - 1024)), 7),  # dq reaches the table
])
def test_bwd_varlen_validation(L, kw, code):
    assert bwd_v(L, **kw) == code


def test_varlen_workspace_is_the_single_sequence_size(L):
    assert L.ul_attn_bwd_workspace_bytes(1, 1000, 8, 2, 128, B.UL_BF16) >= 2 * 8 * 1000 * 4


@pytest.mark.parametrize("fn", ["ul_relayout_s2h", "ul_relayout_h2s"])
@pytest.mark.parametrize("args,code", [
    ((0, 1, 3, 64, 32, 128, 4, 1), 1),
    ((A, A + BIG, 0, 64, 32, 128, 4, 1), 2),
    ((A, A + BIG, 3, 64, 32, 0, 4, 1), 2),
    ((A, A + BIG, 3, 64, 30, 128, 4, 1), 3),   # H % P
    ((A, A + BIG, 3, 66, 32, 128, 4, 1), 3),   # N % P
    ((A, A + BIG, 3, 64, 32, 128, 0, 1), 3),
    ((A, A + BIG, 3, 64, 32, 128, 64, 1), 3),  # P > H: num_heads >= sp_size violated
    ((A, A + BIG, 3, 64, 32, 128, 4, 5), 4),
    ((A, A + 4096, 3, 64, 32, 128, 4, 1), 7),  # ranges overlap
])
def test_relayout_validation(L, fn, args, code):
    a = [ctypes.c_void_p(args[0]), ctypes.c_void_p(args[1]), *args[2:], None]
    assert getattr(L, fn)(*a) == code


def test_binding_raises_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(B, "LIB_PATH", tmp_path / "missing.so")
    monkeypatch.setattr(B, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        B.lib()


@pytest.mark.parametrize("fn", ["ul_relayout_s2h_heads", "ul_relayout_h2s_heads"])
@pytest.mark.parametrize("args,code", [
    ((0, A + BIG, 3, 64, 32, 128, 4, 0, 4, 1), 1),
    ((A, A + BIG, 0, 64, 32, 128, 4, 0, 4, 1), 2),
    ((A, A + BIG, 3, 64, 30, 128, 4, 0, 4, 1), 3),   # H % P
    ((A, A + BIG, 3, 66, 32, 128, 4, 0, 4, 1), 3),   # N % P
    ((A, A + BIG, 3, 64, 32, 128, 4, -1, 4, 1), 2),  # h0 < 0
    ((A, A + BIG, 3, 64, 32, 128, 4, 0, 0, 1), 2),   # empty chunk
    ((A, A + BIG, 3, 64, 32, 128, 4, 5, 4, 1), 2),   # past the rank's 8 heads
    ((A, A + BIG, 3, 64, 32, 128, 4, 0, 4, 9), 4),
    ((A, A + 4096, 3, 64, 32, 128, 4, 0, 4, 1), 7),  # ranges overlap
])
def test_relayout_heads_validation(L, fn, args, code):
    a = [ctypes.c_void_p(args[0]), ctypes.c_void_p(args[1]), *args[2:], None]
    assert getattr(L, fn)(*a) == code


def noalloc(L, **kw):
    p = dict(Bsz=1, N=256, Hq=8, Hkv=2, d=128, scale=0.088, causal=1, dtype=B.UL_BF16)
    p.update(kw)
    ptrs = [kw.get(n, addr(i)) for i, n in enumerate(["q", "k", "v", "o", "dout", "lse", "dq", "dk",
                                                      "dv"])]
    return L.ul_attn_bwd_noalloc(*ptrs, p["Bsz"], p["N"], p["Hq"], p["Hkv"], p["d"], p["scale"],
                                 p["causal"], p["dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=ctypes.c_void_p(0)), 1), (dict(dv=ctypes.c_void_p(0)), 1),
    (dict(N=0), 2), (dict(scale=0.0), 2), (dict(Hq=6, Hkv=4), 3), (dict(d=96), 4),
    (dict(dq=ctypes.c_void_p(A + 8)), 5),
    (dict(dk=ctypes.c_void_p(A + 64)), 7),            # dk overlaps q
    (dict(N=1 << 23), 9), (dict(Bsz=9, N=1 << 20, Hq=4, Hkv=1), 9),  # beyond the fixed scratch
    # bf16 statistics are addressed with 32-bit offsets: N < 2^30 (fp32 is not limited)
    (dict(N=1 << 30, Hq=1, Hkv=1, d=64), 2), (dict(N=1 << 30, Hq=1, Hkv=1, d=64, dtype=B.UL_F32), 9),
])
def test_noalloc_validation(L, kw, code):
    """ul_attn_bwd_noalloc validates before touching the runtime; a problem whose statistics
    exceed the fixed scratch is rejected with UL_ERR_SCRATCH."""
    assert noalloc(L, **kw) == code


def test_noalloc_scratch_limit_matches_workspace_size(L):
    """The largest accepted problem is the one whose backward workspace fits the scratch."""
    rows_max = B.NOALLOC_SCRATCH_BYTES // 8
    assert L.ul_attn_bwd_workspace_bytes(1, rows_max // 4, 4, 1, 128, B.UL_BF16) <= B.NOALLOC_SCRATCH_BYTES
    assert L.ul_attn_bwd_workspace_bytes(1, rows_max // 4 + 64, 4, 1, 128, B.UL_BF16) > B.NOALLOC_SCRATCH_BYTES
    assert noalloc(L, N=rows_max // 4 + 64, Hq=4, Hkv=1) == 9
