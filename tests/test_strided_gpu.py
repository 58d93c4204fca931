"""GPU parity of the token-strided entry points (ul_attn_fwd_strided, ul_attn_bwd_strided).

A rank's attention reads its head slice straight out of sequence-sharded world tensors and
writes O, dQ, dK and dV straight into world-layout buffers, so that no relayout pass runs on
either side of it.  Heads are independent and the kernels do the same per-(head, block) work
whatever the strides, so every check here is bit-identical:

* against the relayout path (s2h, dense per-rank attention, h2s), for separate world Q/K/V
  tensors and for a packed [N][P*(Hq + 2 Hkv)][d] QKV tensor whose gradient is written into
  one packed buffer (disjoint head slices of one allocation);
* heads of a world buffer outside the rank's slice are left untouched (NaN poison);
* at the metric shape (N = 65536, world 32 query / 8 KV heads, P = 4) the last rank's
  strided call equals the dense call on contiguous copies of its slices.

Each rank's strided results are also compared element by element with the float64 oracle
on that rank's head slice (ragged N, GQA, causal and full, bf16 and fp32, separate world
tensors and a packed QKV tensor), at the path's tolerances.
"""

import math

import numpy as np
import pytest

from oracle import attention as OA
from ulysses_sequence_parallelism_attn_amd import synth

from . import helpers as H

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _B():
    from ulysses_sequence_parallelism_attn_amd import binding

    return binding


def _bits(t):
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


def _same(a, b, what):
    assert torch.equal(_bits(a), _bits(b)), what


def _world(shape, dtype, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    x32 = rng.standard_normal(shape).astype(np.float32)
    return H.to_device(synth.encode(x32, dtype), dtype)


def _relayout_path(Qw, Kw, Vw, dOw, P, scale):
    """Per-rank dense attention on s2h outputs, results h2s'd back to world layout."""
    B = _B()
    yq, yk, yv, ydo = (B.relayout_s2h(x, P) for x in (Qw, Kw, Vw, dOw))  # [1, P, N, H/P, d]
    outs = {n: torch.empty_like(y) for n, y in (("o", yq), ("dq", yq), ("dk", yk), ("dv", yv))}
    lses = []
    for r in range(P):
        q, k, v, do = (y[0, r][None].contiguous() for y in (yq, yk, yv, ydo))
        o, lse = B.attn_fwd(q, k, v, scale, True, split=False)  # the strided call's rounding
        dq, dk, dv = B.attn_bwd(q, k, v, o, do, lse, scale, True)
        for n, t in (("o", o), ("dq", dq), ("dk", dk), ("dv", dv)):
            outs[n][0, r] = t[0]
        lses.append(lse)
    back = {n: B.relayout_h2s(y) for n, y in outs.items()}
    return back, lses


@pytest.mark.parametrize("dtype,N,Hq,Hkv,d,P", [
    ("bf16", 700, 4, 2, 128, 2),
    ("bf16", 332, 8, 2, 64, 4),
    ("f32", 200, 2, 1, 64, 2),
])
def test_fused_relayout_matches_relayout_path(dtype, N, Hq, Hkv, d, P):
    """Separate world Q, K, V, dO, O, dQ, dK, dV tensors; each rank's head slice is a view."""
    B = _B()
    print(f"[strided] separate world tensors {dtype} N={N} Hq={Hq} Hkv={Hkv} d={d} P={P}", flush=True)
    scale = 1.0 / math.sqrt(d)
    Qw = _world((1, N, P * Hq, d), dtype, 901)
    Kw = _world((1, N, P * Hkv, d), dtype, 902)
    Vw = _world((1, N, P * Hkv, d), dtype, 903)
    dOw = _world((1, N, P * Hq, d), dtype, 904)
    ref, ref_lse = _relayout_path(Qw[0:1], Kw[0:1], Vw[0:1], dOw[0:1], P, scale)

    Ow = torch.full_like(Qw, float("nan"))
    dQw = torch.full_like(Qw, float("nan"))
    dKw = torch.full_like(Kw, float("nan"))
    dVw = torch.full_like(Vw, float("nan"))
    for r in range(P):
        qs, ks = slice(r * Hq, (r + 1) * Hq), slice(r * Hkv, (r + 1) * Hkv)
        q, k, v, do = Qw[:, :, qs], Kw[:, :, ks], Vw[:, :, ks], dOw[:, :, qs]
        o, lse = B.attn_fwd(q, k, v, scale, True, out=Ow[:, :, qs])
        B.attn_bwd(q, k, v, Ow[:, :, qs], do, lse, scale, True, dq=dQw[:, :, qs], dk=dKw[:, :, ks],
                   dv=dVw[:, :, ks])
        torch.cuda.synchronize()
        _same(lse, ref_lse[r], f"lse rank {r}")
        if r == 0 and P > 1:  # the other ranks' heads are still untouched
            assert torch.isnan(Ow[:, :, Hq:]).all() and torch.isnan(dQw[:, :, Hq:]).all()
            assert torch.isnan(dKw[:, :, Hkv:]).all() and torch.isnan(dVw[:, :, Hkv:]).all()
    for n, x in (("o", Ow), ("dq", dQw), ("dk", dKw), ("dv", dVw)):
        _same(x, ref[n], n)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_fused_relayout_packed_qkv(dtype):
    """Q, K and V are head slices of one packed [N][P*(Hq + 2 Hkv)][d] tensor and dQ, dK, dV
    are written into one packed gradient buffer of the same layout."""
    B = _B()
    N, Hq, Hkv, P = 518, 4, 1, 2
    d = 128 if dtype == "bf16" else 64
    print(f"[strided] packed qkv {dtype} N={N} Hq={Hq} Hkv={Hkv} d={d} P={P}", flush=True)
    scale = 1.0 / math.sqrt(d)
    Hw, Kw_ = P * Hq, P * Hkv
    X = _world((1, N, Hw + 2 * Kw_, d), dtype, 911)  # [q heads | k heads | v heads]
    dOw = _world((1, N, Hw, d), dtype, 914)
    Qw, Kw, Vw = X[:, :, :Hw], X[:, :, Hw:Hw + Kw_], X[:, :, Hw + Kw_:]
    ref, _ = _relayout_path(Qw.contiguous(), Kw.contiguous(), Vw.contiguous(), dOw, P, scale)

    Ow = torch.full_like(dOw, float("nan"))
    dX = torch.full_like(X, float("nan"))
    for r in range(P):
        qs = slice(r * Hq, (r + 1) * Hq)
        ks = slice(Hw + r * Hkv, Hw + (r + 1) * Hkv)
        vs = slice(Hw + Kw_ + r * Hkv, Hw + Kw_ + (r + 1) * Hkv)
        q, k, v = X[:, :, qs], X[:, :, ks], X[:, :, vs]
        o, lse = B.attn_fwd(q, k, v, scale, True, out=Ow[:, :, qs])
        B.attn_bwd(q, k, v, Ow[:, :, qs], dOw[:, :, qs], lse, scale, True, dq=dX[:, :, qs],
                   dk=dX[:, :, ks], dv=dX[:, :, vs])
    torch.cuda.synchronize()
    _same(Ow, ref["o"], "o")
    _same(dX[:, :, :Hw], ref["dq"], "dq")
    _same(dX[:, :, Hw:Hw + Kw_], ref["dk"], "dk")
    _same(dX[:, :, Hw + Kw_:], ref["dv"], "dv")


def test_fused_relayout_metric_shape_last_rank():
    """N = 65536, world 32 query / 8 KV heads, P = 4: rank 3 reads its 8 query / 2 KV heads
    at world token strides (the largest head offsets) and matches the dense call."""
    B = _B()
    N, P, Hq, Hkv, d = 65536, 4, 8, 2, 128
    r = P - 1
    print(f"[strided] metric shape N={N} world {P * Hq}/{P * Hkv} rank {r}", flush=True)
    scale = 1.0 / math.sqrt(d)
    g = torch.Generator(device="cuda").manual_seed(921)
    Qw = torch.randn((1, N, P * Hq, d), generator=g, device="cuda").to(torch.bfloat16)
    Kw = torch.randn((1, N, P * Hkv, d), generator=g, device="cuda").to(torch.bfloat16)
    Vw = torch.randn((1, N, P * Hkv, d), generator=g, device="cuda").to(torch.bfloat16)
    dOw = torch.randn((1, N, P * Hq, d), generator=g, device="cuda").to(torch.bfloat16)
    qs, ks = slice(r * Hq, (r + 1) * Hq), slice(r * Hkv, (r + 1) * Hkv)
    q, k, v, do = Qw[:, :, qs], Kw[:, :, ks], Vw[:, :, ks], dOw[:, :, qs]
    Ow = torch.full_like(Qw, float("nan"))
    dQw = torch.full_like(Qw, float("nan"))
    dKw = torch.full_like(Kw, float("nan"))
    dVw = torch.full_like(Vw, float("nan"))
    o_s, lse_s = B.attn_fwd(q, k, v, scale, True, out=Ow[:, :, qs])
    B.attn_bwd(q, k, v, Ow[:, :, qs], do, lse_s, scale, True, dq=dQw[:, :, qs], dk=dKw[:, :, ks],
               dv=dVw[:, :, ks])
    qc, kc, vc, doc = (t.contiguous() for t in (q, k, v, do))
    o_d, lse_d = B.attn_fwd(qc, kc, vc, scale, True, split=False)
    dq_d, dk_d, dv_d = B.attn_bwd(qc, kc, vc, o_d, doc, lse_d, scale, True)
    torch.cuda.synchronize()
    _same(lse_s, lse_d, "lse")
    _same(Ow[:, :, qs], o_d, "o")
    _same(dQw[:, :, qs], dq_d, "dq")
    _same(dKw[:, :, ks], dk_d, "dk")
    _same(dVw[:, :, ks], dv_d, "dv")
    assert torch.isnan(Ow[:, :, : r * Hq]).all() and torch.isnan(dKw[:, :, : r * Hkv]).all()


# ---------------------------------------------------------------------------- against the oracle


def _world_host(shape, dtype, seed):
    """Stored world tensor (bf16 bits or float32) from seeded normals."""
    return synth.encode(synth.normal_f32(shape, seed), dtype)


def _check_rank(got: dict, st: dict, dtype, scale, causal, label):
    """Compare one rank's strided results with the float64 oracle on its head slice."""
    w = {n: OA.widen(a, dtype) for n, a in st.items()}
    dq, dk, dv, o, lse = OA.attn_bwd(w["q"], w["k"], w["v"], w["dout"], scale, causal)
    ref = {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}
    g = {n: H.to_f64(t) for n, t in got.items()}
    for n, x in g.items():
        assert np.isfinite(x).all(), f"{label}: {n} has non-finite values"
    if dtype == "f32":
        for n in ("o", "lse", "dq", "dk", "dv"):
            H.check_max_abs(g[n], ref[n], H.TOL_F32, f"{label} {n}")
    else:
        H.check_o_bf16(g["o"], ref["o"], f"{label} O")
        H.check_max_abs(g["lse"], ref["lse"], H.TOL_BF16_LSE, f"{label} lse")
        for n in ("dq", "dk", "dv"):
            H.check_rel_l2(g[n], ref[n], H.TOL_BF16_GRAD_RL2, f"{label} {n}")


@pytest.mark.parametrize("dtype,N,Hq,Hkv,d,P,causal", [
    ("bf16", 700, 4, 2, 128, 2, True),
    ("bf16", 332, 8, 2, 64, 4, True),
    ("bf16", 300, 4, 1, 128, 2, False),
    ("f32", 200, 2, 1, 64, 2, True),
    ("f32", 150, 4, 2, 128, 2, False),
])
def test_strided_matches_oracle(dtype, N, Hq, Hkv, d, P, causal):
    """Every rank reads its head slice from world tensors [1, N, P*H, d] at the world token
    stride and writes O, dQ, dK, dV into world buffers; each slice is compared with the
    oracle on that slice."""
    B = _B()
    label = f"strided-vs-oracle {dtype} N={N} {Hq}q{Hkv}kv d={d} P={P} {'causal' if causal else 'full'}"
    print(f"[strided] {label}", flush=True)
    scale = 1.0 / math.sqrt(d)
    host = {"q": _world_host((1, N, P * Hq, d), dtype, 931), "k": _world_host((1, N, P * Hkv, d), dtype, 932),
            "v": _world_host((1, N, P * Hkv, d), dtype, 933),
            "dout": _world_host((1, N, P * Hq, d), dtype, 934)}
    Qw, Kw, Vw, dOw = (H.to_device(host[n], dtype) for n in ("q", "k", "v", "dout"))
    Ow, dQw = torch.full_like(Qw, float("nan")), torch.full_like(Qw, float("nan"))
    dKw, dVw = torch.full_like(Kw, float("nan")), torch.full_like(Vw, float("nan"))
    for r in range(P):
        qs, ks = slice(r * Hq, (r + 1) * Hq), slice(r * Hkv, (r + 1) * Hkv)
        q, k, v, do = Qw[:, :, qs], Kw[:, :, ks], Vw[:, :, ks], dOw[:, :, qs]
        assert q.stride(1) == P * Hq * d and not q.is_contiguous()
        _, lse = B.attn_fwd(q, k, v, scale, causal, out=Ow[:, :, qs])
        B.attn_bwd(q, k, v, Ow[:, :, qs], do, lse, scale, causal, dq=dQw[:, :, qs],
                   dk=dKw[:, :, ks], dv=dVw[:, :, ks])
        torch.cuda.synchronize()
        st = {"q": host["q"][:, :, qs], "k": host["k"][:, :, ks], "v": host["v"][:, :, ks],
              "dout": host["dout"][:, :, qs]}
        got = {"o": Ow[:, :, qs], "lse": lse, "dq": dQw[:, :, qs], "dk": dKw[:, :, ks],
               "dv": dVw[:, :, ks]}
        _check_rank(got, st, dtype, scale, causal, f"{label} rank {r}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_strided_packed_qkv_matches_oracle(dtype):
    """Q, K, V as head slices of one packed [1, N, P*(Hq + 2 Hkv), d] tensor, gradients into
    one packed buffer: each rank's results against the oracle."""
    B = _B()
    N, Hq, Hkv, P = 389, 4, 2, 2
    d = 128 if dtype == "bf16" else 64
    print(f"[strided] packed qkv vs oracle {dtype} N={N}", flush=True)
    scale = 1.0 / math.sqrt(d)
    Hw, Kw_ = P * Hq, P * Hkv
    Xh = _world_host((1, N, Hw + 2 * Kw_, d), dtype, 941)
    dOh = _world_host((1, N, Hw, d), dtype, 944)
    X, dOw = H.to_device(Xh, dtype), H.to_device(dOh, dtype)
    Ow = torch.full_like(dOw, float("nan"))
    dX = torch.full_like(X, float("nan"))
    for r in range(P):
        qs = slice(r * Hq, (r + 1) * Hq)
        ks = slice(Hw + r * Hkv, Hw + (r + 1) * Hkv)
        vs = slice(Hw + Kw_ + r * Hkv, Hw + Kw_ + (r + 1) * Hkv)
        q, k, v = X[:, :, qs], X[:, :, ks], X[:, :, vs]
        _, lse = B.attn_fwd(q, k, v, scale, True, out=Ow[:, :, qs])
        B.attn_bwd(q, k, v, Ow[:, :, qs], dOw[:, :, qs], lse, scale, True, dq=dX[:, :, qs],
                   dk=dX[:, :, ks], dv=dX[:, :, vs])
        torch.cuda.synchronize()
        st = {"q": Xh[:, :, qs], "k": Xh[:, :, ks], "v": Xh[:, :, vs], "dout": dOh[:, :, qs]}
        got = {"o": Ow[:, :, qs], "lse": lse, "dq": dX[:, :, qs], "dk": dX[:, :, ks], "dv": dX[:, :, vs]}
        _check_rank(got, st, dtype, scale, True, f"packed {dtype} rank {r}")
