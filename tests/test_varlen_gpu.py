"""GPU parity of the packed variable-length entry points (ul_attn_fwd_varlen, ul_attn_bwd_varlen).

* Element by element against the float64 varlen oracle (oracle/varlen.py) for ragged length
  mixes with empty, one-token, tile-aligned and unaligned sequences: bf16 (GQA 8/2, d = 128,
  causal; 4/1, d = 64, non-causal) and fp32 (d = 64).  Outputs are NaN-poisoned first, so an
  unwritten element fails.
* At the metric size (65536 packed tokens of a seeded length mix, 8q/2kv, d = 128, bf16), each
  sequence's results are bit-identical to the plain (B = 1) call on that sequence alone: the
  kernels do the same per-(head, block) work for a sequence wherever it sits in the packed
  axis, and the plain path is pinned to the oracle by test_attn_gpu.py.
* Tokens that no sequence covers stay unwritten.
"""

import math

import numpy as np
import pytest

from oracle import attention as OA
from oracle import varlen as OV
from ulysses_sequence_parallelism_attn_amd import synth

from . import helpers as H

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _B():
    from ulysses_sequence_parallelism_attn_amd import binding

    return binding


def _bits(t):
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


def _inputs(T, Hq, Hkv, d, dtype, seed):
    st = synth.custom_inputs(1, T, Hq, Hkv, d, dtype, seed)
    return {n: a[0] for n, a in st.items()}  # [T, H, d]


def _run(st, dtype, cu_np, max_len, scale, causal):
    B = _B()
    q, k, v, do = (H.to_device(st[n], dtype) for n in ("q", "k", "v", "dout"))
    cu = torch.from_numpy(cu_np).cuda()
    T, Hq = q.shape[0], q.shape[1]
    o = torch.full_like(q, float("nan"))
    lse = torch.full((Hq, T), float("nan"), device="cuda")
    B.attn_fwd_varlen(q, k, v, cu, max_len, scale, causal, out=o, lse=lse)
    dq = torch.full_like(q, float("nan"))
    dk = torch.full_like(k, float("nan"))
    dv = torch.full_like(v, float("nan"))
    B.attn_bwd_varlen(q, k, v, o, do, lse, cu, max_len, scale, causal, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return {"q": q, "k": k, "v": v, "dout": do, "o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}


CASES = [
    ("bf16", (1, 63, 0, 64, 65, 200, 17, 512, 129), 8, 2, 128, True),
    ("bf16", (100, 1, 33, 250, 64), 4, 1, 64, False),
    ("f32", (1, 31, 64, 100, 0, 7), 4, 2, 64, True),
]


@pytest.mark.parametrize("dtype,lengths,Hq,Hkv,d,causal", CASES)
def test_varlen_full_parity(dtype, lengths, Hq, Hkv, d, causal):
    T = int(sum(lengths))
    print(f"[varlen] {dtype} lengths={lengths} Hq={Hq} Hkv={Hkv} d={d} causal={causal}", flush=True)
    st = _inputs(T, Hq, Hkv, d, dtype, seed=400 + T)
    cu = synth.cu_seqlens(lengths)
    scale = 1.0 / math.sqrt(d)
    gpu = _run(st, dtype, cu, max(lengths), scale, causal)
    w = H.widen_inputs(st, dtype)
    dq, dk, dv, o, lse = OV.attn_varlen_bwd(w["q"], w["k"], w["v"], w["dout"], cu, scale, causal)
    got = {n: H.to_f64(gpu[n]) for n in ("o", "lse", "dq", "dk", "dv")}
    for n, x in got.items():
        assert np.isfinite(x).all(), f"{n}: unwritten or non-finite elements"
    if dtype == "f32":
        for n, ref in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv)):
            H.check_max_abs(got[n], ref, H.TOL_F32, f"varlen {n}")
    else:
        H.check_o_bf16(got["o"], o, "varlen O")
        H.check_max_abs(got["lse"], lse, H.TOL_BF16_LSE, "varlen lse")
        for n, ref in (("dq", dq), ("dk", dk), ("dv", dv)):
            H.check_rel_l2(got[n], ref, H.TOL_BF16_GRAD_RL2, f"varlen {n}")
            # every sequence on its own, not just the total (a one-token sequence has dQ = dK = 0
            # exactly, so its float64 reference is rounding noise and is skipped)
            for s in range(len(lengths)):
                a, b = cu[s], cu[s + 1]
                if b > a and np.linalg.norm(ref[a:b]) > 1e-6 * np.linalg.norm(ref):
                    H.check_rel_l2(got[n][a:b], ref[a:b], H.TOL_BF16_GRAD_RL2, f"varlen {n} seq {s}")


def test_varlen_metric_size_matches_per_sequence_calls():
    """65536 packed tokens of the seeded length mix equal the plain call on each sequence
    (its forward without the key-range split, which packed calls do not take): O, lse and
    dQ bit for bit.  dK and dV to 1e-3 relative L2: a plain call on a sequence
    this short runs its longest key blocks one query head at a time and sums the heads'
    fp32 partials afterwards, a different summation order from the packed call's (which the
    float64 oracle checks on its own in test_varlen_full_parity)."""
    B = _B()
    lengths = synth.length_mix(65536, seed=3008)
    cu = synth.cu_seqlens(lengths)
    T, Hq, Hkv, d = int(cu[-1]), 8, 2, 128
    print(f"[varlen] metric size: {len(lengths)} sequences, max {lengths.max()}", flush=True)
    scale = 1.0 / math.sqrt(d)
    g = torch.Generator(device="cuda").manual_seed(3009)
    q = torch.randn((T, Hq, d), generator=g, device="cuda").to(torch.bfloat16)
    k = torch.randn((T, Hkv, d), generator=g, device="cuda").to(torch.bfloat16)
    v = torch.randn((T, Hkv, d), generator=g, device="cuda").to(torch.bfloat16)
    do = torch.randn((T, Hq, d), generator=g, device="cuda").to(torch.bfloat16)
    cu_t = torch.from_numpy(cu).cuda()
    o, lse = B.attn_fwd_varlen(q, k, v, cu_t, int(lengths.max()), scale, True)
    dq, dk, dv = B.attn_bwd_varlen(q, k, v, o, do, lse, cu_t, int(lengths.max()), scale, True)
    torch.cuda.synchronize()
    for s in range(len(lengths)):
        a, b = int(cu[s]), int(cu[s + 1])
        sl = lambda t: t[a:b][None].contiguous()
        o1, l1 = B.attn_fwd(sl(q), sl(k), sl(v), scale, True, split=False)
        dq1, dk1, dv1 = B.attn_bwd(sl(q), sl(k), sl(v), o1, sl(do), l1, scale, True)
        torch.cuda.synchronize()
        for name, x, r in (("o", o[a:b], o1[0]), ("dq", dq[a:b], dq1[0]), ("lse", lse[:, a:b], l1[0])):
            assert torch.equal(_bits(x.contiguous()), _bits(r.contiguous())), f"seq {s} {name}"
        for name, x, r in (("dk", dk[a:b], dk1[0]), ("dv", dv[a:b], dv1[0])):
            x32, r32 = x.float(), r.float()
            rel = float((x32 - r32).norm() / r32.norm())
            assert rel <= 1e-3, f"seq {s} {name}: rel-L2 {rel:.3g} against the plain call"


def test_varlen_uncovered_tokens_stay_unwritten():
    """A table that ends before the last token (and starts past the first) leaves the
    uncovered tokens as they were, and the covered ones equal the same table shifted."""
    B = _B()
    T, Hq, Hkv, d = 300, 4, 2, 128
    st = _inputs(T, Hq, Hkv, d, "bf16", seed=450)
    q, k, v, do = (H.to_device(st[n], "bf16") for n in ("q", "k", "v", "dout"))
    cu = torch.tensor([20, 20, 150, 260], dtype=torch.int32, device="cuda")
    o = torch.full_like(q, float("nan"))
    lse = torch.full((Hq, T), float("nan"), device="cuda")
    B.attn_fwd_varlen(q, k, v, cu, 130, None, True, out=o, lse=lse)
    dq = torch.full_like(q, float("nan"))
    dk = torch.full_like(k, float("nan"))
    dv = torch.full_like(v, float("nan"))
    B.attn_bwd_varlen(q, k, v, o, do, lse, cu, 130, None, True, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    for t in (o, dq, dk, dv):
        assert torch.isnan(t[:20]).all() and torch.isnan(t[260:]).all()
        assert not torch.isnan(t[20:260]).any()
    assert torch.isnan(lse[:, :20]).all() and torch.isnan(lse[:, 260:]).all()
    # the same sequences packed from token 0
    sub = lambda t: t[20:260].contiguous()
    cu0 = torch.tensor([0, 0, 130, 240], dtype=torch.int32, device="cuda")
    o2, l2 = B.attn_fwd_varlen(sub(q), sub(k), sub(v), cu0, 130)
    dq2, dk2, dv2 = B.attn_bwd_varlen(sub(q), sub(k), sub(v), o2, sub(do), l2, cu0, 130)
    torch.cuda.synchronize()
    for x, r in ((o[20:260], o2), (dq[20:260], dq2), (dk[20:260], dk2), (dv[20:260], dv2)):
        assert torch.equal(_bits(x.contiguous()), _bits(r))
    assert torch.equal(lse[:, 20:260].contiguous(), l2)
