"""GPU parity of ul_attn_fwd / ul_attn_bwd against the float64 oracle.

* Full comparison (every row, every gradient element) for the tiny fp32 workload, the
  N = 8192 bf16 rank, and a sweep of ragged / GQA / head-dim / non-causal / batched shapes
  that span several tiles and a ragged tail.
* At N = 65536, 98304 and 1048576 (the launch configuration the benchmark times): 512
  seeded rows per head plus fixed edge rows for O, lse and dQ; dK and dV at 512 seeded keys
  per KV head drawn over the whole sequence plus keys 0, 1, 127, 128 and N/2 (over the last
  16384 positions at N = 1048576), against values the oracle stored for exactly these inputs
  (tests/golden/make_dkdv_samples.py; a key near the start needs the statistics of every
  query row, minutes of fp64 CPU work); the last 64 keys against the oracle run here; and
  exact gradient identities on the full tensors.
* Determinism, full coverage of the outputs (NaN poison), causality and the Ulysses
  composition (per-rank attention on the relayout equals attention over all heads).
"""

import math
import os

import numpy as np
import pytest

from oracle import attention as OA
from oracle import native as ON
from ulysses_sequence_parallelism_attn_amd import synth

from . import helpers as H

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _B():
    from ulysses_sequence_parallelism_attn_amd import binding

    return binding


def _run_gpu(st, dtype, scale, causal, poison=True):
    B = _B()
    q, k, v, do = (H.to_device(st[n], dtype) for n in ("q", "k", "v", "dout"))
    o = torch.full_like(q, float("nan")) if poison else None
    lse = torch.full((q.shape[0], q.shape[2], q.shape[1]), float("nan"), device="cuda") if poison else None
    o, lse = B.attn_fwd(q, k, v, scale, causal, out=o, lse=lse)
    dq = torch.full_like(q, float("nan")) if poison else None
    dk = torch.full_like(k, float("nan")) if poison else None
    dv = torch.full_like(v, float("nan")) if poison else None
    dq, dk, dv = B.attn_bwd(q, k, v, o, do, lse, scale, causal, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return {"q": q, "k": k, "v": v, "dout": do, "o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}


def _compare_full(gpu, ref, dtype, label):
    o, lse, dq, dk, dv = (H.to_f64(gpu[n]) for n in ("o", "lse", "dq", "dk", "dv"))
    for n, x in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv)):
        assert np.isfinite(x).all(), f"{label}: {n} has non-finite values (unwritten elements?)"
    if dtype == "f32":
        H.check_max_abs(o, ref["o"], H.TOL_F32, f"{label} O")
        H.check_max_abs(lse, ref["lse"], H.TOL_F32, f"{label} lse")
        H.check_max_abs(dq, ref["dq"], H.TOL_F32, f"{label} dQ")
        H.check_max_abs(dk, ref["dk"], H.TOL_F32, f"{label} dK")
        H.check_max_abs(dv, ref["dv"], H.TOL_F32, f"{label} dV")
    else:
        H.check_o_bf16(o, ref["o"], f"{label} O")
        H.check_max_abs(lse, ref["lse"], H.TOL_BF16_LSE, f"{label} lse")
        H.check_rel_l2(dq, ref["dq"], H.TOL_BF16_GRAD_RL2, f"{label} dQ")
        H.check_rel_l2(dk, ref["dk"], H.TOL_BF16_GRAD_RL2, f"{label} dK")
        H.check_rel_l2(dv, ref["dv"], H.TOL_BF16_GRAD_RL2, f"{label} dV")


def _oracle_full(st, dtype, scale, causal):
    w = H.widen_inputs(st, dtype)
    dq, dk, dv, o, lse = OA.attn_bwd(w["q"], w["k"], w["v"], w["dout"], scale, causal)
    return {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}


# ---------------------------------------------------------------------------- full parity


@pytest.mark.parametrize("wid", [1, 2])
def test_workload_full_parity(wid):
    wl = synth.WORKLOADS[wid]
    print(f"[parity] workload {wl.name}", flush=True)
    st = synth.attn_inputs(wl)
    gpu = _run_gpu(st, wl.dtype, wl.scale, wl.causal)
    _compare_full(gpu, _oracle_full(st, wl.dtype, wl.scale, wl.causal), wl.dtype, wl.name)


SWEEP = [
    # (B, N, Hq, Hkv, d, dtype, causal)
    (1, 1, 4, 1, 128, "bf16", True),
    (1, 65, 8, 2, 128, "bf16", True),
    (1, 1000, 8, 2, 128, "bf16", True),
    (2, 333, 4, 1, 64, "bf16", True),
    (1, 517, 8, 1, 128, "bf16", True),    # 8 query heads per KV head
    (1, 300, 4, 2, 128, "bf16", True),    # 2 query heads per KV head
    (1, 260, 4, 4, 64, "bf16", True),     # no grouping
    (1, 300, 8, 2, 128, "bf16", False),   # full attention
    (1, 200, 4, 2, 128, "f32", True),
    (2, 150, 4, 1, 64, "f32", False),
    (1, 129, 2, 2, 64, "f32", True),
]


@pytest.mark.parametrize("Bsz,N,Hq,Hkv,d,dtype,causal", SWEEP)
def test_shape_sweep_full_parity(Bsz, N, Hq, Hkv, d, dtype, causal):
    label = f"B{Bsz}-N{N}-{Hq}q{Hkv}kv-d{d}-{dtype}-{'causal' if causal else 'full'}"
    print(f"[parity] {label}", flush=True)
    st = synth.custom_inputs(Bsz, N, Hq, Hkv, d, dtype, seed=N * 7 + Hq)
    scale = 1.0 / math.sqrt(d)
    gpu = _run_gpu(st, dtype, scale, causal)
    _compare_full(gpu, _oracle_full(st, dtype, scale, causal), dtype, label)


# ---------------------------------------------------------------------------- split key range


SPLIT_SWEEP = [
    # (B, N, Hq, Hkv, d): query blocks of 64 rows (4+ query heads per KV head), 128 rows (2)
    # or 256 rows (1); 16 .. 128 blocks, ragged last blocks
    (1, 1000, 8, 2, 128),
    (1, 2100, 4, 2, 128),
    (1, 4100, 2, 2, 64),
    (2, 1500, 8, 2, 64),
    (1, 8192, 8, 1, 128),
]


@pytest.mark.parametrize("Bsz,N,Hq,Hkv,d", SPLIT_SWEEP)
def test_split_forward_matches_oracle(Bsz, N, Hq, Hkv, d):
    """ul_attn_fwd_ws, which runs the upper query blocks as two key-range halves combined
    afterwards, and ul_attn_fwd, which does not, both against the float64 oracle on every
    row; a NaN-filled workspace and NaN-poisoned outputs must leave no trace."""
    B = _B()
    label = f"split B{Bsz}-N{N}-{Hq}q{Hkv}kv-d{d}"
    print(f"[parity] {label}", flush=True)
    need = B.fwd_workspace_bytes(Bsz, N, Hq, Hkv, d, B.UL_BF16)
    assert need > 0, "these sizes are meant to split"
    st = synth.custom_inputs(Bsz, N, Hq, Hkv, d, "bf16", seed=N * 11 + Hq, with_dout=False)
    scale = 1.0 / math.sqrt(d)
    q, k, v = (H.to_device(st[n], "bf16") for n in ("q", "k", "v"))
    ws = torch.full((need // 4,), float("nan"), device="cuda").view(torch.uint8)
    res = {}
    for split in (True, False):
        o = torch.full_like(q, float("nan"))
        lse = torch.full((Bsz, Hq, N), float("nan"), device="cuda")
        B.attn_fwd(q, k, v, scale, True, out=o, lse=lse, split=split, workspace=ws if split else None)
        torch.cuda.synchronize()
        res[split] = (H.to_f64(o), H.to_f64(lse))
    w = H.widen_inputs(st, "bf16")
    o_ref, lse_ref = OA.attn_fwd(w["q"], w["k"], w["v"], scale, True)
    for split, (o, lse) in res.items():
        assert np.isfinite(o).all() and np.isfinite(lse).all(), f"{label} split={split}"
        H.check_o_bf16(o, o_ref, f"{label} O split={split}")
        H.check_max_abs(lse, lse_ref, H.TOL_BF16_LSE, f"{label} lse split={split}")
    # the lower half of the query blocks is never split: bit-identical on both paths, and the
    # split rows differ from the unsplit ones only by rounding
    grp = Hq // Hkv
    rows_per_blk = 32 * 8 // (4 if grp % 4 == 0 else 2 if grp % 2 == 0 else 1)
    lo = (-(-N // rows_per_blk) + 1) // 2 * rows_per_blk
    assert np.array_equal(res[True][0][:, :lo], res[False][0][:, :lo]), f"{label}: unsplit rows differ"
    assert np.array_equal(res[True][1][:, :, :lo], res[False][1][:, :, :lo]), f"{label}: unsplit lse differ"
    assert not np.array_equal(res[True][0][:, lo:], res[False][0][:, lo:]), f"{label}: split path not taken"


# ---------------------------------------------------------------------------- large N, sampled


def _invariants(gpu, wl):
    """Exact identities of the gradient, checked on the full GPU tensors in float64."""
    q, k, dq, dk, dv, do = (H.to_f64(gpu[n]) for n in ("q", "k", "dq", "dk", "dv", "dout"))
    r = wl.Hq // wl.Hkv
    out = {}
    for g in range(wl.Hkv):
        hs = slice(g * r, (g + 1) * r)
        dkg, dvg = dk[0, :, g], dv[0, :, g]
        res_k = np.linalg.norm(dkg.sum(axis=0)) / np.linalg.norm(dkg)
        res_v = np.linalg.norm(dvg.sum(axis=0) - do[0, :, hs].sum(axis=(0, 1))) / np.linalg.norm(dvg)
        a = np.sum(dq[0, :, hs] * q[0, :, hs])
        c = np.sum(dkg * k[0, :, g])
        res_s = abs(a - c) / (np.linalg.norm(dq[0, :, hs]) * np.linalg.norm(q[0, :, hs]))
        out[g] = (res_k, res_v, res_s)
        assert res_k <= H.TOL_BF16_GRAD_RL2, f"sum_j dK_j = 0 violated: {res_k:.3g}"
        assert res_v <= H.TOL_BF16_GRAD_RL2, f"sum_j dV_j = sum dO violated: {res_v:.3g}"
        assert res_s <= H.TOL_BF16_GRAD_RL2, f"<dQ,Q> = <dK,K> violated: {res_s:.3g}"
    return out


GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _check_stored_dkdv(gpu, wl):
    """dK and dV of the GPU at the keys the oracle's stored file holds, per KV head."""
    path = os.path.join(GOLDEN, f"dkdv_samples_w{wl.wid}.npz")
    with np.load(path, allow_pickle=False) as z:
        for g in range(wl.Hkv):
            keys = z[f"keys_g{g}"]
            dk_ref, dv_ref = z[f"dk_g{g}"].astype(np.float64), z[f"dv_g{g}"].astype(np.float64)
            dk = H.to_f64(gpu["dk"][0, keys, g])
            dv = H.to_f64(gpu["dv"][0, keys, g])
            rk = H.check_rel_l2(dk, dk_ref, H.TOL_BF16_GRAD_RL2, f"{wl.name} dK sampled keys g{g}")
            rv = H.check_rel_l2(dv, dv_ref, H.TOL_BF16_GRAD_RL2, f"{wl.name} dV sampled keys g{g}")
            # the first keys carry the longest sums: report them on their own as well
            first = keys < 256
            if first.any():
                H.check_rel_l2(dk[first], dk_ref[first], H.TOL_BF16_GRAD_RL2, f"{wl.name} dK first keys g{g}")
                H.check_rel_l2(dv[first], dv_ref[first], H.TOL_BF16_GRAD_RL2, f"{wl.name} dV first keys g{g}")
            print(f"[parity] {wl.name} g{g}: {len(keys)} keys [{keys.min()}, {keys.max()}] "
                  f"dK rel-L2 {rk:.3g} dV rel-L2 {rv:.3g}", flush=True)


@pytest.mark.parametrize("wid", [3, 4, 5])
def test_large_workload_sampled_parity(wid):
    wl = synth.WORKLOADS[wid]
    print(f"[parity] workload {wl.name}: generating inputs", flush=True)
    st = synth.attn_inputs(wl)
    gpu = _run_gpu(st, wl.dtype, wl.scale, wl.causal, poison=False)
    print(f"[parity] {wl.name}: GPU fwd+bwd done; oracle on sampled rows", flush=True)
    w = H.widen_inputs({n: st[n] for n in ("q", "k", "v", "dout")}, wl.dtype)
    del st
    o_all = gpu["o"]
    for h in range(wl.Hq):
        rows = np.union1d(synth.sample_rows(wl, h), synth.fixed_rows(wl.N))
        g = h // (wl.Hq // wl.Hkv)
        # one-head views keep the oracle's work to this head's rows
        qh, doh = w["q"][:, :, h:h + 1], w["dout"][:, :, h:h + 1]
        kg, vg = w["k"][:, :, g:g + 1], w["v"][:, :, g:g + 1]
        o_ref, lse_ref = OA.attn_fwd(qh, kg, vg, wl.scale, wl.causal, rows)
        o_gpu = H.to_f64(o_all[:, rows, h:h + 1])
        lse_gpu = H.to_f64(gpu["lse"][:, h:h + 1, rows])
        H.check_o_bf16(o_gpu, o_ref, f"{wl.name} O head {h}")
        H.check_max_abs(lse_gpu, lse_ref, H.TOL_BF16_LSE, f"{wl.name} lse head {h}")
        # dQ rows need D = dO . O of the oracle's own O
        dq_ref = OA.dq_rows(qh, kg, vg, doh, wl.scale, wl.causal, rows)
        dq_gpu = H.to_f64(gpu["dq"][:, rows, h:h + 1])
        H.check_rel_l2(dq_gpu, dq_ref, H.TOL_BF16_GRAD_RL2, f"{wl.name} dQ head {h}")
    # dK / dV at the stored sampled keys of every KV head (whole range; last 16K at 1M)
    _check_stored_dkdv(gpu, wl)
    # the last 64 keys of every KV head: their causal sums cover only the last rows
    keys = np.arange(wl.N - 64, wl.N)
    dk_ref, dv_ref = OA.dkdv_rows(w["q"], w["k"], w["v"], w["dout"], wl.scale, wl.causal, keys)
    H.check_rel_l2(H.to_f64(gpu["dk"][:, keys]), dk_ref, H.TOL_BF16_GRAD_RL2, f"{wl.name} dK tail")
    H.check_rel_l2(H.to_f64(gpu["dv"][:, keys]), dv_ref, H.TOL_BF16_GRAD_RL2, f"{wl.name} dV tail")
    print(f"[parity] {wl.name}: invariants {_invariants(gpu, wl)}", flush=True)


# ---------------------------------------------------------------------------- properties


def test_deterministic_bitwise():
    wl = synth.WORKLOADS[2]
    st = synth.custom_inputs(1, 2048, 8, 2, 128, "bf16", seed=77)
    a = _run_gpu(st, "bf16", wl.scale, True, poison=False)
    b = _run_gpu(st, "bf16", wl.scale, True, poison=True)
    for n in ("o", "lse", "dq", "dk", "dv"):
        assert torch.equal(a[n].view(torch.uint8) if a[n].dtype != torch.float32 else a[n].view(torch.int32),
                           b[n].view(torch.uint8) if b[n].dtype != torch.float32 else b[n].view(torch.int32)), n


def test_causality_bitwise():
    """Changing keys and values after row i leaves rows <= i bit-identical."""
    B = _B()
    st = synth.custom_inputs(1, 700, 8, 2, 128, "bf16", seed=78, with_dout=False)
    q, k, v = (H.to_device(st[n], "bf16") for n in ("q", "k", "v"))
    o1, l1 = B.attn_fwd(q, k, v)
    i = 389
    k2, v2 = k.clone(), v.clone()
    k2[:, i + 1:] = -k2[:, i + 1:] * 3
    v2[:, i + 1:] = v2[:, i + 1:] + 5
    o2, l2 = B.attn_fwd(q, k2, v2)
    torch.cuda.synchronize()
    assert torch.equal(o1[:, : i + 1].view(torch.int16), o2[:, : i + 1].view(torch.int16))
    assert torch.equal(l1[:, :, : i + 1], l2[:, :, : i + 1])
    assert not torch.equal(o1[:, i + 1:].view(torch.int16), o2[:, i + 1:].view(torch.int16))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ulysses_composition(dtype):
    """Per-rank attention on the head-sharded relayout, relayouted back, equals attention
    over all heads at once (bit-identical: heads are independent)."""
    B = _B()
    wl = synth.WORKLOADS[1]
    C, N, Hh, d, P = wl.relayout
    rng = np.random.Generator(np.random.PCG64(79))
    x32 = rng.standard_normal((C, N, Hh, d)).astype(np.float32)
    x = H.to_device(synth.encode(x32, dtype), dtype)
    o_full, _ = B.attn_fwd(x[0:1], x[1:2], x[2:3])
    y = B.relayout_s2h(x, P)  # [3, P, N, H/P, d]
    outs = torch.empty((1, P, N, Hh // P, d), dtype=x.dtype, device="cuda")
    for r in range(P):
        o_r, _ = B.attn_fwd(y[0, r][None].contiguous(), y[1, r][None].contiguous(), y[2, r][None].contiguous())
        outs[0, r] = o_r[0]
    back = B.relayout_h2s(outs)
    torch.cuda.synchronize()
    assert torch.equal(back, o_full)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_backward_stages_match_single_call(dtype):
    """Prep, dQ and dK/dV run as separate calls -- dK/dV first, and on a second stream --
    give the bit-identical result of the one-call backward."""
    B = _B()
    d = 128 if dtype == "bf16" else 64
    st = synth.custom_inputs(1, 700, 8, 2, d, dtype, seed=81)
    scale = 1.0 / math.sqrt(d)
    ref = _run_gpu(st, dtype, scale, True, poison=False)
    q, k, v, o, do, lse = (ref[n] for n in ("q", "k", "v", "o", "dout", "lse"))
    dq = torch.full_like(q, float("nan"))
    dk = torch.full_like(k, float("nan"))
    dv = torch.full_like(v, float("nan"))
    ws = torch.empty(B.workspace_bytes(1, 700, 8, 2, d, B.UL_BF16 if dtype == "bf16" else B.UL_F32),
                     dtype=torch.uint8, device="cuda")
    B.attn_bwd(q, k, v, o, do, lse, scale, True, workspace=ws, dq=dq, dk=dk, dv=dv, stages=B.UL_BWD_PREP)
    side = torch.cuda.Stream()
    prep_done = torch.cuda.Event()
    prep_done.record()
    side.wait_event(prep_done)
    B.attn_bwd(q, k, v, o, do, lse, scale, True, workspace=ws, dq=dq, dk=dk, dv=dv,
               stages=B.UL_BWD_DKDV, stream=side)
    B.attn_bwd(q, k, v, o, do, lse, scale, True, workspace=ws, dq=dq, dk=dk, dv=dv, stages=B.UL_BWD_DQ)
    torch.cuda.synchronize()
    for n, x in (("dq", dq), ("dk", dk), ("dv", dv)):
        a = x.view(torch.int16) if x.dtype == torch.bfloat16 else x.view(torch.int32)
        r = ref[n].view(torch.int16) if x.dtype == torch.bfloat16 else ref[n].view(torch.int32)
        assert torch.equal(a, r), n
