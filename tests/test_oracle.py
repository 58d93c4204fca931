"""Pins for the fp64 oracle, independent of the oracle itself (CPU only).

Each test ties the oracle to something it does not contain: a closed form of
softmax attention, a hand-derived example, a library routine (torch's CPU
attention and autograd, numpy's transpose), finite differences, or an exact
invariant of the mathematics.  The mutation tests at the end plant plausible
mistakes in a copy of the oracle and check that a pin catches each one.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import attention as OA
from oracle import native as ON
from ulysses_sequence_parallelism_attn_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed, scale=1.0):
    return scale * np.random.Generator(np.random.PCG64(seed)).standard_normal(shape)


def _qkv(B, N, Hq, Hkv, d, seed=0):
    return (_rand((B, N, Hq, d), seed), _rand((B, N, Hkv, d), seed + 1),
            _rand((B, N, Hkv, d), seed + 2), _rand((B, N, Hq, d), seed + 3))


# ----------------------------------------------------------------------------- closed forms


@pytest.mark.parametrize("causal", [True, False])
def test_uniform_scores_give_prefix_mean_of_v(causal):
    """Q = 0 makes every visible score 0: P_ij = 1/(#visible), O_i = mean of visible V rows,
    lse_i = ln(#visible)."""
    B, N, Hq, Hkv, d = 2, 37, 4, 2, 8
    q, k, v, _ = _qkv(B, N, Hq, Hkv, d, 10)
    q[:] = 0.0
    o, lse = OA.attn_fwd(q, k, v, 0.3, causal)
    for h in range(Hq):
        g = h // 2
        for i in range(N):
            cnt = i + 1 if causal else N
            np.testing.assert_allclose(o[:, i, h], v[:, :cnt, g].mean(axis=1), rtol=0, atol=1e-13)
            np.testing.assert_allclose(lse[:, h, i], math.log(cnt), rtol=0, atol=1e-13)


def test_equal_keys_give_prefix_mean_and_shifted_lse():
    """All K rows equal to one vector c: every visible score of row i is scale*q_i.c, so
    O_i is the prefix mean of V and lse_i = scale*q_i.c + ln(i+1)."""
    B, N, Hq, Hkv, d = 1, 29, 2, 1, 16
    q, k, v, _ = _qkv(B, N, Hq, Hkv, d, 20)
    c = _rand(d, 99)
    k[:] = c
    scale = 0.25
    o, lse = OA.attn_fwd(q, k, v, scale, True)
    for h in range(Hq):
        for i in range(N):
            np.testing.assert_allclose(o[0, i, h], v[0, : i + 1, 0].mean(axis=0), atol=1e-13)
            np.testing.assert_allclose(lse[0, h, i], scale * q[0, i, h] @ c + math.log(i + 1),
                                       atol=1e-12)


def test_one_hot_dominant_score_returns_that_v_row():
    """K_{j*} = c * Q_i with a score gap >= 40 over every other visible key: O_i = V_{j*}
    to within exp(-40) * i * max|V|."""
    N, d = 50, 8
    q, k, v, _ = _qkv(1, N, 1, 1, d, 30)
    q *= 0.1
    k *= 0.1
    i, jstar = 41, 17
    k[0, jstar, 0] = 60.0 * q[0, i, 0] / (q[0, i, 0] @ q[0, i, 0])  # s_i,j* = 60 (scale 1)
    o, _ = OA.attn_fwd(q, k, v, 1.0, True)
    s = q[0, i, 0] @ k[0, : i + 1, 0].T
    gap = s[jstar] - np.delete(s, jstar).max()
    assert gap >= 40
    bound = math.exp(-40) * (i + 1) * np.abs(v).max()
    np.testing.assert_allclose(o[0, i, 0], v[0, jstar, 0], rtol=0, atol=bound)


def test_first_causal_row_is_v0_exactly():
    q, k, v, _ = _qkv(2, 17, 4, 2, 8, 40)
    o, lse = OA.attn_fwd(q, k, v, 0.7, True)
    for h in range(4):
        assert np.array_equal(o[:, 0, h], v[:, 0, h // 2])
        np.testing.assert_allclose(lse[:, h, 0], 0.7 * np.einsum("be,be->b", q[:, 0, h], k[:, 0, h // 2]),
                                   atol=1e-14)


@pytest.mark.parametrize("causal", [True, False])
def test_probability_rows_sum_to_one(causal):
    q, k, v, _ = _qkv(1, 23, 2, 2, 8, 50)
    P = OA.probabilities(q, k, 0.5, causal)
    np.testing.assert_allclose(P.sum(axis=-1), 1.0, rtol=0, atol=1e-14)
    if causal:
        assert np.all(np.triu(P[0, 0], 1) == 0)
    v1 = np.ones_like(v)
    o, _ = OA.attn_fwd(q, k, v1, 0.5, causal)
    np.testing.assert_allclose(o, 1.0, rtol=0, atol=1e-14)


def _torch_probabilities(q, k, scale, causal):
    """Softmax of the scaled, masked scores by torch's CPU softmax (a library routine), with
    each KV head repeated for its query heads."""
    tq = torch.tensor(q).permute(0, 2, 1, 3)  # [B, Hq, N, d]
    tk = torch.tensor(k).permute(0, 2, 1, 3)
    tk = tk.repeat_interleave(q.shape[2] // k.shape[2], dim=1)
    s = scale * (tq @ tk.transpose(-1, -2))
    if causal:
        N = q.shape[1]
        s = s.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), float("-inf"))
    return torch.softmax(s, dim=-1).numpy()


@pytest.mark.parametrize("shape,causal", [((1, 23, 2, 2, 8), True), ((2, 31, 4, 1, 16), True),
                                          ((1, 17, 6, 2, 8), False)])
def test_probabilities_match_torch_softmax(shape, causal):
    """P from the oracle equals torch's softmax of the scaled scores (GQA via repeated KV
    heads), and P V equals the oracle's forward output."""
    B, N, Hq, Hkv, d = shape
    q, k, v, _ = _qkv(B, N, Hq, Hkv, d, 51)
    P = OA.probabilities(q, k, 0.37, causal)
    np.testing.assert_allclose(P, _torch_probabilities(q, k, 0.37, causal), rtol=0, atol=1e-14)
    o, _ = OA.attn_fwd(q, k, v, 0.37, causal)
    vr = np.repeat(v, Hq // Hkv, axis=2).transpose(0, 2, 1, 3)  # [B, Hq, N, d]
    np.testing.assert_allclose((P @ vr).transpose(0, 2, 1, 3), o, rtol=0, atol=1e-13)


@pytest.mark.parametrize("mistake", ["scale", "group", "mask"])
def test_probabilities_planted_mistakes_are_caught(monkeypatch, mistake):
    """A wrong scale, group map or mask in the oracle's P fails the torch comparison."""
    q, k, _, _ = _qkv(1, 23, 4, 2, 8, 52)
    ref = _torch_probabilities(q, k, 0.5, True)
    if mistake == "scale":
        P = OA.probabilities(q, k, 0.5 * 1.01, True)
    else:
        if mistake == "group":
            monkeypatch.setattr(OA, "_group", lambda h, Hq, Hkv: h % Hkv)
        else:
            monkeypatch.setattr(OA, "_visible",
                                lambda rows, N, causal: np.arange(N)[None, :] < rows[:, None])
        P = OA.probabilities(q, k, 0.5, True)
    assert not (np.abs(P - ref) <= 1e-3).all()  # an all-masked row gives NaN: also a miss


def test_lse_bounds():
    """max_j s_ij <= lse_i <= max_j s_ij + ln(i+1)."""
    B, N, Hq, Hkv, d = 1, 64, 2, 1, 16
    q, k, v, _ = _qkv(B, N, Hq, Hkv, d, 60)
    scale = 0.25
    _, lse = OA.attn_fwd(q, k, v, scale, True)
    for h in range(Hq):
        s = scale * q[0, :, h] @ k[0, :, 0].T
        for i in range(N):
            m = s[i, : i + 1].max()
            assert m - 1e-13 <= lse[0, h, i] <= m + math.log(i + 1) + 1e-13


def test_causality_is_bit_exact():
    """Changing keys/values after row i leaves row i's output and lse bit-identical."""
    B, N, Hq, Hkv, d = 1, 40, 2, 1, 8
    q, k, v, _ = _qkv(B, N, Hq, Hkv, d, 70)
    o1, l1 = OA.attn_fwd(q, k, v, 0.3, True)
    i = 25
    k2, v2 = k.copy(), v.copy()
    k2[:, i + 1:] = _rand(k2[:, i + 1:].shape, 71, 5.0)
    v2[:, i + 1:] = _rand(v2[:, i + 1:].shape, 72, 5.0)
    o2, l2 = OA.attn_fwd(q, k2, v2, 0.3, True)
    assert np.array_equal(o1[:, : i + 1], o2[:, : i + 1])
    assert np.array_equal(l1[:, :, : i + 1], l2[:, :, : i + 1])
    assert not np.array_equal(o1[:, i + 1:], o2[:, i + 1:])


def test_hand_worked_example():
    with open(os.path.join(GOLDEN, "hand_worked_example.json")) as f:
        ex = json.load(f)

    def val(x):
        if isinstance(x, (int, float)):
            return float(x)
        return {"ln3": math.log(3), "ln4": math.log(4), "0.75*ln3": 0.75 * math.log(3)}[x]

    inp = ex["inputs"]
    q = np.array([val(x) for x in inp["q"]]).reshape(1, 2, 1, 1)
    k = np.array([val(x) for x in inp["k"]]).reshape(1, 2, 1, 1)
    v = np.array([val(x) for x in inp["v"]]).reshape(1, 2, 1, 1)
    do = np.array([val(x) for x in inp["dout"]]).reshape(1, 2, 1, 1)
    exp = {n: np.array([val(x) for x in xs]) for n, xs in ex["expected"].items()}
    o, lse = OA.attn_fwd(q, k, v, inp["scale"], inp["causal"])
    np.testing.assert_allclose(o.ravel(), exp["o"], atol=1e-14)
    np.testing.assert_allclose(lse.ravel(), exp["lse"], atol=1e-14)
    dq, dk, dv, _, _ = OA.attn_bwd(q, k, v, do, inp["scale"], inp["causal"])
    np.testing.assert_allclose(dq.ravel(), exp["dq"], atol=1e-14)
    np.testing.assert_allclose(dk.ravel(), exp["dk"], atol=1e-14)
    np.testing.assert_allclose(dv.ravel(), exp["dv"], atol=1e-14)


# ----------------------------------------------------------------------------- library routine


def _torch_ref(q, k, v, do, scale, causal):
    """torch CPU float64 attention (library routine) with K/V repeated per group."""
    Hq, Hkv = q.shape[2], k.shape[2]
    tq = torch.tensor(q).permute(0, 2, 1, 3).contiguous().requires_grad_(True)
    tk = torch.tensor(k).permute(0, 2, 1, 3).contiguous().requires_grad_(True)
    tv = torch.tensor(v).permute(0, 2, 1, 3).contiguous().requires_grad_(True)
    kr = tk.repeat_interleave(Hq // Hkv, dim=1)
    vr = tv.repeat_interleave(Hq // Hkv, dim=1)
    o = torch.nn.functional.scaled_dot_product_attention(tq, kr, vr, is_causal=causal, scale=scale)
    o.backward(torch.tensor(do).permute(0, 2, 1, 3))
    _, lse = torch.ops.aten._scaled_dot_product_flash_attention_for_cpu(
        tq.detach(), kr.detach(), vr.detach(), 0.0, causal, scale=scale)[:2]
    tr = lambda t: t.detach().permute(0, 2, 1, 3).numpy()
    return tr(o), lse.numpy(), tr(tq.grad), tr(tk.grad), tr(tv.grad)


@pytest.mark.parametrize("shape,causal", [((1, 64, 4, 4, 16), True), ((2, 97, 8, 2, 32), True),
                                          ((1, 256, 4, 1, 64), True), ((1, 50, 4, 2, 16), False)])
def test_matches_torch_cpu_float64(shape, causal):
    B, N, Hq, Hkv, d = shape
    q, k, v, do = _qkv(B, N, Hq, Hkv, d, 80)
    scale = 1 / math.sqrt(d)
    to, tl, tdq, tdk, tdv = _torch_ref(q, k, v, do, scale, causal)
    o, lse = OA.attn_fwd(q, k, v, scale, causal)
    np.testing.assert_allclose(o, to, atol=1e-12)
    np.testing.assert_allclose(lse, tl, atol=1e-12)
    dq, dk, dv, o2, lse2 = OA.attn_bwd(q, k, v, do, scale, causal)
    np.testing.assert_allclose(dq, tdq, atol=1e-11)
    np.testing.assert_allclose(dk, tdk, atol=1e-11)
    np.testing.assert_allclose(dv, tdv, atol=1e-11)
    assert np.array_equal(o2, o) and np.array_equal(lse2, lse)


# ----------------------------------------------------------------------------- finite differences


def test_gradients_match_central_differences():
    """dL/d(Q,K,V) of L = <dO, O> against central differences, h = 1e-6, fp64."""
    B, N, Hq, Hkv, d = 1, 8, 2, 1, 4
    q, k, v, do = _qkv(B, N, Hq, Hkv, d, 90)
    scale = 0.5
    dq, dk, dv, _, _ = OA.attn_bwd(q, k, v, do, scale, True)

    def L(q_, k_, v_):
        return float(np.sum(do * OA.attn_fwd(q_, k_, v_, scale, True)[0]))

    h = 1e-6
    for name, arr, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            a1, a2 = arr.copy(), arr.copy()
            a1[idx] += h
            a2[idx] -= h
            args1 = {"q": q, "k": k, "v": v}
            args2 = dict(args1)
            args1[name], args2[name] = a1, a2
            num[idx] = (L(**{n + "_": x for n, x in args1.items()}) -
                        L(**{n + "_": x for n, x in args2.items()})) / (2 * h)
        err = np.abs(num - grad).max() / max(np.abs(grad).max(), 1e-300)
        assert err <= 1e-7, (name, err)


# ----------------------------------------------------------------------------- invariants


def test_backward_invariants():
    """Exact identities of the gradient:
    sum_j dK_j = 0 (shifting every key by the same vector changes no probability);
    sum_j dV_j = sum over the group's heads of sum_i dO_i (rows of P sum to 1);
    <dQ, Q> = <dK, K> per KV group (invariance to Q -> aQ, K -> K/a)."""
    B, N, Hq, Hkv, d = 2, 70, 8, 2, 16
    q, k, v, do = _qkv(B, N, Hq, Hkv, d, 100)
    dq, dk, dv, _, _ = OA.attn_bwd(q, k, v, do, 0.25, True)
    r = Hq // Hkv
    for g in range(Hkv):
        heads = slice(g * r, (g + 1) * r)
        np.testing.assert_allclose(dk[:, :, g].sum(axis=1), 0.0, atol=1e-12)
        np.testing.assert_allclose(dv[:, :, g].sum(axis=1), do[:, :, heads].sum(axis=(1, 2)),
                                   atol=1e-11)
        for b in range(B):
            a = np.sum(dq[b, :, heads] * q[b, :, heads])
            c = np.sum(dk[b, :, g] * k[b, :, g])
            np.testing.assert_allclose(a, c, rtol=1e-11, atol=1e-11)


def test_backward_closed_forms():
    """Q = 0: dK = 0 and dV_j = sum_{h in group} sum_{i >= j} dO_i / (i+1).
    All K rows equal: dQ = 0."""
    B, N, Hq, Hkv, d = 1, 33, 4, 2, 8
    q, k, v, do = _qkv(B, N, Hq, Hkv, d, 110)
    q0 = np.zeros_like(q)
    _, dk, dv, _, _ = OA.attn_bwd(q0, k, v, do, 0.5, True)
    np.testing.assert_allclose(dk, 0.0, atol=1e-14)
    w = 1.0 / (np.arange(N) + 1.0)
    for g in range(Hkv):
        s = do[0, :, 2 * g: 2 * g + 2].sum(axis=1) * w[:, None]  # [N, d]
        expect = np.cumsum(s[::-1], axis=0)[::-1]
        np.testing.assert_allclose(dv[0, :, g], expect, atol=1e-13)
    ke = k.copy()
    ke[:] = k[:, :1]
    dq, _, _, _, _ = OA.attn_bwd(q, ke, v, do, 0.5, True)
    np.testing.assert_allclose(dq, 0.0, atol=1e-13)


def test_gqa_equals_mha_with_repeated_kv():
    B, N, Hq, Hkv, d = 1, 45, 8, 2, 16
    q, k, v, do = _qkv(B, N, Hq, Hkv, d, 120)
    kr, vr = np.repeat(k, 4, axis=2), np.repeat(v, 4, axis=2)
    o1, l1 = OA.attn_fwd(q, k, v, 0.25, True)
    o2, l2 = OA.attn_fwd(q, kr, vr, 0.25, True)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    dq1, dk1, dv1, _, _ = OA.attn_bwd(q, k, v, do, 0.25, True)
    dq2, dk2, dv2, _, _ = OA.attn_bwd(q, kr, vr, do, 0.25, True)
    np.testing.assert_allclose(dq1, dq2, atol=1e-13)
    np.testing.assert_allclose(dk1, dk2.reshape(B, N, Hkv, 4, d).sum(axis=3), atol=1e-12)
    np.testing.assert_allclose(dv1, dv2.reshape(B, N, Hkv, 4, d).sum(axis=3), atol=1e-12)


def test_ulysses_composition_is_exact():
    """Head independence: attention per rank on the head-sharded relayout, relayouted back,
    equals attention over all heads at once (bit-identical in the oracle)."""
    C, N, H, d, P = 3, 64, 8, 16, 4
    x = _rand((C, N, H, d), 130)
    q, k, v = x[0][None], x[1][None], x[2][None]
    o_full, _ = OA.attn_fwd(q, k, v, 0.25, True)
    y = ON.relayout_s2h(x, P)  # [C, P, N, H/P, d]
    outs = np.empty((1, P, N, H // P, d))
    for r in range(P):
        outs[0, r], _ = OA.attn_fwd(y[0, r][None], y[1, r][None], y[2, r][None], 0.25, True)
    assert np.array_equal(ON.relayout_h2s(outs)[0], o_full[0])


# ----------------------------------------------------------------------------- subsets and brute force


def test_row_subsets_match_full_results():
    B, N, Hq, Hkv, d = 1, 300, 4, 1, 16
    q, k, v, do = _qkv(B, N, Hq, Hkv, d, 140)
    rows = np.array([0, 1, 63, 64, 150, 298, 299])
    o, lse = OA.attn_fwd(q, k, v, 0.25, True)
    o_r, lse_r = OA.attn_fwd(q, k, v, 0.25, True, rows)
    np.testing.assert_allclose(o_r, o[:, rows], atol=1e-14)
    np.testing.assert_allclose(lse_r, lse[:, :, rows], atol=1e-14)
    dq, dk, dv, _, _ = OA.attn_bwd(q, k, v, do, 0.25, True)
    np.testing.assert_allclose(OA.dq_rows(q, k, v, do, 0.25, True, rows), dq[:, rows], atol=1e-12)
    keys = np.array([5, 200, 290, 299])
    dk_r, dv_r = OA.dkdv_rows(q, k, v, do, 0.25, True, keys)
    np.testing.assert_allclose(dk_r, dk[:, keys], atol=1e-12)
    np.testing.assert_allclose(dv_r, dv[:, keys], atol=1e-12)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("causal", [True, False])
def test_scalar_brute_force_agrees(dtype, causal):
    """The scalar C loops (no matrix library) agree with the matrix formulation, reading the
    same stored inputs."""
    B, N, Hq, Hkv, d = 1, 48, 4, 2, 16
    st = synth.custom_inputs(B, N, Hq, Hkv, d, dtype, seed=7)
    w = {n: OA.widen(a, dtype) for n, a in st.items()}
    o, lse = OA.attn_fwd(w["q"], w["k"], w["v"], 0.25, causal)
    o2, lse2 = ON.brute_fwd(st["q"], st["k"], st["v"], dtype, 0.25, causal)
    np.testing.assert_allclose(o2, o, atol=1e-13)
    np.testing.assert_allclose(lse2, lse, atol=1e-13)
    dq, dk, dv, _, _ = OA.attn_bwd(w["q"], w["k"], w["v"], w["dout"], 0.25, causal)
    dq2, dk2, dv2 = ON.brute_bwd(st["q"], st["k"], st["v"], st["dout"], dtype, 0.25, causal)
    np.testing.assert_allclose(dq2, dq, atol=1e-12)
    np.testing.assert_allclose(dk2, dk, atol=1e-12)
    np.testing.assert_allclose(dv2, dv, atol=1e-12)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("causal", [True, False])
def test_scalar_row_subsets_agree(dtype, causal):
    """The scalar C row-subset loops (forward rows, dQ rows, dK/dV key rows with the row
    statistics recomputed per row or precomputed) agree with the matrix row functions the
    long-sequence parity checks use, on unsorted subsets that include the first and the last
    positions."""
    B, N, Hq, Hkv, d = 2, 70, 4, 2, 16
    st = synth.custom_inputs(B, N, Hq, Hkv, d, dtype, seed=9)
    w = {n: OA.widen(a, dtype) for n, a in st.items()}
    rows = np.array([69, 0, 33, 1, 64, 63])
    o, lse = OA.attn_fwd(w["q"], w["k"], w["v"], 0.3, causal, rows)
    o2, lse2 = ON.brute_fwd_rows(st["q"], st["k"], st["v"], dtype, 0.3, causal, rows)
    np.testing.assert_allclose(o2, o, atol=1e-13)
    np.testing.assert_allclose(lse2, lse, atol=1e-13)
    dq = OA.dq_rows(w["q"], w["k"], w["v"], w["dout"], 0.3, causal, rows)
    dq2 = ON.brute_dq_rows(st["q"], st["k"], st["v"], st["dout"], dtype, 0.3, causal, rows)
    np.testing.assert_allclose(dq2, dq, atol=1e-12)
    keys = np.array([0, 69, 12, 40])
    dk, dv = OA.dkdv_rows(w["q"], w["k"], w["v"], w["dout"], 0.3, causal, keys)
    for pre in (False, True):
        dk2, dv2 = ON.brute_dkdv_rows(st["q"], st["k"], st["v"], st["dout"], dtype, 0.3, causal,
                                      keys, precomputed_stats=pre)
        np.testing.assert_allclose(dk2, dk, atol=1e-12)
        np.testing.assert_allclose(dv2, dv, atol=1e-12)


def test_row_chunking_does_not_change_results(monkeypatch):
    """Blocking the rows differently (the memory bound of the matrix oracle) gives the same
    values: every row is computed on its own."""
    B, N, Hq, Hkv, d = 1, 90, 2, 1, 8
    q, k, v, do = _qkv(B, N, Hq, Hkv, d, 141)
    ref = OA.attn_bwd(q, k, v, do, 0.3, True)
    keys = np.array([0, 45, 89])
    ref_kv = OA.dkdv_rows(q, k, v, do, 0.3, True, keys)
    monkeypatch.setattr(OA, "_BLOCK_ELEMS", 7 * N)  # 7-row blocks
    got = OA.attn_bwd(q, k, v, do, 0.3, True)
    for a, b in zip(got, ref):
        np.testing.assert_allclose(a, b, atol=1e-13)
    for a, b in zip(OA.dkdv_rows(q, k, v, do, 0.3, True, keys), ref_kv):
        np.testing.assert_allclose(a, b, atol=1e-13)


def test_sampled_keys_cover_the_range():
    """The seeded key sample holds 512 distinct keys plus the fixed ones, inside the window."""
    wl = synth.WORKLOADS[3]
    keys = synth.sample_keys(wl, 0)
    assert len(keys) >= 512 and np.all(np.diff(keys) > 0)
    assert {0, 1, 127, 128, wl.N // 2, wl.N - 1} <= set(keys.tolist())
    assert keys.min() == 0 and keys.max() == wl.N - 1
    assert not np.array_equal(keys, synth.sample_keys(wl, 1))
    w5 = synth.WORKLOADS[5]
    k5 = synth.sample_keys(w5, 0, window=16384)
    assert k5.min() == w5.N - 16384 and k5.max() == w5.N - 1 and len(k5) >= 512


def test_stored_dkdv_samples_match_the_seeded_key_draw():
    """The stored file's keys are the seeded draw of synth.sample_keys (so its values belong
    to these inputs' sampled keys), and every workload above has a file."""
    for wid, window in ((3, None), (4, None), (5, 16384)):
        wl = synth.WORKLOADS[wid]
        with np.load(os.path.join(GOLDEN, f"dkdv_samples_w{wid}.npz"), allow_pickle=False) as z:
            for g in range(wl.Hkv):
                assert np.array_equal(z[f"keys_g{g}"], synth.sample_keys(wl, g, window=window))
                assert z[f"dk_g{g}"].shape == (len(z[f"keys_g{g}"]), wl.d)


def test_widen_is_exact():
    x = synth.normal_f32((1000,), 5)
    b = synth.f32_to_bf16_bits(x)
    w = OA.widen(b, "bf16")
    t = torch.tensor(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(w, t)  # torch's float32 -> bf16 rounding is also nearest-even
    assert np.array_equal(OA.widen(x, "f32"), x.astype(np.float64))


# ----------------------------------------------------------------------------- relayout


@pytest.mark.parametrize("C,N,H,d,P", [(3, 256, 4, 64, 2), (1, 12, 6, 3, 3), (2, 8, 8, 4, 8),
                                       (3, 16, 4, 8, 1)])
@pytest.mark.parametrize("dtype", [np.uint16, np.uint32, np.uint8])
def test_relayout_matches_numpy_transpose(C, N, H, d, P, dtype):
    rng = np.random.Generator(np.random.PCG64(150))
    x = rng.integers(0, np.iinfo(dtype).max, size=(C, N, H, d), dtype=dtype)
    y = ON.relayout_s2h(x, P)
    ref = x.reshape(C, N, P, H // P, d).transpose(0, 2, 1, 3, 4)
    assert np.array_equal(y, ref)
    assert np.array_equal(ON.relayout_h2s(y), x)
    z = rng.integers(0, np.iinfo(dtype).max, size=y.shape, dtype=dtype)
    assert np.array_equal(ON.relayout_s2h(ON.relayout_h2s(z), P), z)
    if P == 1:
        assert np.array_equal(y[:, 0], x)


def test_relayout_adjointness():
    """<s2h x, y> = <x, h2s y>: the adjoint of the permutation is its inverse, which is what
    the backward pass of each exchange applies."""
    C, N, H, d, P = 2, 16, 8, 4, 4
    x = _rand((C, N, H, d), 160)
    y = _rand((C, P, N, H // P, d), 161)
    np.testing.assert_allclose(np.sum(ON.relayout_s2h(x, P) * y), np.sum(x * ON.relayout_h2s(y)),
                               rtol=1e-12)


def test_relayout_rejects_bad_shapes():
    x = np.zeros((1, 8, 6, 2), dtype=np.uint16)
    with pytest.raises(ValueError):
        ON.relayout_s2h(x, 4)  # 6 heads not divisible by 4
    with pytest.raises(ValueError):
        ON.relayout_s2h(np.zeros((1, 6, 8, 2), np.uint16), 4)  # 6 tokens not divisible by 4


@pytest.mark.parametrize("C,N,H,d,P,h0,Hc", [(3, 16, 8, 4, 2, 1, 2), (1, 12, 6, 3, 3, 0, 1),
                                             (2, 8, 16, 8, 4, 2, 2), (3, 4, 4, 5, 1, 0, 4)])
@pytest.mark.parametrize("dtype", [np.uint16, np.uint32])
def test_head_chunk_relayout_matches_numpy_slice(C, N, H, d, P, h0, Hc, dtype):
    """The head-chunk exchange is a slice of the heads inside every rank's slice, then the
    same transpose (a library routine)."""
    rng = np.random.Generator(np.random.PCG64(155))
    x = rng.integers(0, np.iinfo(dtype).max, size=(C, N, H, d), dtype=dtype)
    y = ON.relayout_s2h_heads(x, P, h0, Hc)
    ref = x.reshape(C, N, P, H // P, d)[:, :, :, h0:h0 + Hc].transpose(0, 2, 1, 3, 4)
    assert np.array_equal(y, ref)


def test_head_chunks_compose_to_the_full_exchange():
    """Chunks that partition each rank's slice, put side by side, are the full s2h; writing
    them back with h2s_heads over a garbage-filled tensor rebuilds the input exactly, and a
    single chunk's write leaves every other head untouched."""
    C, N, H, d, P = 2, 12, 12, 3, 3
    Hs = H // P
    rng = np.random.Generator(np.random.PCG64(156))
    x = rng.integers(0, 65535, size=(C, N, H, d), dtype=np.uint16)
    chunks = [(0, 1), (1, 2), (3, 1)]  # (h0, Hc) covering 0 .. Hs-1
    parts = [ON.relayout_s2h_heads(x, P, h0, Hc) for h0, Hc in chunks]
    assert np.array_equal(np.concatenate(parts, axis=3), ON.relayout_s2h(x, P))
    back = rng.integers(0, 65535, size=x.shape, dtype=np.uint16)
    before = back.copy()
    ON.relayout_h2s_heads(parts[1], back, 1)
    owned = np.zeros(H, bool)
    for r in range(P):
        owned[r * Hs + 1: r * Hs + 3] = True
    assert np.array_equal(back[:, :, ~owned], before[:, :, ~owned])
    assert np.array_equal(back[:, :, owned], x[:, :, owned])
    for (h0, Hc), y in zip(chunks, parts):
        ON.relayout_h2s_heads(y, back, h0)
    assert np.array_equal(back, x)


def test_head_chunk_relayout_rejects_bad_ranges():
    x = np.zeros((1, 8, 8, 2), dtype=np.uint16)
    for h0, Hc in ((-1, 1), (0, 0), (3, 2), (4, 1)):  # rank slices hold 4 heads at P = 2
        with pytest.raises(RuntimeError):
            ON.relayout_s2h_heads(x, 2, h0, Hc)


# ----------------------------------------------------------------------------- planted mistakes


def _mutated(monkeypatch, which):
    """Plant one plausible mistake in the oracle (CPU only)."""
    orig_pdd = OA._p_dp_ds
    orig_group = OA._group
    orig_vis = OA._visible
    if which == "sign_of_D":
        def bad(qh_r, kg, vg, do_r, lse_r, D_r, rows, scale, causal):
            p, dp, ds = orig_pdd(qh_r, kg, vg, do_r, lse_r, D_r, rows, scale, causal)
            return p, dp, p * (dp + D_r[:, None])
        monkeypatch.setattr(OA, "_p_dp_ds", bad)
    elif which == "dropped_D":
        def bad(qh_r, kg, vg, do_r, lse_r, D_r, rows, scale, causal):
            p, dp, ds = orig_pdd(qh_r, kg, vg, do_r, lse_r, D_r, rows, scale, causal)
            return p, dp, p * dp
        monkeypatch.setattr(OA, "_p_dp_ds", bad)
    elif which == "transposed_p":
        def bad(qh_r, kg, vg, do_r, lse_r, D_r, rows, scale, causal):
            p, dp, ds = orig_pdd(qh_r, kg, vg, do_r, lse_r, D_r, rows, scale, causal)
            return p.T, dp, ds  # square at this size: dV = P dO instead of P^T dO
        monkeypatch.setattr(OA, "_p_dp_ds", bad)
    elif which == "group_mapping":
        monkeypatch.setattr(OA, "_group", lambda h, Hq, Hkv: h % Hkv)
    elif which == "mask_off_by_one":
        def bad(rows, N, causal):
            m = orig_vis(rows, N, causal)
            return np.arange(N)[None, :] < rows[:, None] + 2 if causal else m
        monkeypatch.setattr(OA, "_visible", bad)
    else:
        raise ValueError(which)
    return orig_group


@pytest.mark.parametrize("which", ["sign_of_D", "dropped_D", "transposed_p", "group_mapping",
                                   "mask_off_by_one"])
def test_planted_mistakes_are_caught(monkeypatch, which):
    B, N, Hq, Hkv, d = 1, 64, 4, 2, 16
    q, k, v, do = _qkv(B, N, Hq, Hkv, d, 170)
    scale = 0.25
    ref = _torch_ref(q, k, v, do, scale, True)
    _mutated(monkeypatch, which)
    o, lse = OA.attn_fwd(q, k, v, scale, True)
    dq, dk, dv, _, _ = OA.attn_bwd(q, k, v, do, scale, True)
    errs = [np.abs(a - b).max() for a, b in zip((o, lse, dq, dk, dv), ref)]
    assert max(errs) > 1e-3, errs
