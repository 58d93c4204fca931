"""Pins of the packed variable-length oracle (oracle/varlen.py), CPU only.

The oracle writes the block-diagonal mask over the whole packed token axis.  It is pinned to
things other than itself:
* the per-sequence oracle (oracle/attention.py, itself pinned to closed forms, a library
  routine and finite differences) applied to each sequence sliced out on its own;
* torch CPU float64 scaled_dot_product_attention with an explicit block-diagonal mask plus
  autograd (a library routine);
* exact identities: isolation between sequences (bit-exact), the per-sequence gradient
  sums, and tokens outside every sequence;
* central finite differences of L = <dO, O>;
* a planted mistake (the sequence term of the mask dropped) that these checks catch.
"""


import numpy as np
import pytest
import torch

from oracle import attention as OA
from oracle import varlen as OV


def _rand(shape, seed):
    return np.random.Generator(np.random.PCG64(seed)).standard_normal(shape)


def _packed(T, Hq, Hkv, d, seed):
    return (_rand((T, Hq, d), seed), _rand((T, Hkv, d), seed + 1), _rand((T, Hkv, d), seed + 2),
            _rand((T, Hq, d), seed + 3))


def _cu(lengths):
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)


LENGTHS = [1, 63, 0, 64, 65, 30]


@pytest.mark.parametrize("causal", [True, False])
def test_single_sequence_equals_plain_oracle(causal):
    T, Hq, Hkv, d = 90, 4, 2, 16
    q, k, v, do = _packed(T, Hq, Hkv, d, 300)
    dq, dk, dv, o, lse = OV.attn_varlen_bwd(q, k, v, do, [0, T], 0.25, causal)
    rdq, rdk, rdv, ro, rlse = OA.attn_bwd(q[None], k[None], v[None], do[None], 0.25, causal)
    for a, b in ((o, ro[0]), (lse, rlse[0]), (dq, rdq[0]), (dk, rdk[0]), (dv, rdv[0])):
        np.testing.assert_allclose(a, b, atol=1e-12)


@pytest.mark.parametrize("causal", [True, False])
def test_matches_per_sequence_oracle(causal):
    Hq, Hkv, d = 4, 1, 8
    cu = _cu(LENGTHS)
    T = int(cu[-1])
    q, k, v, do = _packed(T, Hq, Hkv, d, 310)
    dq, dk, dv, o, lse = OV.attn_varlen_bwd(q, k, v, do, cu, 0.3, causal)
    for s in range(len(LENGTHS)):
        a, b = cu[s], cu[s + 1]
        if a == b:
            continue
        rdq, rdk, rdv, ro, rlse = OA.attn_bwd(q[None, a:b], k[None, a:b], v[None, a:b],
                                              do[None, a:b], 0.3, causal)
        np.testing.assert_allclose(o[a:b], ro[0], atol=1e-12)
        np.testing.assert_allclose(lse[:, a:b], rlse[0], atol=1e-12)
        np.testing.assert_allclose(dq[a:b], rdq[0], atol=1e-11)
        np.testing.assert_allclose(dk[a:b], rdk[0], atol=1e-11)
        np.testing.assert_allclose(dv[a:b], rdv[0], atol=1e-11)


def _torch_block_diag(q, k, v, do, cu, scale, causal):
    """torch CPU float64 SDPA with an explicit boolean block-diagonal mask, plus autograd."""
    T, Hq, _ = q.shape
    Hkv = k.shape[1]
    seg = np.full(T, -1)
    for s in range(len(cu) - 1):
        seg[cu[s]:cu[s + 1]] = s
    allow = torch.tensor((seg[:, None] == seg[None, :]) &
                         (np.tril(np.ones((T, T), bool)) if causal else True))
    tq = torch.tensor(q).permute(1, 0, 2).contiguous().requires_grad_(True)
    tk = torch.tensor(k).permute(1, 0, 2).contiguous().requires_grad_(True)
    tv = torch.tensor(v).permute(1, 0, 2).contiguous().requires_grad_(True)
    kr = tk.repeat_interleave(Hq // Hkv, dim=0)
    vr = tv.repeat_interleave(Hq // Hkv, dim=0)
    o = torch.nn.functional.scaled_dot_product_attention(tq, kr, vr, attn_mask=allow, scale=scale)
    o.backward(torch.tensor(do).permute(1, 0, 2))
    tr = lambda t: t.detach().permute(1, 0, 2).numpy()
    return tr(o), tr(tq.grad), tr(tk.grad), tr(tv.grad)


@pytest.mark.parametrize("causal", [True, False])
def test_matches_torch_block_diagonal_sdpa(causal):
    Hq, Hkv, d = 4, 2, 16
    lengths = [5, 17, 1, 40]  # every token covered (SDPA gives NaN for fully masked rows)
    cu = _cu(lengths)
    T = int(cu[-1])
    q, k, v, do = _packed(T, Hq, Hkv, d, 320)
    to, tdq, tdk, tdv = _torch_block_diag(q, k, v, do, cu, 0.25, causal)
    dq, dk, dv, o, _ = OV.attn_varlen_bwd(q, k, v, do, cu, 0.25, causal)
    np.testing.assert_allclose(o, to, atol=1e-12)
    np.testing.assert_allclose(dq, tdq, atol=1e-11)
    np.testing.assert_allclose(dk, tdk, atol=1e-11)
    np.testing.assert_allclose(dv, tdv, atol=1e-11)


def test_sequences_are_isolated_bitwise():
    """Changing every input of one sequence leaves every other sequence's results bit-identical."""
    Hq, Hkv, d = 2, 1, 8
    cu = _cu(LENGTHS)
    T = int(cu[-1])
    q, k, v, do = _packed(T, Hq, Hkv, d, 330)
    r1 = OV.attn_varlen_bwd(q, k, v, do, cu, 0.3, True)
    a, b = cu[3], cu[4]
    q2, k2, v2, do2 = (x.copy() for x in (q, k, v, do))
    for x in (q2, k2, v2, do2):
        x[a:b] = -3 * x[a:b] + 1
    r2 = OV.attn_varlen_bwd(q2, k2, v2, do2, cu, 0.3, True)
    keep = np.r_[0:a, b:T]
    for x1, x2 in zip(r1, r2):
        if x1.shape[0] == T:
            assert np.array_equal(x1[keep], x2[keep])
            assert not np.array_equal(x1[a:b], x2[a:b])
        else:  # lse [Hq, T]
            assert np.array_equal(x1[:, keep], x2[:, keep])


def test_per_sequence_gradient_identities():
    """Within each sequence and KV group: sum_j dK_j = 0 (a shift of that sequence's keys
    changes no probability) and sum_j dV_j = sum of the group's dO over the sequence (rows
    of P sum to 1 inside the sequence)."""
    Hq, Hkv, d = 4, 2, 8
    cu = _cu(LENGTHS)
    T = int(cu[-1])
    q, k, v, do = _packed(T, Hq, Hkv, d, 340)
    _, dk, dv, _, _ = OV.attn_varlen_bwd(q, k, v, do, cu, 0.4, True)
    for s in range(len(LENGTHS)):
        a, b = cu[s], cu[s + 1]
        for g in range(Hkv):
            heads = slice(g * 2, g * 2 + 2)
            np.testing.assert_allclose(dk[a:b, g].sum(axis=0), 0.0, atol=1e-12)
            np.testing.assert_allclose(dv[a:b, g].sum(axis=0), do[a:b, heads].sum(axis=(0, 1)),
                                       atol=1e-12)


def test_tokens_outside_every_sequence():
    """cu need not cover the whole axis: uncovered tokens give NaN outputs and no gradient,
    and the covered ones are unaffected."""
    Hq, Hkv, d = 2, 2, 4
    T = 20
    q, k, v, do = _packed(T, Hq, Hkv, d, 350)
    cu = [3, 8, 15]
    dq, dk, dv, o, lse = OV.attn_varlen_bwd(q, k, v, do, cu, 0.5, True)
    out = np.r_[0:3, 15:20]
    assert np.isnan(o[out]).all() and np.isnan(lse[:, out]).all()
    assert (dq[out] == 0).all() and (dk[out] == 0).all() and (dv[out] == 0).all()
    ref = OV.attn_varlen_bwd(q[3:15], k[3:15], v[3:15], do[3:15], [0, 5, 12], 0.5, True)
    for x, r in zip((dq, dk, dv, o), ref[:4]):  # equal up to the products' summation order
        np.testing.assert_allclose(x[3:15], r, atol=1e-13)


def test_varlen_gradients_match_central_differences():
    Hq, Hkv, d = 2, 1, 3
    cu = _cu([3, 1, 4])
    T = int(cu[-1])
    q, k, v, do = _packed(T, Hq, Hkv, d, 360)
    dq, dk, dv, _, _ = OV.attn_varlen_bwd(q, k, v, do, cu, 0.7, True)

    def L(args):
        return float(np.sum(do * OV.attn_varlen_fwd(args["q"], args["k"], args["v"], cu, 0.7,
                                                     True)[0]))

    h = 1e-6
    base = {"q": q, "k": k, "v": v}
    for name, grad in (("q", dq), ("k", dk), ("v", dv)):
        num = np.zeros_like(base[name])
        for idx in np.ndindex(num.shape):
            a1, a2 = dict(base), dict(base)
            a1[name] = base[name].copy()
            a2[name] = base[name].copy()
            a1[name][idx] += h
            a2[name][idx] -= h
            num[idx] = (L(a1) - L(a2)) / (2 * h)
        err = np.abs(num - grad).max() / np.abs(grad).max()
        assert err <= 1e-7, (name, err)


def test_planted_mask_mistake_is_caught(monkeypatch):
    """Dropping the same-sequence term of the mask (plain causal attention over the packed
    axis) is caught by the library cross-check."""
    Hq, Hkv, d = 2, 1, 8
    cu = _cu([10, 20, 7])
    T = int(cu[-1])
    q, k, v, do = _packed(T, Hq, Hkv, d, 370)
    to, tdq, tdk, tdv = _torch_block_diag(q, k, v, do, cu, 0.35, True)

    def plain_causal(seg, rows, causal):
        return np.arange(len(seg))[None, :] <= rows[:, None]

    monkeypatch.setattr(OV, "_mask", plain_causal)
    dq, dk, dv, o, _ = OV.attn_varlen_bwd(q, k, v, do, cu, 0.35, True)
    errs = [np.abs(a - b).max() for a, b in ((o, to), (dq, tdq), (dk, tdk), (dv, tdv))]
    assert max(errs) > 1e-3, errs
