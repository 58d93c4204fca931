"""CPU tests of the binding's argument checks (no GPU, no library call).

Every public call of the binding checks that its tensors agree with q (or with the relayout
input) in shape, dtype and device before any ctypes call, so that no mis-shaped buffer can
reach a kernel.  The checks are pure Python; here they run on host tensors with
device_type="cpu", and a tensor on the meta device stands in for one on another device.
"""

import pytest
import torch

from ulysses_sequence_parallelism_attn_amd import binding as B

bf, f32 = torch.bfloat16, torch.float32


def _fwd(B_=1, N=40, Hq=8, Hkv=2, d=128, dt=bf):
    q = torch.empty(B_, N, Hq, d, dtype=dt)
    k = torch.empty(B_, N, Hkv, d, dtype=dt)
    v = torch.empty(B_, N, Hkv, d, dtype=dt)
    o = torch.empty(B_, N, Hq, d, dtype=dt)
    lse = torch.empty(B_, Hq, N, dtype=f32)
    return dict(q=q, k=k, v=v, out=o, lse=lse)


def _bwd(**kw):
    a = _fwd(**kw)
    q, k = a["q"], a["k"]
    return dict(q=q, k=k, v=a["v"], o=a["out"], dout=torch.empty_like(q), lse=a["lse"],
                dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(k))


def test_forward_accepts_matching_tensors():
    B.check_attn_fwd(**_fwd(), device_type="cpu")
    B.check_attn_fwd(**_fwd(B_=2, N=7, Hq=4, Hkv=4, d=64, dt=f32), device_type="cpu")
    # a rank's head slice of a world tensor (token-strided view) is accepted
    world = torch.empty(1, 40, 32, 128, dtype=bf)
    a = _fwd()
    a["q"] = world[:, :, 8:16]
    B.check_attn_fwd(**a, device_type="cpu")


@pytest.mark.parametrize("name,bad", [
    ("k", torch.empty(1, 39, 2, 128, dtype=bf)),       # short k
    ("v", torch.empty(1, 40, 1, 128, dtype=bf)),       # v does not match k
    ("k", torch.empty(1, 40, 2, 64, dtype=bf)),        # head dim differs from q
    ("k", torch.empty(2, 40, 2, 128, dtype=bf)),       # batch differs
    ("out", torch.empty(1, 40, 8, 127, dtype=bf)),     # short out
    ("out", torch.empty(1, 40, 8, 128, dtype=f32)),    # out dtype
    ("lse", torch.empty(1, 8, 39, dtype=f32)),         # short lse
    ("lse", torch.empty(1, 40, 8, dtype=f32)),         # lse in the wrong layout
    ("lse", torch.empty(1, 8, 40, dtype=torch.float64)),
    ("lse", torch.empty(1, 8, 80, dtype=f32)[:, :, ::2]),  # non-contiguous lse
    ("k", torch.empty(1, 40, 2, 128, dtype=f32)),      # fp32 k with bf16 q
    ("v", torch.empty(1, 40, 2, 128, dtype=bf, device="meta")),  # another device
])
def test_forward_rejects(name, bad):
    a = _fwd()
    a[name] = bad
    with pytest.raises(ValueError):
        B.check_attn_fwd(**a, device_type="cpu")


def test_forward_rejects_unsupported_dtype_and_rank():
    a = {n: t.to(torch.float16) if n != "lse" else t for n, t in _fwd().items()}
    with pytest.raises(ValueError):
        B.check_attn_fwd(**a, device_type="cpu")
    a = _fwd()
    a["q"] = a["q"][0]
    with pytest.raises(ValueError):
        B.check_attn_fwd(**a, device_type="cpu")


def test_device_type_is_enforced():
    with pytest.raises(ValueError):
        B.check_attn_fwd(**_fwd())  # host tensors where device tensors are required


@pytest.mark.parametrize("name,shape,dtype", [
    ("dout", (1, 40, 8, 64), bf), ("dq", (1, 40, 2, 128), bf), ("dk", (1, 40, 8, 128), bf),
    ("dv", (1, 41, 2, 128), bf), ("dq", (1, 40, 8, 128), f32), ("dout", (1, 40, 8, 128), f32),
])
def test_backward_rejects(name, shape, dtype):
    a = _bwd()
    B.check_attn_bwd(**a, device_type="cpu")
    a[name] = torch.empty(*shape, dtype=dtype)
    with pytest.raises(ValueError):
        B.check_attn_bwd(**a, device_type="cpu")


def test_workspace_checks():
    q = torch.empty(1, 4, 2, 64, dtype=bf)
    B.check_workspace(torch.empty(512, dtype=torch.uint8), 512, q, device_type="cpu")
    for ws in (torch.empty(511, dtype=torch.uint8), torch.empty(512, dtype=torch.int8),
               torch.empty(1024, dtype=torch.uint8)[::2]):
        with pytest.raises(ValueError):
            B.check_workspace(ws, 512, q, device_type="cpu")


def _varlen(T=100, Hq=8, Hkv=2, d=128):
    return dict(q=torch.empty(T, Hq, d, dtype=bf), k=torch.empty(T, Hkv, d, dtype=bf),
                v=torch.empty(T, Hkv, d, dtype=bf), out=torch.empty(T, Hq, d, dtype=bf),
                lse=torch.empty(Hq, T, dtype=f32),
                cu_seqlens=torch.tensor([0, 30, 100], dtype=torch.int32))


@pytest.mark.parametrize("name,bad", [
    ("k", torch.empty(99, 2, 128, dtype=bf)),
    ("out", torch.empty(100, 8, 64, dtype=bf)),
    ("lse", torch.empty(100, 8, dtype=f32)),
    ("cu_seqlens", torch.tensor([0, 30, 100], dtype=torch.int64)),
    ("cu_seqlens", torch.empty(0, dtype=torch.int32)),
    ("q", torch.empty(100, 16, 128, dtype=bf)[:, ::2]),
])
def test_varlen_rejects(name, bad):
    a = _varlen()
    B.check_attn_varlen(**a, device_type="cpu")
    a[name] = bad
    with pytest.raises(ValueError):
        B.check_attn_varlen(**a, device_type="cpu")


def test_varlen_gradients_checked():
    a = _varlen()
    q, k = a["q"], a["k"]
    good = (torch.empty_like(q), torch.empty_like(q), torch.empty_like(k), torch.empty_like(k))
    B.check_attn_varlen(**a, device_type="cpu", grads=good)
    bad = (good[0], good[1], torch.empty(100, 2, 64, dtype=bf), good[3])
    with pytest.raises(ValueError):
        B.check_attn_varlen(**a, device_type="cpu", grads=bad)


def test_relayout_checks():
    x = torch.empty(3, 16, 8, 64, dtype=bf)
    B.check_relayout(x, torch.empty(3, 4, 16, 2, 64, dtype=bf), (3, 4, 16, 2, 64), "cpu")
    for out in (torch.empty(3, 4, 16, 2, 63, dtype=bf), torch.empty(3, 4, 16, 2, 64, dtype=f32),
                torch.empty(3, 4, 16, 4, 64, dtype=bf)[:, :, :, ::2]):
        with pytest.raises(ValueError):
            B.check_relayout(x, out, (3, 4, 16, 2, 64), "cpu")
    with pytest.raises(ValueError):
        B.check_relayout(x[:, :, ::2], torch.empty(3, 4, 16, 1, 64, dtype=bf), (3, 4, 16, 1, 64),
                         "cpu")


def test_public_calls_check_before_the_library(monkeypatch):
    """Mis-shaped calls raise ValueError before the binding touches the library."""

    def no_lib():
        raise AssertionError("the library was called")

    monkeypatch.setattr(B, "lib", no_lib)
    a = _fwd()
    with pytest.raises(ValueError):
        B.attn_fwd(a["q"], a["k"][:, :-1], a["v"])
    g = _bwd()
    with pytest.raises(ValueError):
        B.attn_bwd(g["q"], g["k"], g["v"], g["o"], g["dout"], g["lse"], dq=g["dq"][:, :-1])
    with pytest.raises(ValueError):
        B.relayout_s2h(torch.empty(3, 16, 8, 64, dtype=bf), 4,
                       out=torch.empty(3, 4, 16, 2, 32, dtype=bf))
    with pytest.raises(ValueError):
        B.relayout_h2s(torch.empty(3, 4, 16, 2, 64, dtype=bf),
                       out=torch.empty(3, 16, 8, 32, dtype=bf))
    v = _varlen()
    with pytest.raises(ValueError):
        B.attn_fwd_varlen(v["q"], v["k"], v["v"], v["cu_seqlens"], 70)
