"""GPU test of ul_attn_bwd_noalloc (the backward that allocates nothing).

It runs through the C ABI and must give, call after call, exactly what ul_attn_bwd gives
for the same inputs: the same kernels read the statistics from the library's fixed per-GPU
scratch instead of a caller workspace.  Two calls in a row share that scratch, the second
with a smaller problem, so stale contents of the first call must not leak into it.
ul_attn_bwd itself is pinned to the float64 oracle by test_attn_gpu.py.
"""

import math

import pytest

from ulysses_sequence_parallelism_attn_amd import synth

from . import helpers as H

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _B():
    from ulysses_sequence_parallelism_attn_amd import binding

    return binding


def _bits(t):
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


def _case(Bsz, N, Hq, Hkv, d, dtype, seed):
    B = _B()
    st = synth.custom_inputs(Bsz, N, Hq, Hkv, d, dtype, seed=seed)
    q, k, v, do = (H.to_device(st[n], dtype) for n in ("q", "k", "v", "dout"))
    scale = 1.0 / math.sqrt(d)
    o, lse = B.attn_fwd(q, k, v, scale, True)
    return q, k, v, o, do, lse, scale


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_matches_workspace_backward_twice(dtype):
    """Two consecutive no-allocation calls (the second smaller) against ul_attn_bwd."""
    B = _B()
    d = 128 if dtype == "bf16" else 64
    cases = [(1, 1300, 8, 2, d, 11), (2, 300, 4, 1, d, 12)]  # second call: fewer rows
    for Bsz, N, Hq, Hkv, dd, seed in cases:
        print(f"[noalloc] {dtype} B={Bsz} N={N} {Hq}q{Hkv}kv d={dd}", flush=True)
        q, k, v, o, do, lse, scale = _case(Bsz, N, Hq, Hkv, dd, dtype, seed)
        ref = B.attn_bwd(q, k, v, o, do, lse, scale, True)
        got = [torch.full_like(t, float("nan")) for t in ref]
        B.attn_bwd_noalloc(q, k, v, o, do, lse, scale, True, dq=got[0], dk=got[1], dv=got[2])
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv"), got, ref):
            assert torch.equal(_bits(a), _bits(b)), f"{name} differs from ul_attn_bwd"


def test_noalloc_rejects_problems_beyond_the_scratch():
    """A problem whose statistics exceed the fixed scratch raises UL_ERR_SCRATCH and
    leaves the outputs untouched (checked on the host before any launch)."""
    B = _B()
    # B*Hq*N = 32M + 64 rows of statistics, past the 256 MiB scratch; head_dim 64 tensors
    Bsz, N, Hq, Hkv, d = 1, (1 << 23) + 16, 4, 1, 64
    q = torch.zeros((Bsz, N, Hq, d), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((Bsz, N, Hkv, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((Bsz, Hq, N), dtype=torch.float32, device="cuda")
    dq = torch.full_like(q, 7.0)
    with pytest.raises(B.UlError) as e:
        B.attn_bwd_noalloc(q, k, k.clone(), q.clone(), q.clone(), lse, 0.125, True, dq=dq)
    assert e.value.name == "UL_ERR_SCRATCH"
    torch.cuda.synchronize()
    assert bool((dq == 7.0).all())
