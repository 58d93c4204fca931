"""GPU test: one rank's step captured in a HIP graph replays exactly what eager calls give.

The library allocates nothing, synchronises nothing and issues no memset, so every entry
point can be recorded into a graph once its buffers exist: the exchange (s2h), the forward
with its key-range split workspace, the backward with its workspace (whose short-sequence
plan merges both passes and sums head-split partials), the backward without a workspace
(ul_attn_bwd_noalloc, for callers that cannot allocate), and the reverse exchange.  The graph
is replayed three times with the program's own eager work and synchronisations in between,
and every replay must be bit-identical to the eager results.  The eager calls are pinned to
the float64 oracle by the other GPU tests.
"""

import math

import numpy as np
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


@pytest.mark.parametrize("N", [4096, 1000])
def test_step_replays_bit_identically_in_a_hip_graph(N):
    B = _B()
    Hq, Hkv, d, P = 8, 2, 128, 4
    print(f"[graph] N={N}", flush=True)
    scale = 1.0 / math.sqrt(d)
    st = synth.custom_inputs(1, N, Hq, Hkv, d, "bf16", seed=N + 17)
    q, k, v, do = (H.to_device(st[n], "bf16") for n in ("q", "k", "v", "dout"))
    rng = np.random.Generator(np.random.PCG64(N + 18))
    x = torch.from_numpy(rng.integers(-32768, 32767, size=(3, N, 16, d), dtype=np.int16)).cuda().view(torch.bfloat16)
    fws_n = B.fwd_workspace_bytes(1, N, Hq, Hkv, d, B.UL_BF16)
    assert fws_n > 0, "the forward of these sizes takes its split path"
    fws = torch.empty(fws_n, dtype=torch.uint8, device="cuda")
    bws = torch.empty(B.workspace_bytes(1, N, Hq, Hkv, d, B.UL_BF16), dtype=torch.uint8, device="cuda")
    out = {
        "y": torch.empty((3, P, N, 16 // P, d), dtype=torch.bfloat16, device="cuda"),
        "x2": torch.empty_like(x),
        "o": torch.empty_like(q),
        "lse": torch.empty((1, Hq, N), dtype=torch.float32, device="cuda"),
        "dq": torch.empty_like(q), "dk": torch.empty_like(k), "dv": torch.empty_like(v),
        "dq2": torch.empty_like(q), "dk2": torch.empty_like(k), "dv2": torch.empty_like(v),
    }

    def step():
        B.relayout_s2h(x, P, out=out["y"])
        B.attn_fwd(q, k, v, scale, True, out=out["o"], lse=out["lse"], workspace=fws)
        B.attn_bwd(q, k, v, out["o"], do, out["lse"], scale, True, workspace=bws, dq=out["dq"],
                   dk=out["dk"], dv=out["dv"])
        B.attn_bwd_noalloc(q, k, v, out["o"], do, out["lse"], scale, True, dq=out["dq2"],
                           dk=out["dk2"], dv=out["dv2"])
        B.relayout_h2s(out["y"], out=out["x2"])

    # eager reference (also resolves the no-alloc scratch address before capture)
    step()
    torch.cuda.synchronize()
    ref = {n: t.clone() for n, t in out.items()}
    assert torch.equal(_bits(ref["x2"]), _bits(x)), "h2s(s2h(x)) is x"
    for n in ("dq", "dk", "dv"):
        assert torch.equal(_bits(ref[n]), _bits(ref[n + "2"])), f"no-alloc {n} differs from ul_attn_bwd"

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in out.values():  # poison every output between replays
            t.view(torch.uint8).fill_(0xFF)
        scratch = torch.randn((1 << 20,), device="cuda").sum()  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(scratch)
        for n, t in out.items():
            assert torch.equal(_bits(t), _bits(ref[n])), f"replay {rep}: {n} differs from the eager call"
