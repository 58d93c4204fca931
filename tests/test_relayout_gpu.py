"""GPU parity of ul_relayout_s2h / ul_relayout_h2s against the scalar oracle: byte-equal.

Inputs are random bit patterns (every 16- or 32-bit pattern, NaN payloads included), so any
misplaced element or any pass through float registers changes the bytes.
"""

import numpy as np
import pytest

from oracle import native as ON
from ulysses_sequence_parallelism_attn_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _bits_to_device(bits: np.ndarray, dtype: str):
    t = torch.from_numpy(bits)
    return (t.view(torch.bfloat16) if dtype == "bf16" else t.view(torch.float32)).cuda()


def _device_bits(t, dtype: str) -> np.ndarray:
    host = t.cpu()
    return (host.view(torch.uint16) if dtype == "bf16" else host.view(torch.int32)).numpy().view(
        np.uint16 if dtype == "bf16" else np.uint32)


def _run_case(C, N, H, d, P, dtype, seed):
    from ulysses_sequence_parallelism_attn_amd import binding as B

    x = synth.random_bits((C, N, H, d), dtype, seed)
    y_ref = ON.relayout_s2h(x, P)
    xd = _bits_to_device(x, dtype)
    yd = B.relayout_s2h(xd, P)
    torch.cuda.synchronize()
    assert np.array_equal(_device_bits(yd, dtype), y_ref), "s2h differs from the oracle"
    # inverse on an independent head-sharded tensor, and the round trip
    z = synth.random_bits((C, P, N, H // P, d), dtype, seed + 1)
    zd = _bits_to_device(z, dtype)
    xz = B.relayout_h2s(zd)
    back = B.relayout_h2s(yd)
    torch.cuda.synchronize()
    assert np.array_equal(_device_bits(xz, dtype), ON.relayout_h2s(z)), "h2s differs from the oracle"
    assert np.array_equal(_device_bits(back, dtype), x), "h2s(s2h(x)) != x"


@pytest.mark.parametrize("C,N,H,d,P,dtype", [
    (3, 256, 4, 64, 2, "f32"),     # tiny fp32 workload's QKV stack
    (3, 4096, 32, 128, 8, "bf16"), # SP=8 slice shape
    (2, 12, 6, 3, 3, "bf16"),      # odd P, 12-byte segments (4-byte units)
    (1, 6, 3, 1, 3, "bf16"),       # 2-byte segments
    (1, 10, 4, 5, 2, "f32"),       # 40-byte segments
    (3, 64, 8, 128, 1, "bf16"),    # P = 1 is the identity layout
    (1, 1024, 8, 64, 8, "f32"),    # one head per rank
])
def test_relayout_small_shapes(C, N, H, d, P, dtype):
    _run_case(C, N, H, d, P, dtype, seed=1000 + N + H)


def test_relayout_full_size_qkv_stack():
    """The [3, 65536, 32, 128] bf16 stack at P = 4: byte-equal both ways."""
    wl = synth.WORKLOADS[3]
    C, N, H, d, P = wl.relayout
    _run_case(C, N, H, d, P, "bf16", seed=synth.seed_of(3, synth.SLOT_RELAYOUT))


def test_relayout_is_deterministic_and_writes_everything():
    from ulysses_sequence_parallelism_attn_amd import binding as B

    x = _bits_to_device(synth.random_bits((3, 512, 16, 128), "bf16", 5), "bf16")
    y1 = torch.full((3, 4, 512, 4, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    B.relayout_s2h(x, 4, out=y1)
    y2 = B.relayout_s2h(x, 4)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    assert torch.equal(B.relayout_h2s(y1).view(torch.int16), x.view(torch.int16))
