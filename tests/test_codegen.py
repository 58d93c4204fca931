"""The dK/dV producer's early barrier, checked on the compiled gfx950 code (CPU only).

Before the barrier that hands its P / dS fragments to the consumers, a dK/dV producer waits
only until its own P / dS writes have retired, and leaves the LDS reads it issued after them
in flight (`s_waitcnt lgkmcnt(K)` rather than lgkmcnt(0); the same instruction may also wait on
the producer's own tile loads, `vmcnt(n)`).  That retires every write only
while the compiled code keeps three facts, which this test checks in the assembly of every
kernel that contains the producer (the dK/dV kernels and the merged backward kernel,
head_dim 64 and 128):
* between the last LDS write before the wait and the wait there are at least K LDS reads and
  no other LDS or scalar-memory operation (LDS operations retire in order, so once at most K
  are outstanding, everything before the last K reads, the writes included, has retired);
* the wait is the instruction right before the barrier (so nothing touches LDS in between);
* no scalar memory operation is issued after the kernel's first barrier (lgkmcnt then counts
  LDS operations only).  This one is checked on the standalone dK/dV kernels: the merged
  kernel also holds the dQ body, whose scalar loads are on a branch that no dK/dV workgroup
  takes, while its dK/dV body is the same inlined code.
K is the count the source defines, kReadsAfterPds, read from the source.
"""

import re
import shutil
import subprocess
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
CSRC = ROOT / "ulysses_sequence_parallelism_attn_amd" / "csrc"


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not Path(hipcc).exists():
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / "attn_bwd.s"
    subprocess.run([hipcc, "--offload-arch=gfx950", "-O3", "-std=c++20", "-Xclang", "-target-feature",
                    "-Xclang", "-packed-fp32-ops", f"-I{ROOT / 'include'}", "--cuda-device-only", "-S",
                    str(CSRC / "attn_bwd.hip"), "-o", str(out)], check=True, capture_output=True)
    return out.read_text()


def _kernels(text):
    """Lines of each dK/dV-containing kernel, by symbol (labels kept: they end basic blocks)."""
    out = {}
    for m in re.finditer(r"^(_Z\S*dkdv_bf16_kernel\S*):", text, re.M):
        body = text[m.end():text.index(".Lfunc_end", m.end())]  # every exit of the kernel
        out[m.group(1)] = [ln.strip() for ln in body.split("\n")
                           if ln.strip() and not ln.strip().startswith((";", ".p2align", ".loc", ".file"))]
    return out


def _is_label(x):
    return x.endswith(":") and not x.startswith("s_")


LDS = re.compile(r"^ds_")
SMEM = re.compile(r"^s_(load|buffer_load|store|buffer_store|atomic)")


def _const(src, name):
    """An integer constant of the source, following a definition by another constant's name."""
    v = re.search(rf"constexpr int {name} = (\w+);", src).group(1)
    return int(v) if v.isdigit() else _const(src, v)


def _expected_count():
    return _const((CSRC / "attn_bwd.hip").read_text(), "kReadsAfterPds")


def test_producer_waits_retire_exactly_the_pds_writes(asm):
    kernels = _kernels(asm)
    assert len(kernels) == 4, sorted(kernels)  # dkdv<64>, dkdv<128>, dq_dkdv<64>, dq_dkdv<128>
    K = _expected_count()
    assert 0 < K < 15  # lgkmcnt(15) encodes "no wait"
    for name, ins in kernels.items():
        # the producer's hand-over waits: lgkmcnt(K) right before a barrier (a
        # compiler-placed wait with the same count elsewhere guards a register use)
        wait = re.compile(rf"^s_waitcnt (vmcnt\(\d+\) )?lgkmcnt\({K}\)$")
        waits = [i for i, x in enumerate(ins) if wait.match(x) and ins[i + 1].startswith("s_barrier")]
        checked = 0
        for i in waits:
            # the straight-line code that every path runs right before the wait: back to
            # the nearest label, branch or barrier
            j = i - 1
            while j >= 0 and not (_is_label(ins[j]) or ins[j].startswith(("s_barrier", "s_branch",
                                                                           "s_cbranch"))):
                j -= 1
            seg = ins[j + 1:i]
            lds = [x for x in seg if LDS.match(x)]
            assert not any(SMEM.match(x) for x in seg), (name, i)
            if not any(x.startswith("ds_write") for x in lds) and len(lds) < K:
                continue  # too short to decide on its own (the iteration whose stores are dropped)
            # the last K LDS operations before the wait are reads: every earlier one retires
            assert len(lds) >= K and all(x.startswith("ds_read") for x in lds[-K:]), (name, i, lds[-K - 2:])
            checked += 1
        # one per unrolled producer iteration; the compiler may peel the first iteration,
        # whose stores (P = dS = 0 over LDS that is already zero) it can drop
        assert checked >= 5, (name, checked)
        if "dq_dkdv" not in name:
            first_barrier = next(i for i, x in enumerate(ins) if x.startswith("s_barrier"))
            assert not any(SMEM.match(x) for x in ins[first_barrier:]), name


def _metadata(text):
    """Per-kernel (.name -> {field: value}) from the code object's metadata block."""
    out = {}
    for blk in re.split(r"\n\s*- \.", text[text.index("amdhsa.kernels:"):]):
        name = re.search(r"\.name:\s+(\S+)", blk)
        if not name:
            continue
        fields = {k: int(v) for k, v in re.findall(r"\.?(vgpr_spill_count|sgpr_spill_count|vgpr_count|"
                                                   r"private_segment_fixed_size):\s+(\d+)", "." + blk)}
        out[name.group(1)] = fields
    return out


@pytest.fixture(scope="module")
def fwd_asm(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not Path(hipcc).exists():
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / "attn_fwd.s"
    subprocess.run([hipcc, "--offload-arch=gfx950", "-O3", "-std=c++20", "-Xclang", "-target-feature",
                    "-Xclang", "-packed-fp32-ops", f"-I{ROOT / 'include'}", "--cuda-device-only", "-S",
                    str(CSRC / "attn_fwd.hip"), "-o", str(out)], check=True, capture_output=True)
    return out.read_text()


def test_bf16_attention_kernels_keep_everything_in_registers(asm, fwd_asm):
    """Every bf16 attention kernel (forward, dQ, dK/dV and the merged backward, head_dim 64 and
    128) fits its registers without spilling to scratch memory: a spill inside their loops
    costs scratch traffic on every step (the merged backward kernel once spilled 49 registers,
    9 % of its time at N = 8192)."""
    meta = {**_metadata(asm), **_metadata(fwd_asm)}
    bf16 = {n: f for n, f in meta.items() if "bf16_kernel" in n}
    assert len(bf16) == 8, sorted(bf16)  # fwd, dq, dkdv, dq_dkdv x head_dim 64, 128
    for n, f in bf16.items():
        assert f["vgpr_spill_count"] == 0, (n, f)
        assert f["private_segment_fixed_size"] == 0, (n, f)
