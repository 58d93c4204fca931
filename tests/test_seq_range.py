"""The packed-sequence table clamp (seq_range in csrc/ul_internal.h), run on the host.

The varlen kernels read their table from device memory, so the host cannot validate it;
instead every kernel maps its sequence through seq_range, which must keep every token range
inside [0, total] and no longer than the caller's maximum for ANY table contents.  This
compiles that same header function for the CPU and checks the bound on random and
adversarial tables (negative, decreasing, past-the-end and INT32 extreme entries), plus the
exact ranges of well-formed tables.
"""

import shutil
import subprocess

import numpy as np
import pytest

from pathlib import Path

HERE = Path(__file__).resolve().parent
SRC = HERE / "native" / "seq_range_host.cpp"


@pytest.fixture(scope="module")
def exe(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not Path(hipcc).exists():
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("seqrange") / "seq_range_host"
    # host-only HIP compile: the header's HIP attributes, no device code
    subprocess.run([hipcc, "-O1", "-std=c++20", "-x", "hip", "--cuda-host-only", str(SRC), "-o",
                    str(out)], check=True, capture_output=True)
    return out


def _run(exe, cases):
    text = "".join(f"{t} {N} {Hq} {len(cu) - 1} " + " ".join(str(int(x)) for x in cu) + "\n"
                   for t, N, Hq, cu in cases)
    res = subprocess.run([str(exe)], input=text, capture_output=True, text=True, check=True)
    rows = [tuple(int(x) for x in line.split()) for line in res.stdout.splitlines()]
    out, i = [], 0
    for t, N, Hq, cu in cases:
        out.append(rows[i:i + len(cu) - 1])
        i += len(cu) - 1
    return out


def test_well_formed_tables_give_their_ranges(exe):
    cu = [0, 5, 5, 70, 300]
    (got,) = _run(exe, [(300, 230, 4, cu)])
    for b, (tok0, ln, lse0, st0, hs) in enumerate(got):
        assert (tok0, ln) == (cu[b], cu[b + 1] - cu[b])
        assert lse0 == tok0 and st0 == tok0 and hs == 300


def test_fixed_length_batches_without_a_table(exe):
    res = subprocess.run([str(exe)], input="-1 700 8 3\n", capture_output=True, text=True,
                         check=True)
    rows = [tuple(int(x) for x in line.split()) for line in res.stdout.splitlines()]
    for b, (tok0, ln, lse0, st0, hs) in enumerate(rows):
        assert (tok0, ln, lse0, st0, hs) == (b * 700, 700, b * 8 * 700, 2 * b * 8 * 700, 700)


def test_any_table_stays_inside_the_tensors(exe):
    rng = np.random.Generator(np.random.PCG64(700))
    extremes = np.array([-2**31, -1, 0, 1, 2**31 - 1], dtype=np.int64)
    cases = []
    for _ in range(300):
        total = int(rng.integers(1, 5000))
        N = int(rng.integers(1, total + 1))
        n = int(rng.integers(1, 12))
        kind = rng.integers(0, 3)
        if kind == 0:    # arbitrary values around the valid range
            cu = rng.integers(-total, 2 * total + 1, size=n + 1)
        elif kind == 1:  # decreasing
            cu = np.sort(rng.integers(-10, total + 10, size=n + 1))[::-1]
        else:            # int32 extremes mixed in
            cu = rng.choice(np.concatenate([extremes, rng.integers(0, total + 1, size=4)]), n + 1)
        cases.append((total, N, 4, cu))
    for (total, N, _, cu), got in zip(cases, _run(exe, cases)):
        for tok0, ln, lse0, st0, hs in got:
            assert 0 <= tok0 <= total and 0 <= ln <= N and tok0 + ln <= total
            assert lse0 == tok0 and st0 == tok0 and hs == total
