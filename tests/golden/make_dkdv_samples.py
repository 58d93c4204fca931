#!/usr/bin/env python3
"""Write the stored expected dK/dV rows at sampled keys for the long workloads.

The fp64 oracle needs the statistics (lse, D) of every query row that sees a key, i.e. a
full forward over the sequence, to give dK and dV of a key near the start.  That takes
minutes of CPU at N = 65536 and 98304, far too long for a test, so this script computes
them once from the oracle alone and stores the results next to it:

    tests/golden/dkdv_samples_w<id>.npz   keys_g<g>, dk_g<g>, dv_g<g> (float32), meta

Keys per KV head g: 512 drawn uniformly (seeded, ``synth.sample_keys``) plus the fixed
keys {0, 1, 127, 128, N/2}; for the million-token workload the draws come from the last
16384 positions, where the query rows that see a key are few enough to run through the
oracle here.  Every value comes from ``oracle.attention.dkdv_rows`` on the seeded inputs;
the only arithmetic outside the oracle is the sum of the per-query-head contributions of
a KV group (the oracle's dkdv_rows sums the same terms when given the group's heads at
once; it is split by head here so the heads run in parallel processes).

Usage: python tests/golden/make_dkdv_samples.py [workload ids ...]   (default 3 4 5)
On a host where freshly touched memory is slow, MALLOC_MMAP_MAX_=0 and a large
MALLOC_TRIM_THRESHOLD_ keep numpy's freed blocks for reuse.
"""

from __future__ import annotations

import multiprocessing as mp
import os
import sys
import time
from pathlib import Path

import numpy as np

ROOT = Path(__file__).resolve().parents[2]
sys.path.insert(0, str(ROOT))

from oracle import attention as OA  # noqa: E402
from ulysses_sequence_parallelism_attn_amd import synth  # noqa: E402

OUT = Path(__file__).resolve().parent
WINDOW = {3: None, 4: None, 5: 16384}

_ST: dict = {}


def _head_job(args):
    wid, h, keys = args
    wl = synth.WORKLOADS[wid]
    g = h // (wl.Hq // wl.Hkv)
    st = _ST[wid]
    one = lambda name, hh: OA.widen(np.ascontiguousarray(st[name][:, :, hh:hh + 1]), wl.dtype)
    t0 = time.time()
    dk, dv = OA.dkdv_rows(one("q", h), one("k", g), one("v", g), one("dout", h), wl.scale,
                          wl.causal, keys)
    print(f"  w{wid} head {h}: {len(keys)} keys in {time.time() - t0:.0f} s", flush=True)
    return h, dk[0, :, 0], dv[0, :, 0]


def make(wid: int, procs: int) -> Path:
    wl = synth.WORKLOADS[wid]
    t0 = time.time()
    _ST[wid] = synth.attn_inputs(wl)
    print(f"w{wid} {wl.name}: inputs in {time.time() - t0:.0f} s", flush=True)
    keys = {g: synth.sample_keys(wl, g, window=WINDOW[wid]) for g in range(wl.Hkv)}
    grp = wl.Hq // wl.Hkv
    jobs = [(wid, h, keys[h // grp]) for h in range(wl.Hq)]
    ctx = mp.get_context("fork")
    with ctx.Pool(min(procs, len(jobs))) as pool:
        parts = pool.map(_head_job, jobs, chunksize=1)
    out = {}
    for g in range(wl.Hkv):
        dk = sum(p[1] for p in parts if p[0] // grp == g)
        dv = sum(p[2] for p in parts if p[0] // grp == g)
        out[f"keys_g{g}"] = keys[g]
        out[f"dk_g{g}"] = dk.astype(np.float32)
        out[f"dv_g{g}"] = dv.astype(np.float32)
    out["meta"] = np.array(f"{wl.name}; window={WINDOW[wid]}; oracle.attention.dkdv_rows, fp64, "
                           f"stored as float32")
    path = OUT / f"dkdv_samples_w{wid}.npz"
    np.savez_compressed(path, **out)
    del _ST[wid]
    print(f"w{wid}: wrote {path} in {time.time() - t0:.0f} s", flush=True)
    return path


if __name__ == "__main__":
    ids = [int(a) for a in sys.argv[1:]] or [3, 4, 5]
    procs = int(os.environ.get("PROCS", "8"))
    for wid in ids:
        make(wid, procs)
