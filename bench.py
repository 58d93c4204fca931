#!/usr/bin/env python3
"""Benchmark of the per-rank Ulysses hot path on one MI355X.

One step is one pass of the whole path over one batch of synthetic input:

  1. ul_relayout_s2h of a [3, 65536, 32, 128] bf16 QKV stack at P = 4
     (the sequence -> head exchange, as a single-GPU permutation);
  2. ul_attn_fwd: causal attention for one SP=4 rank of a Llama-3.1-8B-shaped layer
     (N = 65536, 8 query heads, 2 KV heads, head_dim 128, bf16);
  3. ul_attn_bwd: its dQ, dK, dV;
  4. ul_relayout_h2s of the [3, 4, 65536, 8, 128] head-sharded stack (the reverse exchange).

The headline value is counted attention FLOPs per second over whole steps: causal
forward 2*N^2*Hq*d plus backward 2.5x that (7*N^2*Hq*d per step), in TFLOP/s.  The
relayouts add time but no FLOPs.  Inputs are resident in HBM before timing starts.

Prints ONE JSON line (rank 0).  Runs on one GPU only.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

METRIC = "causal attn fwd+bwd TFLOP/s and % bf16 MFMA peak at N=64K, 8q/2kv heads"
PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 4096 dense bf16 FLOP/clk/CU x 2.4 GHz
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
TRAFFIC_FILE = ROOT / "profiles" / "traffic.json"
KERNEL_SOURCES = ["attn_fwd.hip", "attn_bwd.hip", "relayout.hip", "mfma_tile.h"]


def kernel_hash() -> str:
    h = hashlib.sha256()
    for n in KERNEL_SOURCES:
        h.update((ROOT / "ulysses_sequence_parallelism_attn_amd" / "csrc" / n).read_bytes())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str) -> float | None:
    """HBM bytes per launch from the committed PMC measurement, if the kernels are unchanged."""
    try:
        rec = json.loads(TRAFFIC_FILE.read_text())
    except (OSError, ValueError):
        return None
    if rec.get("kernel_hash") != kernel_hash():
        return None
    v = rec.get("bytes_per_launch", {}).get(kernel)
    return float(v) if v is not None else None


def cpu_baseline(st: dict, wl, n_prefix: int) -> dict:
    """Time the float64 oracle on a causal prefix of the workload's own inputs."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import attention as OA

    w = {n: OA.widen(a[:, :n_prefix], wl.dtype) for n, a in st.items()}
    t0 = time.perf_counter()
    OA.attn_bwd(w["q"], w["k"], w["v"], w["dout"], wl.scale, True)  # forward + backward
    dt = time.perf_counter() - t0
    flops = 7.0 * n_prefix ** 2 * wl.Hq * wl.d
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"float64 oracle forward+backward on the causal prefix N={n_prefix} of the "
                   f"N={wl.N} inputs (all {wl.Hq} query / {wl.Hkv} KV heads, d={wl.d}); "
                   f"{dt:.1f} s wall, rate in counted FLOPs (7*N^2*Hq*d)"),
        "seconds": dt,
    }


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=3, help="attention workload id (default 3)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-prefix", type=int, default=8192)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run one 1 GiB device-to-device copy first (a known-size reference for "
                         "HBM byte counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (--gpus {args.gpus}, WORLD_SIZE {world} requested); "
              "the multi-GPU exchange is not part of this build.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from ulysses_sequence_parallelism_attn_amd import binding as B
    from ulysses_sequence_parallelism_attn_amd import synth

    wl = synth.WORKLOADS[args.workload]
    rl = synth.WORKLOADS[3].relayout  # (C, N, H, d, P)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    st = synth.attn_inputs(wl)
    up = lambda a: torch.from_numpy(a).view(torch.bfloat16).to(dev)
    q, k, v, do = (up(st[n]) for n in ("q", "k", "v", "dout"))
    C, Nr, Hr, dr, P = rl
    gen = torch.Generator(device=dev)
    gen.manual_seed(synth.seed_of(3, synth.SLOT_RELAYOUT))
    x = torch.randint(-32768, 32767, (C, Nr, Hr, dr), dtype=torch.int16, device=dev,
                      generator=gen).view(torch.bfloat16)
    y = torch.empty((C, P, Nr, Hr // P, dr), dtype=torch.bfloat16, device=dev)
    x2 = torch.empty_like(x)
    o = torch.empty_like(q)
    lse = torch.empty((wl.B, wl.Hq, wl.N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(B.workspace_bytes(wl.B, wl.N, wl.Hq, wl.Hkv, wl.d, B.UL_BF16),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        src.fill_(1)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        B.relayout_s2h(x, P, out=y)
        if ev is not None:
            ev[1].record(stream)
        B.attn_fwd(q, k, v, wl.scale, True, out=o, lse=lse)
        if ev is not None:
            ev[2].record(stream)
        B.attn_bwd(q, k, v, o, do, lse, wl.scale, True, workspace=ws, dq=dq, dk=dk, dv=dv)
        if ev is not None:
            ev[3].record(stream)
        B.relayout_h2s(y, out=x2)
        if ev is not None:
            ev[4].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        step(evs[i])
    t_end.record(stream)
    torch.cuda.synchronize()

    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps
    parts = {"relayout_s2h": [], "attn_fwd": [], "attn_bwd": [], "relayout_h2s": []}
    for e in evs:
        for j, name in enumerate(parts):
            parts[name].append(e[j].elapsed_time(e[j + 1]))
    avg = {n: sum(v) / len(v) for n, v in parts.items()}

    f_fwd = wl.flops_fwd()
    f_bwd = wl.flops_bwd()
    flops_step = f_fwd + f_bwd
    value = flops_step / (ms_per_step * 1e-3) / 1e12
    rl_bytes = 2.0 * C * Nr * Hr * dr * 2
    roof = {
        "attn_bwd": {"bound": "mfma", "achieved": f_bwd / (avg["attn_bwd"] * 1e-3) / 1e12,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s"},
        "attn_fwd": {"bound": "mfma", "achieved": f_fwd / (avg["attn_fwd"] * 1e-3) / 1e12,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s"},
        "relayout_s2h": {"bound": "hbm", "achieved": rl_bytes / (avg["relayout_s2h"] * 1e-3) / 1e9,
                         "peak": PEAK_HBM_GBS, "unit": "GB/s"},
        "relayout_h2s": {"bound": "hbm", "achieved": rl_bytes / (avg["relayout_h2s"] * 1e-3) / 1e9,
                         "peak": PEAK_HBM_GBS, "unit": "GB/s"},
    }
    for n, r in roof.items():
        r["frac"] = r["achieved"] / r["peak"]
        r["ms"] = avg[n]
        r["traffic"] = measured_traffic(n)
    dominant = max(avg, key=avg.get)
    dom = dict(roof[dominant])
    dom.pop("ms")
    dom["kernel"] = dominant

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) Q/K/V/dO; random-bit relayout stack)",
        "config": {"workload": wl.name, "B": wl.B, "seq_len": wl.N, "q_heads": wl.Hq,
                   "kv_heads": wl.Hkv, "head_dim": wl.d, "causal": True,
                   "relayout": {"shape": [C, Nr, Hr, dr], "P": P}, "parallelism": "sp4-rank-share"},
        "pct_bf16_peak": 100.0 * value / PEAK_BF16_TFLOPS,
        "attn_fwd_bwd_tflops": flops_step / ((avg["attn_fwd"] + avg["attn_bwd"]) * 1e-3) / 1e12,
        "tokens_per_s": wl.B * wl.N / (ms_per_step * 1e-3),
        "roofline": dom,
        "roofline_all": roof,
        "kernel_hash": kernel_hash(),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(st, wl, min(args.cpu_prefix, wl.N))
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
