#!/usr/bin/env python3
"""Benchmark of the per-rank Ulysses hot path on one MI355X.

One step is one pass of the whole path over one batch of synthetic input:

  1. ul_relayout_s2h of the layer's [3, N, 32, 128] bf16 QKV stack at P = 4 (P = 8 for the
     4q/1kv rank) (the sequence -> head exchange, as a single-GPU permutation);
  2. ul_attn_fwd: causal attention for one SP=4 rank of a Llama-3.1-8B-shaped layer
     (N = 65536, 8 query heads, 2 KV heads, head_dim 128, bf16);
  3. ul_attn_bwd: its dQ, dK, dV;
  4. ul_relayout_h2s of the [3, P, N, 32/P, 128] head-sharded stack (the reverse exchange).

A second measurement, `fused_relayout`, times the same rank's forward and backward through
the token-strided entry points on sequence-sharded world tensors, i.e. the step with both
relayouts fused into the attention's own loads and stores.  A third, `varlen`, times forward
and backward over the same 65536 tokens packed as variable-length sequences.  A fourth,
`head_chunked`, runs the whole step one KV group at a time through head-chunk exchanges,
so the exchange buffer holds one chunk of heads.

The backward runs as its three C-ABI stages (D/lse preparation, the dQ pass, the dK/dV
pass) with events between them, so each kernel's duration is measured on the stream it
runs on; the `roofline` object reports the longest one against its peak.

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
KERNEL_SOURCES = ["attn_fwd.hip", "attn_bwd.hip", "relayout.hip", "mfma_tile.h", "ul_internal.h"]


def _code_only(text: str) -> str:
    """C++ source without its comments and blank lines (string and character literals kept
    as written), so that a comment edit does not count as a kernel change."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return "\n".join(ln.rstrip() for ln in "".join(out).splitlines() if ln.strip())


def kernel_hash() -> str:
    h = hashlib.sha256()
    for n in KERNEL_SOURCES:
        h.update(_code_only((ROOT / "ulysses_sequence_parallelism_attn_amd" / "csrc" / n).read_text()).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str) -> float | None:
    """HBM bytes per launch from the committed PMC measurement, if it was taken on this
    workload and the kernels are unchanged."""
    try:
        rec = json.loads(TRAFFIC_FILE.read_text())
    except (OSError, ValueError):
        return None
    if rec.get("kernel_hash") != kernel_hash() or rec.get("workload") != workload:
        return None
    v = rec.get("bytes_per_launch", {}).get(kernel)
    return float(v) if v is not None else None


# rocprofv3 kernel names -> the names used in the roofline objects
KERNEL_NAMES = [
    ("relayout32_kernel<unsigned int __vector(4), true>", "relayout_s2h"),
    ("relayout32_kernel<unsigned int __vector(4), false>", "relayout_h2s"),
    ("attn_fwd_bf16_kernel<128>", "attn_fwd"),
    ("bwd_pre_kernel", "attn_bwd_prep"),
    ("attn_bwd_dq_bf16_kernel<128>", "attn_bwd_dq"),
    ("attn_bwd_dkdv_bf16_kernel<128>", "attn_bwd_dkdv"),
]
CALIBRATION_KERNEL = "__amd_rocclr_copyBuffer"
CALIBRATION_BYTES = float(1 << 30)


def _pmc_per_kernel(csv_path: Path, counter: str) -> dict:
    """Mean counter value per dispatch for each known kernel, and the value of the calibration
    copy: the first copy dispatch of the run (later copies have other sizes)."""
    import csv

    acc: dict = {}
    rows = sorted(csv.DictReader(open(csv_path)), key=lambda r: int(r["Dispatch_Id"]))
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        name = r["Kernel_Name"]
        key = CALIBRATION_KERNEL if CALIBRATION_KERNEL in name else None
        for pat, short in KERNEL_NAMES:
            if pat in name:
                key = short
        if key is None or (key == CALIBRATION_KERNEL and key in acc):
            continue
        acc.setdefault(key, []).append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def ingest_pmc(fetch_dir: str, write_dir: str, workload: str) -> dict:
    """HBM bytes per launch from a FETCH_SIZE run and a WRITE_SIZE run (KiB per dispatch),
    each scaled by what the same counter reads for the 1 GiB calibration copy."""
    fetch = _pmc_per_kernel(next(Path(fetch_dir).rglob("*counter_collection.csv")), "FETCH_SIZE")
    write = _pmc_per_kernel(next(Path(write_dir).rglob("*counter_collection.csv")), "WRITE_SIZE")
    f_cal = CALIBRATION_BYTES / (fetch[CALIBRATION_KERNEL] * 1024.0)
    w_cal = CALIBRATION_BYTES / (write[CALIBRATION_KERNEL] * 1024.0)
    rec = {"kernel_hash": kernel_hash(), "workload": workload,
           "calibration": {"kernel": CALIBRATION_KERNEL, "bytes": CALIBRATION_BYTES,
                           "fetch_kib": fetch[CALIBRATION_KERNEL], "write_kib": write[CALIBRATION_KERNEL],
                           "fetch_factor": f_cal, "write_factor": w_cal},
           "fetch_bytes": {}, "write_bytes": {}, "bytes_per_launch": {}}
    for _, short in KERNEL_NAMES:
        if short in fetch and short in write:
            fb, wb = fetch[short] * 1024.0 * f_cal, write[short] * 1024.0 * w_cal
            rec["fetch_bytes"][short] = fb
            rec["write_bytes"][short] = wb
            rec["bytes_per_launch"][short] = fb + wb
    return rec


N_XCD = 8          # GRBM_GUI_ACTIVE is summed over the XCDs; one XCD's count is the clock
N_SIMD = 256 * 4   # SQ_VALU_MFMA_BUSY_CYCLES is summed over every SIMD


def summarize_pmc(dirs: list) -> str:
    """Per-kernel counters of rocprofv3 --pmc runs (last dispatch of each kernel) as a markdown
    table, with the derived MFMA utilisation (busy cycles over one XCD's active cycles times
    the SIMD count), shader clock and MFMA rate."""
    import csv

    vals: dict = {}
    ms: dict = {}
    for d in dirs:
        f = next(Path(d).rglob("*counter_collection.csv"))
        for r in sorted(csv.DictReader(open(f)), key=lambda r: int(r["Dispatch_Id"])):
            key = next((short for pat, short in KERNEL_NAMES if pat in r["Kernel_Name"]), None)
            if key is None:
                continue
            vals.setdefault(key, {})[r["Counter_Name"]] = float(r["Counter_Value"])
            ms.setdefault(key, {})[d] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e6
    lines = ["| kernel | ms | clock (GHz) | MFMA busy | MFMA TFLOP/s | VALU instr / MFMA | LDS instr / MFMA "
             "| LDS bank conflicts / LDS active cycles | MFMA-VALU co-issue cycles / MFMA busy |",
             "|---|---|---|---|---|---|---|---|---|"]
    for _, key in KERNEL_NAMES:
        if key not in vals:
            continue
        v = vals[key]
        t = sum(ms[key].values()) / len(ms[key])
        gui = v.get("GRBM_GUI_ACTIVE", 0.0) / N_XCD
        busy = v.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0)
        mops = v.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0)
        n_mfma = mops * 512 / (2 * 32 * 32 * 16)
        cell = lambda x: f"{x:.3g}" if x is not None else "-"
        util = busy / (gui * N_SIMD) if gui and "SQ_VALU_MFMA_BUSY_CYCLES" in v else None
        valu = (v["SQ_INSTS_VALU"] - n_mfma) / n_mfma if n_mfma and "SQ_INSTS_VALU" in v else None
        lds = v["SQ_INSTS_LDS"] / n_mfma if n_mfma and "SQ_INSTS_LDS" in v else None
        bank = (v["SQ_LDS_BANK_CONFLICT"] / v["SQ_LDS_IDX_ACTIVE"]
                if v.get("SQ_LDS_IDX_ACTIVE") else None)
        coex = v["SQ_VALU_MFMA_COEXEC_CYCLES"] / busy if busy and "SQ_VALU_MFMA_COEXEC_CYCLES" in v else None
        lines.append(f"| {key} | {t:.3f} | {cell(gui / (t * 1e-3) / 1e9 if gui else None)} | "
                     f"{cell(util)} | {cell(mops * 512 / (t * 1e-3) / 1e12 if mops else None)} | "
                     f"{cell(valu)} | {cell(lds)} | {cell(bank)} | {cell(coex)} |")
    raw = ["", "Raw counters (last dispatch of each kernel):", ""]
    names = sorted({c for v in vals.values() for c in v})
    raw.append("| kernel | " + " | ".join(names) + " |")
    raw.append("|---|" + "---|" * len(names))
    for _, key in KERNEL_NAMES:
        if key in vals:
            raw.append(f"| {key} | " + " | ".join(f"{vals[key].get(c, float('nan')):.4g}" for c in names) + " |")
    return "\n".join(lines + raw)


def cpu_model() -> str:
    """The host CPU's model name (lscpu, else /proc/cpuinfo)."""
    import subprocess

    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(st: dict, wl, n_prefix: int, relayout_shape=None) -> dict:
    """Time the float64 oracle on a causal prefix of the workload's own inputs; also the
    oracle's full forward+backward of the N = 8192 rank workload and its scalar index-loop
    relayout over the workload's exchange tensor, as reported context."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import attention as OA
    from oracle import native as ON
    from ulysses_sequence_parallelism_attn_amd import synth

    w = {n: OA.widen(a[:, :n_prefix], wl.dtype) for n, a in st.items()}
    t0 = time.perf_counter()
    OA.attn_bwd(w["q"], w["k"], w["v"], w["dout"], wl.scale, True)  # forward + backward
    dt = time.perf_counter() - t0
    del w
    flops = 7.0 * n_prefix ** 2 * wl.Hq * wl.d
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    out = {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": len(os.sched_getaffinity(0)),
        "blas_threads": int(threads),
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": (f"float64 oracle forward+backward on the causal prefix N={n_prefix} of the "
                   f"N={wl.N} inputs (all {wl.Hq} query / {wl.Hkv} KV heads, d={wl.d}); "
                   f"{dt:.1f} s wall, rate in counted FLOPs (7*N^2*Hq*d)"),
        "seconds": dt,
    }
    # the full N = 8192 rank workload, forward + backward
    w2 = synth.WORKLOADS[2]
    s2 = synth.attn_inputs(w2)
    ww = {n: OA.widen(a, w2.dtype) for n, a in s2.items()}
    del s2
    t0 = time.perf_counter()
    OA.attn_bwd(ww["q"], ww["k"], ww["v"], ww["dout"], w2.scale, True)
    t2 = time.perf_counter() - t0
    del ww
    out["full_n8192"] = {"workload": w2.name, "seconds": t2,
                         "tflops": (w2.flops_fwd() + w2.flops_bwd()) / t2 / 1e12}
    # the scalar C relayout (one element per iteration, OpenMP over the outer loops)
    if relayout_shape is not None:
        C, N, H, d, P = relayout_shape
        x = np.random.Generator(np.random.PCG64(7)).integers(0, 1 << 16, size=(C, N, H, d),
                                                             dtype=np.uint16)
        t0 = time.perf_counter()
        ON.relayout_s2h(x, P)
        tr = time.perf_counter() - t0
        nbytes = 2.0 * x.nbytes
        out["relayout_s2h_scalar"] = {"shape": [C, N, H, d], "P": P, "seconds": tr,
                                      "GB/s": nbytes / tr / 1e9,
                                      "omp_threads": int(os.environ.get("OMP_NUM_THREADS", "0"))
                                      or len(os.sched_getaffinity(0))}
    return out


def copy_ceiling(torch, x, reps: int = 10) -> dict:
    """A plain device-to-device copy of the relayout's bytes (torch's copy kernel): the
    practical ceiling an HBM-bound permutation of that size can approach, for context."""
    src = x.view(-1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    stream = torch.cuda.current_stream()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for _ in range(reps):
        dst.copy_(src)
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / reps
    nbytes = 2.0 * src.numel() * src.element_size()
    del dst
    return {"ms": ms, "GB/s": nbytes / (ms * 1e-3) / 1e9, "bytes": nbytes,
            "frac_of_hbm_peak": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS}


def fused_step(B, torch, q, k, v, do, wl, P, args, ms_relayout_path) -> dict:
    """The same rank's forward and backward with the relayouts fused away: the token-strided
    calls read the rank's head slice (rank P-1, the largest offsets) straight out of
    sequence-sharded world tensors [B, N, P*H, d] and write O, dQ, dK, dV into world-layout
    buffers.  Timed like the main step (warmup, then `steps` back-to-back passes)."""
    dev = q.device
    r = P - 1
    qs, ks = slice(r * wl.Hq, (r + 1) * wl.Hq), slice(r * wl.Hkv, (r + 1) * wl.Hkv)
    shape_q, shape_kv = (wl.B, wl.N, P * wl.Hq, wl.d), (wl.B, wl.N, P * wl.Hkv, wl.d)
    Qw, Ow, dOw, dQw = (torch.empty(shape_q, dtype=q.dtype, device=dev) for _ in range(4))
    Kw, Vw, dKw, dVw = (torch.empty(shape_kv, dtype=q.dtype, device=dev) for _ in range(4))
    Qw[:, :, qs].copy_(q)
    dOw[:, :, qs].copy_(do)
    Kw[:, :, ks].copy_(k)
    Vw[:, :, ks].copy_(v)
    views = dict(q=Qw[:, :, qs], k=Kw[:, :, ks], v=Vw[:, :, ks], o=Ow[:, :, qs], do=dOw[:, :, qs],
                 dq=dQw[:, :, qs], dk=dKw[:, :, ks], dv=dVw[:, :, ks])
    lse = torch.empty((wl.B, wl.Hq, wl.N), dtype=torch.float32, device=dev)
    ws = torch.empty(B.workspace_bytes(wl.B, wl.N, wl.Hq, wl.Hkv, wl.d, B.UL_BF16),
                     dtype=torch.uint8, device=dev)
    vw = views  # short name for the step body

    def step():
        B.attn_fwd(vw["q"], vw["k"], vw["v"], wl.scale, True, out=vw["o"], lse=lse)
        B.attn_bwd(vw["q"], vw["k"], vw["v"], vw["o"], vw["do"], lse, wl.scale, True, workspace=ws,
                   dq=vw["dq"], dk=vw["dk"], dv=vw["dv"])

    for _ in range(args.warmup):
        step()
    stream = torch.cuda.current_stream()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for _ in range(args.steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    return {"ms_per_step": ms,
            "tflops": (wl.flops_fwd() + wl.flops_bwd()) / (ms * 1e-3) / 1e12,
            "tokens_per_s": wl.B * wl.N / (ms * 1e-3),
            "speedup_vs_relayout_path": ms_relayout_path / ms,
            "rank": r, "q_tok_stride": views["q"].stride(1), "kv_tok_stride": views["k"].stride(1)}


def chunked_step(B, torch, q, k, v, do, wl, x, P, args, ms_whole) -> dict:
    """The step with the rank's heads taken one KV group at a time: for each group, the
    head-chunk exchange of the QKV stack into a buffer of that group's heads, forward and
    backward on the group, and the reverse exchange of the chunk.  Same bytes and FLOPs as
    the whole-slice step; the exchange buffer holds one chunk."""
    C, N, H, d = x.shape
    Hs = H // P
    groups = wl.Hkv
    hc = Hs // groups  # heads of the stack per chunk
    grp = wl.Hq // wl.Hkv
    ybuf = torch.empty((C, P, N, hc, d), dtype=x.dtype, device=x.device)
    x2 = torch.empty_like(x)
    parts = []
    for gi in range(groups):
        qs, ks = slice(gi * grp, (gi + 1) * grp), slice(gi, gi + 1)
        t = {"q": q[:, :, qs].contiguous(), "k": k[:, :, ks].contiguous(),
             "v": v[:, :, ks].contiguous(), "do": do[:, :, qs].contiguous()}
        t["o"] = torch.empty_like(t["q"])
        t["dq"], t["dk"], t["dv"] = (torch.empty_like(t[n]) for n in ("q", "k", "v"))
        t["lse"] = torch.empty((wl.B, grp, wl.N), dtype=torch.float32, device=q.device)
        t["ws"] = torch.empty(B.workspace_bytes(wl.B, wl.N, grp, 1, wl.d, B.UL_BF16),
                              dtype=torch.uint8, device=q.device)
        parts.append(t)

    def step():
        for gi, t in enumerate(parts):
            B.relayout_s2h_heads(x, P, gi * hc, hc, out=ybuf)
            B.attn_fwd(t["q"], t["k"], t["v"], wl.scale, True, out=t["o"], lse=t["lse"])
            B.attn_bwd(t["q"], t["k"], t["v"], t["o"], t["do"], t["lse"], wl.scale, True,
                       workspace=t["ws"], dq=t["dq"], dk=t["dk"], dv=t["dv"])
            B.relayout_h2s_heads(ybuf, x2, gi * hc)

    for _ in range(args.warmup):
        step()
    stream = torch.cuda.current_stream()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for _ in range(args.steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    return {"ms_per_step": ms,
            "tflops": (wl.flops_fwd() + wl.flops_bwd()) / (ms * 1e-3) / 1e12,
            "chunks": groups, "heads_per_chunk": {"stack": hc, "q": grp, "kv": 1},
            "exchange_buffer_bytes": ybuf.numel() * ybuf.element_size(),
            "whole_slice_buffer_bytes": C * P * N * Hs * d * x.element_size(),
            "time_vs_whole_slice": ms / ms_whole}


VARLEN_SEED = 3008  # seed of the packed-sequence length mix


def varlen_step(B, torch, synth, q, k, v, do, wl, args) -> dict:
    """Forward and backward over the same 65536 tokens split into packed variable-length
    sequences (the seeded log-uniform length mix of synth.length_mix), through the varlen
    entry points.  Counted FLOPs are 7*len^2*Hq*d summed over the sequences."""
    lengths = synth.length_mix(wl.N, VARLEN_SEED)
    cu = torch.from_numpy(synth.cu_seqlens(lengths)).to(q.device)
    mx = int(lengths.max())
    qv, kv, vv, dov = (t[0] for t in (q, k, v, do))  # [T, H, d], dense
    o = torch.empty_like(qv)
    lse = torch.empty((wl.Hq, wl.N), dtype=torch.float32, device=q.device)
    dq, dk, dv = torch.empty_like(qv), torch.empty_like(kv), torch.empty_like(vv)
    ws = torch.empty(B.workspace_bytes(1, wl.N, wl.Hq, wl.Hkv, wl.d, B.UL_BF16),
                     dtype=torch.uint8, device=q.device)

    def step():
        B.attn_fwd_varlen(qv, kv, vv, cu, mx, wl.scale, True, out=o, lse=lse)
        B.attn_bwd_varlen(qv, kv, vv, o, dov, lse, cu, mx, wl.scale, True, workspace=ws, dq=dq,
                          dk=dk, dv=dv)

    for _ in range(args.warmup):
        step()
    stream = torch.cuda.current_stream()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for _ in range(args.steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    flops = float(sum(7.0 * int(n) * int(n) * wl.Hq * wl.d for n in lengths))
    return {"ms_per_step": ms, "tflops": flops / (ms * 1e-3) / 1e12,
            "tokens_per_s": wl.N / (ms * 1e-3), "n_seqs": int(len(lengths)),
            "max_seqlen": mx, "min_seqlen": int(lengths.min()), "length_mix_seed": VARLEN_SEED,
            "counted_flop": flops}


def graph_step(torch, step, args, ms_eager) -> dict:
    """The same step (the calls of `step`, without its per-stage events) captured once in a
    HIP graph and replayed: the library allocates, synchronises and memsets nothing, so the
    whole step is one graph launch per iteration."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(args.warmup):
        g.replay()
    stream = torch.cuda.current_stream()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for _ in range(args.steps):
        g.replay()
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    del g
    return {"ms_per_step": ms, "time_vs_eager": ms / ms_eager}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=3, help="attention workload id (default 3)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fused", action="store_true",
                    help="skip the strided (relayout-free) variant of the step")
    ap.add_argument("--no-varlen", action="store_true",
                    help="skip the packed variable-length variant of the step")
    ap.add_argument("--no-chunked", action="store_true",
                    help="skip the head-chunked variant of the step")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the HIP-graph replay of the step")
    ap.add_argument("--no-copy-ceiling", action="store_true",
                    help="skip the device-copy reference for the relayout's bytes")
    ap.add_argument("--cpu-prefix", type=int, default=16384)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run one 1 GiB device-to-device copy first (a known-size reference for "
                         "HBM byte counters)")
    ap.add_argument("--summarize-pmc", nargs="+", metavar="PMC_DIR",
                    help="print a markdown table of the attention kernels' counters from rocprofv3 "
                         "--pmc output folders and exit")
    ap.add_argument("--ingest-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/traffic.json from two rocprofv3 --pmc output folders "
                         "(FETCH_SIZE run, WRITE_SIZE run, both with --copy-calibration) and exit")
    args = ap.parse_args()

    if args.summarize_pmc:
        print(summarize_pmc(args.summarize_pmc))
        return 0

    if args.ingest_pmc:
        from ulysses_sequence_parallelism_attn_amd import synth

        rec = ingest_pmc(*args.ingest_pmc, synth.WORKLOADS[args.workload].name)
        TRAFFIC_FILE.parent.mkdir(exist_ok=True)
        TRAFFIC_FILE.write_text(json.dumps(rec, indent=1) + "\n")
        print(json.dumps(rec["bytes_per_launch"]))
        return 0

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (--gpus {args.gpus}, WORLD_SIZE {world} requested); "
              "the multi-GPU exchange is not implemented here.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from ulysses_sequence_parallelism_attn_amd import binding as B
    from ulysses_sequence_parallelism_attn_amd import synth

    wl = synth.WORKLOADS[args.workload]
    rl = wl.exchange  # (C, N, H, d, P) of this workload's own QKV-stack exchange
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    st = synth.attn_inputs(wl)
    up = lambda a: torch.from_numpy(a).view(torch.bfloat16).to(dev)
    q, k, v, do = (up(st[n]) for n in ("q", "k", "v", "dout"))
    C, Nr, Hr, dr, P = rl
    gen = torch.Generator(device=dev)
    gen.manual_seed(synth.seed_of(wl.wid, synth.SLOT_RELAYOUT))
    x = torch.randint(-32768, 32767, (C, Nr, Hr, dr), dtype=torch.int16, device=dev,
                      generator=gen).view(torch.bfloat16)
    y = torch.empty((C, P, Nr, Hr // P, dr), dtype=torch.bfloat16, device=dev)
    x2 = torch.empty_like(x)
    o = torch.empty_like(q)
    lse = torch.empty((wl.B, wl.Hq, wl.N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(B.workspace_bytes(wl.B, wl.N, wl.Hq, wl.Hkv, wl.d, B.UL_BF16),
                     dtype=torch.uint8, device=dev)
    # the forward's key-range split takes a workspace at shorter N (none at N = 65536)
    fws_bytes = B.fwd_workspace_bytes(wl.B, wl.N, wl.Hq, wl.Hkv, wl.d, B.UL_BF16)
    fws = torch.empty(fws_bytes, dtype=torch.uint8, device=dev) if fws_bytes else None
    stream = torch.cuda.current_stream()
    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        src.fill_(1)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # One step: relayout s2h, forward, the backward's stages, relayout h2s.  The backward
    # runs as C-ABI stage calls that launch exactly what ul_attn_bwd launches, so that each
    # kernel is bracketed by its own events on the stream it is launched on: PREP, then DQ
    # and DKDV as separate calls where ul_attn_bwd launches them separately, or as one DQ|DKDV
    # call where it merges them into one launch (its rule: fewer 128-key dK/dV blocks than
    # four per compute unit).
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    merged_bwd = -(-wl.N // 128) * wl.B * wl.Hkv < 4 * cus

    def bwd_stage(stage):
        return lambda: B.attn_bwd(q, k, v, o, do, lse, wl.scale, True, workspace=ws, dq=dq, dk=dk,
                                  dv=dv, stages=stage)

    names = ["relayout_s2h", "attn_fwd", "attn_bwd_prep"]
    calls = [
        lambda: B.relayout_s2h(x, P, out=y),
        lambda: B.attn_fwd(q, k, v, wl.scale, True, out=o, lse=lse, workspace=fws),
        bwd_stage(B.UL_BWD_PREP),
    ]
    if merged_bwd:
        names += ["attn_bwd_dq_dkdv"]
        calls += [bwd_stage(B.UL_BWD_DQ | B.UL_BWD_DKDV)]
    else:
        names += ["attn_bwd_dq", "attn_bwd_dkdv"]
        calls += [bwd_stage(B.UL_BWD_DQ), bwd_stage(B.UL_BWD_DKDV)]
    names += ["relayout_h2s"]
    calls += [lambda: B.relayout_h2s(y, out=x2)]

    def step(ev=None):
        for j, call in enumerate(calls):
            if ev is not None:
                ev[j].record(stream)
            call()
        if ev is not None:
            ev[len(calls)].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)]
           for _ in range(args.steps)]
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
    avg = {n: sum(e[j].elapsed_time(e[j + 1]) for e in evs) / args.steps for j, n in enumerate(names)}

    # Algorithmic work per launch.  Attention counts 2d FLOPs per multiply-add over the
    # visible (query, key) pairs: forward S and O (4d per pair); the dQ pass S, dP and dQ
    # (6d); the dK/dV pass S, dP, dV and dK (8d).  The headline counts the backward as
    # 10d per pair (S and dP once), so the two passes together do 14d of it.
    pairs_x_heads = wl.flops_fwd() / (4.0 * wl.d)
    f_fwd = wl.flops_fwd()
    f_bwd = wl.flops_bwd()
    flops_step = f_fwd + f_bwd
    value = flops_step / (ms_per_step * 1e-3) / 1e12
    rl_bytes = 2.0 * C * Nr * Hr * dr * 2
    rows = wl.B * wl.N * wl.Hq
    prep_bytes = 2.0 * rows * wl.d * 2 + rows * 4 + 2 * rows * 4  # o, dout read; lse read; lse2, D written

    def mfma(flop, n, performed=None):
        r = {"bound": "mfma", "achieved": flop / (avg[n] * 1e-3) / 1e12, "peak": PEAK_BF16_TFLOPS,
             "unit": "TFLOP/s", "algorithmic": flop}
        if performed is not None:
            r["performed"] = performed
            r["achieved_performed"] = performed / (avg[n] * 1e-3) / 1e12
            r["frac_performed"] = r["achieved_performed"] / PEAK_BF16_TFLOPS
        return r

    def hbm(nbytes, n):
        return {"bound": "hbm", "achieved": nbytes / (avg[n] * 1e-3) / 1e9, "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "algorithmic": nbytes}

    roof = {
        "relayout_s2h": hbm(rl_bytes, "relayout_s2h"),
        "attn_fwd": mfma(f_fwd, "attn_fwd"),
        "attn_bwd_prep": hbm(prep_bytes, "attn_bwd_prep"),
    }
    if merged_bwd:
        # one launch does both passes: 10d per pair counted, 14d performed
        roof["attn_bwd_dq_dkdv"] = mfma(10.0 * wl.d * pairs_x_heads, "attn_bwd_dq_dkdv",
                                        14.0 * wl.d * pairs_x_heads)
    else:
        # the method counts the dQ pass only for its dQ contraction (2d per pair; S and dP
        # are counted once, in dK/dV); it performs S, dP and dQ (6d per pair)
        roof["attn_bwd_dq"] = mfma(2.0 * wl.d * pairs_x_heads, "attn_bwd_dq", 6.0 * wl.d * pairs_x_heads)
        roof["attn_bwd_dkdv"] = mfma(8.0 * wl.d * pairs_x_heads, "attn_bwd_dkdv")
    roof["relayout_h2s"] = hbm(rl_bytes, "relayout_h2s")
    for n, r in roof.items():
        r["frac"] = r["achieved"] / r["peak"]
        r["ms"] = avg[n]
        r["traffic"] = measured_traffic(n, wl.name)
    dominant = max(avg, key=avg.get)
    dom = {k2: roof[dominant][k2] for k2 in ("bound", "achieved", "peak", "unit", "frac", "traffic")}
    dom["kernel"] = dominant
    dom["ms"] = avg[dominant]

    attn_ms = sum(t for n, t in avg.items() if n.startswith("attn_"))
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
                   "relayout": {"shape": [C, Nr, Hr, dr], "P": P}, "parallelism": f"sp{P}-rank-share"},
        "pct_bf16_peak": 100.0 * value / PEAK_BF16_TFLOPS,
        "attn_fwd_bwd_ms": attn_ms,
        "attn_fwd_bwd_tflops": flops_step / (attn_ms * 1e-3) / 1e12,
        "tokens_per_s": wl.B * wl.N / (ms_per_step * 1e-3),
        "roofline": dom,
        "roofline_all": roof,
        "kernel_hash": kernel_hash(),
        "bwd_launch": "dq+dkdv merged" if merged_bwd else "dq, dkdv separate",
        "fwd_split": bool(fws_bytes),
    }
    if not args.no_graph:
        out["graph"] = graph_step(torch, step, args, ms_per_step)
    if not args.no_copy_ceiling:
        out["copy_ceiling"] = copy_ceiling(torch, x)
    if not args.no_fused:
        out["fused_relayout"] = fused_step(B, torch, q, k, v, do, wl, P, args, ms_per_step)
    if not args.no_varlen:
        out["varlen"] = varlen_step(B, torch, synth, q, k, v, do, wl, args)
    if not args.no_chunked:
        del y, x2
        out["head_chunked"] = chunked_step(B, torch, q, k, v, do, wl, x, P, args, ms_per_step)
    if not args.no_cpu_baseline:
        del x
        torch.cuda.empty_cache()
        out["cpu_baseline"] = cpu_baseline(st, wl, min(args.cpu_prefix, wl.N),
                                           synth.WORKLOADS[3].exchange)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
