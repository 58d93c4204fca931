"""Host-side logic of bench.py (CPU only): the one-GPU refusal, the ingestion of rocprofv3
counter files into per-launch HBM bytes, and the hash gate on the stored traffic figures."""

import csv
import json
import subprocess
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
sys.path.insert(0, str(ROOT))
import bench  # noqa: E402
from ulysses_sequence_parallelism_attn_amd import synth  # noqa: E402


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout == ""


def _write_counters(d: Path, counter: str, rows):
    d.mkdir(parents=True)
    with open(d / "run_counter_collection.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (name, value) in enumerate(rows):
            w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": name, "Counter_Name": counter,
                        "Counter_Value": value})


def test_ingest_scales_by_the_first_calibration_copy(tmp_path):
    cal = "__amd_rocclr_copyBuffer"
    fwd = "void ul::(anonymous namespace)::attn_fwd_bf16_kernel<128>(ul::(anonymous namespace)::FwdParams)"
    dkdv = "void ul::(anonymous namespace)::attn_bwd_dkdv_bf16_kernel<128>(ul::(anonymous namespace)::DkvParams)"
    # the 1 GiB calibration copy reads 2^19 KiB of FETCH_SIZE (factor 2) and 2^20 KiB of
    # WRITE_SIZE (factor 1); a later copy of another size must not replace it
    _write_counters(tmp_path / "F", "FETCH_SIZE",
                    [(cal, 524288.0), (fwd, 1000.0), (fwd, 3000.0), (dkdv, 10.0), (cal, 7.0)])
    _write_counters(tmp_path / "W", "WRITE_SIZE",
                    [(cal, 1048576.0), (fwd, 100.0), (fwd, 300.0), (dkdv, 1.0), (cal, 9.0)])
    rec = bench.ingest_pmc(str(tmp_path / "F"), str(tmp_path / "W"), "wl-x")
    assert rec["workload"] == "wl-x"
    assert rec["calibration"]["fetch_factor"] == pytest.approx(2.0)
    assert rec["calibration"]["write_factor"] == pytest.approx(1.0)
    # per launch: the mean over dispatches, in KiB, times 1024 and the factor
    assert rec["fetch_bytes"]["attn_fwd"] == pytest.approx(2000.0 * 1024 * 2.0)
    assert rec["write_bytes"]["attn_fwd"] == pytest.approx(200.0 * 1024)
    assert rec["bytes_per_launch"]["attn_fwd"] == pytest.approx(2000.0 * 2048 + 200.0 * 1024)
    assert rec["bytes_per_launch"]["attn_bwd_dkdv"] == pytest.approx(10.0 * 2048 + 1.0 * 1024)
    assert rec["kernel_hash"] == bench.kernel_hash()
    assert "relayout_s2h" not in rec["bytes_per_launch"]  # not in the files, not invented


def test_traffic_is_reported_only_for_the_measured_sources(tmp_path, monkeypatch):
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps({"kernel_hash": bench.kernel_hash(), "workload": "wl-a",
                             "bytes_per_launch": {"attn_fwd": 5.0}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", f)
    assert bench.measured_traffic("attn_fwd", "wl-a") == 5.0
    assert bench.measured_traffic("attn_bwd_dq", "wl-a") is None
    assert bench.measured_traffic("attn_fwd", "wl-b") is None  # another workload's bytes
    f.write_text(json.dumps({"kernel_hash": "0" * 16, "workload": "wl-a",
                             "bytes_per_launch": {"attn_fwd": 5.0}}))
    assert bench.measured_traffic("attn_fwd", "wl-a") is None
    f.write_text("not json")
    assert bench.measured_traffic("attn_fwd", "wl-a") is None


def test_committed_traffic_matches_the_kernel_sources():
    rec = json.loads(bench.TRAFFIC_FILE.read_text())
    assert rec["kernel_hash"] == bench.kernel_hash(), "profiles/traffic.json is stale: re-run the counter passes"
    assert rec["workload"] == synth.WORKLOADS[3].name


def test_kernel_hash_ignores_comments_but_not_code():
    src = 'int a = 1; // note\n/* block\n comment */ const char *s = "// kept"; char q = \'/\';\n\n  int b;'
    same = '// header\nint a = 1;\n const char *s = "// kept"; char q = \'/\';\nint b;   /* tail */'
    assert bench._code_only(src).split() == bench._code_only(same).split()
    assert bench._code_only(src) != bench._code_only(src.replace('"// kept"', '"// changed"'))
    assert bench._code_only(src) != bench._code_only(src.replace("int b;", "int c;"))
