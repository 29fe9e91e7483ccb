"""Host logic of bench.py (CPU only): the one-GPU refusal, the algorithmic
byte counts behind the roofline numerator, and the rocprofv3 summarizers on
small synthetic CSV files."""
from __future__ import annotations

import csv
import json
import os
import subprocess
import sys
from types import SimpleNamespace

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_block_bytes_counts_q_planes_and_lut_q():
    # 64 rows x 256 columns at q = 3: 3 planes of 64 * 256 / 8 bytes + 64 rows x 8 fp16 entries
    assert bench.block_bytes(64, 256, 3) == 3 * 64 * 256 // 8 + 64 * 8 * 2
    # at q = 8 the planes are the parent codes themselves (one byte per weight)
    assert bench.block_bytes(10, 32, 8) == 10 * 32 + 10 * 256 * 2


def test_step_bytes_counts_only_active_experts():
    shape = SimpleNamespace(H=64, I=32, I_shared=0, top_k=2, E=4)
    wq = np.array([[3, 4], [8, 8], [5, 6], [7, 3]])
    offsets = np.array([0, 3, 3, 4, 4])  # experts 0 and 2 active (3 and 1 assignments), 1 and 3 idle
    T = 2
    b = bench.step_bytes(shape, wq, offsets, T)
    gu = bench.block_bytes(64, 64, 3) + bench.block_bytes(64, 64, 5)
    dn = bench.block_bytes(64, 32, 4) + bench.block_bytes(64, 32, 6)
    assert b["active"] == 2
    assert b["weights"] == gu + dn
    rows_h = T * 2 * 32
    assert b["gate_up"] == gu + T * 64 * 2 + rows_h * 2
    assert b["down"] == dn + rows_h * 2 + T * 2 * 64 * 4
    assert b["path"] == gu + dn + 2 * T * 64 * 2 + T * 4 * 4


def test_step_bytes_adds_the_shared_expert_at_8_bits():
    shape = SimpleNamespace(H=64, I=32, I_shared=96, top_k=1, E=2)
    wq = np.array([[3, 3], [3, 3]])
    offsets = np.array([0, 1, 1])
    b = bench.step_bytes(shape, wq, offsets, 1)
    assert b["weights"] == (bench.block_bytes(64, 64, 3) + bench.block_bytes(64, 32, 3)
                            + bench.block_bytes(192, 64, 8) + bench.block_bytes(64, 96, 8))


def _write_csv(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0].keys()))
        w.writeheader()
        w.writerows(rows)


def test_pmc_summary_scales_by_the_copy_kernel(tmp_path, monkeypatch):
    fetch, write = str(tmp_path / "f"), str(tmp_path / "w")
    gu = "void pw::ffn_gemv_kernel<0, 4, true>(pw::FfnArgs)"
    dn = "void pw::ffn_gemv_kernel<1, 2, false, false>(pw::FfnArgs)"
    cp = "__amd_rocclr_copyBuffer"
    # the counters see half the copied bytes on fetch and all of them on write
    _write_csv(os.path.join(fetch, "run_counter_collection.csv"), [
        {"Kernel_Name": gu, "Counter_Name": "FETCH_SIZE", "Counter_Value": "1000"},
        {"Kernel_Name": gu, "Counter_Name": "FETCH_SIZE", "Counter_Value": "1200"},
        {"Kernel_Name": dn, "Counter_Name": "FETCH_SIZE", "Counter_Value": "300"},
        {"Kernel_Name": cp, "Counter_Name": "FETCH_SIZE", "Counter_Value": str(512 * 1024)},
        {"Kernel_Name": cp, "Counter_Name": "FETCH_SIZE", "Counter_Value": "10"},  # small staging copy, ignored
    ])
    _write_csv(os.path.join(write, "run_counter_collection.csv"), [
        {"Kernel_Name": gu, "Counter_Name": "WRITE_SIZE", "Counter_Value": "50"},
        {"Kernel_Name": dn, "Counter_Name": "WRITE_SIZE", "Counter_Value": "20"},
        {"Kernel_Name": cp, "Counter_Name": "WRITE_SIZE", "Counter_Value": str(1024 * 1024)},
    ])
    out = str(tmp_path / "traffic.md")
    monkeypatch.setattr(bench, "kernel_sha", lambda: "abc")
    bench.summarize_pmc(fetch, write, out, "cmd f", "cmd w", 1024, {"gate_up": 2.0e6, "down": 1.0e6})
    line = [l for l in open(out) if l.startswith("TRAFFIC_JSON:")][0]
    t = json.loads(line.split(":", 1)[1])
    assert abs(t["scale_fetch"] - 2.0) < 1e-12 and abs(t["scale_write"] - 1.0) < 1e-12
    assert abs(t["gate_up"]["fetch_bytes"] - 1100 * 2.0 * 1024) < 1e-6
    assert abs(t["gate_up"]["write_bytes"] - 50 * 1024) < 1e-6
    assert abs(t["down"]["traffic_bytes"] - (300 * 2.0 + 20) * 1024) < 1e-6
    assert t["down"]["algorithmic_bytes"] == 1.0e6
    assert t["kernel_sha"] == "abc"
    # read back only while the kernel source is the one profiled
    monkeypatch.setattr(bench, "TRAFFIC_MD", out)
    assert bench.stored_traffic()["gate_up"]["write_bytes"] == t["gate_up"]["write_bytes"]
    monkeypatch.setattr(bench, "kernel_sha", lambda: "changed")
    assert bench.stored_traffic() is None


def test_trace_and_counter_summaries(tmp_path):
    trace = str(tmp_path / "t")
    _write_csv(os.path.join(trace, "bench_kernel_stats.csv"), [
        {"Name": "void pw::ffn_gemv_kernel<0, 4, true>(pw::FfnArgs)", "Calls": "10", "AverageNs": "21000",
         "TotalDurationNs": "210000", "Percentage": "60.0"},
        {"Name": "__amd_rocclr_fillBufferAligned", "Calls": "2", "AverageNs": "1000",
         "TotalDurationNs": "2000", "Percentage": "1.0"},
    ])
    out = str(tmp_path / "trace.md")
    bench.summarize_trace(trace, out, "cmd")
    text = open(out).read()
    assert "| void pw::ffn_gemv_kernel<0, 4, true> | 10 | 21.00 | 0.21 | 60.0 |" in text
    assert "fillBuffer" not in text
    t = json.loads([l for l in text.splitlines() if l.startswith("TRACE_JSON:")][0].split(":", 1)[1])
    assert t["average_us"] == {"ffn_gemv_kernel<0, 4, true>": 21.0}

    pmc = str(tmp_path / "c")
    k = "void pw::ffn_prefill_kernel<0>(pw::FfnArgs)"
    _write_csv(os.path.join(pmc, "run_counter_collection.csv"), [
        {"Kernel_Name": k, "Counter_Name": "SQ_WAVE_CYCLES", "Counter_Value": "1000"},
        {"Kernel_Name": k, "Counter_Name": "SQ_WAIT_ANY", "Counter_Value": "250"},
        {"Kernel_Name": k, "Counter_Name": "SQ_WAVE_CYCLES", "Counter_Value": "3000"},
        {"Kernel_Name": k, "Counter_Name": "SQ_WAIT_ANY", "Counter_Value": "750"},
    ])
    out2 = str(tmp_path / "counters.md")
    bench.summarize_counters([pmc], out2, ["cmd"], "title")
    text = open(out2).read()
    assert "| void pw::ffn_prefill_kernel<0> | 2 | 500 | 2000 |" in text  # columns sorted by name
    assert "| void pw::ffn_prefill_kernel<0> | 25.0% |" in text
