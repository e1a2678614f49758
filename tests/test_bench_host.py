"""The host side of bench.py, without a GPU: the one-GPU guard, the CPU oracle
baseline's fields, and the traffic record's consistency rules."""

from __future__ import annotations

import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""


def test_cpu_baseline_fields():
    cb = bench.cpu_baseline("qk_4k", budget_s=0.5)
    assert cb["kind"] == "oracle" and cb["unit"] == "GB/s" and cb["cores"] == 1
    assert cb["value"] > 0 and cb["rows_per_s"] > 0
    assert "tokens" in cb["sample"] and "numpy oracle" in cb["sample"]


def test_traffic_record_is_consistent():
    """The committed counter summary covers the headline kernel at its grid, its
    bytes are calibrated reads plus writes, and the bench reports them only
    while the kernel sources hash to the recorded value."""
    with open(bench.TRAFFIC_FILE) as f:
        t = json.load(f)
    assert t["kernel"].startswith("rows_kernel<") and t["grid"] == "262144"
    assert t["traffic_bytes_per_launch"] == t["fetch_bytes_per_launch"] + t["write_bytes_per_launch"]
    assert abs(t["fetch_bytes_per_launch"] - t["fetch_kib_per_dispatch"] * 1024 * t["fetch_scale"]) <= 1
    assert t["algorithmic_bytes_per_launch"] == 65667584
    # counters within 1 % of the algorithmic bytes (no re-reads)
    assert abs(t["traffic_bytes_per_launch"] / t["algorithmic_bytes_per_launch"] - 1) < 0.01
    fresh = t["kernel_source_sha256"] == bench.kernel_source_hash()
    assert (bench.measured_traffic() is not None) == fresh


def test_summary_arithmetic():
    s = bench._summary({"workload": "w", "ms": 0.01, "bytes": 80_000_000, "rows": 1000, "sets": 3})
    assert s["us_per_call"] == 10.0 and s["GB/s"] == 8000.0 and s["pct_of_peak"] == 100.0
    assert s["rows_per_s"] == 1e8 and s["rotated_sets"] == 3
