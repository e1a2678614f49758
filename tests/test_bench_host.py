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
    cb = bench.cpu_baseline("qk_4k", single_s=0.3, multi_s=0.3, max_procs=2)
    assert cb["kind"] == "oracle" and cb["unit"] == "GB/s"
    assert cb["value"] > 0 and cb["rows_per_s"] > 0
    assert "tokens" in cb["sample"] and "numpy oracle" in cb["sample"]
    assert cb["single_thread"]["cores"] == 1 and cb["single_thread"]["value"] > 0
    assert cb["cores"] == min(2, cb["cores_available"]) and cb["cpu_model"]


def test_cpu_baseline_single_process():
    cb = bench.cpu_baseline("qk_4k", single_s=0.3, multi_s=0.3, max_procs=1)
    assert cb["cores"] == 1 and cb["value"] == cb["single_thread"]["value"]


def test_timer_queues_a_lead_in_before_the_start_event():
    """The timed window opens on a busy queue: untimed launches go out after the
    warm-up's last synchronisation and before the start event, and exactly
    ``steps`` launches fall between the two events."""
    log = []

    class Ev:
        def __init__(self, **kw):
            pass

        def record(self):
            log.append("event")

        def elapsed_time(self, other):
            return 1.0

    class Cuda:
        Event = Ev

        @staticmethod
        def synchronize():
            log.append("sync")

    class Torch:
        cuda = Cuda

    ms = bench._timed(Torch, [lambda: log.append("launch")], steps=7, warmup=3, warm_ms=0.0, lead_ms=0.0)
    assert ms == 1.0 / 7
    first_event = log.index("event")
    last_sync_before = max(i for i, e in enumerate(log[:first_event]) if e == "sync")
    assert log[last_sync_before + 1:first_event].count("launch") >= 16  # the lead-in
    second_event = log.index("event", first_event + 1)
    assert log[first_event + 1:second_event] == ["launch"] * 7


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
