#!/usr/bin/env python3
"""Benchmark: QK-norm + RoPE + FP8 prologue, 4096 tokens x (32 q + 8 kv) heads x 128, on one MI355X.

One step = one ``rnq_qk_norm_rope_fp8`` call over the whole batch (RMSNorm ->
NeoX RoPE -> per-row FP8 for every (token, head) row). Inputs are seeded
synthetic tensors already resident in HBM; several input/output sets are
rotated so the working set (> 512 MB) does not stay in the 256 MB Infinity
Cache between steps.

Prints ONE JSON line: achieved GB/s (algorithmic bytes / step time), % of the
8 TB/s HBM peak, rows/s, the roofline of the kernel (average launch time from
HIP events on the launch stream), and the CPU oracle timed on a bounded sample.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "achieved HBM GB/s (% of peak) + rows/s, QK-norm+RoPE+FP8 4096tok×40h×128"
PEAK_HBM_GBS = 8000.0
KERNEL_SOURCES = ("fp8_quant_amd/csrc/rnq_rows.hip", "fp8_quant_amd/csrc/rnq_device.h",
                  "fp8_quant_amd/csrc/rnq_launch.h", "fp8_quant_amd/build.py")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_qk_4k.json")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None
    when the counters were taken on a different kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return t.get("traffic_bytes_per_launch")


def cpu_baseline(workload_name: str, budget_s: float = 12.0) -> dict:
    """The CPU oracle (as it stands) on a bounded sample of the same workload."""
    import numpy as np

    import oracle
    import workloads
    from fp8_quant_amd import ledger

    d = workloads.generate(workload_name)
    T = d["tokens"]
    qb, kb = workloads.bits(d["q"]), workloads.bits(d["k"])
    wq, wk = workloads.bits(d["wq"]), workloads.bits(d["wk"])
    cos, sin = d["cos"].numpy(), d["sin"].numpy()
    chunk = 256
    done = 0
    t0 = time.perf_counter()
    while done < T and time.perf_counter() - t0 < budget_s:
        hi = min(done + chunk, T)
        oracle.qk_norm_rope_fp8(qb[done:hi], kb[done:hi], wq, wk, cos, sin, tokens=np.arange(done, hi))
        done = hi
    dt = time.perf_counter() - t0
    b = ledger.qk_bytes(done, d["q_heads"], d["kv_heads"], d["head_dim"], d["rope_dim"])
    return {
        "value": round(b["total"] / dt / 1e9, 6),
        "unit": "GB/s",
        "rows_per_s": round(b["rows"] / dt, 1),
        "cores": 1,
        "kind": "oracle",
        "sample": f"first {done} of {T} tokens ({b['rows']} rows), numpy oracle, one pass, {dt:.1f} s",
    }


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="qk_4k")
    ap.add_argument("--sets", type=int, default=0, help="rotated input/output sets (0 = enough for > 512 MB)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "the path shards by token with no exchange, see DESIGN.md", file=sys.stderr)
        return 2

    import torch

    import fp8_quant_amd as rnq
    import workloads
    from fp8_quant_amd import ledger

    wl = workloads.WORKLOADS[args.workload]
    assert wl.kind == "qk", "the bench times the QK-norm + RoPE + FP8 path"
    d = workloads.generate(args.workload)
    T, Hq, Hk, D, R = d["tokens"], d["q_heads"], d["kv_heads"], d["head_dim"], d["rope_dim"]
    led = ledger.qk_bytes(T, Hq, Hk, D, R)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    n_sets = args.sets or max(2, -(-512 * 2**20 // led["total"]) + 1)
    sets = []
    for _ in range(n_sets):
        sets.append({
            "q": d["q"].to(dev), "k": d["k"].to(dev),
            "q8": torch.empty((T, Hq, D), dtype=torch.uint8, device=dev),
            "k8": torch.empty((T, Hk, D), dtype=torch.uint8, device=dev),
            "qs": torch.empty((T, Hq), dtype=torch.float32, device=dev),
            "ks": torch.empty((T, Hk), dtype=torch.float32, device=dev),
        })
    wq, wk = d["wq"].to(dev), d["wk"].to(dev)
    cos, sin = d["cos"].to(dev), d["sin"].to(dev)
    torch.cuda.synchronize()

    def step(i):
        s = sets[i % n_sets]
        rnq.rnq_qk_norm_rope_fp8(s["q"], s["k"], wq, wk, cos, sin, s["q8"], s["k8"], s["qs"], s["ks"],
                                 eps=wl.eps, fp8_max=wl.fp8_max)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    K = args.steps
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for i in range(K):
        starts[i].record()
        step(args.warmup + i)
        ends[i].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    per_launch_ms = [starts[i].elapsed_time(ends[i]) for i in range(K)]
    region_ms = starts[0].elapsed_time(ends[-1])
    ms_per_step = region_ms / K
    kern_ms = sum(per_launch_ms) / K
    per_launch_sorted = sorted(per_launch_ms)

    value = led["total"] / (ms_per_step * 1e-3) / 1e9
    achieved = led["total"] / (kern_ms * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{args.workload}: QK-norm+RoPE+FP8, {T} tokens x ({Hq} q + {Hk} kv) heads x {D}, "
                        f"rope {R}, bf16 in, e4m3fn + fp32 scale per row out",
            "tokens": T, "q_heads": Hq, "kv_heads": Hk, "head_dim": D, "rope_dim": R,
            "rotated_sets": n_sets,
        },
        "pct_of_peak": round(100.0 * value / PEAK_HBM_GBS, 2),
        "rows_per_s": round(led["rows"] / (ms_per_step * 1e-3), 1),
        "bytes_per_step": led["total"],
        "kernel_ms": {"mean": round(kern_ms, 6), "p10": round(per_launch_sorted[K // 10], 6),
                      "p50": round(per_launch_sorted[K // 2], 6), "p90": round(per_launch_sorted[(9 * K) // 10], 6)},
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": measured_traffic(),
        },
        "host_wall_s": round(wall, 4),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.workload)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    raise SystemExit(main())
