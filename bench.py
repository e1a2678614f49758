#!/usr/bin/env python3
"""Benchmark: QK-norm + RoPE + FP8 prologue, 4096 tokens x (32 q + 8 kv) heads x 128, on one MI355X.

One step = one ``rnq_qk_norm_rope_fp8`` call over the whole batch (RMSNorm ->
NeoX RoPE -> per-row FP8 for every (token, head) row). Inputs are seeded
synthetic tensors already resident in HBM; several input/output sets are
rotated so the working set (> 512 MB) does not stay in the 256 MB Infinity
Cache between steps. The K timed steps are launched back to back with
pre-marshalled arguments between two events on the launch stream, so the
time per step is the kernel's own time (the host stays ahead of the GPU).
Every path warms up for its warm-up steps and at least 40 ms of back-to-back
launches, past the GPU's power-management transient at the onset of load
(~15 ms, during which kernels run up to ~30 % slower); the timed steps
measure the steady state.

Prints ONE JSON line: achieved GB/s (algorithmic bytes / step time), % of the
8 TB/s HBM peak, rows/s, the roofline of the kernel, the other paths of the
library measured the same way, and the CPU oracle timed on a bounded sample.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "achieved HBM GB/s (% of peak) + rows/s, QK-norm+RoPE+FP8 4096tok×40h×128"
PEAK_HBM_GBS = 8000.0
KERNEL_SOURCES = ("fp8_quant_amd/csrc/rnq_rows.h", "fp8_quant_amd/csrc/rnq_rows_inst.h",
                  "fp8_quant_amd/csrc/rnq_rows.hip", "fp8_quant_amd/csrc/rnq_rows_quant.hip",
                  "fp8_quant_amd/csrc/rnq_device.h", "fp8_quant_amd/csrc/rnq_launch.h", "fp8_quant_amd/build.py")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_qk_4k.json")
WARM_MS = 40.0  # the onset-of-load transient lasts ~15 ms
LEAD_MS = 0.5  # untimed work queued ahead of the start event
# Rotate input/output sets until they hold at least this many bytes: the inputs
# must come from HBM, not the 256 MB Infinity Cache, and so must the outputs go
# to it. Outputs are a third or more of a path's bytes, so 2 GiB of sets keeps
# them well past the cache too: ordinary and device-scope stores allocate there,
# and with 600 MB of sets (about 220 MB of outputs) their lines could stay
# resident and never reach HBM inside the timed window (4096 x 4096 backward:
# 0.47 us faster with ordinary stores at 600 MB, no faster at 4 GB).
ROTATE_BYTES = 2 * 2**30
MAX_SETS = 256
COPY_BYTES = 256 * 2**20  # size of the plain copy used to calibrate the HBM byte counters


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


# ------------------------------------------------------------------ GPU timing


def _timed(torch, launches, steps, warmup, warm_ms=None, lead_ms=LEAD_MS):
    """Warm up (``warmup`` launches, and at least ``warm_ms`` of back-to-back
    work, so that every path is timed past the power-management transient at
    the onset of load, whatever its launch length), then time ``steps``
    back-to-back launches (rotating over the prepared launchers) between two
    events on the launch stream; ms per step. Each launcher holds
    pre-marshalled arguments, so the host enqueues a call in a few
    microseconds and the GPU runs the kernels back to back.

    After the warm-up's final synchronisation the queue is empty; a lead-in of
    untimed launches (about ``lead_ms`` of GPU work, judged from the warm-up's
    pace) is enqueued before the start event, so that the timed window opens
    on a busy GPU with the host already ahead of it: the host-side latency of
    submitting the first launch then falls outside the window, which matters
    when only a few steps are timed."""
    if warm_ms is None:
        warm_ms = WARM_MS
    n = len(launches)
    t0 = time.perf_counter()
    i = 0
    while i < warmup or (time.perf_counter() - t0) * 1e3 < warm_ms:
        launches[i % n]()
        i += 1
        if i % 256 == 0:
            torch.cuda.synchronize()  # (keeps the host clock on the GPU's pace)
    torch.cuda.synchronize()
    per_launch_ms = (time.perf_counter() - t0) * 1e3 / max(i, 1)
    lead = max(16, min(4096, math.ceil(lead_ms / max(per_launch_ms, 1e-4))))
    for j in range(lead):
        launches[(i + j) % n]()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for k in range(steps):
        launches[(i + lead + k) % n]()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def _n_sets(nbytes: int) -> int:
    return max(1, min(MAX_SETS, math.ceil(ROTATE_BYTES / max(nbytes, 1))))


def input_hashes(workloads, d, names):
    """SHA-256 of each named host input buffer (the bytes both the GPU and the oracle read)."""
    out = {}
    for k in names:
        t = d.get(k)
        if t is not None:
            # 16-bit floats, fp32 and bytes through workloads.bits; integer indices as they are
            out[k] = workloads.sha256(t.numpy() if not t.is_floating_point() else t)
    return out


def bench_qk(torch, rnq, workloads, ledger, name, steps, warmup, hashes=False):
    wl = workloads.WORKLOADS[name]
    d = workloads.generate(name)
    sha = input_hashes(workloads, d, ("q", "k", "wq", "wk", "cos", "sin", "qkv", "positions")) if hashes else None
    T, Hq, Hk, D, R = d["tokens"], d["q_heads"], d["kv_heads"], d["head_dim"], d["rope_dim"]
    led = ledger.qk_bytes(T, Hq, Hk, D, R, write_y=wl.write_y)
    pos_cpu = d.get("positions")
    if pos_cpu is not None:
        led = ledger.gathered_table_adjust(led, T, R, len(set(pos_cpu.tolist())))
    dev = torch.device("cuda:0")
    n_sets = _n_sets(led["total"])
    sets = []
    for _ in range(n_sets):
        if wl.fused_qkv:
            # q and k are views into one fused projection output (v columns are not read)
            qkv = d["qkv"].to(dev)
            q, k = qkv[:, : Hq * D].view(T, Hq, D), qkv[:, Hq * D : (Hq + Hk) * D].view(T, Hk, D)
        else:
            q, k = d["q"].to(dev), d["k"].to(dev) if Hk else None
        s = {"q": q, "k": k,
             "q8": torch.empty((T, Hq, D), dtype=torch.uint8, device=dev),
             "k8": torch.empty((T, Hk, D), dtype=torch.uint8, device=dev) if Hk else None,
             "qs": torch.empty((T, Hq), dtype=torch.float32, device=dev),
             "ks": torch.empty((T, Hk), dtype=torch.float32, device=dev) if Hk else None}
        s["qy"] = torch.empty((T, Hq, D), dtype=q.dtype, device=dev) if wl.write_y else None
        sets.append(s)
    wq = d["wq"].to(dev)
    wk = d["wk"].to(dev) if Hk else None
    cos, sin = d["cos"].to(dev), d["sin"].to(dev)
    pos = None if pos_cpu is None else pos_cpu.to(dev)
    del d

    if wl.fused_qkv or pos is not None:
        launches = [rnq.prepare_qk_norm_rope_fp8_ex(s["q"], s["k"], wq, wk, cos, sin, s["q8"], s["k8"], s["qs"],
                                                    s["ks"], s["qy"], None, positions=pos, eps=wl.eps,
                                                    fp8_max=wl.fp8_max) for s in sets]
    else:
        launches = [rnq.prepare_qk_norm_rope_fp8(s["q"], s["k"], wq, wk, cos, sin, s["q8"], s["k8"], s["qs"],
                                                 s["ks"], s["qy"], None, eps=wl.eps, fp8_max=wl.fp8_max)
                    for s in sets]
    ms = _timed(torch, launches, steps, warmup)
    out = {"workload": name, "ms": ms, "bytes": led["total"], "rows": led["rows"], "sets": n_sets}
    if sha is not None:
        out["inputs_sha256"] = sha
    del sets
    torch.cuda.empty_cache()
    return out


def bench_norm_rope(torch, rnq, workloads, ledger, name, steps, warmup):
    d = workloads.generate(name)
    M, N, R = d["rows"], d["width"], d["rope_dim"]
    led = ledger.norm_rope_bytes(M, N, R, d["rows_per_token"])
    pos_cpu = d.get("positions")
    if pos_cpu is not None:
        led = ledger.gathered_table_adjust(led, M // d["rows_per_token"], R, len(set(pos_cpu.tolist())))
    dev = torch.device("cuda:0")
    n_sets = _n_sets(led["total"])
    sets = [{"x": d["x"].to(dev), "y": torch.empty_like(d["x"], device=dev),
             "cos": d["cos"].to(dev), "sin": d["sin"].to(dev)} for _ in range(n_sets)]
    w = d["w"].to(dev)
    if pos_cpu is not None:
        pos = pos_cpu.to(dev)
        launches = [rnq.prepare_rmsnorm_rope_ex(s["x"], w, s["cos"], s["sin"], s["y"], positions=pos,
                                                rows_per_token=d["rows_per_token"]) for s in sets]
    else:
        launches = [rnq.prepare_rmsnorm_rope(s["x"], w, s["cos"], s["sin"], s["y"],
                                             rows_per_token=d["rows_per_token"]) for s in sets]
    ms = _timed(torch, launches, steps, warmup)
    del sets
    torch.cuda.empty_cache()
    return {"workload": name, "ms": ms, "bytes": led["total"], "rows": led["rows"], "sets": n_sets}


def bench_grouped(torch, rnq, workloads, ledger, name, steps, warmup):
    wl = workloads.WORKLOADS[name]
    d = workloads.generate(name)
    M, N, R, G = d["rows"], d["width"], d["rope_dim"], d["group_size"]
    led = ledger.grouped_bytes(M, N, R, G, d["rows_per_token"], write_y=wl.write_y)
    dev = torch.device("cuda:0")
    n_sets = _n_sets(led["total"])
    sets = [{"x": d["x"].to(dev), "cos": d["cos"].to(dev), "sin": d["sin"].to(dev),
             "codes": torch.empty((M, N), dtype=torch.uint8, device=dev),
             "scales": torch.empty((M, N // G), dtype=torch.float32, device=dev),
             "y": torch.empty_like(d["x"], device=dev) if wl.write_y else None} for _ in range(n_sets)]
    w = d["w"].to(dev)

    launches = [rnq.prepare_rmsnorm_rope_fp8_grouped(s["x"], w, s["cos"], s["sin"], s["codes"], s["scales"], s["y"],
                                                     group_size=G, rows_per_token=d["rows_per_token"],
                                                     eps=wl.eps, fp8_max=wl.fp8_max) for s in sets]
    ms = _timed(torch, launches, steps, warmup)
    del sets
    torch.cuda.empty_cache()
    return {"workload": name, "ms": ms, "bytes": led["total"], "rows": led["rows"], "sets": n_sets}


def bench_fusion(torch, rnq, workloads, ledger, steps, warmup):
    """The chapter 13 ledger page's norm+rope+quant plan on nrq_4k: fused (one kernel,
    one FP8 scale per row) against the three-kernel plan; and the chapter 28 designs
    A / B / C (1, 8, 40 rows per workgroup) on qk_4k against the row kernel."""
    from fp8_quant_amd import baselines

    wl = workloads.WORKLOADS["nrq_4k"]
    d = workloads.generate("nrq_4k")
    M, N, R = d["rows"], d["width"], d["rope_dim"]
    fused_b = ledger.norm_rope_quant_bytes(M, N, R)
    unfused_b = ledger.norm_rope_quant_bytes(M, N, R, unfused=True)
    dev = torch.device("cuda:0")
    n_sets = _n_sets(unfused_b["total"])
    sets = [{"x": d["x"].to(dev), "codes": torch.empty((M, N), dtype=torch.uint8, device=dev),
             "scales": torch.empty((M, 1), dtype=torch.float32, device=dev),
             "normed": torch.empty_like(d["x"], device=dev), "rotated": torch.empty_like(d["x"], device=dev)}
            for _ in range(n_sets)]
    w, cos, sin = d["w"].to(dev), d["cos"].to(dev), d["sin"].to(dev)
    fused = [rnq.prepare_rmsnorm_rope_fp8_grouped(s["x"], w, cos, sin, s["codes"], s["scales"], None, group_size=N,
                                                  eps=wl.eps, fp8_max=wl.fp8_max) for s in sets]
    unfused = [baselines.prepare_norm_rope_quant_unfused(s["x"], w, cos, sin, s["normed"], s["rotated"], s["codes"],
                                                         s["scales"].view(M), eps=wl.eps, fp8_max=wl.fp8_max)
               for s in sets]
    ms_f = _timed(torch, fused, steps, warmup)
    ms_u = _timed(torch, unfused, steps, warmup)
    del sets, fused, unfused
    torch.cuda.empty_cache()
    paths = [
        {"workload": "nrq_4k fused (1 kernel)", "ms": ms_f, "bytes": fused_b["total"], "rows": M, "sets": n_sets},
        {"workload": "nrq_4k unfused (3 kernels)", "ms": ms_u, "bytes": unfused_b["total"], "rows": M,
         "sets": n_sets},
    ]
    summary = {"plan": "norm+rope+quant 4096x4096 bf16, rope 128, per-row scale",
               "fused_us": round(ms_f * 1e3, 3), "unfused_us": round(ms_u * 1e3, 3),
               "measured_time_ratio": round(ms_u / ms_f, 3),
               "ledger_bytes_ratio": round(unfused_b["total"] / fused_b["total"], 3)}

    # designs A / B / C at the qk_4k shape (outputs equal the row kernel's)
    dq = workloads.generate("qk_4k")
    T, Hq, Hk, D, Rq = dq["tokens"], dq["q_heads"], dq["kv_heads"], dq["head_dim"], dq["rope_dim"]
    led = ledger.qk_bytes(T, Hq, Hk, D, Rq)
    n_sets = _n_sets(led["total"])
    qsets = [{"q": dq["q"].to(dev), "k": dq["k"].to(dev),
              "q8": torch.empty((T, Hq, D), dtype=torch.uint8, device=dev),
              "k8": torch.empty((T, Hk, D), dtype=torch.uint8, device=dev),
              "qs": torch.empty((T, Hq), dtype=torch.float32, device=dev),
              "ks": torch.empty((T, Hk), dtype=torch.float32, device=dev)} for _ in range(n_sets)]
    wq, wk, qc, qsn = dq["wq"].to(dev), dq["wk"].to(dev), dq["cos"].to(dev), dq["sin"].to(dev)
    designs = {}
    for label, rpb in (("A", 1), ("B", 8), ("C", Hq + Hk)):
        launches = [baselines.prepare_qk_design(s["q"], s["k"], wq, wk, qc, qsn, s["q8"], s["k8"], s["qs"], s["ks"],
                                                rows_per_block=rpb) for s in qsets]
        ms = _timed(torch, launches, steps, warmup)
        designs[label] = round(ms * 1e3, 3)
        paths.append({"workload": f"qk_4k design {label} ({rpb} rows per workgroup)", "ms": ms,
                      "bytes": led["total"], "rows": led["rows"], "sets": n_sets})
    del qsets
    torch.cuda.empty_cache()
    summary["qk_4k_designs_us"] = designs
    return paths, summary


def bench_rope_bwd(torch, rnq, workloads, ledger, name, steps, warmup):
    d = workloads.generate(name)
    M, N, R, rpt = d["rows"], d["width"], d["rope_dim"], d["rows_per_token"]
    led = ledger.rope_bwd_bytes(M, N, R, rpt)
    dev = torch.device("cuda:0")
    n_sets = _n_sets(led["total"])
    ws_bytes = rnq.rnq_rmsnorm_bwd_workspace_size(M, N)
    g = torch.Generator("cpu").manual_seed(91)
    gy = torch.randn(d["x"].shape, generator=g).to(d["x"].dtype)
    sets = [{"x": d["x"].to(dev), "gy": gy.to(dev), "cos": d["cos"].to(dev), "sin": d["sin"].to(dev),
             "gx": torch.empty_like(d["x"], device=dev), "gw": torch.empty((N,), dtype=torch.float32, device=dev),
             "ws": torch.empty((max(ws_bytes, 16) // 4,), dtype=torch.float32, device=dev)} for _ in range(n_sets)]
    w = d["w"].to(dev)
    launches = [rnq.prepare_rmsnorm_rope_bwd(s["x"], w, s["gy"], s["cos"], s["sin"], s["gx"], s["gw"], s["ws"],
                                             rows_per_token=rpt) for s in sets]
    ms = _timed(torch, launches, steps, warmup)
    del sets
    torch.cuda.empty_cache()
    return {"workload": name + " rope bwd", "ms": ms, "bytes": led["total"], "rows": M, "sets": n_sets,
            "workspace_bytes_each_way": ws_bytes}


def bench_rmsnorm(torch, rnq, workloads, ledger, name, steps, warmup):
    d = workloads.generate(name)
    M, N = d["rows"], d["width"]
    fwd = ledger.rmsnorm_fwd_bytes(M, N)
    bwd = ledger.rmsnorm_bwd_bytes(M, N)
    dev = torch.device("cuda:0")
    n_sets = _n_sets(bwd["total"])
    ws_bytes = rnq.rnq_rmsnorm_bwd_workspace_size(M, N)
    sets = [{"x": d["x"].to(dev), "gy": d["grad_y"].to(dev), "y": torch.empty_like(d["x"], device=dev),
             "gx": torch.empty_like(d["x"], device=dev),
             "gw": torch.empty((N,), dtype=torch.float32, device=dev),
             "ws": torch.empty((max(ws_bytes, 16) // 4,), dtype=torch.float32, device=dev)} for _ in range(n_sets)]
    w = d["w"].to(dev)

    ms_f = _timed(torch, [rnq.prepare_rmsnorm_fwd(s["x"], w, s["y"]) for s in sets], steps, warmup)
    ms_b = _timed(torch, [rnq.prepare_rmsnorm_bwd(s["x"], w, s["gy"], s["gx"], s["gw"], s["ws"]) for s in sets],
                  steps, warmup)
    del sets
    torch.cuda.empty_cache()
    return [
        {"workload": name + " fwd", "ms": ms_f, "bytes": fwd["total"], "rows": M, "sets": n_sets},
        {"workload": name + " bwd", "ms": ms_b, "bytes": bwd["total"], "rows": M, "sets": n_sets,
         "workspace_bytes_each_way": ws_bytes},
    ]


def bench_wide_norm_rope(torch, rnq, workloads, ledger, name, steps, warmup):
    """Path R on rows wider than a head (the fusion page's check shape scaled to the
    ledger page's plan: 4096 x 4096 bf16, rope 128, one table row per row)."""
    return bench_norm_rope(torch, rnq, workloads, ledger, name, steps, warmup)


ONLY_PATHS = {
    "qk_4k": lambda t, r, w, l, s, wu: [bench_qk(t, r, w, l, "qk_4k", s, wu)],
    "qk_small": lambda t, r, w, l, s, wu: [bench_qk(t, r, w, l, "qk_small", s, wu)],
    "qk_4k_fused": lambda t, r, w, l, s, wu: [bench_qk(t, r, w, l, "qk_4k_fused", s, wu)],
    "qk_64k": lambda t, r, w, l, s, wu: [bench_qk(t, r, w, l, "qk_64k", s, wu)],
    "rmsnorm_4k": lambda t, r, w, l, s, wu: bench_rmsnorm(t, r, w, l, "rmsnorm_4k", s, wu),
    "norm_rope_fp16": lambda t, r, w, l, s, wu: [bench_norm_rope(t, r, w, l, "norm_rope_fp16", s, wu)],
    "norm_rope_pos": lambda t, r, w, l, s, wu: [bench_norm_rope(t, r, w, l, "norm_rope_pos", s, wu)],
    "norm_rope_4k": lambda t, r, w, l, s, wu: [bench_wide_norm_rope(t, r, w, l, "norm_rope_4k", s, wu)],
    "rope_bwd": lambda t, r, w, l, s, wu: [bench_rope_bwd(t, r, w, l, "norm_rope_fp16", s, wu)],
    "rope_bwd_4k": lambda t, r, w, l, s, wu: [bench_rope_bwd(t, r, w, l, "norm_rope_4k", s, wu)],
    "grouped_4k": lambda t, r, w, l, s, wu: [bench_grouped(t, r, w, l, "grouped_4k", s, wu)],
}


def _summary(r):
    gbs = r["bytes"] / (r["ms"] * 1e-3) / 1e9
    out = {"workload": r["workload"], "us_per_call": round(r["ms"] * 1e3, 3), "GB/s": round(gbs, 1),
           "pct_of_peak": round(100 * gbs / PEAK_HBM_GBS, 2), "rows_per_s": round(r["rows"] / (r["ms"] * 1e-3), 1),
           "bytes": r["bytes"], "rotated_sets": r["sets"]}
    for k in ("workspace_bytes_each_way",):
        if k in r:
            out[k] = r[k]
    return out


def _with_floor(torch, summary, steps, warmup):
    """A path's summary with the memory floor for its own byte count, measured in the same run."""
    fl = bench_floor(torch, summary["bytes"], steps, warmup, with_empty=False)
    summary["floor"] = {"stream_us": fl["stream_us"], "d2d_copy_us": fl["d2d_copy_us"],
                        "stream_over_kernel": round(fl["stream_us"] / summary["us_per_call"], 3)}
    return summary


# ---------------------------------------------------------------- CPU oracle


def bench_floor(torch, total_bytes, steps, warmup, with_empty=True):
    """Memory floors for ``total_bytes`` of traffic, measured the same way as the
    kernels: rnq_baseline_stream_policy reading 2/3 and writing 1/3 of the bytes
    (rounded to whole 2 KB blocks; the headline moves 44.0 MB in and 21.6 MB
    out), no arithmetic, rotated like the headline, timed with nontemporal and
    with device-scope stores (the faster one is the floor); the runtime's own
    device-to-device copy (torch ``copy_``, i.e. hipMemcpyAsync) of half the
    bytes (read once, written once: the same total); and the cost of an empty
    launch."""
    from fp8_quant_amd import baselines

    src_bytes = (2 * total_bytes // 3) // 2048 * 2048
    n_sets = _n_sets(src_bytes * 3 // 2)
    dev = torch.device("cuda:0")
    sets = [(torch.empty(src_bytes, dtype=torch.uint8, device=dev).fill_(i + 1),
             torch.empty(src_bytes // 2, dtype=torch.uint8, device=dev)) for i in range(n_sets)]
    # the faster of two store policies (nontemporal, device scope): which one
    # wins depends on the size
    ms_nt = _timed(torch, [baselines.prepare_stream(a, b, store_policy=0) for a, b in sets], steps, warmup)
    ms_dev = _timed(torch, [baselines.prepare_stream(a, b, store_policy=1) for a, b in sets], steps, warmup)
    ms = min(ms_nt, ms_dev)
    del sets
    torch.cuda.empty_cache()
    moved = src_bytes * 3 // 2
    copy_bytes = total_bytes // 2 // 256 * 256
    n_sets = _n_sets(2 * copy_bytes)
    csets = [(torch.empty(copy_bytes, dtype=torch.uint8, device=dev).fill_(i + 1),
              torch.empty(copy_bytes, dtype=torch.uint8, device=dev)) for i in range(n_sets)]
    ms_copy = _timed(torch, [(lambda a=a, b=b: b.copy_(a)) for a, b in csets], steps, warmup)
    del csets
    torch.cuda.empty_cache()
    out = {"stream_us": round(ms * 1e3, 3), "stream_bytes": moved,
           "stream_nontemporal_us": round(ms_nt * 1e3, 3), "stream_device_scope_us": round(ms_dev * 1e3, 3),
           "stream_GB/s": round(moved / (ms * 1e-3) / 1e9, 1),
           "stream_pct_of_peak": round(100.0 * moved / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 2),
           "d2d_copy_us": round(ms_copy * 1e3, 3), "d2d_copy_bytes_moved": 2 * copy_bytes,
           "d2d_copy_GB/s": round(2 * copy_bytes / (ms_copy * 1e-3) / 1e9, 1),
           "d2d_copy_pct_of_peak": round(100.0 * 2 * copy_bytes / (ms_copy * 1e-3) / 1e9 / PEAK_HBM_GBS, 2),
           "kernel": "rnq_baseline_stream_policy (one 2 KB block in, 1 KB out per wave, 16-byte nontemporal loads; "
                     "the faster of nontemporal and device-scope stores); "
                     "d2d copy: torch copy_ (hipMemcpyAsync device to device)"}
    if with_empty:
        out["empty_launch_us"] = round(_timed(torch, [baselines.prepare_stream(None)], steps, warmup) * 1e3, 3)
    return out


_CPU = {}  # the sample a forked oracle worker reads (set before the pool forks)


def _oracle_run(start_token: int, budget_s: float):
    """Oracle calls on 256-token chunks from ``start_token`` on (wrapping), for about
    ``budget_s`` seconds; returns (tokens done, seconds)."""
    import numpy as np

    import oracle

    d = _CPU
    T = d["T"]
    tokens = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        lo = (start_token + tokens) % T
        hi = min(lo + 256, T)
        oracle.qk_norm_rope_fp8(d["q"][lo:hi], d["k"][lo:hi], d["wq"], d["wk"], d["cos"], d["sin"],
                                tokens=np.arange(lo, hi))
        tokens += hi - lo
    return tokens, time.perf_counter() - t0


def _oracle_worker(a):
    return _oracle_run(*a)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform

    return platform.processor() or "unknown"


def cpu_baseline(workload_name: str, single_s: float = 4.0, multi_s: float = 1.5, max_procs: int = 16) -> dict:
    """The CPU oracle (as it stands) on a bounded sample of the same workload,
    256-token chunks at a time: once in this process (one thread: numpy's
    elementwise loops are single-threaded), then in one forked process per
    available core (at most ``max_procs``), each on its own token range, for
    about ``multi_s`` seconds. Runs before anything touches the GPU (the
    workers are plain forks that only run numpy). ``value`` is the all-cores
    figure; the one-thread figure is kept beside it."""
    import multiprocessing

    import workloads
    from fp8_quant_amd import ledger

    d = workloads.generate(workload_name)
    T = d["tokens"]
    _CPU.update(T=T, q=workloads.bits(d["q"]), k=workloads.bits(d["k"]), wq=workloads.bits(d["wq"]),
                wk=workloads.bits(d["wk"]), cos=d["cos"].numpy(), sin=d["sin"].numpy())
    Hq, Hk, D, R = d["q_heads"], d["kv_heads"], d["head_dim"], d["rope_dim"]
    del d

    def rate(tokens, dt):
        b = ledger.qk_bytes(tokens, Hq, Hk, D, R)
        return b["total"] / dt / 1e9, b["rows"] / dt, b["rows"]

    tok1, dt1 = _oracle_run(0, single_s)
    gbs1, rows1, nrows1 = rate(tok1, dt1)
    single = {"value": round(gbs1, 6), "unit": "GB/s", "rows_per_s": round(rows1, 1), "cores": 1,
              "sample": f"{tok1} tokens ({nrows1} rows) in {dt1:.1f} s"}
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    procs = max(1, min(max_procs, avail))
    multi = None
    if procs > 1:
        ctx = multiprocessing.get_context("fork")
        t0 = time.perf_counter()
        with ctx.Pool(procs) as pool:
            res = pool.map_async(_oracle_worker, [((i * T) // procs, multi_s) for i in range(procs)]).get(
                timeout=120)
        wall = time.perf_counter() - t0
        tokm = sum(t for t, _ in res)
        span = max(dt for _, dt in res)
        gbsm, rowsm, nrowsm = rate(tokm, span)
        multi = {"value": round(gbsm, 6), "rows_per_s": round(rowsm, 1), "cores": procs, "tokens": tokm,
                 "rows": nrowsm, "seconds": round(span, 2), "wall_with_fork_s": round(wall, 2)}
    _CPU.clear()
    best = multi if multi is not None else single
    return {
        "value": best["value"],
        "unit": "GB/s",
        "rows_per_s": best["rows_per_s"],
        "cores": best["cores"],
        "kind": "oracle",
        "sample": (f"numpy oracle on 256-token chunks of {workload_name} ({T} tokens): "
                   + (f"{multi['tokens']} tokens ({multi['rows']} rows) over {procs} processes, one per core, "
                      f"each ~{multi_s:.1f} s on its own token range; " if multi else "")
                   + f"one thread alone: {tok1} tokens ({nrows1} rows) in {dt1:.1f} s"),
        "single_thread": single,
        "cpu_model": cpu_model(),
        "cores_available": avail,
    }


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    # defaults: ~30 ms of warm-up launches, past the GPU's power-management
    # transient at the onset of load (kernels run up to ~30 % slower for the
    # first ~15 ms), then ~30 ms timed
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=2000)
    ap.add_argument("--workload", default="qk_4k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-paths", action="store_true", help="time only the headline workload")
    ap.add_argument("--fusion-only", action="store_true",
                    help="time only the fused / unfused plan and the designs A/B/C; print their summary")
    ap.add_argument("--only", default="",
                    help="comma-separated paths to time alone, each with its same-run floor (one of: "
                         + ", ".join(ONLY_PATHS) + "); prints their summaries")
    ap.add_argument("--warm-ms", type=float, default=WARM_MS,
                    help="least warm-up of back-to-back launches per timed path, in ms (default %(default)s: past the "
                         "power-management transient; counter passes, which do not time, can take 0)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run a plain 256 MiB device copy three times (counter calibration) and exit")
    args = ap.parse_args()
    globals()["WARM_MS"] = args.warm_ms  # (read by _timed at each call)

    if args.calibrate_copy:
        import torch

        # three sources, each evicted from the 256 MB Infinity Cache by 1 GiB of
        # other writes before it is copied, so every copy reads from HBM
        srcs = [torch.full((COPY_BYTES,), 7 + i, dtype=torch.uint8, device="cuda:0") for i in range(3)]
        dst = torch.empty_like(srcs[0])
        scratch = torch.empty((4 * COPY_BYTES,), dtype=torch.uint8, device="cuda:0")
        for a in srcs:
            scratch.fill_(1)
            torch.cuda.synchronize()
            dst.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": COPY_BYTES, "copies": 3}))
        return 0

    if args.gpus != 1:
        print(f"bench.py: runs on one GPU only (asked for --gpus {args.gpus}); "
              "the rows are independent and the path would shard by token with no exchange", file=sys.stderr)
        return 2

    # the CPU oracle first, before anything touches the GPU (its workers are forks)
    cpu = None if args.no_cpu_baseline or args.fusion_only else cpu_baseline(args.workload)

    import torch

    import fp8_quant_amd as rnq
    import workloads
    from fp8_quant_amd import ledger

    torch.cuda.set_device(0)
    # every launch and event goes to one created stream (default priority): the
    # legacy null stream adds about a microsecond of synchronisation per launch
    torch.cuda.set_stream(torch.cuda.Stream(device=0))
    if args.fusion_only:
        fpaths, fsum = bench_fusion(torch, rnq, workloads, ledger, args.steps, args.warmup)
        print(json.dumps({"fusion": fsum, "paths": [_summary(r) for r in fpaths]}), flush=True)
        return 0
    if args.only:
        out = []
        for name in args.only.split(","):
            if name not in ONLY_PATHS:
                print(f"bench.py: unknown path {name!r} (one of {', '.join(ONLY_PATHS)})", file=sys.stderr)
                return 2
            for r in ONLY_PATHS[name](torch, rnq, workloads, ledger, args.steps, args.warmup):
                out.append(_with_floor(torch, _summary(r), args.steps, args.warmup))
        print(json.dumps({"paths": out}), flush=True)
        return 0
    head = bench_qk(torch, rnq, workloads, ledger, args.workload, args.steps, args.warmup, hashes=True)
    wl = workloads.WORKLOADS[args.workload]
    ms = head["ms"]
    value = head["bytes"] / (ms * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{args.workload}: QK-norm+RoPE+FP8, {wl.tokens} tokens x ({wl.q_heads} q + "
                        f"{wl.kv_heads} kv) heads x {wl.head_dim}, rope {wl.rope_dim}, bf16 in, "
                        f"e4m3fn + fp32 scale per row out",
            "tokens": wl.tokens, "q_heads": wl.q_heads, "kv_heads": wl.kv_heads,
            "head_dim": wl.head_dim, "rope_dim": wl.rope_dim,
        },
        "pct_of_peak": round(100.0 * value / PEAK_HBM_GBS, 2),
        "rows_per_s": round(head["rows"] / (ms * 1e-3), 1),
        "bytes_per_step": head["bytes"],
        "rotated_sets": head["sets"],
        "inputs_sha256": head["inputs_sha256"],
        "roofline": {
            "bound": "hbm",
            "achieved": round(value, 2),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(value / PEAK_HBM_GBS, 4),
            "traffic": measured_traffic(),
        },
    }
    if not args.no_other_paths:
        out["floor"] = bench_floor(torch, head["bytes"], args.steps, args.warmup)
        out["floor"]["kernel_over_stream_floor"] = round(ms * 1e3 / out["floor"]["stream_us"], 3)
        out["floor"]["kernel_over_d2d_copy"] = round(ms * 1e3 / out["floor"]["d2d_copy_us"], 3)
        paths = []
        steps, warm = max(10, args.steps // 4), max(2, args.warmup // 4)
        paths.append(_summary(bench_qk(torch, rnq, workloads, ledger, "qk_small", steps, warm)))
        # (every path but the small ones with the memory floor for its own byte count, timed in this run)
        paths += [_with_floor(torch, _summary(r), steps, warm)
                  for r in bench_rmsnorm(torch, rnq, workloads, ledger, "rmsnorm_4k", steps, warm)]
        paths.append(_with_floor(torch, _summary(bench_norm_rope(torch, rnq, workloads, ledger, "norm_rope_fp16",
                                                                 steps, warm)), steps, warm))
        paths.append(_with_floor(torch, _summary(bench_grouped(torch, rnq, workloads, ledger, "grouped_4k", steps, warm)),
                                 steps, warm))
        paths.append(_with_floor(torch, _summary(bench_rope_bwd(torch, rnq, workloads, ledger, "norm_rope_fp16", steps,
                                                                warm)), steps, warm))
        paths.append(_with_floor(torch, _summary(bench_norm_rope(torch, rnq, workloads, ledger, "norm_rope_4k", steps,
                                                                 warm)), steps, warm))
        paths.append(_with_floor(torch, _summary(bench_rope_bwd(torch, rnq, workloads, ledger, "norm_rope_4k", steps,
                                                                warm)), steps, warm))
        paths.append(_summary(bench_qk(torch, rnq, workloads, ledger, "qk_4k_fused", steps, warm)))
        paths.append(_with_floor(torch, _summary(bench_norm_rope(torch, rnq, workloads, ledger, "norm_rope_pos",
                                                                 steps, warm)), steps, warm))
        fpaths, fsum = bench_fusion(torch, rnq, workloads, ledger, steps, warm)
        paths += [_summary(r) for r in fpaths]
        out["fusion"] = fsum
        s64 = max(5, steps // 5)
        big = _summary(bench_qk(torch, rnq, workloads, ledger, "qk_64k", s64, 20))
        fl = bench_floor(torch, big["bytes"], s64, 20, with_empty=False)
        big["floor"] = {"stream_us": fl["stream_us"], "d2d_copy_us": fl["d2d_copy_us"],
                        "kernel_over_stream_floor": round(big["us_per_call"] / fl["stream_us"], 3)}
        paths.append(big)
        out["other_paths"] = paths
    out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    raise SystemExit(main())
