"""Summaries of rocprofv3 output for the measurement record (host-side only).

* ``stats``   - per-kernel call count and durations from a ``--kernel-trace``
  run (``*_kernel_trace.csv``), as a short Markdown table;
* ``counters`` - every (kernel, grid) of a run with its calibrated HBM read
  and write bytes per dispatch (two ``--pmc`` passes, as for ``traffic``), as
  a Markdown table;
* ``traffic`` - HBM bytes per launch of the row kernel from two ``--pmc``
  passes (FETCH_SIZE, then WRITE_SIZE, both in KiB per dispatch), each scaled
  by what the same counter reads for a plain copy of known size, written as
  JSON together with a hash of the kernel sources (the bench reports the
  figure only while the sources are unchanged).

Usage::

    python -m fp8_quant_amd.profiling stats TRACE_CSV OUT_MD --command "..."
    python -m fp8_quant_amd.profiling counters FETCH_CSV WRITE_CSV COPY_FETCH_CSV COPY_WRITE_CSV \
        COPY_BYTES OUT_MD --command "..." [--sq SQ_CSV]
    python -m fp8_quant_amd.profiling traffic FETCH_CSV WRITE_CSV COPY_FETCH_CSV COPY_WRITE_CSV \
        COPY_BYTES OUT_JSON --kernel rows_kernel --grid 1310720 --command "..."
"""

from __future__ import annotations

import argparse
import csv
import json
import os
import statistics
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _rows(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def kernel_stats(trace_csv: str) -> list[dict]:
    rows = _rows(trace_csv)
    by = {}
    for r in rows:
        d = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        key = (r["Kernel_Name"], r.get("Grid_Size_X") or r.get("Grid_Size", ""))
        by.setdefault(key, []).append(d)
    out = []
    for (name, grid), ds in sorted(by.items(), key=lambda kv: -sum(kv[1])):
        out.append({
            "kernel": name, "grid": grid, "calls": len(ds), "avg_ns": sum(ds) / len(ds),
            "median_ns": statistics.median(ds), "min_ns": min(ds), "max_ns": max(ds), "total_ns": sum(ds),
        })
    return out


def counter_per_dispatch(counter_csv: str, counter: str, kernel_sub: str, grid: str | None = None) -> float:
    vals = {}
    for r in _rows(counter_csv):
        if r["Counter_Name"] != counter or kernel_sub not in r["Kernel_Name"]:
            continue
        g = r.get("Grid_Size") or r.get("Grid_Size_X")
        if grid is not None and g != grid:
            continue
        # a dispatch may report one row per agent-level instance; add them per dispatch
        vals[r["Dispatch_Id"]] = vals.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    if not vals:
        raise ValueError(f"no {counter} rows for kernel matching {kernel_sub!r} (grid {grid})")
    return statistics.median(vals.values())


def headline_lines(trace_csv: str, kernel_sub: str, grid: str, timed: int, bench_us=None, block: int = 500) -> list:
    """The headline kernel's timed launches (the last ``timed`` of its dispatches at ``grid``):
    duration statistics, gaps, the span per launch, and the median per stretch of ``block``
    launches over the whole run (the onset-of-load transient)."""
    ev = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in _rows(trace_csv)
                if kernel_sub in r["Kernel_Name"] and (r.get("Grid_Size_X") or r.get("Grid_Size")) == grid)
    if len(ev) < timed:
        return []
    t = ev[-timed:]
    d = sorted(e - s for s, e in t)
    q = lambda f: d[min(len(d) - 1, int(f * len(d)))] / 1e3
    gaps = sorted(t[i + 1][0] - t[i][1] for i in range(len(t) - 1))
    span = (t[-1][1] - t[0][0]) / timed / 1e3
    out = [
        "",
        f"Headline kernel (grid {grid} threads): {len(ev)} launches ({len(ev) - timed} warm-up + {timed} timed), "
        "back to back.",
        f"Over the {timed} timed launches: mean {statistics.mean(d) / 1e3:.2f} us, median {statistics.median(d) / 1e3:.2f} us,",
        f"p10 {q(0.1):.2f} us, p90 {q(0.9):.2f} us; median gap between kernels {statistics.median(gaps) / 1e3:.2f} us;",
        f"first start to last end / {timed} = {span:.2f} us per launch"
        + (f" (the bench's own figure in this run: {bench_us:.2f} us)." if bench_us else "."),
        "",
        f"Duration by stretch of the whole run (median of each block of {block} launches, start time of the block):",
        "",
        "| start | median us |",
        "|---|---|",
    ]
    t0 = ev[0][0]
    for i in range(0, len(ev) - block + 1, block):
        blk = ev[i : i + block]
        out.append(f"| {(blk[0][0] - t0) / 1e6:.1f} ms | {statistics.median(e - s for s, e in blk) / 1e3:.2f} |")
    return out


def write_stats_md(trace_csv: str, out_md: str, command: str, top: int = 16, headline=None) -> None:
    st = kernel_stats(trace_csv)
    lines = [
        "# rocprofv3 kernel trace summary",
        "",
        f"Command: `{command}`",
        "",
        "| kernel | grid | calls | avg us | median us | min us | max us |",
        "|---|---|---|---|---|---|---|",
    ]
    for s in st[:top]:
        name = s["kernel"].replace("|", "\\|")
        if len(name) > 90:
            name = name[:87] + "..."
        lines.append(f"| `{name}` | {s['grid']} | {s['calls']} | {s['avg_ns'] / 1e3:.2f} | "
                     f"{s['median_ns'] / 1e3:.2f} | {s['min_ns'] / 1e3:.2f} | {s['max_ns'] / 1e3:.2f} |")
    if headline:
        lines += headline_lines(trace_csv, *headline)
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


def _per_kernel(counter_csv: str, counter: str) -> dict:
    """(kernel, grid) -> median over dispatches of the counter summed per dispatch."""
    per = {}
    for r in _rows(counter_csv):
        if r["Counter_Name"] != counter:
            continue
        key = (r["Kernel_Name"], r.get("Grid_Size") or r.get("Grid_Size_X"), r.get("Workgroup_Size", ""))
        d = per.setdefault(key, {})
        d[r["Dispatch_Id"]] = d.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    return {k: statistics.median(v.values()) for k, v in per.items()}


SQ_COLUMNS = ("SQ_INSTS_VALU", "SQ_INSTS_SALU", "SQ_INSTS_VMEM", "SQ_INSTS_LDS", "SQ_WAVE_CYCLES")


def write_counters_md(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, copy_bytes, out_md, command,
                      sq_csv=None, skip=("copyBuffer", "FillFunctor")) -> None:
    """Calibrated HBM bytes per dispatch of every (kernel, grid); with ``sq_csv``
    (an SQ counter pass of the same command) also the waves and the instruction
    mix per wave."""
    cf = counter_per_dispatch(copy_fetch_csv, "FETCH_SIZE", "copy", None)
    cw = counter_per_dispatch(copy_write_csv, "WRITE_SIZE", "copy", None)
    f_scale, w_scale = copy_bytes / (cf * 1024.0), copy_bytes / (cw * 1024.0)
    fetch, write = _per_kernel(fetch_csv, "FETCH_SIZE"), _per_kernel(write_csv, "WRITE_SIZE")
    sq = {c: _per_kernel(sq_csv, c) for c in ("SQ_WAVES",) + SQ_COLUMNS} if sq_csv else None
    lines = [
        "# HBM bytes per dispatch by kernel (rocprofv3 FETCH_SIZE / WRITE_SIZE, calibrated)"
        + (" and instruction mix per wave" if sq else ""),
        "",
        f"Command: `{command}` (one pass per counter group), and `python3 bench.py --calibrate-copy` under",
        f"FETCH_SIZE and WRITE_SIZE for the calibration: a {copy_bytes}-byte copy reads {cf:.0f} KiB and writes",
        f"{cw:.0f} KiB as counted, so FETCH is scaled by {f_scale:.4f} and WRITE by {w_scale:.4f}. Medians over",
        "the profiled dispatches of each (kernel, grid).",
        "",
    ]
    head = "| kernel | grid (threads) | workgroup | read MB | written MB | total MB |"
    rule = "|---|---|---|---|---|---|"
    if sq:
        head += " waves | " + " | ".join(c[3:].replace("INSTS_", "").lower() + " / wave" for c in SQ_COLUMNS) + " |"
        rule += "---|" * (1 + len(SQ_COLUMNS))
    lines += [head, rule]
    for key in sorted(fetch, key=lambda k: -fetch[k]):
        if any(t in key[0] for t in skip) or key not in write:
            continue
        rd = fetch[key] * 1024.0 * f_scale / 1e6
        wr = write[key] * 1024.0 * w_scale / 1e6
        name = key[0].replace("|", "\\|")
        if len(name) > 80:
            name = name[:77] + "..."
        row = f"| `{name}` | {key[1]} | {key[2]} | {rd:.2f} | {wr:.2f} | {rd + wr:.2f} |"
        if sq:
            waves = sq["SQ_WAVES"].get(key)
            if waves:
                row += f" {waves:.0f} | " + " | ".join(f"{sq[c].get(key, float('nan')) / waves:.1f}" for c in SQ_COLUMNS) + " |"
            else:
                row += " |" * (1 + len(SQ_COLUMNS))
        lines.append(row)
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


def write_traffic_json(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, copy_bytes, out_json,
                       kernel_sub, grid, command, algorithmic_bytes=None) -> dict:
    sys.path.insert(0, ROOT)
    import bench  # the kernel-source hash the bench compares against

    fetch_kib = counter_per_dispatch(fetch_csv, "FETCH_SIZE", kernel_sub, grid)
    write_kib = counter_per_dispatch(write_csv, "WRITE_SIZE", kernel_sub, grid)
    cf = counter_per_dispatch(copy_fetch_csv, "FETCH_SIZE", "copy", None)
    cw = counter_per_dispatch(copy_write_csv, "WRITE_SIZE", "copy", None)
    f_scale = copy_bytes / (cf * 1024.0)
    w_scale = copy_bytes / (cw * 1024.0)
    fetch_b = fetch_kib * 1024.0 * f_scale
    write_b = write_kib * 1024.0 * w_scale
    rec = {
        "kernel": kernel_sub,
        "grid": grid,
        "command": command,
        "fetch_kib_per_dispatch": fetch_kib,
        "write_kib_per_dispatch": write_kib,
        "copy_bytes": copy_bytes,
        "copy_fetch_kib": cf,
        "copy_write_kib": cw,
        "fetch_scale": f_scale,
        "write_scale": w_scale,
        "fetch_bytes_per_launch": round(fetch_b),
        "write_bytes_per_launch": round(write_b),
        "traffic_bytes_per_launch": round(fetch_b + write_b),
        "algorithmic_bytes_per_launch": algorithmic_bytes,
        "kernel_source_sha256": bench.kernel_source_hash(),
    }
    with open(out_json, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    return rec


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    a = sub.add_parser("stats")
    a.add_argument("trace_csv")
    a.add_argument("out_md")
    a.add_argument("--command", required=True)
    a.add_argument("--headline", nargs=3, metavar=("KERNEL", "GRID", "TIMED"),
                   help="add the timed-launch statistics of this kernel at this grid")
    a.add_argument("--bench-us", type=float, default=None)
    c = sub.add_parser("counters")
    for n in ("fetch_csv", "write_csv", "copy_fetch_csv", "copy_write_csv"):
        c.add_argument(n)
    c.add_argument("copy_bytes", type=int)
    c.add_argument("out_md")
    c.add_argument("--command", required=True)
    c.add_argument("--sq", default=None, help="an SQ counter pass of the same command (instruction mix per wave)")
    b = sub.add_parser("traffic")
    for n in ("fetch_csv", "write_csv", "copy_fetch_csv", "copy_write_csv"):
        b.add_argument(n)
    b.add_argument("copy_bytes", type=int)
    b.add_argument("out_json")
    b.add_argument("--kernel", default="rows_kernel")
    b.add_argument("--grid", default=None)
    b.add_argument("--algorithmic-bytes", type=int, default=None)
    b.add_argument("--command", required=True)
    args = ap.parse_args(argv)
    if args.cmd == "stats":
        hl = None if not args.headline else (args.headline[0], args.headline[1], int(args.headline[2]), args.bench_us)
        write_stats_md(args.trace_csv, args.out_md, args.command, headline=hl)
    elif args.cmd == "counters":
        write_counters_md(args.fetch_csv, args.write_csv, args.copy_fetch_csv, args.copy_write_csv, args.copy_bytes,
                          args.out_md, args.command, sq_csv=args.sq)
    else:
        rec = write_traffic_json(args.fetch_csv, args.write_csv, args.copy_fetch_csv, args.copy_write_csv,
                                 args.copy_bytes, args.out_json, args.kernel, args.grid, args.command,
                                 args.algorithmic_bytes)
        print(json.dumps(rec, indent=1))
    return 0


if __name__ == "__main__":
    raise SystemExit(main())
