"""Summaries of rocprofv3 output (CSV format) for the kernels of this library.

    python rocprof_summary.py stats DIR
        Per-kernel table from DIR's *_kernel_stats.csv (calls, average and
        total duration), as markdown.

    python rocprof_summary.py shapes DIR [--only SUBSTR]
        Per (kernel, grid) table from DIR's *_kernel_trace.csv: the same
        kernel launched at different shapes gets one row per grid, with the
        number of dispatches and their median and minimum duration.

    python rocprof_summary.py counters DIR [DIR ...] [--only SUBSTR]
        Per (kernel, grid) averages per dispatch of every counter in the
        DIRs' *_counter_collection.csv (one --pmc pass per DIR), with the
        ratios that read directly: VALU and LDS instructions and MFMAs per
        wave, share of wave cycles waiting on a dependency, share of LDS
        cycles lost to bank conflicts.

    python rocprof_summary.py traffic \\
        --fetch DIR --write DIR --copy-fetch DIR --copy-write DIR \\
        --kernel SUBSTR --copy-bytes B --source FILE --algo-bytes A --out JSON
        HBM bytes per dispatch of the kernels whose name contains SUBSTR, from
        two --pmc runs (FETCH_SIZE, WRITE_SIZE: KiB per dispatch), each scaled
        by the same counter's reading for a plain device copy of B bytes (the
        copy's dispatches are the largest of its runs).  Writes JSON with the
        scaled read and write bytes per dispatch, the scale factors, the
        algorithmic bytes per dispatch A, and the sha256 of FILE (the kernel's
        source, so that a reader can tell when the figures went stale).
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys


XCDS = 8          # MI355X: accelerator complex dies
SIMDS = 1024      # 256 compute units x 4 SIMDs


def _csv_rows(directory: str, suffix: str):
    files = sorted(glob.glob(os.path.join(directory, "**", "*" + suffix), recursive=True))
    if not files:
        raise SystemExit(f"no *{suffix} under {directory}")
    rows = []
    for f in files:
        with open(f, newline="") as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def kernel_stats(directory: str):
    rows = _csv_rows(directory, "_kernel_stats.csv")
    out = []
    for r in rows:
        out.append(dict(name=r["Name"], calls=int(r["Calls"]), avg_ns=float(r["AverageNs"]),
                        total_ns=float(r["TotalDurationNs"]), min_ns=float(r["MinNs"]),
                        max_ns=float(r["MaxNs"]), pct=float(r["Percentage"])))
    out.sort(key=lambda d: -d["total_ns"])
    return out


def stats_markdown(directory: str) -> str:
    lines = ["| kernel | calls | avg us | min us | max us | total ms | % |",
             "|---|---:|---:|---:|---:|---:|---:|"]
    for d in kernel_stats(directory):
        name = d["name"].replace("|", "\\|")
        if len(name) > 110:
            name = name[:107] + "..."
        lines.append(f"| `{name}` | {d['calls']} | {d['avg_ns'] / 1e3:.3f} | "
                     f"{d['min_ns'] / 1e3:.3f} | {d['max_ns'] / 1e3:.3f} | "
                     f"{d['total_ns'] / 1e6:.3f} | {d['pct']:.2f} |")
    return "\n".join(lines)


def shapes_markdown(directory: str, only: str = "") -> str:
    rows = _csv_rows(directory, "_kernel_trace.csv")
    groups = {}
    for r in rows:
        name = r["Kernel_Name"]
        if only and only not in name:
            continue
        grid = (int(r["Grid_Size_X"]), int(r.get("Grid_Size_Y", 1) or 1),
                int(r.get("Grid_Size_Z", 1) or 1))
        wg = int(r["Workgroup_Size_X"]) * int(r.get("Workgroup_Size_Y", 1) or 1)
        d = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        groups.setdefault((name, grid, wg), []).append(d)
    lines = ["| kernel | grid (threads x, y, z) | workgroup | dispatches | median us | min us |",
             "|---|---|---:|---:|---:|---:|"]
    for (name, grid, wg), ds in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        ds.sort()
        short = name.replace("|", "\\|")
        if len(short) > 90:
            short = short[:87] + "..."
        lines.append(f"| `{short}` | {grid[0]} x {grid[1]} x {grid[2]} | {wg} | {len(ds)} | "
                     f"{ds[len(ds) // 2] / 1e3:.3f} | {ds[0] / 1e3:.3f} |")
    return "\n".join(lines)


def counters_markdown(directories, only: str = "") -> str:
    sums = {}
    for directory in directories:
        for r in _csv_rows(directory, "_counter_collection.csv"):
            name = r["Kernel_Name"]
            if only and only not in name:
                continue
            key = (name, int(r["Grid_Size"]), int(r["Workgroup_Size"]))
            cnt = sums.setdefault(key, {})
            c = cnt.setdefault(r["Counter_Name"], [0.0, set()])
            c[0] += float(r["Counter_Value"])
            c[1].add((directory, r.get("Process_Id", ""), r["Dispatch_Id"]))
    lines = []
    for (name, grid, wg), cnt in sorted(sums.items()):
        avg = {k: v[0] / len(v[1]) for k, v in cnt.items()}
        short = name.replace("|", "\\|")
        if len(short) > 90:
            short = short[:87] + "..."
        lines.append(f"### `{short}`, grid {grid} threads, workgroup {wg}")
        lines.append("")
        lines.append("| counter | per dispatch |")
        lines.append("|---|---:|")
        for k in sorted(avg):
            lines.append(f"| {k} | {avg[k]:.0f} |")
        waves = avg.get("SQ_WAVES")
        derived = []
        if waves:
            for k, label in (("SQ_INSTS_VALU", "VALU instructions per wave"),
                             ("SQ_INSTS_LDS", "LDS instructions per wave"),
                             ("SQ_INSTS_MFMA", "MFMA instructions per wave")):
                if k in avg:
                    derived.append((label, f"{avg[k] / waves:.1f}"))
        if "SQ_WAIT_INST_ANY" in avg and avg.get("SQ_WAVE_CYCLES"):
            derived.append(("wave cycles waiting on a dependency",
                            f"{avg['SQ_WAIT_INST_ANY'] / avg['SQ_WAVE_CYCLES']:.2f}"))
        if "SQ_VALU_MFMA_BUSY_CYCLES" in avg and avg.get("GRBM_GUI_ACTIVE"):
            # GRBM_GUI_ACTIVE sums the elapsed cycles of the 8 XCDs; the MFMA
            # busy cycles are summed over all 1024 SIMDs (256 CUs x 4)
            elapsed = avg["GRBM_GUI_ACTIVE"] / XCDS
            derived.append(("matrix cores busy (share of SIMD cycles)",
                            f"{avg['SQ_VALU_MFMA_BUSY_CYCLES'] / (elapsed * SIMDS):.3f}"))
        if "SQ_LDS_BANK_CONFLICT" in avg and avg.get("SQ_LDS_IDX_ACTIVE"):
            derived.append(("LDS cycles lost to bank conflicts",
                            f"{avg['SQ_LDS_BANK_CONFLICT'] / avg['SQ_LDS_IDX_ACTIVE']:.2f}"))
        for label, v in derived:
            lines.append(f"| {label} | {v} |")
        lines.append("")
    return "\n".join(lines)


def _counter_per_dispatch(directory: str, counter: str):
    """{dispatch id: (kernel name, value)} for one counter."""
    rows = _csv_rows(directory, "_counter_collection.csv")
    out = {}
    for r in rows:
        if r.get("Counter_Name") != counter:
            continue
        did = (r.get("Process_Id", ""), r["Dispatch_Id"])
        name = r["Kernel_Name"]
        out[did] = (name, out.get(did, (name, 0.0))[1] + float(r["Counter_Value"]))
    return out


def _avg_for(d, substr):
    vals = [v for name, v in d.values() if substr in name]
    if not vals:
        raise SystemExit(f"no dispatch of a kernel containing {substr!r}")
    return sum(vals) / len(vals), len(vals)


def _copy_reading(d, copies: int = 10):
    vals = sorted((v for _, v in d.values()), reverse=True)[:copies]
    return sum(vals) / len(vals)


def traffic(args) -> dict:
    fetch_kib, n_fetch = _avg_for(_counter_per_dispatch(args.fetch, "FETCH_SIZE"), args.kernel)
    write_kib, n_write = _avg_for(_counter_per_dispatch(args.write, "WRITE_SIZE"), args.kernel)
    copy_fetch_kib = _copy_reading(_counter_per_dispatch(args.copy_fetch, "FETCH_SIZE"))
    copy_write_kib = _copy_reading(_counter_per_dispatch(args.copy_write, "WRITE_SIZE"))
    # bytes per KiB the counter reports, from the copy of known size
    f_scale = args.copy_bytes / copy_fetch_kib
    w_scale = args.copy_bytes / copy_write_kib
    read_b = fetch_kib * f_scale
    write_b = write_kib * w_scale
    with open(args.source, "rb") as fh:
        sha = hashlib.sha256(fh.read()).hexdigest()
    return {
        "kernel": args.kernel,
        "dispatches_fetch": n_fetch,
        "dispatches_write": n_write,
        "fetch_kib_per_dispatch": round(fetch_kib, 3),
        "write_kib_per_dispatch": round(write_kib, 3),
        "copy_bytes": args.copy_bytes,
        "copy_fetch_kib": round(copy_fetch_kib, 3),
        "copy_write_kib": round(copy_write_kib, 3),
        "fetch_bytes_per_counted_kib": round(f_scale, 3),
        "write_bytes_per_counted_kib": round(w_scale, 3),
        "read_bytes_per_launch": round(read_b, 1),
        "write_bytes_per_launch": round(write_b, 1),
        "bytes_per_launch": round(read_b + write_b, 1),
        "algorithmic_bytes_per_launch": args.algo_bytes,
        "traffic_over_algorithmic": round((read_b + write_b) / args.algo_bytes, 4)
        if args.algo_bytes else None,
        "kernel_source": os.path.relpath(os.path.abspath(args.source),
                                         os.path.dirname(os.path.abspath(__file__))),
        "kernel_source_sha256": sha,
    }


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    sh = sub.add_parser("shapes")
    sh.add_argument("dir")
    sh.add_argument("--only", default="")
    c = sub.add_parser("counters")
    c.add_argument("dir", nargs="+")
    c.add_argument("--only", default="")
    t = sub.add_parser("traffic")
    for k in ("--fetch", "--write", "--copy-fetch", "--copy-write", "--kernel", "--source", "--out"):
        t.add_argument(k, required=True)
    t.add_argument("--copy-bytes", type=float, required=True)
    t.add_argument("--algo-bytes", type=float, default=0.0)
    args = ap.parse_args(argv)
    if args.cmd == "stats":
        print(stats_markdown(args.dir))
    elif args.cmd == "shapes":
        print(shapes_markdown(args.dir, args.only))
    elif args.cmd == "counters":
        print(counters_markdown(args.dir, args.only))
    else:
        res = traffic(args)
        with open(args.out, "w") as fh:
            json.dump(res, fh, indent=1)
            fh.write("\n")
        json.dump(res, sys.stdout, indent=1)
        print()


if __name__ == "__main__":
    main()
