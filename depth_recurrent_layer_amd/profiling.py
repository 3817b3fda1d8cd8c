"""Helpers to turn rocprofv3 CSV output into short summaries (kernel times, HBM traffic).

    python -m depth_recurrent_layer_amd.profiling stats <kernel_stats.csv> <title> <command>
    python -m depth_recurrent_layer_amd.profiling traffic <class> <kernel substring>
        <fetch_counter.csv> <write_counter.csv> <copy_fetch.csv> <copy_write.csv> <copy_bytes>
        <command...>

Both print markdown; the traffic summary ends in a json block that the benchmark reads.

FETCH_SIZE / WRITE_SIZE are read per dispatch (KiB) and scaled by what the same counters
report for a plain device copy of known size.  The summary records a digest of the kernel
sources; a later source change makes the stored traffic stale (the benchmark then reports
null).
"""
from __future__ import annotations

import csv
import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))


def source_digest() -> str:
    """sha256 over the library sources (any kernel change invalidates stored counters)."""
    h = hashlib.sha256()
    csrc = os.path.join(HERE, "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".h", ".cpp")):
            with open(os.path.join(csrc, name), "rb") as fh:
                h.update(name.encode())
                h.update(fh.read())
    return h.hexdigest()


def kernel_stats_md(csv_path: str, title: str, command: str, top: int = 16) -> str:
    rows = list(csv.DictReader(open(csv_path)))
    out = [f"# {title}", "", "Command (repository root, one MI355X):", "", "```", command, "```",
           "", "| kernel | calls | total us | avg us | min us | max us | % |",
           "|---|---|---|---|---|---|---|"]
    for r in rows[:top]:
        n = r["Name"] if len(r["Name"]) < 90 else r["Name"][:87] + "..."
        out.append(f"| `{n}` | {r['Calls']} | {int(r['TotalDurationNs']) / 1e3:.1f} | "
                   f"{float(r['AverageNs']) / 1e3:.2f} | {int(r['MinNs']) / 1e3:.2f} | "
                   f"{int(r['MaxNs']) / 1e3:.2f} | {r['Percentage']} |")
    return "\n".join(out) + "\n"


def counter_per_dispatch(csv_path: str, counter: str, kernel_substr: str) -> list:
    """Counter values (KiB) of every dispatch whose kernel name contains kernel_substr."""
    vals = {}
    for r in csv.DictReader(open(csv_path)):
        name = r.get("Kernel_Name", "")
        if kernel_substr not in name or r.get("Counter_Name") != counter:
            continue
        key = r.get("Dispatch_Id") or r.get("Correlation_Id")
        vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
    return list(vals.values())


def traffic_summary(kclass, kernel_substr, fetch_csv, write_csv, copy_fetch_csv,
                    copy_write_csv, copy_bytes, command):
    copy_f = counter_per_dispatch(copy_fetch_csv, "FETCH_SIZE", "")
    copy_w = counter_per_dispatch(copy_write_csv, "WRITE_SIZE", "")
    # the largest dispatches of the calibration run are the copies of known size
    kf = copy_bytes / (max(copy_f) * 1024.0)
    kw = copy_bytes / (max(copy_w) * 1024.0)
    f = counter_per_dispatch(fetch_csv, "FETCH_SIZE", kernel_substr)
    w = counter_per_dispatch(write_csv, "WRITE_SIZE", kernel_substr)
    fetch = sum(f) / len(f) * 1024.0 * kf
    write = sum(w) / len(w) * 1024.0 * kw
    return {"class": kclass, "kernel": kernel_substr, "dispatches": len(f),
            "fetch_bytes_per_launch": fetch, "write_bytes_per_launch": write,
            "bytes_per_launch": fetch + write, "copy_scale_fetch": kf, "copy_scale_write": kw,
            "copy_bytes": copy_bytes, "source_sha256": source_digest(), "command": command}


if __name__ == "__main__":
    mode = sys.argv[1]
    if mode == "stats":
        sys.stdout.write(kernel_stats_md(sys.argv[2], sys.argv[3], sys.argv[4]))
    elif mode == "traffic":
        s = traffic_summary(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5], sys.argv[6],
                            sys.argv[7], float(sys.argv[8]), " ".join(sys.argv[9:]))
        print(f"# HBM traffic of `{s['kernel']}` ({s['class']})\n")
        print("FETCH_SIZE and WRITE_SIZE (KiB per dispatch) from two separate rocprofv3 --pmc "
              "runs, scaled by the same counters over a plain device copy of "
              f"{s['copy_bytes'] / 2**20:.0f} MiB (fetch x{s['copy_scale_fetch']:.4f}, "
              f"write x{s['copy_scale_write']:.4f}).\n")
        print(f"- dispatches: {s['dispatches']}")
        print(f"- fetch per launch: {s['fetch_bytes_per_launch'] / 2**20:.2f} MiB")
        print(f"- write per launch: {s['write_bytes_per_launch'] / 2**20:.2f} MiB")
        print(f"- commands: {s['command']}\n")
        print("```json\n" + json.dumps(s, indent=1) + "\n```")
    else:
        raise SystemExit(__doc__)
