"""Helpers to turn rocprofv3 CSV output into short summaries (kernel times, HBM traffic).

    python -m depth_recurrent_layer_amd.profiling stats <kernel_stats.csv> <title> <command>
    python -m depth_recurrent_layer_amd.profiling launches <kernel_trace.csv> <title> <command>
    python -m depth_recurrent_layer_amd.profiling traffic <class> <kernel substring>
        <fetch_counter.csv> <write_counter.csv> <copy_fetch.csv> <copy_write.csv> <copy_bytes>
        <command...>
    python -m depth_recurrent_layer_amd.profiling traffic-all <workload> <out dir>
        <fetch_counter.csv> <write_counter.csv> <copy_fetch.csv> <copy_write.csv> <copy_bytes>
        <command...>
    python -m depth_recurrent_layer_amd.profiling mfma <workload> <out dir> <counter.csv>
        <command...>

All print markdown (traffic-all writes one file per kernel class); a traffic summary ends
in a json block that the benchmark reads.

FETCH_SIZE / WRITE_SIZE are read per dispatch (KiB) and scaled by what the same counters
report for a plain device copy of known size.  The summary records a digest of the
sources of its kernel class; a later change to them makes the stored traffic stale (the
benchmark then reports null).
"""
from __future__ import annotations

import csv
import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))

# Sources of each timed kernel class (besides the shared device header), and per workload
# the kernel-name substring that picks a class's dispatches in a counter file (the
# launches choose their GEMM instances and the attention kernels by shape).
CLASS_SOURCES = {
    "qkv_proj": ["gemm.hip"], "out_proj": ["gemm.hip"], "seq_attn": ["attn.hip"],
    "depth_attn": ["attn.hip"], "attention": ["attn.hip"], "route": ["route.hip"],
    "expert_ffn": ["expert_ffn.hip"], "combine": ["moe.hip"],
}
SHARED_SOURCES = ["common.h"]
WORKLOAD_KERNELS = {
    "small": {
        "qkv_proj": "Li32ELi64ELi4ELi2ELi128ELi2ELi2ELb1",  # the 8-wave QKV instance (mangled)
        "out_proj": "GemmCfg<32, 32, 2, 2, 128, 4, 2, false>",
        "seq_attn": "sa_flash_kernel",
        "depth_attn": "depth_attn_kernel",
        "attention": "attn_pair_kernel",   # SA and DA in one launch
        "route": "router_fused_bf16_kernel",
        "expert_ffn": "expert_ffn_kernel",
        "combine": "combine_norm_kernel",
    },
    "deep": {
        "qkv_proj": "Li64ELi64ELi4ELi4ELi128ELi2ELi1ELb1",  # the 16-wave 256 x 256 instance
        "out_proj": "GemmCfg<64, 64, 4, 4, 128, 2, 1, false>",  # float output, 256 x 256
        "seq_attn": "sa_flash2_kernel",    # two query sets per wave (separate launches)
        "depth_attn": "depth_attn_kernel",
        "attention": "attn_pair2_kernel",  # SA and DA blocks interleaved in one launch
        "route": "router_fused_bf16_kernel",
        "expert_ffn": "expert_ffn_kernel",
        "combine": "combine_norm_kernel",
    },
}
# classes bound by the matrix cores (their MFMA-busy share is summarised)
MFMA_CLASSES = ["qkv_proj", "out_proj", "seq_attn", "attention", "expert_ffn"]
CLASS_KERNELS = WORKLOAD_KERNELS["small"]


def source_digest(kclass: str | None = None) -> str:
    """sha256 over the sources of one kernel class (every library source when None): a
    change to them invalidates that class's stored counters."""
    h = hashlib.sha256()
    csrc = os.path.join(HERE, "csrc")
    if kclass is None:
        names = sorted(n for n in os.listdir(csrc) if n.endswith((".hip", ".h", ".cpp")))
    else:
        names = sorted(CLASS_SOURCES[kclass] + SHARED_SOURCES)
    for name in names:
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


def launch_stats_md(trace_csv: str, title: str, command: str, top: int = 24,
                    only: str | None = None) -> str:
    """Per (kernel, grid) durations from a kernel trace: one kernel launched with several
    shapes (the projections of the different wirings, say) gets one row per shape.
    only: keep the kernels whose name contains it (shares are then of their total)."""
    groups = {}
    for r in csv.DictReader(open(trace_csv)):
        if only and only not in r["Kernel_Name"]:
            continue
        grid = (f"{int(r['Grid_Size_X']) // max(1, int(r['Workgroup_Size_X']))}x"
                f"{int(r['Grid_Size_Y']) // max(1, int(r['Workgroup_Size_Y']))}"
                f"x{int(r['Workgroup_Size_X'])}")
        key = (r["Kernel_Name"], grid)
        groups.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    total = sum(sum(v) for v in groups.values())
    rows = sorted(groups.items(), key=lambda kv: -sum(kv[1]))[:top]
    out = [f"# {title}", "", "Command (repository root, one MI355X):", "", "```", command, "```",
           "", "Durations per kernel and launch shape (blocks x, blocks y, threads per block)" +
           (f"; only kernels named `{only}`, shares of their total." if only else "."),
           "", "| kernel | shape | calls | total us | avg us | min us | max us | % |",
           "|---|---|---|---|---|---|---|---|"]
    for (name, grid), d in rows:
        n = name if len(name) < 90 else name[:87] + "..."
        out.append(f"| `{n}` | {grid} | {len(d)} | {sum(d) / 1e3:.1f} | {sum(d) / len(d) / 1e3:.2f} "
                   f"| {min(d) / 1e3:.2f} | {max(d) / 1e3:.2f} | {100.0 * sum(d) / total:.2f} |")
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
    if not f or not w:
        return None  # the class did not run in the profiled command
    fetch = sum(f) / len(f) * 1024.0 * kf
    write = sum(w) / len(w) * 1024.0 * kw
    return {"class": kclass, "kernel": kernel_substr, "dispatches": len(f),
            "fetch_bytes_per_launch": fetch, "write_bytes_per_launch": write,
            "bytes_per_launch": fetch + write, "copy_scale_fetch": kf, "copy_scale_write": kw,
            "copy_bytes": copy_bytes, "source_sha256": source_digest(kclass), "command": command}


def counters_per_class(csv_path: str, kernels: dict) -> dict:
    """Per kernel class: {counter: value summed over the class's dispatches}, and the
    dispatch count."""
    out = {}
    for r in csv.DictReader(open(csv_path)):
        name = r.get("Kernel_Name", "")
        for kclass, sub in kernels.items():
            if sub in name:
                d = out.setdefault(kclass, {"dispatches": set()})
                d["dispatches"].add(r.get("Dispatch_Id") or r.get("Correlation_Id"))
                c = r["Counter_Name"]
                d[c] = d.get(c, 0.0) + float(r["Counter_Value"])
                break
    for d in out.values():
        d["dispatches"] = len(d["dispatches"])
    return out


def mfma_busy_md(kclass, workload, d, kernel, command) -> str:
    """SQ_VALU_MFMA_BUSY_CYCLES over the busy cycles of the CUs' four SIMDs
    (4 x SQ_BUSY_CU_CYCLES): the share of cycles in which a SIMD's matrix core works,
    while the kernel occupies the CU."""
    busy = d["SQ_VALU_MFMA_BUSY_CYCLES"] / (4.0 * d["SQ_BUSY_CU_CYCLES"])
    per = {k: v / d["dispatches"] for k, v in d.items() if k != "dispatches"}
    s = {"class": kclass, "workload": workload, "kernel": kernel,
         "dispatches": d["dispatches"], "mfma_busy": busy, "per_dispatch": per,
         "source_sha256": source_digest(kclass), "command": command}
    if per.get("SQ_INSTS_MFMA"):
        s["valu_per_mfma"] = per.get("SQ_INSTS_VALU", 0.0) / per["SQ_INSTS_MFMA"]
    out = [f"# MFMA busy share of `{kernel}` ({kclass}, {workload} workload)", "",
           "SQ_VALU_MFMA_BUSY_CYCLES / (4 x SQ_BUSY_CU_CYCLES), summed over the class's "
           "dispatches in one rocprofv3 --pmc run: the share of the cycles in which a CU "
           "runs the kernel that its four SIMDs' matrix cores are busy.", "",
           f"- dispatches: {d['dispatches']}",
           f"- MFMA busy: {busy:.3f}"]
    if "valu_per_mfma" in s:
        out.append(f"- VALU instructions per MFMA instruction: {s['valu_per_mfma']:.2f}")
    out += [f"- command: {command}", "", "```json", json.dumps(s, indent=1), "```"]
    return "\n".join(out) + "\n"


def traffic_md(s) -> str:
    out = [f"# HBM traffic of `{s['kernel']}` ({s['class']})", "",
           "FETCH_SIZE and WRITE_SIZE (KiB per dispatch) from two separate rocprofv3 --pmc "
           "runs, scaled by the same counters over a plain device copy of "
           f"{s['copy_bytes'] / 2**20:.0f} MiB (fetch x{s['copy_scale_fetch']:.4f}, "
           f"write x{s['copy_scale_write']:.4f}).", "",
           f"- dispatches: {s['dispatches']}",
           f"- fetch per launch: {s['fetch_bytes_per_launch'] / 2**20:.2f} MiB",
           f"- write per launch: {s['write_bytes_per_launch'] / 2**20:.2f} MiB",
           f"- commands: {s['command']}", "", "```json", json.dumps(s, indent=1), "```"]
    return "\n".join(out) + "\n"


if __name__ == "__main__":
    mode = sys.argv[1]
    if mode == "stats":
        sys.stdout.write(kernel_stats_md(sys.argv[2], sys.argv[3], sys.argv[4]))
    elif mode == "launches":
        sys.stdout.write(launch_stats_md(sys.argv[2], sys.argv[3], sys.argv[4]))
    elif mode == "lib-launches":  # the library's own kernels only (names in dreamer::)
        sys.stdout.write(launch_stats_md(sys.argv[2], sys.argv[3], sys.argv[4], top=64,
                                         only="dreamer"))
    elif mode == "traffic":
        s = traffic_summary(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5], sys.argv[6],
                            sys.argv[7], float(sys.argv[8]), " ".join(sys.argv[9:]))
        sys.stdout.write(traffic_md(s))
    elif mode == "mfma":
        workload, out_dir, pmc_csv = sys.argv[2], sys.argv[3], sys.argv[4]
        kernels = WORKLOAD_KERNELS[workload]
        per = counters_per_class(pmc_csv, kernels)
        for kclass in MFMA_CLASSES:
            if kclass not in per or "SQ_VALU_MFMA_BUSY_CYCLES" not in per[kclass]:
                continue
            path = os.path.join(out_dir, f"{kclass}_{workload}_mfma_busy.md")
            md = mfma_busy_md(kclass, workload, per[kclass], kernels[kclass],
                              " ".join(sys.argv[5:]))
            with open(path, "w") as fh:
                fh.write(md)
            print(kclass, md.splitlines()[5])
    elif mode == "traffic-all":
        workload, out_dir = sys.argv[2], sys.argv[3]
        for kclass, kname in WORKLOAD_KERNELS[workload].items():
            s = traffic_summary(kclass, kname, sys.argv[4], sys.argv[5], sys.argv[6],
                                sys.argv[7], float(sys.argv[8]), " ".join(sys.argv[9:]))
            path = os.path.join(out_dir, f"{kclass}_{workload}_hbm_traffic.md")
            if s is None:  # no dispatches of this class: drop an older summary
                if os.path.exists(path):
                    os.remove(path)
                print(kclass, "not run")
                continue
            with open(path, "w") as fh:
                fh.write(traffic_md(s))
            print(kclass, s["dispatches"], round(s["bytes_per_launch"] / 2**20, 2), "MiB")
    else:
        raise SystemExit(__doc__)
