"""Summaries of rocprofv3 output for the profiles/ folder, and the kernel-source hash
that ties a counter summary to the kernel it was taken on.

    python -m block_sparse_attention_tok_amd.profsum stats  KERNEL_STATS_CSV --title T --command C --out FILE
    python -m block_sparse_attention_tok_amd.profsum traffic --kernel K --fetch CSV --write CSV \
        --copy-fetch CSV --copy-write CSV --copy-bytes N --title T --cmds CMD1 CMD2 CMD3 CMD4 --out FILE

`traffic` scales FETCH_SIZE and WRITE_SIZE (KiB per dispatch) by what the same
counters read for a plain device copy of known size, and records the source hash
of the kernel; bench.py reports the traffic only while that hash still matches.
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import os
import statistics

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

# Sources that determine each profiled kernel's code.
KERNEL_SOURCES = {
    "sol_fused_kernel": ["csrc/fused.hip", "csrc/pipe.h", "csrc/common.h", "csrc/kernels.h"],
    "sol2_fused_kernel": ["csrc/sol2.hip", "csrc/pipe.h", "csrc/common.h", "csrc/kernels.h"],
}


def source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel]:
        with open(os.path.join(HERE, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _per_dispatch(path: str, kernel: str, counter: str):
    tot = collections.defaultdict(float)
    for r in csv.DictReader(open(path)):
        if kernel in r["Kernel_Name"] and r["Counter_Name"] == counter:
            tot[r["Dispatch_Id"]] += float(r["Counter_Value"])
    return list(tot.values())


def traffic_summary(kernel, fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, copy_bytes):
    """Per-launch HBM bytes of `kernel` from FETCH_SIZE / WRITE_SIZE, copy-calibrated."""
    cf = statistics.median(_per_dispatch(copy_fetch_csv, "copyBuffer", "FETCH_SIZE"))
    cw = statistics.median(_per_dispatch(copy_write_csv, "copyBuffer", "WRITE_SIZE"))
    f_factor = copy_bytes / (cf * 1024.0)
    w_factor = copy_bytes / (cw * 1024.0)
    fetch = _per_dispatch(fetch_csv, kernel, "FETCH_SIZE")
    write = _per_dispatch(write_csv, kernel, "WRITE_SIZE")
    fb = statistics.median(fetch) * 1024.0 * f_factor
    wb = statistics.median(write) * 1024.0 * w_factor
    return {"fetch_factor": f_factor, "write_factor": w_factor, "fetch_dispatches": len(fetch),
            "write_dispatches": len(write), "fetch_bytes_per_launch": fb, "write_bytes_per_launch": wb,
            "traffic_bytes_per_launch": fb + wb}


def read_traffic(path: str, kernel: str):
    """Traffic bytes per launch from a summary written by `traffic`, or None if the file
    is missing or the kernel's sources changed since the counters were taken."""
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and line.strip().startswith("- "):
            k, v = line.strip()[2:].split(":", 1)
            vals[k.strip()] = v.strip().strip("`")
    if vals.get("source_hash") != source_hash(kernel):
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _stats_md(csv_path, title, cmd):
    rows = list(csv.DictReader(open(csv_path)))
    out = [f"# {title}", "", "Command (from the repository root on the GPU box; R = repository root):", "",
           f"    {cmd}", "", "| Kernel | Calls | Average (us) | Min (us) | Max (us) | Share |",
           "|---|---:|---:|---:|---:|---:|"]
    for r in rows:
        name = r["Name"].replace("(anonymous namespace)::", "").split("(")[0]
        out.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | {float(r['MinNs']) / 1e3:.1f} | "
                   f"{float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.1f}% |")
    return "\n".join(out) + "\n"


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="action", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--title", required=True)
    s.add_argument("--command", required=True)
    s.add_argument("--out", required=True)
    t = sub.add_parser("traffic")
    for a in ("--kernel", "--fetch", "--write", "--copy-fetch", "--copy-write", "--title", "--out"):
        t.add_argument(a, required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--cmds", nargs=4, required=True, help="the four rocprofv3 commands")
    a = ap.parse_args()
    if a.action == "stats":
        open(a.out, "w").write(_stats_md(a.csv, a.title, a.command))
        return
    r = traffic_summary(a.kernel, a.fetch, a.write, a.copy_fetch, a.copy_write, a.copy_bytes)
    lines = [f"# {a.title}", "", "Commands (from the repository root on the GPU box; R = repository root):", ""]
    lines += [f"    {c}" for c in a.cmds]
    lines += ["", "FETCH_SIZE / WRITE_SIZE are KiB per dispatch; each is scaled by what the same counter reads",
              f"for a plain device copy of {a.copy_bytes} bytes (medians over the dispatches).", "",
              f"- kernel: `{a.kernel}`",
              f"- source_hash: `{source_hash(a.kernel)}`",
              f"- fetch_factor: {r['fetch_factor']:.4f}",
              f"- write_factor: {r['write_factor']:.4f}",
              f"- dispatches: {r['fetch_dispatches']} (fetch run), {r['write_dispatches']} (write run)",
              f"- fetch_bytes_per_launch: {r['fetch_bytes_per_launch']:.6g}",
              f"- write_bytes_per_launch: {r['write_bytes_per_launch']:.6g}",
              f"- traffic_bytes_per_launch: {r['traffic_bytes_per_launch']:.6g}", ""]
    open(a.out, "w").write("\n".join(lines))


if __name__ == "__main__":
    main()
