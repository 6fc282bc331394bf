"""Short markdown summaries of rocprofv3 CSV output (for the profiles/ folder).

    python -m routing_grouped_gemm_router_amd.rocprof_summary stats DIR TITLE CMD > out.md
    python -m routing_grouped_gemm_router_amd.rocprof_summary pmc FETCH_DIR WRITE_DIR \
        KERNEL COPY_BYTES TITLE CMD_FETCH CMD_WRITE > out.md

`stats` tabulates DIR/run_kernel_stats.csv (from --kernel-trace --stats
--output-format csv). `pmc` reads two --pmc runs (FETCH_SIZE, then
WRITE_SIZE; counter values in KiB per dispatch), averages them over the
dispatches whose name contains KERNEL, and scales each by what the same
counter reads for the largest device copy of COPY_BYTES bytes in the same
run. The result carries the hash of the GEMM sources it was measured on, so
a reader can tell whether it still describes the current kernel.

Only reads the CSV files; runs nothing.
"""
from __future__ import annotations

import csv
import hashlib
import os
import sys
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))
# the sources that make up the grouped GEMM kernel
GEMM_SOURCES = ("csrc/gemm.hip", "csrc/common.h", "../include/moe.h")


def gemm_source_hash() -> str:
    h = hashlib.sha256()
    for rel in GEMM_SOURCES:
        with open(os.path.join(PKG, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _short(name: str, n: int = 96) -> str:
    name = name.replace("|", "/")
    return name if len(name) <= n else name[:n] + "..."


def stats(d: str, title: str, cmd: str, top: int = 24) -> str:
    rows = list(csv.DictReader(open(os.path.join(d, "run_kernel_stats.csv"))))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    out = [f"# {title}", "", "Command (one MI355X):", "", "```", cmd, "```", "",
           "| kernel | calls | avg us | min us | max us | total us | % |",
           "|---|---|---|---|---|---|---|"]
    for r in rows[:top]:
        out.append(f"| `{_short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                   f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                   f"{float(r['TotalDurationNs']) / 1e3:.1f} | {float(r['Percentage']):.1f} |")
    return "\n".join(out) + "\n"


def _per_dispatch(d: str, counter: str):
    vals = defaultdict(float)
    names = {}
    for r in csv.DictReader(open(os.path.join(d, "run_counter_collection.csv"))):
        if r["Counter_Name"] != counter:
            continue
        i = int(r["Dispatch_Id"])
        vals[i] += float(r["Counter_Value"])       # summed over the agent's instances
        names[i] = r["Kernel_Name"]
    return vals, names


def pmc(fetch_dir: str, write_dir: str, kernel: str, copy_bytes: int, title: str,
        cmd_fetch: str, cmd_write: str) -> str:
    res = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        vals, names = _per_dispatch(d, counter)
        kv = [vals[i] * 1024 for i in vals if kernel in names[i]]
        copies = [vals[i] * 1024 for i in vals if "copyBuffer" in names[i]]
        if not kv or not copies:
            raise SystemExit(f"{counter}: no '{kernel}' or copy dispatch in {d}")
        copy_read = max(copies)
        res[counter] = (sum(kv) / len(kv), len(kv), copy_read, copy_bytes / copy_read)
    fetch, nf, cf, kf = res["FETCH_SIZE"]
    write, nw, cw, kw = res["WRITE_SIZE"]
    traffic = fetch * kf + write * kw
    out = [f"# {title}", "",
           "HBM bytes per launch of the kernel from two counter runs, each scaled by",
           "what the same counter reads for a device copy of known size in that run.", "",
           "Commands (one MI355X):", "", "```", cmd_fetch, cmd_write, "```", "",
           "| counter | kernel dispatches | raw bytes / launch | copy of "
           f"{copy_bytes / 2**20:.0f} MiB reads | scale | bytes / launch |",
           "|---|---|---|---|---|---|",
           f"| FETCH_SIZE | {nf} | {fetch:.4g} | {cf:.4g} | {kf:.3f} | {fetch * kf:.4g} |",
           f"| WRITE_SIZE | {nw} | {write:.4g} | {cw:.4g} | {kw:.3f} | {write * kw:.4g} |", "",
           f"traffic_bytes_per_launch = {traffic:.6g}",
           f"gemm_source_hash = {gemm_source_hash()}", ""]
    return "\n".join(out)


def read_traffic(md_path: str):
    """(bytes per launch, source hash) from a pmc summary, or None."""
    if not os.path.exists(md_path):
        return None
    t = hs = None
    for line in open(md_path):
        if line.startswith("traffic_bytes_per_launch ="):
            t = float(line.split("=")[1])
        elif line.startswith("gemm_source_hash ="):
            hs = line.split("=")[1].strip()
    return (t, hs) if t is not None and hs else None


if __name__ == "__main__":
    if sys.argv[1] == "stats":
        sys.stdout.write(stats(sys.argv[2], sys.argv[3], sys.argv[4]))
    elif sys.argv[1] == "pmc":
        sys.stdout.write(pmc(sys.argv[2], sys.argv[3], sys.argv[4], int(sys.argv[5]), sys.argv[6],
                             sys.argv[7], sys.argv[8]))
    else:
        raise SystemExit(__doc__)
