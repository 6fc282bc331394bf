"""Short markdown summaries of rocprofv3 CSV output (for the profiles/ folder).

    python -m routing_grouped_gemm_router_amd.rocprof_summary stats DIR TITLE CMD > out.md
    python -m routing_grouped_gemm_router_amd.rocprof_summary pmc FETCH_DIR WRITE_DIR \
        KERNEL[#n/p] COPY_BYTES TITLE CMD_FETCH CMD_WRITE > out.md
    python -m routing_grouped_gemm_router_amd.rocprof_summary api DIR_A DIR_B STEPS_A STEPS_B \
        TITLE CMD_A CMD_B > out.md
    python -m routing_grouped_gemm_router_amd.rocprof_summary sq DIR TITLE CMD [NAMES] > out.md
    python -m routing_grouped_gemm_router_amd.rocprof_summary counters FETCH_DIR WRITE_DIR \
        LABEL=KERNEL[#n/p];... COPY_BYTES TITLE CMD_FETCH CMD_WRITE > out.md

`stats` tabulates DIR/run_kernel_stats.csv (from --kernel-trace --stats
--output-format csv). `pmc` reads two --pmc runs (FETCH_SIZE, then
WRITE_SIZE; counter values in KiB per dispatch), averages them over the
dispatches whose name contains KERNEL (with #n/p: the n-th of every p such
dispatches), and scales each by what the same
counter reads for the largest device copy of COPY_BYTES bytes in the same
run. The result carries the hash of the GEMM sources it was measured on, so
a reader can tell whether it still describes the current kernel. `api`
compares the HIP API call counts of two runs that differ only in their
number of timed steps (what one step issues); `sq` tabulates SQ counters
per kernel; `counters` tabulates the scaled FETCH_SIZE / WRITE_SIZE of several
kernels of one step (the row movers and quantisers) and carries the hash of
their sources.

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
GEMM_SOURCES = ("csrc/gemm.hip", "csrc/copy_plan.h", "csrc/common.h", "csrc/mx_encode.h",
                "../include/moe.h")
# the sources of the row movers, the routing kernels and the MXFP8 quantisers
ROW_SOURCES = ("csrc/rows.hip", "csrc/route.hip", "csrc/mxfp8.hip", "csrc/common.h",
               "csrc/mx_encode.h", "../include/moe.h")


def source_hash(sources) -> str:
    h = hashlib.sha256()
    for rel in sources:
        with open(os.path.join(PKG, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def gemm_source_hash() -> str:
    return source_hash(GEMM_SOURCES)


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


def _select(kernel: str):
    """KERNEL[#n/p]: dispatches whose name contains KERNEL; with #n/p only
    the n-th of every p of them in dispatch order (e.g. the second of the two
    weight-gradient launches of each step, which share one kernel name)."""
    if "#" in kernel:
        name, sel = kernel.rsplit("#", 1)
        n, p = (int(v) for v in sel.split("/"))
        return name, n, p
    return kernel, 0, 1


def pmc(fetch_dir: str, write_dir: str, kernel: str, copy_bytes: int, title: str,
        cmd_fetch: str, cmd_write: str) -> str:
    res = {}
    kname, nth, period = _select(kernel)
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        vals, names = _per_dispatch(d, counter)
        ids = sorted(i for i in vals if kname in names[i])
        kv = [vals[i] * 1024 for j, i in enumerate(ids) if j % period == nth]
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


def _scaled(d: str, counter: str, copy_bytes: int):
    """Per-dispatch bytes of one counter run, scaled by the copy calibration."""
    vals, names = _per_dispatch(d, counter)
    copies = [vals[i] * 1024 for i in vals if "copyBuffer" in names[i]]
    if not copies:
        raise SystemExit(f"{counter}: no copy dispatch in {d}")
    scale = copy_bytes / max(copies)
    return {i: v * 1024 * scale for i, v in vals.items()}, names, scale


def counters(fetch_dir: str, write_dir: str, specs, copy_bytes: int, title: str, cmd_fetch: str,
             cmd_write: str) -> str:
    """Scaled read and written bytes per launch of several kernels; specs are
    LABEL=KERNEL[#n/p] strings (see _select)."""
    rd, rnames, rs = _scaled(fetch_dir, "FETCH_SIZE", copy_bytes)
    wr, wnames, ws = _scaled(write_dir, "WRITE_SIZE", copy_bytes)
    out = [f"# {title}", "",
           "HBM bytes per launch from two counter runs (FETCH_SIZE, then WRITE_SIZE),",
           f"each scaled by what the counter reads for a {copy_bytes / 2**20:.0f} MiB device copy in",
           f"that run (reads x{rs:.3f}, writes x{ws:.3f}).", "",
           "Commands (one MI355X):", "", "```", cmd_fetch, cmd_write, "```", "",
           "| role | kernel | launches | read bytes / launch | written bytes / launch |",
           "|---|---|---|---|---|"]
    for spec in specs:
        label, kernel = spec.split("=", 1)
        kname, nth, period = _select(kernel)
        per = []
        for vals, names in ((rd, rnames), (wr, wnames)):
            ids = sorted(i for i in vals if kname in names[i])
            kv = [vals[i] for j, i in enumerate(ids) if j % period == nth]
            if not kv:
                raise SystemExit(f"no '{kernel}' dispatch")
            per.append((sum(kv) / len(kv), len(kv)))
        out.append(f"| {label} | `{_short(kname, 60)}` | {per[0][1]} | {per[0][0]:.4g} | {per[1][0]:.4g} |")
    out += ["", f"row_source_hash = {source_hash(ROW_SOURCES)}", ""]
    return "\n".join(out)


def api_diff(d_small: str, d_large: str, n_small: int, n_large: int, title: str, cmd_small: str,
             cmd_large: str) -> str:
    """HIP API calls of two runs that differ only in their number of timed
    steps: the difference per extra step is what one step issues."""
    def calls(d):
        return {r["Name"]: int(r["Calls"])
                for r in csv.DictReader(open(os.path.join(d, "run_hip_api_stats.csv")))}
    a, b = calls(d_small), calls(d_large)
    extra = n_large - n_small
    out = [f"# {title}", "", "Commands (one MI355X):", "", "```", cmd_small, cmd_large, "```", "",
           f"| HIP API call | {n_small} steps | {n_large} steps | per extra step |",
           "|---|---|---|---|"]
    for n in sorted(set(a) | set(b)):
        out.append(f"| `{n}` | {a.get(n, 0)} | {b.get(n, 0)} | {(b.get(n, 0) - a.get(n, 0)) / extra:g} |")
    return "\n".join(out) + "\n"


def sq(d: str, title: str, cmd: str, select=None) -> str:
    """SQ counters averaged per kernel name (all dispatches of each name)."""
    vals = defaultdict(lambda: defaultdict(float))
    names = {}
    for r in csv.DictReader(open(os.path.join(d, "run_counter_collection.csv"))):
        i = int(r["Dispatch_Id"])
        vals[i][r["Counter_Name"]] += float(r["Counter_Value"])
        names[i] = r["Kernel_Name"]
    groups = defaultdict(list)
    for i in sorted(vals):
        if select and not any(s in names[i] for s in select):
            continue
        groups[_short(names[i].split("(")[0], 60)].append(vals[i])
    cols = sorted({c for g in groups.values() for x in g for c in x})
    out = [f"# {title}", "", "Command (one MI355X):", "", "```", cmd, "```", "",
           "Per launch (summed over the GPU's counter instances, averaged over the launches).", "",
           "| kernel | launches | " + " | ".join(c.replace("SQ_", "") for c in cols) + " |",
           "|---|---|" + "---|" * len(cols)]
    for k, lst in groups.items():
        out.append(f"| `{k}` | {len(lst)} | " +
                   " | ".join(f"{sum(x.get(c, 0) for x in lst) / len(lst):.4g}" for c in cols) + " |")
    out += ["", f"gemm_source_hash = {gemm_source_hash()}"]
    return "\n".join(out) + "\n"


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
    elif sys.argv[1] == "api":
        sys.stdout.write(api_diff(sys.argv[2], sys.argv[3], int(sys.argv[4]), int(sys.argv[5]),
                                  sys.argv[6], sys.argv[7], sys.argv[8]))
    elif sys.argv[1] == "sq":
        sys.stdout.write(sq(sys.argv[2], sys.argv[3], sys.argv[4],
                            sys.argv[5].split(",") if len(sys.argv) > 5 else None))
    elif sys.argv[1] == "counters":
        sys.stdout.write(counters(sys.argv[2], sys.argv[3], sys.argv[4].split(";"), int(sys.argv[5]),
                                  sys.argv[6], sys.argv[7], sys.argv[8]))
    elif sys.argv[1] == "pmc":
        sys.stdout.write(pmc(sys.argv[2], sys.argv[3], sys.argv[4], int(sys.argv[5]), sys.argv[6],
                             sys.argv[7], sys.argv[8]))
    else:
        raise SystemExit(__doc__)
