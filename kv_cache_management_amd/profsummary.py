"""Summaries of rocprofv3 CSV output for the R-SWA kernels.

    python -m kv_cache_management_amd.profsummary trace DIR --kernel decode_split --last N \
        --command "<the rocprofv3 command>" [--out FILE]
    python -m kv_cache_management_amd.profsummary pmc --fetch DIR --write DIR \
        --copy-fetch DIR --copy-write DIR --kernel decode_split --last N \
        --algorithmic-bytes B --command "..." [--out FILE]

`counters` sums the counters of `--pmc` runs over a kernel's last dispatches.
`trace` reads a `--kernel-trace --stats --output-format csv` directory and
reports rocprofv3's own per-kernel statistics plus the mean duration of the
last N dispatches of one kernel (the measured steps of a benchmark run come
last, or use --measured-grid).  `pmc` reads `--pmc FETCH_SIZE` and `--pmc WRITE_SIZE` runs of the
benchmark and of a plain 1 GiB device copy, scales each counter by what it
reads for the copy of known size, and reports HBM bytes per dispatch.
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import statistics
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
COPY_BYTES = 1 << 30


def _one(pattern: str) -> str:
    hits = sorted(glob.glob(pattern, recursive=True))
    if not hits:
        raise SystemExit(f"no file matches {pattern}")
    return hits[0]


def kernel_source_sha(kernel: str) -> str:
    src = {"decode_split": "rswa_decode.hip", "prefill_mfma": "rswa_prefill_mfma.hip"}[kernel]
    data = open(os.path.join(PKG, "csrc", src), "rb").read()
    return hashlib.sha256(data).hexdigest()[:16]


def trace_summary(d: str, kernel: str, last: int, command: str, max_grid: bool = False) -> str:
    stats = list(csv.DictReader(open(_one(os.path.join(d, "**", "*kernel_stats.csv")))))
    trace = list(csv.DictReader(open(_one(os.path.join(d, "**", "*kernel_trace.csv")))))
    lines = [f"# rocprofv3 kernel trace: {kernel} ({os.path.basename(d.rstrip('/'))})", "",
             "Command:", "", "```", command, "```", "",
             "rocprofv3 --stats (all dispatches):", "",
             "| kernel | calls | avg us | min us | max us | % time |", "|---|---|---|---|---|---|"]
    for r in stats[:12]:
        name = r["Name"]
        short = name if len(name) < 70 else name[:67] + "..."
        lines.append(f"| `{short}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{float(r['Percentage']):.2f} |")
    sel = [r for r in trace if kernel in r.get("Kernel_Name", "")]
    sel.sort(key=lambda r: int(r["Start_Timestamp"]))
    what = "all dispatches"
    if max_grid:
        # The measured decode steps all run the full batch with one plan, so
        # their grid is the most frequent one.
        gsz = lambda r: int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
        counts = {}
        for r in sel:
            counts[gsz(r)] = counts.get(gsz(r), 0) + 1
        gmode = max(counts, key=counts.get)
        sel = [r for r in sel if gsz(r) == gmode]
        what = f"dispatches with the full-batch grid ({gmode} work-items)"
    durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in sel]
    tail = durs[-last:] if last else durs
    if last:
        what += f", last {len(tail)}"
    lines += ["", f"`{kernel}`, {what}: {len(tail)} dispatches, "
              f"mean {statistics.mean(tail):.2f} us, median {statistics.median(tail):.2f} us, "
              f"min {min(tail):.2f} us, max {max(tail):.2f} us.", ""]
    return "\n".join(lines)


def _pmc_rows(d: str, counter: str, kernel: str):
    rows = list(csv.DictReader(open(_one(os.path.join(d, "**", "*counter_collection.csv")))))
    out = []
    for r in rows:
        if r.get("Counter_Name") != counter:
            continue
        if kernel and kernel not in r.get("Kernel_Name", ""):
            continue
        out.append((int(r.get("Dispatch_Id", 0)), float(r["Counter_Value"]), r.get("Kernel_Name", "")))
    out.sort()
    return out


def pmc_summary(fetch: str, write: str, copy_fetch: str, copy_write: str, kernel: str, last: int,
                algorithmic: float, command: str, launches_note: str = "") -> str:
    cf = _pmc_rows(copy_fetch, "FETCH_SIZE", "")
    cw = _pmc_rows(copy_write, "WRITE_SIZE", "")
    # the copy kernel: the dispatches that moved about 1 GiB
    cf_big = [v for _, v, _ in cf if v > 0.25 * COPY_BYTES / 1024]
    cw_big = [v for _, v, _ in cw if v > 0.25 * COPY_BYTES / 1024]
    f_scale = COPY_BYTES / (statistics.mean(cf_big) * 1024)
    w_scale = COPY_BYTES / (statistics.mean(cw_big) * 1024)
    f = [v for _, v, _ in _pmc_rows(fetch, "FETCH_SIZE", kernel)]
    w = [v for _, v, _ in _pmc_rows(write, "WRITE_SIZE", kernel)]
    f_tail = f[-last:] if last else f
    w_tail = w[-last:] if last else w
    fetch_b = statistics.mean(f_tail) * 1024 * f_scale
    write_b = statistics.mean(w_tail) * 1024 * w_scale
    rec = {"kernel": kernel, "kernel_source_sha256_16": kernel_source_sha(kernel),
           "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
           "hbm_fetch_bytes_per_launch": int(fetch_b), "hbm_write_bytes_per_launch": int(write_b),
           "hbm_bytes_per_launch": int(fetch_b + write_b),
           "algorithmic_bytes_per_launch": int(algorithmic), "launches_averaged": len(f_tail),
           "launches_note": launches_note or f"last {len(f_tail)} dispatches of the profiled run"}
    lines = [f"# rocprofv3 PMC: HBM traffic of {kernel}", "", "Commands:", "", "```", command, "```", "",
             f"Copy calibration (1 GiB read + 1 GiB written by one copy kernel): FETCH_SIZE reads "
             f"{1 / f_scale:.3f}x and WRITE_SIZE {1 / w_scale:.3f}x the true bytes, so they are scaled by "
             f"{f_scale:.3f} and {w_scale:.3f}.", "",
             f"`{kernel}`, mean over the last {len(f_tail)} dispatches (the measured steps):", "",
             "| quantity | bytes per launch |", "|---|---|",
             f"| HBM fetch (scaled FETCH_SIZE) | {fetch_b:,.0f} |",
             f"| HBM write (scaled WRITE_SIZE) | {write_b:,.0f} |",
             f"| algorithmic K+V read | {algorithmic:,.0f} |",
             f"| fetch / algorithmic | {fetch_b / algorithmic:.4f} |", "",
             f"<!-- traffic {json.dumps(rec)} -->", ""]
    return "\n".join(lines)


def counters_summary(dirs, kernel: str, last: int, command: str) -> str:
    """Sums of every counter over the last `last` dispatches of `kernel` in
    each --pmc run directory, plus the ratios used to read them."""
    vals = {}
    for d in dirs:
        rows = list(csv.DictReader(open(_one(os.path.join(d, "**", "*counter_collection.csv")))))
        rows = [r for r in rows if kernel in r.get("Kernel_Name", "")]
        ids = sorted({int(r["Dispatch_Id"]) for r in rows})
        keep = set(ids[-last:] if last else ids)
        for r in rows:
            if int(r["Dispatch_Id"]) in keep:
                vals[r["Counter_Name"]] = vals.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    lines = [command, f"({kernel}: sums over the last {last or 'all'} dispatch(es) of each run)", ""]
    lines += [f"{k} {int(v)}" for k, v in sorted(vals.items())]
    wave = vals.get("SQ_WAVE_CYCLES")
    if wave:
        for k in ("SQ_WAIT_INST_ANY", "SQ_WAIT_ANY", "SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_VALU",
                  "SQ_ACTIVE_INST_LDS", "SQ_WAIT_INST_LDS"):
            if k in vals:
                lines.append(f"{k} / SQ_WAVE_CYCLES = {vals[k] / wave:.3f}")
    if "SQ_INSTS_MFMA" in vals and "SQ_INSTS_VALU" in vals:
        lines.append(f"(SQ_INSTS_VALU - SQ_INSTS_MFMA) / SQ_INSTS_MFMA = "
                     f"{(vals['SQ_INSTS_VALU'] - vals['SQ_INSTS_MFMA']) / vals['SQ_INSTS_MFMA']:.2f}")
    return "\n".join(lines) + "\n"


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("dir")
    t.add_argument("--kernel", required=True)
    t.add_argument("--last", type=int, default=0)
    t.add_argument("--command", required=True)
    t.add_argument("--measured-grid", dest="max_grid", action="store_true",
                   help="only dispatches with the kernel's most frequent grid (the "
                        "full-batch measured steps)")
    t.add_argument("--out")
    p = sub.add_parser("pmc")
    for k in ("fetch", "write", "copy-fetch", "copy-write"):
        p.add_argument(f"--{k}", required=True)
    p.add_argument("--kernel", required=True)
    p.add_argument("--last", type=int, default=0)
    p.add_argument("--algorithmic-bytes", type=float, required=True)
    p.add_argument("--command", required=True)
    p.add_argument("--launches-note", default="",
                   help="which launches were averaged (recorded beside the traffic)")
    p.add_argument("--out")
    c = sub.add_parser("counters")
    c.add_argument("dirs", nargs="+")
    c.add_argument("--kernel", required=True)
    c.add_argument("--last", type=int, default=1)
    c.add_argument("--command", required=True)
    c.add_argument("--out")
    a = ap.parse_args(argv)
    if a.cmd == "trace":
        text = trace_summary(a.dir, a.kernel, a.last, a.command, a.max_grid)
    elif a.cmd == "counters":
        text = counters_summary(a.dirs, a.kernel, a.last, a.command)
    else:
        text = pmc_summary(a.fetch, a.write, a.copy_fetch, a.copy_write, a.kernel, a.last,
                           a.algorithmic_bytes, a.command, a.launches_note)
    if a.out:
        open(a.out, "w").write(text)
    else:
        sys.stdout.write(text)


if __name__ == "__main__":
    main()
