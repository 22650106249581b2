"""Summaries of rocprofv3 CSV output for the step kernel (text + traffic JSON).

Usage (after rocprofv3 runs with ``--output-format csv``):

  python -m long_sequence_causal_cp_amd.prof_summary stats KERNEL_STATS_CSV --cmd "..."
  python -m long_sequence_causal_cp_amd.prof_summary traffic --fetch F.csv --write W.csv \
      --copy-fetch CF.csv --copy-write CW.csv --workload s32k_cp8 --cmd-fetch "..." ...

``traffic`` calibrates the two L2-to-HBM byte counters (FETCH_SIZE and
WRITE_SIZE, KiB per dispatch) against a plain device copy of known size: the
factor is known bytes / counted bytes for that copy.  The step kernel's
per-launch HBM traffic is then the mean over its dispatches of
factor_fetch * FETCH_SIZE + factor_write * WRITE_SIZE.  The JSON records the
SHA-256 of the kernel source it was measured on, so that a benchmark can
refuse to report traffic taken on a different kernel.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import statistics
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
# the translation unit of each measured kernel family and the headers it includes
KERNEL_SOURCES = tuple(os.path.join(HERE, "csrc", f)
                       for f in ("cp_attn_kernels.hip", "cp_attn_tile.h", "cp_attn_internal.h", "cp_job_map.h"))
BWD_SOURCES = tuple(os.path.join(HERE, "csrc", f)
                    for f in ("cp_attn_bwd.hip", "cp_attn_tile.h", "cp_attn_internal.h", "cp_job_map.h"))


def sources_for(kernel: str):
    return BWD_SOURCES if kernel.startswith("bwd_") else KERNEL_SOURCES


def kernel_source_sha256(paths=KERNEL_SOURCES) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _rows(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _per_dispatch(path, counter, name_substr):
    vals = []
    for r in _rows(path):
        if r["Counter_Name"] == counter and name_substr in r["Kernel_Name"]:
            vals.append((int(r["Dispatch_Id"]), int(r["Grid_Size"]), float(r["Counter_Value"])))
    return vals


def stats_text(stats_csv: str, cmd: str, top: int = 6) -> str:
    rows = _rows(stats_csv)
    out = [f"command: {cmd}", "", f"{'kernel':70s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} "
           f"{'max_us':>10s} {'pct':>6s}"]
    for r in rows[:top]:
        name = r["Name"]
        name = name if len(name) <= 70 else name[:67] + "..."
        out.append(f"{name:70s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.2f} "
                   f"{float(r['MinNs']) / 1e3:10.2f} {float(r['MaxNs']) / 1e3:10.2f} "
                   f"{float(r['Percentage']):6.2f}")
    return "\n".join(out) + "\n"


def traffic(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, copy_bytes, kernel="step_kernel"):
    cf = [v for _, _, v in _per_dispatch(copy_fetch_csv, "FETCH_SIZE", "copyBuffer")]
    cw = [v for _, _, v in _per_dispatch(copy_write_csv, "WRITE_SIZE", "copyBuffer")]
    if not cf or not cw:
        raise SystemExit("no copy-probe dispatches found")
    f_fetch = copy_bytes / (statistics.fmean(cf) * 1024.0)
    f_write = copy_bytes / (statistics.fmean(cw) * 1024.0)
    kf = _per_dispatch(fetch_csv, "FETCH_SIZE", kernel)
    kw = _per_dispatch(write_csv, "WRITE_SIZE", kernel)
    if not kf or not kw:
        raise SystemExit(f"no {kernel} dispatches found")
    fetch_b = statistics.fmean(v for _, _, v in kf) * 1024.0 * f_fetch
    write_b = statistics.fmean(v for _, _, v in kw) * 1024.0 * f_write
    by_grid = {}
    for _, g, v in kf:
        by_grid.setdefault(g, [[], []])[0].append(v)
    for _, g, v in kw:
        by_grid.setdefault(g, [[], []])[1].append(v)
    grids = {str(g): {"dispatches": len(a), "fetch_bytes": statistics.fmean(a) * 1024.0 * f_fetch,
                      "write_bytes": statistics.fmean(b) * 1024.0 * f_write}
             for g, (a, b) in sorted(by_grid.items()) if a and b}
    return {
        "factor_fetch": f_fetch, "factor_write": f_write,
        "fetch_bytes_per_launch": fetch_b, "write_bytes_per_launch": write_b,
        "bytes_per_launch": fetch_b + write_b, "dispatches": len(kf), "by_grid_size": grids,
    }


SQ_NAMES = ["SQ_WAVES", "SQ_INSTS_MFMA", "SQ_INSTS_VALU", "SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT", "SQ_BUSY_CYCLES",
            "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE"]


def sq_text(pmc_csv: str, cmd: str, kernel: str = "step_kernel", n_xcd: int = 8, n_simd: int = 1024) -> str:
    """Per-dispatch means of the SQ counters and the MFMA-busy fraction.

    GRBM_GUI_ACTIVE is summed over the XCDs, so cycles per XCD = value / n_xcd;
    MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (cycles per XCD * n_simd).
    """
    agg = {}
    for r in _rows(pmc_csv):
        if kernel in r["Kernel_Name"]:
            agg.setdefault(int(r["Grid_Size"]), {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    out = [f"command: {cmd}", f"kernel: every dispatch whose name contains '{kernel}'; mean per dispatch", ""]
    for grid, counters in sorted(agg.items()):
        out.append(f"grid {grid} threads:")
        vals = {n: statistics.fmean(counters[n]) for n in SQ_NAMES if n in counters}
        for n in SQ_NAMES:
            if n in vals:
                out.append(f"  {n:28s} {vals[n]:16.1f}   ({len(counters[n])} dispatches)")
        if "GRBM_GUI_ACTIVE" in vals and "SQ_VALU_MFMA_BUSY_CYCLES" in vals:
            per_xcd = vals["GRBM_GUI_ACTIVE"] / n_xcd
            out.append(f"  derived: cycles per XCD {per_xcd:.0f}; MFMA busy "
                       f"{100 * vals['SQ_VALU_MFMA_BUSY_CYCLES'] / (per_xcd * n_simd):.1f} %")
        if "SQ_WAVES" in vals and vals["SQ_WAVES"] > 0:
            w = vals["SQ_WAVES"]
            out.append(f"  derived: per wave {vals.get('SQ_INSTS_MFMA', 0) / w:.0f} MFMA, "
                       f"{vals.get('SQ_INSTS_VALU', 0) / w:.0f} VALU (incl. MFMA), "
                       f"{vals.get('SQ_INSTS_LDS', 0) / w:.0f} LDS instructions")
        out.append("")
    return "\n".join(out) + "\n"


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="sub", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--cmd", required=True)
    q = sub.add_parser("sq")
    q.add_argument("csv")
    q.add_argument("--cmd", required=True)
    q.add_argument("--kernel", default="step_kernel", help="substring of the kernel name")
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--copy-fetch", required=True)
    t.add_argument("--copy-write", required=True)
    t.add_argument("--copy-bytes", type=int, required=True, help="bytes the copy probe reads (= writes)")
    t.add_argument("--workload", required=True)
    t.add_argument("--commands", required=True, help="the rocprofv3 commands, one string")
    t.add_argument("--json-out", required=True)
    t.add_argument("--kernel", default="step_kernel", help="substring of the kernel name")
    a = ap.parse_args(argv)
    if a.sub == "stats":
        sys.stdout.write(stats_text(a.csv, a.cmd))
        return
    if a.sub == "sq":
        sys.stdout.write(sq_text(a.csv, a.cmd, kernel=a.kernel))
        return
    res = traffic(a.fetch, a.write, a.copy_fetch, a.copy_write, a.copy_bytes, kernel=a.kernel)
    res.update({"workload": a.workload, "kernel": a.kernel, "kernel_source_sha256": kernel_source_sha256(sources_for(a.kernel)),
                "commands": a.commands})
    with open(a.json_out, "w") as f:
        json.dump(res, f, indent=1)
    print(json.dumps(res, indent=1))


if __name__ == "__main__":
    main()
