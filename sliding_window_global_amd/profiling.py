"""Turn rocprofv3 CSV output into the short text summaries kept under profiles/.

Usage (on the CSV files rocprofv3 wrote; see each summary's header for its command):
  python -m sliding_window_global_amd.profiling trace  STATS_CSV OUT --cmd "..."
  python -m sliding_window_global_amd.profiling traffic --kernel NAME --grid N \
      --fetch F.csv --write W.csv --copy-fetch CF.csv --copy-write CW.csv OUT --cmd "..." --cmd "..."
  python -m sliding_window_global_amd.profiling counters --kernel NAME --grid N PMC.csv OUT --cmd "..."

The traffic summary records the SHA-256 of the kernel sources it was measured on, so that
bench.py reports the figure only while those sources are unchanged.
"""

from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import os

PKG = os.path.dirname(os.path.abspath(__file__))
PREFILL_SOURCES = [os.path.join(PKG, "csrc", "prefill_bf16.hip"), os.path.join(PKG, "csrc", "common.h")]
DECODE_SOURCES = [os.path.join(PKG, "csrc", "decode.hip"), os.path.join(PKG, "csrc", "common.h")]
SOURCES = {"prefill": PREFILL_SOURCES, "decode": DECODE_SOURCES,
           "prefill_wide": [os.path.join(PKG, "csrc", "prefill_wide.hip"), os.path.join(PKG, "csrc", "common.h")],
           "decode_wide": [os.path.join(PKG, "csrc", "decode_wide.hip"), os.path.join(PKG, "csrc", "common.h")]}


def sources_sha256(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _per_dispatch(path, kernel, grid, counter, nth=None):
    vals = []
    for r in csv.DictReader(open(path)):
        if kernel in r["Kernel_Name"] and (grid is None or int(r["Grid_Size"]) == grid) \
                and r["Counter_Name"] == counter:
            vals.append(float(r["Counter_Value"]))
    if nth:  # "a:b" keeps matching dispatches a .. b-1 in launch order
        a, b = (int(x) for x in nth.split(":"))
        vals = vals[a:b]
    if not vals:
        raise SystemExit(f"no {counter} rows for {kernel} (grid {grid}) in {path}")
    return sum(vals) / len(vals), len(vals)


def summarize_trace(stats_csv, out, cmds, trace_csv=None, prefix="plamo"):
    """Kernel statistics table; with the per-dispatch trace, also one line per (kernel, grid)
    for the library's kernels (one kernel serves several workloads of different grids)."""
    rows = list(csv.DictReader(open(stats_csv)))
    lines = [f"# rocprofv3 kernel trace summary", ""]
    lines += [f"command: {c}" for c in cmds]
    lines += ["", f"{'kernel':<78} {'calls':>6} {'avg_us':>11} {'min_us':>10} {'max_us':>10} {'pct':>6}"]
    for r in rows:
        lines.append(f"{r['Name'][:78]:<78} {int(r['Calls']):>6} {float(r['AverageNs'])/1e3:>11.2f} "
                     f"{float(r['MinNs'])/1e3:>10.2f} {float(r['MaxNs'])/1e3:>10.2f} {float(r['Percentage']):>6.2f}")
    if trace_csv:
        by = collections.defaultdict(list)
        for r in csv.DictReader(open(trace_csv)):
            name = r["Kernel_Name"]
            if prefix not in name:
                continue
            grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
            by[(name, grid)].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        lines += ["", "per (kernel, grid threads):",
                  f"{'kernel':<66} {'grid':>10} {'calls':>6} {'avg_us':>11} {'min_us':>10} {'max_us':>10}"]
        for (name, grid), v in sorted(by.items(), key=lambda kv: -sum(kv[1])):
            lines.append(f"{name[:66]:<66} {grid:>10} {len(v):>6} {sum(v)/len(v):>11.2f} {min(v):>10.2f} {max(v):>10.2f}")
    open(out, "w").write("\n".join(lines) + "\n")


def summarize_traffic(kernel, grid, fetch, write, copy_fetch, copy_write, out, cmds, copy_bytes=1 << 30,
                      sources=PREFILL_SOURCES, nth=None, algorithmic=None):
    f_kib, nf = _per_dispatch(fetch, kernel, grid, "FETCH_SIZE", nth)
    w_kib, nw = _per_dispatch(write, kernel, grid, "WRITE_SIZE", nth) if write else (0.0, 0)
    cf_kib, _ = _per_dispatch(copy_fetch, "copyBuffer", None, "FETCH_SIZE")
    cw_kib, _ = _per_dispatch(copy_write, "copyBuffer", None, "WRITE_SIZE")
    f_factor = cf_kib * 1024 / copy_bytes
    w_factor = cw_kib * 1024 / copy_bytes
    read_b = f_kib * 1024 / f_factor
    write_b = w_kib * 1024 / w_factor
    lines = ["# HBM traffic per dispatch (rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE, copy-calibrated)", ""]
    lines += [f"command: {c}" for c in cmds]
    lines += ["",
              f"kernel: {kernel}",
              f"grid_threads: {grid}",
              f"fetch_kib_per_dispatch: {f_kib:.1f}  (n={nf})",
              f"write_kib_per_dispatch: {w_kib:.1f}  (n={nw})",
              f"copy_calibration: plain device copy of {copy_bytes} bytes reads FETCH_SIZE {cf_kib:.1f} KiB "
              f"(factor {f_factor:.4f}) and WRITE_SIZE {cw_kib:.1f} KiB (factor {w_factor:.4f})",
              f"hbm_read_bytes_per_launch: {read_b:.0f}",
              f"hbm_write_bytes_per_launch: {write_b:.0f}",
              f"traffic_bytes_per_launch: {read_b + write_b:.0f}",
              *([f"algorithmic_bytes_per_launch: {algorithmic}",
                 f"traffic_over_algorithmic: {(read_b + write_b) / algorithmic:.4f}"] if algorithmic else []),
              f"kernel_source_sha256: {sources_sha256(sources)}"]
    open(out, "w").write("\n".join(lines) + "\n")


def summarize_counters(kernel, grid, pmc_csv, out, cmds):
    agg = collections.defaultdict(list)
    for r in csv.DictReader(open(pmc_csv)):
        if kernel in r["Kernel_Name"] and (grid is None or int(r["Grid_Size"]) == grid):
            agg[r["Counter_Name"]].append(float(r["Counter_Value"]))
    lines = ["# rocprofv3 counters per dispatch (mean over dispatches)", ""]
    lines += [f"command: {c}" for c in cmds]
    lines += ["", f"kernel: {kernel}", f"grid_threads: {grid}", ""]
    for k in sorted(agg):
        v = agg[k]
        lines.append(f"{k:<32} {sum(v)/len(v):.6g}  (n={len(v)})")
    if "SQ_VALU_MFMA_BUSY_CYCLES" in agg and "GRBM_GUI_ACTIVE" in agg:
        busy = sum(agg["SQ_VALU_MFMA_BUSY_CYCLES"]) / len(agg["SQ_VALU_MFMA_BUSY_CYCLES"])
        active = sum(agg["GRBM_GUI_ACTIVE"]) / len(agg["GRBM_GUI_ACTIVE"])
        # GRBM_GUI_ACTIVE is summed over the 8 XCDs; 1024 SIMDs
        lines += ["", f"mfma_busy_fraction: {busy / 1024 / (active / 8):.4f}  "
                      "(SQ_VALU_MFMA_BUSY_CYCLES / 1024 SIMDs / (GRBM_GUI_ACTIVE / 8 XCDs))"]
    open(out, "w").write("\n".join(lines) + "\n")


def read_traffic(path, sources=PREFILL_SOURCES):
    """traffic_bytes_per_launch from a summary, or None if missing or measured on other sources."""
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line:
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip().split()[0] if v.strip() else ""
    if vals.get("kernel_source_sha256") != sources_sha256(sources):
        return None
    try:
        return int(float(vals["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    t = sub.add_parser("trace")
    t.add_argument("stats_csv")
    t.add_argument("out")
    t.add_argument("--trace-csv", default=None)
    t.add_argument("--cmd", action="append", default=[])
    f = sub.add_parser("traffic")
    f.add_argument("--kernel", required=True)
    f.add_argument("--grid", type=int, default=None)
    f.add_argument("--fetch", required=True)
    f.add_argument("--write", default=None)
    f.add_argument("--sources", choices=sorted(SOURCES), default="prefill")
    f.add_argument("--nth", default=None, help="a:b = only matching dispatches a .. b-1")
    f.add_argument("--algorithmic", type=int, default=None)
    f.add_argument("--copy-fetch", required=True)
    f.add_argument("--copy-write", required=True)
    f.add_argument("out")
    f.add_argument("--cmd", action="append", default=[])
    c = sub.add_parser("counters")
    c.add_argument("--kernel", required=True)
    c.add_argument("--grid", type=int, default=None)
    c.add_argument("pmc_csv")
    c.add_argument("out")
    c.add_argument("--cmd", action="append", default=[])
    a = ap.parse_args()
    if a.what == "trace":
        summarize_trace(a.stats_csv, a.out, a.cmd, trace_csv=a.trace_csv)
    elif a.what == "traffic":
        summarize_traffic(a.kernel, a.grid, a.fetch, a.write, a.copy_fetch, a.copy_write, a.out, a.cmd,
                          sources=SOURCES[a.sources], nth=a.nth, algorithmic=a.algorithmic)
    else:
        summarize_counters(a.kernel, a.grid, a.pmc_csv, a.out, a.cmd)


if __name__ == "__main__":
    main()
