"""Summaries of rocprofv3 output for the profiles folder.

  python -m ssd_chunked_scan_03_amd.profsum trace DIR --command "..."
      per-kernel dispatch counts and durations from a `--kernel-trace --stats` run
      (the rocpd SQLite database under DIR), as a markdown table.

  python -m ssd_chunked_scan_03_amd.profsum traffic --fetch DIR --write DIR --kernel NAME
          --workload NAME --copy-bytes N --command-fetch "..." --command-write "..."
      HBM bytes per launch of one kernel from a `--pmc FETCH_SIZE` run and a
      `--pmc WRITE_SIZE` run.  Both counters are scaled by what they read for a plain
      streaming elementwise kernel that reads and writes N bytes in the same run, so
      the result is in bytes the kernel moved, not in counter units.  Writes
      traffic_<kernel>_<workload>.json (read by bench.py) and prints a markdown summary.

  python -m ssd_chunked_scan_03_amd.profsum counters DIR [--kernel REGEX]
      mean value per (kernel, counter) of any `--pmc` run, as a markdown table.

  python -m ssd_chunked_scan_03_amd.profsum mfma DIR --trace DIR --command "..."
      matrix-core use per kernel from a `--pmc SQ_INSTS_VALU_MFMA_MOPS_BF16
      SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE` run: counted flops (MOPS x 512), busy
      cycles as a share of GRBM_GUI_ACTIVE x 256 CUs x 4 SIMDs, and counted TFLOP/s over
      the kernel's average duration in the trace run.
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import re
import sqlite3
import statistics
import sys

from .metrics import kernel_source_hash

CALIBRATION_KERNEL = "neg_kernel"  # torch's elementwise negate: reads N, writes N bytes


def short_name(name: str) -> str:
    """k_out<bf16, 64, 128, false> style name from a mangled or demangled symbol."""
    m = re.search(r"ssd\d*(k_[a-z_]+)", name) or re.search(r"ssd::(k_[a-z_]+)", name)
    if m:
        return m.group(1)
    if "neg_kernel" in name or "neg" in name and "elementwise" in name:
        return CALIBRATION_KERNEL
    return name[:60]


def _db(path):
    dbs = sorted(glob.glob(os.path.join(path, "**", "*.db"), recursive=True))
    if not dbs:
        raise SystemExit(f"no rocpd database under {path}")
    return dbs[0]


def trace_rows(path):
    con = sqlite3.connect(_db(path))
    rows = []
    for name, calls, total, avg, pct in con.execute(
            "select name, total_calls, total_duration, average, percentage from top_kernels"):
        rows.append((short_name(name), name, int(calls), float(total), float(avg), float(pct)))
    res = {}
    for name, grid, lds, vgpr, agpr, sgpr, scratch in con.execute(
            "select name, grid_x, lds_size, vgpr_count, accum_vgpr_count, sgpr_count, scratch_size from kernels"):
        res.setdefault(name, (grid, lds, vgpr, agpr, sgpr, scratch))
    return rows, res


def dispatch_medians(path):
    """Median duration (us) of each kernel's dispatches, from the per-dispatch rows of the
    trace database's kernels view (duration column, else end - start, in ns); {} if the
    view has neither."""
    con = sqlite3.connect(_db(path))
    cols = [r[1] for r in con.execute("pragma table_info(kernels)")]
    if "duration" in cols:
        q = "select name, duration from kernels"
    elif "start" in cols and "end" in cols:
        q = 'select name, "end" - "start" from kernels'
    else:
        return {}
    per = {}
    for name, d in con.execute(q):
        if d is not None:
            per.setdefault(name, []).append(float(d))
    return {name: statistics.median(v) / 1e3 for name, v in per.items()}


def cmd_trace(args):
    rows, res = trace_rows(args.dir)
    print(f"Command (from the repository root on one MI355X):\n\n    {args.command}\n")
    print(f"Kernel sources hash: `{kernel_source_hash()}`\n")
    med = dispatch_medians(args.dir)
    print("| kernel | calls | avg us | median us | total us | share | grid x | LDS B | VGPR | AGPR | SGPR | scratch B |")
    print("|---|---|---|---|---|---|---|---|---|---|---|---|")
    for short, full, calls, total, avg, pct in rows:
        g = res.get(full, ("", "", "", "", "", ""))
        m = f"{med[full]:.2f}" if full in med else "—"
        print(f"| {short} | {calls} | {avg:.2f} | {m} | {total:.1f} | {pct:.1f}% | {g[0]} | {g[1]} | {g[2]} | {g[3]} | "
              f"{g[4]} | {g[5]} |")


def pmc_rows(path):
    files = sorted(glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True))
    if not files:
        raise SystemExit(f"no counter_collection.csv under {path}")
    out = []
    with open(files[0]) as f:
        for r in csv.DictReader(f):
            out.append((r["Kernel_Name"], int(r.get("Dispatch_Id", 0) or 0), r["Counter_Name"],
                        float(r["Counter_Value"])))
    return out


def per_dispatch(path, counter, pick):
    """counter value per dispatch (summed over instances) of the kernels `pick` accepts."""
    acc = {}
    for name, disp, cname, val in pmc_rows(path):
        if cname == counter and pick(name):
            acc[disp] = acc.get(disp, 0.0) + val
    return list(acc.values())


def cmd_traffic(args):
    is_k = lambda n: short_name(n) == args.kernel
    is_cal = lambda n: short_name(n) == CALIBRATION_KERNEL
    res = {}
    for counter, path in (("FETCH_SIZE", args.fetch), ("WRITE_SIZE", args.write)):
        k = per_dispatch(path, counter, is_k)
        c = per_dispatch(path, counter, is_cal)
        if not k or not c:
            raise SystemExit(f"{counter}: {len(k)} dispatches of {args.kernel}, {len(c)} of the calibration kernel")
        kk, cc = statistics.median(k), statistics.median(c)
        factor = args.copy_bytes / (cc * 1024.0)
        res[counter] = {"kernel_kib": kk, "calibration_kib": cc, "factor": factor,
                        "bytes": kk * 1024.0 * factor, "dispatches": len(k)}
    total = res["FETCH_SIZE"]["bytes"] + res["WRITE_SIZE"]["bytes"]
    doc = {"kernel": args.kernel, "workload": args.workload, "kernel_source_hash": kernel_source_hash(),
           "hbm_bytes_per_launch": round(total), "read_bytes": round(res["FETCH_SIZE"]["bytes"]),
           "write_bytes": round(res["WRITE_SIZE"]["bytes"]), "calibration_bytes": args.copy_bytes,
           "counters": res, "command_fetch": args.command_fetch, "command_write": args.command_write}
    out = args.out or os.path.join("profiles", f"traffic_{args.kernel}_{args.workload}.json")
    with open(out, "w") as f:
        json.dump(doc, f, indent=1)
        f.write("\n")
    print(f"HBM traffic of {args.kernel} on {args.workload} (median over dispatches)\n")
    print(f"    {args.command_fetch}\n    {args.command_write}\n")
    print("| counter | kernel KiB | calibration KiB (for %d B) | scale | bytes per launch |" % args.copy_bytes)
    print("|---|---|---|---|---|")
    for c, r in res.items():
        print(f"| {c} | {r['kernel_kib']:.0f} | {r['calibration_kib']:.0f} | {r['factor']:.4f} | {r['bytes']:.4g} |")
    print(f"\nTotal: {total:.4g} bytes per launch; kernel sources hash `{doc['kernel_source_hash']}`.")


def cmd_counters(args):
    agg = {}
    for name, disp, cname, val in pmc_rows(args.dir):
        if args.kernel and not re.search(args.kernel, name):
            continue
        key = (short_name(name), cname)
        agg.setdefault(key, {}).setdefault(disp, 0.0)
        agg[key][disp] += val
    print("| kernel | counter | dispatches | mean per dispatch |")
    print("|---|---|---|---|")
    for (k, c), d in sorted(agg.items()):
        print(f"| {k} | {c} | {len(d)} | {statistics.mean(d.values()):.6g} |")


CUS, SIMDS = 256, 4
BF16_PEAK_TFLOPS = 2500.0


def cmd_mfma(args):
    agg = {}
    for name, disp, cname, val in pmc_rows(args.dir):
        agg.setdefault(short_name(name), {}).setdefault(cname, {}).setdefault(disp, 0.0)
        agg[short_name(name)][cname][disp] += val
    durs = {}
    if args.trace:
        rows, _ = trace_rows(args.trace)
        for short, _full, calls, total, avg, pct in rows:
            durs.setdefault(short, []).append((calls, avg))
    print(f"Command (from the repository root on one MI355X):\n\n    {args.command}\n")
    print(f"Kernel sources hash: `{kernel_source_hash()}`\n")
    print("Counted flops are the bf16 matrix-core operations the kernel issued (MOPS x 512).  The busy column is "
          "SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE x 256 CUs x 4 SIMDs) x 8: GRBM_GUI_ACTIVE reads as the sum "
          "over the 8 XCDs, and with that factor the busy share agrees with the flop-based share.\n")
    print("| kernel | dispatches | counted GFLOP (MOPS x 512) | MFMA busy share | "
          "avg us (trace) | counted TFLOP/s | % of bf16 peak |")
    print("|---|---|---|---|---|---|---|")
    for k, cs in sorted(agg.items()):
        mops = cs.get("SQ_INSTS_VALU_MFMA_MOPS_BF16")
        busy = cs.get("SQ_VALU_MFMA_BUSY_CYCLES")
        act = cs.get("GRBM_GUI_ACTIVE")
        if not mops or not busy or not act or statistics.median(mops.values()) == 0:
            continue
        gf = statistics.median(mops.values()) * 512 / 1e9
        util = 8 * statistics.median(busy.values()) / (statistics.median(act.values()) * CUS * SIMDS)
        avg = None
        if k in durs:
            calls, avg = max(durs[k])  # the most-called instance of that kernel name
        tf = gf / (avg * 1e-6) / 1e3 if avg else None
        print(f"| {k} | {len(mops)} | {gf:.2f} | {100 * util:.1f}% | {avg if avg else float('nan'):.1f} | "
              f"{tf if tf else float('nan'):.1f} | {100 * tf / BF16_PEAK_TFLOPS if tf else float('nan'):.1f}% |")


def main(argv=None):
    ap = argparse.ArgumentParser(prog="profsum")
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("dir")
    t.add_argument("--command", required=True)
    w = sub.add_parser("traffic")
    w.add_argument("--fetch", required=True)
    w.add_argument("--write", required=True)
    w.add_argument("--kernel", required=True)
    w.add_argument("--workload", required=True)
    w.add_argument("--copy-bytes", type=int, required=True)
    w.add_argument("--command-fetch", required=True)
    w.add_argument("--command-write", required=True)
    w.add_argument("--out", default=None)
    c = sub.add_parser("counters")
    c.add_argument("dir")
    c.add_argument("--kernel", default=None)
    m = sub.add_parser("mfma")
    m.add_argument("dir")
    m.add_argument("--trace", default=None)
    m.add_argument("--command", required=True)
    args = ap.parse_args(argv)
    {"trace": cmd_trace, "traffic": cmd_traffic, "counters": cmd_counters, "mfma": cmd_mfma}[args.cmd](args)


if __name__ == "__main__":
    sys.exit(main())
