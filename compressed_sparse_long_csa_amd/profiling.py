"""Summaries of rocprofv3 output for the committed profiles.

  python -m compressed_sparse_long_csa_amd.profiling stats RESULTS_DB
      per-kernel launch count and duration (avg / median / min, microseconds)
      from a `rocprofv3 --kernel-trace` database (its `kernels` view).
      With --split-runs, launches that follow or precede a launch of the same
      kernel (a loop that launches one kernel again and again, as bench.py's
      per-kernel timing does) are counted apart from the rest (the graph of
      the step, where every kernel follows a different one).

  python -m compressed_sparse_long_csa_amd.profiling traffic --kernel SUBSTR \\
      --fetch CSV --write CSV --copy-fetch CSV --copy-write CSV --copy-bytes N \\
      --source FILE [--source FILE ...] --out JSON
      HBM bytes per launch of the kernels whose name contains SUBSTR, from two
      `rocprofv3 --pmc FETCH_SIZE` / `--pmc WRITE_SIZE` runs (KiB per
      dispatch).  Each counter is scaled by what it reads for a plain copy
      kernel that moves a known number of bytes (N read, N written), so the
      figure does not depend on the counter's unit or channel coverage.  The
      record keeps the sha256 of the kernel's source files (concatenated in
      the order given): a reader can tell whether the counters were taken on
      the current kernel.

  python -m compressed_sparse_long_csa_amd.profiling counters --csv CSV \\
      --trace-db RESULTS_DB [--kernel SUBSTR ...]
      MFMA use per kernel from one `rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES
      SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_VALU_MFMA_MOPS_F8
      SQ_INSTS_VALU_MFMA_MOPS_F6F4 ...` run: busy SIMD-cycles and MOPS per
      dispatch (a MOP is 512 FLOPs), against the kernel's average duration in
      a kernel-trace run of the same workload.  busy = busy cycles / (1024
      SIMDs x duration x 2.4 GHz); TFLOP/s per operand type, and the fraction
      of that type's dense peak (BF16 2.5, FP8 5.0, FP6/FP4 10.1 PFLOP/s).
"""
import argparse
import collections
import csv
import hashlib
import json
import sqlite3
import statistics
import sys


def kernel_stats(db, runs=None):
    """runs=None: every launch; True: only launches next to a launch of the
    same kernel (in start order); False: only the others."""
    con = sqlite3.connect(db)
    rows = con.execute("select name, duration from kernels order by start").fetchall()
    d = collections.defaultdict(list)
    for i, (name, dur) in enumerate(rows):
        if runs is not None:
            in_run = ((i > 0 and rows[i - 1][0] == name)
                      or (i + 1 < len(rows) and rows[i + 1][0] == name))
            if in_run != runs:
                continue
        d[name].append(dur / 1000.0)
    tot = sum(sum(v) for v in d.values()) or 1.0
    out = []
    for name, v in sorted(d.items(), key=lambda x: -sum(x[1])):
        out.append(dict(kernel=name, launches=len(v), avg_us=statistics.mean(v),
                        median_us=statistics.median(v), min_us=min(v), share=sum(v) / tot))
    return out


def sources_sha256(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def counter_per_dispatch(path, substr, counter):
    vals = collections.defaultdict(float)
    with open(path) as f:
        for r in csv.DictReader(f):
            if substr in r["Kernel_Name"] and r["Counter_Name"] == counter:
                vals[r["Dispatch_Id"]] += float(r["Counter_Value"])
    if not vals:
        raise SystemExit(f"no {counter} rows for kernels matching {substr!r} in {path}")
    return statistics.mean(vals.values()), len(vals)


SIMDS, CLOCK_GHZ = 1024, 2.4
MOPS_PEAK_TFLOPS = {"SQ_INSTS_VALU_MFMA_MOPS_BF16": ("bf16", 2500.0), "SQ_INSTS_VALU_MFMA_MOPS_F8": ("fp8", 5000.0),
                    "SQ_INSTS_VALU_MFMA_MOPS_F6F4": ("fp6/fp4", 10100.0)}


def counters_table(csv_path, db, substrs=None):
    per = collections.defaultdict(lambda: collections.defaultdict(list))
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            per[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
    dur = {r["kernel"]: r["avg_us"] for r in kernel_stats(db)}
    out = []
    for name, cs in per.items():
        if "SQ_VALU_MFMA_BUSY_CYCLES" not in cs or (substrs and not any(x in name for x in substrs)):
            continue
        busy = statistics.mean(cs["SQ_VALU_MFMA_BUSY_CYCLES"])
        if busy == 0 or name not in dur:
            continue
        us = dur[name]
        row = dict(kernel=name, dispatches=len(cs["SQ_VALU_MFMA_BUSY_CYCLES"]), busy_cycles=busy, avg_us=us,
                   busy_frac=busy / (SIMDS * us * 1e-6 * CLOCK_GHZ * 1e9), types={})
        for c, (ty, peak) in MOPS_PEAK_TFLOPS.items():
            if c in cs:
                fl = statistics.mean(cs[c]) * 512.0
                if fl > 0:
                    tf = fl / (us * 1e-6) / 1e12
                    row["types"][ty] = dict(gflop=fl / 1e9, tflops=tf, frac_of_peak=tf / peak)
        out.append(row)
    return sorted(out, key=lambda r: -r["avg_us"])


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("db")
    s.add_argument("--split-runs", action="store_true")
    t = sub.add_parser("traffic")
    for a in ("--kernel", "--fetch", "--write", "--copy-fetch", "--copy-write", "--out"):
        t.add_argument(a, required=True)
    t.add_argument("--source", action="append", required=True)
    t.add_argument("--copy-kernel", default="MulFunctor",
                   help="name part of the copy kernel (torch's multiply; its fill kernel must not match)")
    t.add_argument("--copy-bytes", type=int, required=True, help="bytes read (= written) per copy launch")
    c = sub.add_parser("counters")
    c.add_argument("--csv", required=True)
    c.add_argument("--trace-db", required=True)
    c.add_argument("--kernel", action="append")
    args = ap.parse_args(argv)
    if args.cmd == "counters":
        print(f"{'kernel':70s} {'disp':>5s} {'avg_us':>8s} {'mfma_busy':>9s}  per type: GFLOP/dispatch, TFLOP/s, of peak")
        for r in counters_table(args.csv, args.trace_db, args.kernel):
            ty = "; ".join(f"{t} {v['gflop']:.3f} GFLOP {v['tflops']:.1f} TF/s {100 * v['frac_of_peak']:.1f}%"
                           for t, v in r["types"].items())
            print(f"{r['kernel'][:70]:70s} {r['dispatches']:5d} {r['avg_us']:8.2f} {100 * r['busy_frac']:8.1f}%  {ty}")
        return
    if args.cmd == "stats":
        parts = ([("launches next to a launch of the same kernel", True),
                  ("all other launches", False)] if args.split_runs else [(None, None)])
        for title, runs in parts:
            if title:
                print(f"# {title}")
            print(f"{'kernel':90s} {'launches':>8s} {'avg_us':>9s} {'median':>9s} {'min':>9s} {'share':>6s}")
            for r in kernel_stats(args.db, runs):
                print(f"{r['kernel'][:90]:90s} {r['launches']:8d} {r['avg_us']:9.2f} {r['median_us']:9.2f} "
                      f"{r['min_us']:9.2f} {100 * r['share']:5.1f}%")
        return
    f_kib, nf = counter_per_dispatch(args.fetch, args.kernel, "FETCH_SIZE")
    w_kib, nw = counter_per_dispatch(args.write, args.kernel, "WRITE_SIZE")
    cf_kib, _ = counter_per_dispatch(args.copy_fetch, args.copy_kernel, "FETCH_SIZE")
    cw_kib, _ = counter_per_dispatch(args.copy_write, args.copy_kernel, "WRITE_SIZE")
    f_scale = args.copy_bytes / (cf_kib * 1024.0)
    w_scale = args.copy_bytes / (cw_kib * 1024.0)
    fetch_b = f_kib * 1024.0 * f_scale
    write_b = w_kib * 1024.0 * w_scale
    sha = sources_sha256(args.source)
    rec = dict(kernel=args.kernel, dispatches=[nf, nw], fetch_kib_per_dispatch=f_kib,
               write_kib_per_dispatch=w_kib, copy_bytes=args.copy_bytes,
               copy_fetch_kib=cf_kib, copy_write_kib=cw_kib, fetch_scale=f_scale,
               write_scale=w_scale, fetch_bytes=fetch_b, write_bytes=write_b,
               bytes_per_launch=fetch_b + write_b, source=args.source, source_sha256=sha)
    with open(args.out, "w") as f:
        json.dump(rec, f, indent=1)
    json.dump(rec, sys.stdout, indent=1)
    print()


if __name__ == "__main__":
    main()
