"""Short text summaries of rocprofv3 output.

    python -m long_context_self_amd.profile_summary stats --csv <kernel_stats.csv | results.db> \\
        --command "<the rocprofv3 command>" --out profiles/<kernel>_<workload>.md
    python -m long_context_self_amd.profile_summary counters --db <results.db> [--db ...] \\
        --kernel <name> [--kernel ...] --command "..." [--command ...] --out profiles/<...>.md
    python -m long_context_self_amd.profile_summary traffic \\
        --fetch <counter_collection.csv | results.db of a FETCH_SIZE run> \\
        --write <counter_collection.csv | results.db of a WRITE_SIZE run> \\
        --copy-bytes <size of the calibration copy> --kernel <name> [--kernel <name> ...] \\
        --algorithmic-bytes <per launch> --command-fetch "..." --command-write "..." \\
        --out profiles/<kernel>_<workload>_traffic.json

`traffic` scales each counter (KiB per dispatch) by what the same counter reads for a
plain device-to-device copy of known size in the same run (the runtime's copy kernel;
the last dispatch of it at least a quarter the size of the largest, since the per-layer
KV replicas made before the calibration copy are copies too),
and sums the named kernels' dispatches into HBM bytes per call.  Each kernel's figure is
the median over its dispatches, so that a one-time first-call path (a workspace that
is not yet initialised, a cold cache) does not stand for the steady per-call traffic;
the mean and the maximum are kept beside it.  The JSON carries a
hash of the kernel sources so that a later source change makes it stale.  Inputs are
either rocprofv3's CSV files or its default SQLite database (`*_results.db`).
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
import sqlite3
import statistics
import sys
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCES = [os.path.join(PKG, "csrc", f) for f in ("attn.hip", "select.hip", "lcs_internal.h")]
SIMDS = 256 * 4          # MI355X: 256 compute units of 4 SIMDs
XCDS = 8                 # GRBM_GUI_ACTIVE as collected per dispatch is the sum over the 8 XCDs
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def _code_only(text: str) -> str:
    """Source text without comments and whitespace: edits to comments leave the
    kernels, and so the counters taken on them, unchanged."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return re.sub(r"\s+", "", text)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f) as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def short_name(n: str) -> str:
    for junk in ("lcs::(anonymous namespace)::", "(lcs::AttnArgs)", "(lcs::SelArgs, int)", "(lcs::SelArgs)",
                 "void "):
        n = n.replace(junk, "")
    return n.strip()


def stats_rows(path: str):
    if not path.endswith(".db"):
        return list(csv.DictReader(open(path)))
    durs = defaultdict(list)
    for name, d in sqlite3.connect(path).execute("select name, duration from kernels"):
        durs[name].append(float(d))
    grand = sum(sum(v) for v in durs.values()) or 1.0
    return [{"Name": k, "Calls": str(len(v)), "AverageNs": sum(v) / len(v), "MedianNs": statistics.median(v),
             "MinNs": min(v), "MaxNs": max(v), "TotalDurationNs": sum(v), "Percentage": 100.0 * sum(v) / grand}
            for k, v in durs.items()]


def stats(args) -> None:
    rows = stats_rows(args.csv)
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    out = [f"# {args.title}", "", "Command (run from the repository root):", "", "```", args.command, "```", "",
           "| kernel | calls | avg us | median us | min us | max us | total us | % |",
           "|---|---:|---:|---:|---:|---:|---:|---:|"]
    for r in rows:
        med = "%.2f" % (float(r["MedianNs"]) / 1e3) if r.get("MedianNs") is not None else "—"
        out.append("| `%s` | %s | %.2f | %s | %.2f | %.2f | %.1f | %.2f |" % (
            short_name(r["Name"])[:70], r["Calls"], float(r["AverageNs"]) / 1e3, med, float(r["MinNs"]) / 1e3,
            float(r["MaxNs"]) / 1e3, float(r["TotalDurationNs"]) / 1e3, float(r["Percentage"])))
    if args.note:
        out += ["", args.note]
    with open(args.out, "w") as fh:
        fh.write("\n".join(out) + "\n")


def per_kernel(path: str, counter: str):
    """kernel name -> list of counter values (KiB), one per dispatch."""
    vals = defaultdict(list)
    if path.endswith(".db"):
        q = "select kernel_name, value from counters_collection where counter_name = ? order by dispatch_id"
        for name, v in sqlite3.connect(path).execute(q, (counter,)):
            vals[short_name(name)].append(float(v))
        return vals
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        vals[short_name(r["Kernel_Name"])].append(float(r["Counter_Value"]))
    return vals


def traffic(args) -> None:
    res = {"kernel_source_hash": kernel_source_hash(), "kernels": {}, "copy_bytes": args.copy_bytes,
           "commands": {"FETCH_SIZE": args.command_fetch, "WRITE_SIZE": args.command_write}}
    total = 0.0
    for counter, path in (("FETCH_SIZE", args.fetch), ("WRITE_SIZE", args.write)):
        vals = per_kernel(path, counter)
        copies = vals.get(COPY_KERNEL, [])
        if not copies:
            sys.exit(f"no {COPY_KERNEL} dispatch with {counter} in {path}")
        # bench.py makes its calibration copy after the per-layer KV replicas (also copies,
        # and larger than it at 128K x 8), so it is the last large copy dispatch
        copy_kib = [c for c in copies if c >= 0.25 * max(copies)][-1]
        factor = (args.copy_bytes / 1024.0) / copy_kib
        res[f"{counter}_copy_kib"] = copy_kib
        res[f"{counter}_factor"] = round(factor, 5)
        for k in args.kernel:
            if k not in vals:
                sys.exit(f"kernel {k!r} has no {counter} values in {path}; have {sorted(vals)}")
            v = vals[k]
            med_kib = statistics.median(v)
            ent = res["kernels"].setdefault(k, {})
            ent[f"{counter}_kib_median"] = round(med_kib, 1)
            ent[f"{counter}_kib_mean"] = round(sum(v) / len(v), 1)
            ent[f"{counter}_kib_max"] = round(max(v), 1)
            ent[f"{counter}_dispatches"] = len(v)
            ent[f"{counter}_bytes_scaled"] = round(med_kib * 1024.0 * factor)
            total += med_kib * 1024.0 * factor
    res["hbm_bytes_per_launch"] = round(total)
    if args.algorithmic_bytes:
        res["algorithmic_bytes_per_launch"] = args.algorithmic_bytes
        res["traffic_over_algorithmic"] = round(total / args.algorithmic_bytes, 4)
    with open(args.out, "w") as fh:
        json.dump(res, fh, indent=1)
        fh.write("\n")


def counters(args) -> None:
    """Per-dispatch medians of every counter in one or more --pmc databases for the named
    kernels (the median, as in `traffic`, so a one-time first-call path does not stand for
    the steady call), with the derived MFMA busy fraction, MFMA bf16 flops and LDS
    bank-conflict rate where their inputs were collected."""
    per = defaultdict(dict)
    for path in args.db:
        rows = sqlite3.connect(path).execute("select kernel_name, counter_name, value from counters_collection")
        acc = defaultdict(list)
        for name, cn, v in rows:
            acc[(short_name(name), cn)].append(float(v))
        for (k, cn), v in acc.items():
            if k in args.kernel:
                per[k][cn] = statistics.median(v)
    out = ["# " + args.title, "", "Commands (run from the repository root):", ""]
    out += ["```"] + list(args.command) + ["```", ""]
    out += ["| kernel | counter | per dispatch (median) |", "|---|---|---:|"]
    for k in args.kernel:
        for cn in sorted(per.get(k, {})):
            out.append(f"| `{k}` | {cn} | {per[k][cn]:.4g} |")
    out += ["", "| kernel | MFMA busy (% of SIMD cycles) | MFMA bf16 GFLOP | LDS bank conflicts / LDS cycles |",
            "|---|---:|---:|---:|"]
    for k in args.kernel:
        c = per.get(k, {})
        busy = (100.0 * c["SQ_VALU_MFMA_BUSY_CYCLES"] / (c["GRBM_GUI_ACTIVE"] / XCDS * SIMDS)
                if "SQ_VALU_MFMA_BUSY_CYCLES" in c and c.get("GRBM_GUI_ACTIVE") else None)
        fl = c["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512 / 1e9 if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in c else None
        lds = (c["SQ_LDS_BANK_CONFLICT"] / c["SQ_LDS_IDX_ACTIVE"]
               if c.get("SQ_LDS_IDX_ACTIVE") and "SQ_LDS_BANK_CONFLICT" in c else None)
        f = lambda x, fmt: "—" if x is None else fmt % x  # noqa: E731
        out.append(f"| `{k}` | {f(busy, '%.1f')} | {f(fl, '%.3f')} | {f(lds, '%.4f')} |")
    if args.note:
        out += ["", args.note]
    with open(args.out, "w") as fh:
        fh.write("\n".join(out) + "\n")


def main(argv=None) -> None:
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = p.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("--csv", required=True)
    s.add_argument("--command", required=True)
    s.add_argument("--title", default="rocprofv3 kernel statistics")
    s.add_argument("--note", default="")
    s.add_argument("--out", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--kernel", action="append", required=True)
    t.add_argument("--algorithmic-bytes", type=int, default=0)
    t.add_argument("--command-fetch", required=True)
    t.add_argument("--command-write", required=True)
    t.add_argument("--out", required=True)
    c = sub.add_parser("counters")
    c.add_argument("--db", action="append", required=True)
    c.add_argument("--kernel", action="append", required=True)
    c.add_argument("--command", action="append", required=True)
    c.add_argument("--title", default="rocprofv3 counters")
    c.add_argument("--note", default="")
    c.add_argument("--out", required=True)
    a = p.parse_args(argv)
    {"stats": stats, "traffic": traffic, "counters": counters}[a.cmd](a)


if __name__ == "__main__":
    main()
