"""Summaries of rocprofv3 output for the committed profiles.

HBM traffic of a kernel from two counter runs (FETCH_SIZE, then WRITE_SIZE,
KiB per dispatch), each scaled by what the same counter reads for a kernel
of known traffic: WRITE_SIZE by a plain 1 GiB device copy (1 GiB written),
FETCH_SIZE by the read-only block gather of bench.py's gather leg (known
bytes, the selected branch's and the decode's access pattern) or, without
one, by the copy (1 GiB read):

    python -m long_context_dynamic_amd.pmc traffic --kernel k_sel_part --name selected \\
        --workload nsa_prefill_64k --fetch DIR --write DIR --gather-fetch DIR --copy-write DIR \\
        --command "..." --out profiles/selected_nsa_prefill_64k_traffic.json

Counters of one kernel (matrix-op utilisation and FLOP, VALU busy, ...)
from one or more --pmc runs, mean per dispatch:

    python -m long_context_dynamic_amd.pmc counters --kernel k_sel --name selected \\
        --workload nsa_prefill_64k --runs DIR [DIR ...] --algorithmic-flop 2.644e12 \\
        --command "..." --out profiles/selected_nsa_prefill_64k_counters.json

Per-kernel durations from a --kernel-trace run (CSV or rocpd database):

    python -m long_context_dynamic_amd.pmc trace DIR

The traffic summary records a hash of the kernel's sources; bench.py reports
the traffic only while the sources still hash the same.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sqlite3
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")

# sources whose text decides each kernel's code
KERNEL_SOURCES = {
    "selected": ["k_prefill.hip", "nsa_prefill.h", "nsa_frag.h", "nsa_tile.h", "nsa_topk.h", "nsa_mfma.h",
                 "nsa_internal.h"],
    "selected_merge": ["k_prefill.hip", "nsa_prefill.h", "nsa_frag.h", "nsa_tile.h", "nsa_topk.h", "nsa_mfma.h",
                       "nsa_internal.h"],
    "cmp_select_window": ["k_prefill.hip", "nsa_prefill.h", "nsa_frag.h", "nsa_tile.h", "nsa_topk.h", "nsa_mfma.h",
                          "nsa_internal.h"],
    "moba_attn": ["k_moba.hip", "nsa_moba.h", "nsa_tile.h", "nsa_mfma.h", "nsa_internal.h"],
    "moba_own_block": ["k_moba.hip", "nsa_moba.h", "nsa_tile.h", "nsa_mfma.h", "nsa_internal.h"],
    "dec_step": ["k_decode.hip", "nsa_decode.h", "nsa_topk.h", "nsa_mfma.h", "nsa_internal.h"],
}

COPY_BYTES = 2 ** 30


def source_hash(name: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[name]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def _short(kernel_name: str) -> str:
    n = re.sub(r"\(anonymous namespace\)::", "", kernel_name)
    return re.sub(r"\(.*", "", n).replace("void ", "")


def counter_means(run_dir: str, counter: str) -> dict:
    """{short kernel name: mean counter value per dispatch} of one --pmc run."""
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {run_dir}")
    acc = {}
    for f in files:
        with open(f) as fh:
            for row in csv.DictReader(fh):
                if row["Counter_Name"] != counter:
                    continue
                k = _short(row["Kernel_Name"])
                s = acc.setdefault(k, [0.0, 0])
                s[0] += float(row["Counter_Value"])
                s[1] += 1
    return {k: v[0] / v[1] for k, v in acc.items()}


def _pick(means: dict, substr: str) -> float:
    hits = [v for k, v in means.items() if substr in k]
    if len(hits) != 1:
        raise KeyError(f"{len(hits)} kernels match {substr!r}: {sorted(means)}")
    return hits[0]


def _copy_value(means: dict) -> float:
    # the device copy is the only elementwise/copy kernel of the copy leg
    hits = [v for k, v in means.items() if "copy" in k.lower() or "elementwise" in k.lower()]
    if not hits:
        raise KeyError(f"no copy kernel among {sorted(means)}")
    return max(hits)


# the gather leg of bench.py: 262144 waves x 4 blocks x 40 KiB per launch
GATHER_BYTES = 262144 * 4 * 40960


def traffic(args) -> dict:
    f_k = _pick(counter_means(args.fetch, "FETCH_SIZE"), args.kernel)
    w_k = _pick(counter_means(args.write, "WRITE_SIZE"), args.kernel)
    w_c = _copy_value(counter_means(args.copy_write, "WRITE_SIZE"))
    write_scale = COPY_BYTES / (w_c * 1024.0)
    if args.gather_fetch:
        f_c = _pick(counter_means(args.gather_fetch, "FETCH_SIZE"), "k_gather")
        fetch_scale = GATHER_BYTES / (f_c * 1024.0)
        cal = {"fetch": "read-only 40 KiB block gather over 1.25 GiB", "FETCH_SIZE_kib": f_c,
               "fetch_bytes": GATHER_BYTES}
    else:
        f_c = _copy_value(counter_means(args.copy_fetch, "FETCH_SIZE"))
        fetch_scale = COPY_BYTES / (f_c * 1024.0)
        cal = {"fetch": "1 GiB device copy", "FETCH_SIZE_kib": f_c, "fetch_bytes": COPY_BYTES}
    cal.update({"fetch_scale": fetch_scale, "write": "1 GiB device copy", "WRITE_SIZE_kib": w_c,
                "write_bytes": COPY_BYTES, "write_scale": write_scale})
    fetch = f_k * 1024.0 * fetch_scale
    write = w_k * 1024.0 * write_scale
    return {
        "kernel": args.name, "kernel_symbol": args.kernel, "workload": args.workload,
        "fetch_bytes_per_launch": fetch, "write_bytes_per_launch": write,
        "traffic_bytes_per_launch": fetch + write,
        "raw_kib_per_dispatch": {"FETCH_SIZE": f_k, "WRITE_SIZE": w_k},
        "calibration": cal,
        "source_hash": source_hash(args.name), "command": args.command,
    }


def all_counter_means(run_dir: str) -> dict:
    """{short kernel name: {counter: mean value per dispatch}} of one --pmc run."""
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {run_dir}")
    acc = {}
    for f in files:
        with open(f) as fh:
            for row in csv.DictReader(fh):
                k = _short(row["Kernel_Name"])
                s = acc.setdefault(k, {}).setdefault(row["Counter_Name"], [0.0, 0])
                s[0] += float(row["Counter_Value"])
                s[1] += 1
    return {k: {c: v[0] / v[1] for c, v in cs.items()} for k, cs in acc.items()}


def counters(args) -> dict:
    """One kernel's counters from one or more --pmc runs (mean per dispatch),
    with the algorithmic FLOP per launch and what the matrix-op count says."""
    vals = {}
    for d in args.runs:
        means = all_counter_means(d)
        hits = [k for k in means if args.kernel in k]
        if len(hits) != 1:
            raise KeyError(f"{len(hits)} kernels match {args.kernel!r} in {d}: {sorted(means)}")
        vals.update(means[hits[0]])
    rec = {"kernel": args.name, "kernel_symbol": args.kernel, "workload": args.workload, "counters": vals,
           "source_hash": source_hash(args.name), "command": args.command}
    if "MfmaFlopsBF16" in vals and args.algorithmic_flop:
        rec["algorithmic_flop_per_launch"] = args.algorithmic_flop
        rec["executed_over_algorithmic"] = vals["MfmaFlopsBF16"] / args.algorithmic_flop
    return rec


def trace_stats(run_dir: str) -> list:
    """[(short name, calls, mean us)] from a --kernel-trace run, longest total first."""
    rows = []
    for f in glob.glob(os.path.join(run_dir, "**", "*kernel_trace.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                rows.append((_short(r["Kernel_Name"]), (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
    for f in glob.glob(os.path.join(run_dir, "**", "*results.db"), recursive=True):
        db = sqlite3.connect(f)
        cols = [c[1] for c in db.execute("pragma table_info(kernels)")]
        name = "name" if "name" in cols else "kernel_name"
        for n, s, e in db.execute(f"select {name}, start, end from kernels"):
            rows.append((_short(n), (e - s) / 1e3))
    agg = {}
    for n, us in rows:
        a = agg.setdefault(n, [0, 0.0])
        a[0] += 1
        a[1] += us
    return sorted(((n, c, t / c) for n, (c, t) in agg.items()), key=lambda x: -x[1] * x[2])


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--kernel", required=True, help="substring of the kernel symbol")
    t.add_argument("--name", required=True, choices=sorted(KERNEL_SOURCES))
    t.add_argument("--workload", required=True)
    for k in ("fetch", "write", "copy_write"):
        t.add_argument("--" + k.replace("_", "-"), dest=k, required=True)
    t.add_argument("--gather-fetch", dest="gather_fetch", default=None,
                   help="FETCH_SIZE run of bench.py --only gather (calibrates FETCH_SIZE)")
    t.add_argument("--copy-fetch", dest="copy_fetch", default=None,
                   help="FETCH_SIZE run of bench.py --only copy (used without --gather-fetch)")
    t.add_argument("--command", default="")
    t.add_argument("--out", required=True)
    c = sub.add_parser("counters")
    c.add_argument("--kernel", required=True, help="substring of the kernel symbol")
    c.add_argument("--name", required=True, choices=sorted(KERNEL_SOURCES))
    c.add_argument("--workload", required=True)
    c.add_argument("--runs", nargs="+", required=True, help="--pmc output directories")
    c.add_argument("--algorithmic-flop", type=float, default=0.0)
    c.add_argument("--command", default="")
    c.add_argument("--out", required=True)
    s = sub.add_parser("trace")
    s.add_argument("dir")
    args = ap.parse_args(argv)
    if args.cmd in ("traffic", "counters"):
        rec = traffic(args) if args.cmd == "traffic" else counters(args)
        with open(args.out, "w") as fh:
            json.dump(rec, fh, indent=1)
        print(json.dumps(rec, indent=1))
    else:
        print("| kernel | calls | avg us |\n|---|---|---|")
        for n, c, us in trace_stats(args.dir):
            print(f"| {n} | {c} | {us:.1f} |")


if __name__ == "__main__":
    sys.exit(main())
