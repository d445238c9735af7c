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

All passes of bench.py legs at once (rocprofv3 started as a child process
for each pass, the summaries written to profiles/, each leg's kernel-trace
table printed):

    python -m long_context_dynamic_amd.pmc collect --legs prefill moba decode --dir prof_out

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


# ------------------------------------------------------------- collection --
# The rocprofv3 passes behind the committed summaries, per bench.py leg:
# FETCH_SIZE and WRITE_SIZE runs, counter sets that each fit the hardware's
# per-block limits (at most 8 SQ, 4 TCC, 4 TCP, 2 TA, 2 GRBM), a kernel
# trace.  Algorithmic FLOP per launch are bench.py's counts for the
# workload (selected: 2.644e12, compressed + window: 2.742e12 at 64k;
# MoBA 32k: 5.369e11 listed blocks, 1.377e11 own block).
PREFILL_SETS = (["MfmaUtil", "MfmaFlopsBF16", "VALUBusy", "SQ_WAIT_INST_ANY", "SQ_WAVES"],
                ["SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_WAIT_ANY", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS",
                 "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VMEM_RD", "SQ_INSTS_LDS", "GRBM_GUI_ACTIVE"],
                ["TA_BUSY_avr", "TCP_TOTAL_CACHE_ACCESSES_sum", "TCP_TCC_READ_REQ_sum", "TCC_HIT_sum", "TCC_MISS_sum",
                 "GRBM_GUI_ACTIVE"])
DECODE_SETS = (["SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_VALU",
                "SQ_INSTS_VMEM_RD", "SQ_INSTS_VALU", "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE"],
               ["TA_BUSY_avr", "TCP_TCC_READ_REQ_sum", "TCC_HIT_sum", "TCC_MISS_sum", "GRBM_GUI_ACTIVE"])
LEGS = {
    "prefill": {"workload": "nsa_prefill_64k", "args": ["--only", "prefill", "--workload", "nsa_prefill_64k"],
                "kernels": [("selected", "k_sel_part<192, 128>", 2.644089e12), ("selected_merge", "k_sel_merge", 0.0),
                            ("cmp_select_window", "k_cmpwin<192, 128, true", 2.742e12)],
                "sets": PREFILL_SETS, "trace_steps": 5},
    "moba": {"workload": "moba_32k", "args": ["--only", "prefill", "--workload", "moba_32k"],
             "kernels": [("moba_attn", "k_moba_attn", 5.36870912e11), ("moba_own_block", "k_moba_diag", 1.37707e11)],
             "sets": PREFILL_SETS, "trace_steps": 5},
    "decode": {"workload": "nsa_decode_64x64k", "args": ["--only", "decode"],
               "kernels": [("dec_step", "k_dec_fused", 0.0)], "sets": DECODE_SETS, "trace_steps": 10},
}


def _run_pass(repo, out_dir, name, prof_args, bench_args, limit):
    """One rocprofv3 pass over bench.py (the program itself after --), in
    /tmp, killed with its process group after limit seconds.  Returns the
    command as recorded in the summaries."""
    import signal
    import subprocess
    import time
    d = os.path.join(out_dir, name)
    cmd = ["rocprofv3"] + prof_args + ["-d", d, "-o", "run", "--output-format", "csv", "--",
                                        "python3", os.path.join(repo, "bench.py")] + bench_args
    env = dict(os.environ, TMPDIR="/tmp")
    t0 = time.time()
    print(f"[pmc] {name}: {' '.join(cmd)}", flush=True)
    p = subprocess.Popen(cmd, cwd="/tmp", env=env, start_new_session=True,
                         stdout=open(d + ".log", "w"), stderr=subprocess.STDOUT)
    try:
        rc = p.wait(timeout=limit)
    except subprocess.TimeoutExpired:
        os.killpg(p.pid, signal.SIGKILL)
        p.wait()
        raise RuntimeError(f"{name}: killed after {limit} s (log {d}.log)")
    if rc != 0 and not glob.glob(os.path.join(d, "**", "*.csv"), recursive=True):
        raise RuntimeError(f"{name}: rocprofv3 exited {rc} with no results (log {d}.log)")
    print(f"[pmc] {name}: done in {time.time() - t0:.0f} s (rc {rc})", flush=True)
    return "cd /tmp && export TMPDIR=/tmp; " + " ".join(cmd).replace(repo, "$REPO")


def collect(args) -> None:
    """Runs the passes of the named legs into args.dir and writes their
    traffic and counter summaries to args.profiles; prints each leg's
    kernel-trace table."""
    repo = os.path.dirname(PKG)
    os.makedirs(args.dir, exist_ok=True)
    lim = args.limit
    cal_f = _run_pass(repo, args.dir, "FETCH_SIZE_gather", ["--pmc", "FETCH_SIZE"],
                      ["--only", "gather", "--steps", "2", "--warmup", "1"], lim)
    cal_w = _run_pass(repo, args.dir, "WRITE_SIZE_copy", ["--pmc", "WRITE_SIZE"],
                      ["--only", "copy", "--steps", "2", "--warmup", "1"], lim)
    for leg in args.legs:
        L = LEGS[leg]
        wl = L["workload"]
        steps = ["--steps", "2", "--warmup", "1"]
        cf = _run_pass(repo, args.dir, f"FETCH_SIZE_{leg}", ["--pmc", "FETCH_SIZE"], L["args"] + steps, lim)
        cw = _run_pass(repo, args.dir, f"WRITE_SIZE_{leg}", ["--pmc", "WRITE_SIZE"], L["args"] + steps, lim)
        tcmd = "; ".join([cf, cw, cal_f, cal_w])
        runs, ccmds = [], []
        for i, s in enumerate(L["sets"]):
            name = f"ctr_{leg}{i + 1}"
            ccmds.append(_run_pass(repo, args.dir, name, ["--pmc"] + s,
                                   L["args"] + ["--steps", "1", "--warmup", "1"], lim))
            runs.append(os.path.join(args.dir, name))
        trace_dir = f"trace_{leg}"
        _run_pass(repo, args.dir, trace_dir, ["--kernel-trace", "--stats"],
                  L["args"] + ["--steps", str(L["trace_steps"]), "--warmup", "2"], lim)
        for name, sym, flop in L["kernels"]:
            ns = argparse.Namespace(kernel=sym, name=name, workload=wl, command=tcmd,
                                    fetch=os.path.join(args.dir, f"FETCH_SIZE_{leg}"),
                                    write=os.path.join(args.dir, f"WRITE_SIZE_{leg}"),
                                    gather_fetch=os.path.join(args.dir, "FETCH_SIZE_gather"), copy_fetch=None,
                                    copy_write=os.path.join(args.dir, "WRITE_SIZE_copy"))
            with open(os.path.join(args.profiles, f"{name}_{wl}_traffic.json"), "w") as fh:
                json.dump(traffic(ns), fh, indent=1)
            ns = argparse.Namespace(kernel=sym, name=name, workload=wl, runs=runs, algorithmic_flop=flop,
                                    command="; ".join(ccmds))
            with open(os.path.join(args.profiles, f"{name}_{wl}_counters.json"), "w") as fh:
                json.dump(counters(ns), fh, indent=1)
            print(f"[pmc] wrote {name}_{wl} traffic and counters", flush=True)
        print(f"[pmc] kernel trace of {leg} ({wl}):\n| kernel | calls | avg us |\n|---|---|---|")
        for n, c, us in trace_stats(os.path.join(args.dir, trace_dir)):
            print(f"| {n} | {c} | {us:.1f} |")
        sys.stdout.flush()


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
    r = sub.add_parser("collect", help="run the rocprofv3 passes of bench.py legs and write their summaries")
    r.add_argument("--legs", nargs="+", choices=sorted(LEGS), required=True)
    r.add_argument("--dir", required=True, help="directory for the raw rocprofv3 output")
    r.add_argument("--profiles", default=os.path.join(os.path.dirname(PKG), "profiles"))
    r.add_argument("--limit", type=int, default=240, help="seconds per pass before it is killed")
    args = ap.parse_args(argv)
    if args.cmd == "collect":
        return collect(args)
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
