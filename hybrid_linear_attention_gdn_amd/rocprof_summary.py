"""Text summaries of rocprofv3 output, for the committed profiles/ directory.

Kernel times of a ``rocprofv3 --kernel-trace --stats`` run::

    python -m hybrid_linear_attention_gdn_amd.rocprof_summary stats RUN_DIR \\
        --command "<the rocprofv3 command>" [--bench-log LOG] \\
        [--window KERNEL FIRST COUNT] > profiles/<kernel>_<workload>_kernel_trace.md

``--window`` adds the mean duration of dispatches FIRST .. FIRST + COUNT - 1
of the kernel, in start order, from the run's kernel_trace.csv: the timed
steps of a bench run that warms up first.

Per-kernel means of a ``rocprofv3 --pmc`` run of rocprofv3's derived metrics
(MfmaUtil, LdsBankConflict, ...)::

    python -m hybrid_linear_attention_gdn_amd.rocprof_summary counters RUN_DIR \
        --command "<the rocprofv3 command>" > profiles/counters_<workload>.md

HBM bytes of one kernel from two ``rocprofv3 --pmc`` runs (FETCH_SIZE, then
WRITE_SIZE), each scaled by what the same counter reads for the elementwise
copy of known size that ``bench.py --copy-mib N`` runs in the same process,
per launch and per step (``--launches-per-step``: the kernel's launches in one
bench step, which repeat identically from step to step)::

    python -m hybrid_linear_attention_gdn_amd.rocprof_summary traffic --fetch DIR --write DIR \\
        --copy-mib N --kernel scan_kernel --stage scan --workload clip_241f --o-dtype fp32 \\
        --launches-per-step 6 --fetch-command "..." --write-command "..." \\
        --json profiles/traffic_scan_clip_241f.json --md profiles/scan_clip_241f_traffic.md

The JSON carries a hash of the kernel's sources (see ``kernel_source_hash``);
``bench.py`` reports the stored bytes only while the hash still matches.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import statistics
import sys

PKG = os.path.dirname(os.path.abspath(__file__))

# Source files of the kernels a profiling stage runs.
_STAGE_SOURCES = {
    (True, "scan"): ["gdn_scan.hip", "gdn_intra.h"],
    (False, "portable"): [],
}
_COMMON = {True: ["gdn_mfma_common.h", "gdn_internal.h"], False: ["gdn_prep.hip", "gdn_portable.hip",
                                                                    "gdn_internal.h"]}


def _code_only(text: str) -> str:
    """C++ source without comments and with whitespace runs collapsed, so that
    editing a comment does not count as changing the kernel."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash(stage: str, mfma: bool) -> str:
    """Short hash of the code (comments excluded) of the kernel that `stage` runs."""
    files = _STAGE_SOURCES.get((mfma, stage), []) + _COMMON[mfma]
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(PKG, "csrc", f)) as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def _one(directory: str, suffix: str) -> str:
    hits = sorted(glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True))
    if not hits:
        raise SystemExit(f"no *{suffix} under {directory}")
    return hits[0]


def short_name(name: str) -> str:
    """Kernel name without argument list and namespaces (templates kept)."""
    n = name.strip().replace("(anonymous namespace)::", "")
    if n.startswith("void "):
        n = n[5:]
    depth, cut = 0, len(n)
    for i, ch in enumerate(n):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            cut = i
            break
    n = n[:cut]
    head, _, tmpl = n.partition("<")
    head = head.split("::")[-1]
    return head + ("<" + tmpl if tmpl else "")


def _bench_json(log: str):
    last = None
    with open(log) as fh:
        for line in fh:
            line = line.strip()
            if line.startswith("{") and '"metric"' in line:
                last = json.loads(line)
    return last


def stats(args) -> str:
    path = _one(args.run_dir, "kernel_stats.csv")
    rows = list(csv.DictReader(open(path)))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    out = ["# rocprofv3 kernel trace", "", "Command (from the repository root, on one MI355X):", "",
           "    " + args.command, "", "| kernel | calls | avg us | min us | max us | share % |",
           "|---|---:|---:|---:|---:|---:|"]
    for r in rows:
        out.append(f"| `{short_name(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                   f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.1f} |")
    if args.bench_log:
        b = _bench_json(args.bench_log)
        rl = (b or {}).get("roofline", {})
        if b and rl.get("launches_per_step"):
            out += ["", f"bench.py's own HIP-event timing in the same run: {1e3 * b.get('ms_per_step', 0.0):.1f} us "
                        f"per step of {rl['launches_per_step']} launches of {rl.get('kernel', '?')} "
                        f"({b.get('value')} {b.get('unit')}; {rl.get('achieved')} GB/s algorithmic)."]
        elif b:
            out += ["", f"bench.py's own HIP-event timing in the same run: {1e3 * b.get('ms_per_step', 0.0):.1f} us "
                        f"per step ({b.get('value')} {b.get('unit')})."]
    if args.window:
        name, first, count = args.window[0], int(args.window[1]), int(args.window[2])
        mean, total = window_mean_us(args.run_dir, name, first, count)
        out += ["", f"Dispatches {first} .. {first + count - 1} of {total} of `{name}` in start order (the timed "
                    f"steps): mean {mean:.1f} us per dispatch."]
    return "\n".join(out) + "\n"


def window_mean_us(directory: str, kernel: str, first: int, count: int):
    """(mean duration in us of dispatches first .. first + count - 1 of the
    kernels whose name contains `kernel`, ordered by start, number of such
    dispatches in the run)."""
    path = _one(directory, "kernel_trace.csv")
    rows = [r for r in csv.DictReader(open(path)) if kernel in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    sel = rows[first:first + count]
    if count <= 0 or len(sel) < count:
        raise SystemExit(f"{len(rows)} dispatches of {kernel}: no window [{first}, {first + count})")
    return statistics.mean((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in sel), len(rows)


def counter_by_kernel(directory: str, counter: str):
    """{short kernel name: [value per dispatch]} for one counter."""
    path = _one(directory, "counter_collection.csv")
    per = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        key = (short_name(r["Kernel_Name"]), r["Dispatch_Id"])
        per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    out = {}
    for (name, _), v in per.items():
        out.setdefault(name, []).append(v)
    return out


# what each derived metric of rocprofv3 means, for the table's legend
_METRIC_NOTES = {
    "MfmaUtil": "% of SIMD-cycles with the matrix core busy (SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE x SIMDs))",
    "LdsBankConflict": "bank-conflict cycles per LDS access cycle (SQ_LDS_BANK_CONFLICT / (SQ_LDS_IDX_ACTIVE - "
                       "SQ_LDS_BANK_CONFLICT))",
    "LDSBankConflict": "% of CU-cycles the LDS spent stalled on bank conflicts",
    "LdsUtil": "% of CU-cycles the LDS was active (SQ_LDS_IDX_ACTIVE / (GRBM_GUI_ACTIVE x CUs))",
    "MfmaFlopsBF16": "bf16 matrix-core flops per dispatch (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512)",
}


def counters(args) -> str:
    path = _one(args.run_dir, "counter_collection.csv")
    per = {}
    names = []
    for r in csv.DictReader(open(path)):
        c = r["Counter_Name"]
        if c not in names:
            names.append(c)
        per.setdefault(short_name(r["Kernel_Name"]), {}).setdefault(c, []).append(float(r["Counter_Value"]))
    out = ["# rocprofv3 counters per kernel", "", "Command (from the repository root, on one MI355X):", "",
           "    " + args.command, "", "Mean over each kernel's dispatches in the run.", "",
           "| kernel | dispatches | " + " | ".join(names) + " |", "|---|---:|" + "---:|" * len(names)]
    for kern, vals in sorted(per.items(), key=lambda kv: kv[0]):
        if all(max(v) == 0.0 for v in vals.values()):
            continue
        n = max(len(v) for v in vals.values())
        cells = []
        for c in names:
            v = statistics.mean(vals[c]) if c in vals else float("nan")
            cells.append(f"{v:.4g}")
        out.append(f"| `{kern}` | {n} | " + " | ".join(cells) + " |")
    out += [""] + [f"- {c}: {_METRIC_NOTES[c]}" for c in names if c in _METRIC_NOTES]
    return "\n".join(out) + "\n"


def _match(table, kernel: str):
    hits = [n for n in table if kernel in n]
    if not hits:
        raise SystemExit(f"kernel {kernel!r} not in {sorted(table)}")
    return hits


def traffic(args):
    fetch = counter_by_kernel(args.fetch, "FETCH_SIZE")
    write = counter_by_kernel(args.write, "WRITE_SIZE")
    known_kib = args.copy_mib * 1024.0
    cal_f = [v for n in _match(fetch, "neg") for v in fetch[n]]
    cal_w = [v for n in _match(write, "neg") for v in write[n]]
    f_factor = known_kib / statistics.mean(cal_f)
    w_factor = known_kib / statistics.mean(cal_w)
    kf = [v for n in _match(fetch, args.kernel) for v in fetch[n]]
    kw = [v for n in _match(write, args.kernel) for v in write[n]]
    fetch_b = statistics.mean(kf) * 1024.0 * f_factor
    write_b = statistics.mean(kw) * 1024.0 * w_factor
    L = args.launches_per_step
    rec = {
        "kernel": args.kernel, "stage": args.stage, "workload": args.workload, "o_dtype": args.o_dtype,
        "bytes_per_launch": round(fetch_b + write_b),
        "fetch_bytes_per_launch": round(fetch_b), "write_bytes_per_launch": round(write_b),
        "launches_per_step": L, "bytes_per_step": round(L * (fetch_b + write_b)),
        "fetch_bytes_per_step": round(L * fetch_b), "write_bytes_per_step": round(L * write_b),
        "fetch_kib_raw": statistics.mean(kf), "write_kib_raw": statistics.mean(kw), "dispatches": [len(kf), len(kw)],
        "calibration": {"copy_mib": args.copy_mib, "fetch_kib_raw": statistics.mean(cal_f),
                        "write_kib_raw": statistics.mean(cal_w), "fetch_factor": f_factor, "write_factor": w_factor},
        "source_hash": kernel_source_hash(args.stage, args.stage != "portable"),
        "commands": [args.fetch_command, args.write_command],
    }
    md = ["# HBM traffic of `" + args.kernel + "` on " + args.workload, "",
          "Two rocprofv3 counter runs (from the repository root, on one MI355X):", "",
          "    " + args.fetch_command, "    " + args.write_command, "",
          f"Calibration: the elementwise copy of {args.copy_mib} MiB that the same process runs reads "
          f"FETCH_SIZE {statistics.mean(cal_f):.0f} KiB and WRITE_SIZE {statistics.mean(cal_w):.0f} KiB for "
          f"{known_kib:.0f} KiB moved each way: factors {f_factor:.3f} (fetch) and {w_factor:.3f} (write).", "",
          "| mean per launch | raw counter (KiB) | scaled bytes | per step (x " + str(L) + ") |",
          "|---|---:|---:|---:|",
          f"| fetched | {statistics.mean(kf):.0f} | {fetch_b:.4g} | {L * fetch_b:.4g} |",
          f"| written | {statistics.mean(kw):.0f} | {write_b:.4g} | {L * write_b:.4g} |",
          f"| total | | {fetch_b + write_b:.4g} | {L * (fetch_b + write_b):.4g} |", "",
          f"Kernel sources hash {rec['source_hash']}; dispatches averaged: {len(kf)} (fetch run), {len(kw)} "
          f"(write run)."]
    with open(args.json, "w") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")
    with open(args.md, "w") as fh:
        fh.write("\n".join(md) + "\n")
    print(json.dumps({k: rec[k] for k in ("bytes_per_step", "fetch_bytes_per_step", "write_bytes_per_step")}))


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("run_dir")
    s.add_argument("--command", required=True)
    s.add_argument("--bench-log")
    s.add_argument("--window", nargs=3, metavar=("KERNEL", "FIRST", "COUNT"))
    c = sub.add_parser("counters")
    c.add_argument("run_dir")
    c.add_argument("--command", required=True)
    t = sub.add_parser("traffic")
    for a in ("--fetch", "--write", "--kernel", "--stage", "--workload", "--fetch-command", "--write-command",
              "--json", "--md"):
        t.add_argument(a, required=True)
    t.add_argument("--o-dtype", default="fp32")
    t.add_argument("--copy-mib", type=int, required=True)
    t.add_argument("--launches-per-step", type=int, default=1)
    args = ap.parse_args(argv)
    if args.cmd == "stats":
        sys.stdout.write(stats(args))
    elif args.cmd == "counters":
        sys.stdout.write(counters(args))
    else:
        traffic(args)


if __name__ == "__main__":
    main()
