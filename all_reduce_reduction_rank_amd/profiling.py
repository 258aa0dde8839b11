"""Summaries of rocprofv3 output for the collective kernels (host only).

Two summaries are made from rocprofv3's CSV output (``-f csv``):

* ``stats``: the per-kernel duration table of a ``--kernel-trace --stats``
  run, as markdown.
* ``traffic``: HBM bytes per launch from two ``--pmc`` runs of one workload
  (``FETCH_SIZE``, then ``WRITE_SIZE``; rocprofv3 reports both in KiB per
  dispatch).  The raw counters are scaled by what the same counters read for
  the library's copy kernel (one rank: read S bytes, write S bytes), so that
  the result is in bytes of the kind the algorithmic figures count.

    python -m all_reduce_reduction_rank_amd.profiling stats KERNEL_STATS_CSV --command "..."
    python -m all_reduce_reduction_rank_amd.profiling traffic --name NAME \\
        --fetch FETCH_CSV --write WRITE_CSV --copy-fetch CSV --copy-write CSV \\
        --copy-bytes S --plan-bytes B --command "..." --out profiles/traffic_NAME.json
"""

import argparse
import csv
import hashlib
import json
import os
import re
import statistics

HERE = os.path.dirname(os.path.abspath(__file__))
KERNEL = "collective_kernel"
KERNEL_SOURCES = ("csrc/kernels.hip", "csrc/device.hpp", "csrc/schedule.hpp", "csrc/plan.hpp")


def _code_only(text):
    """C++ source without comments and with whitespace collapsed: what the
    compiler sees, so that editing a comment keeps a counter summary valid.
    (The kernel sources hold no string literal with a comment marker.)"""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_hash():
    """Hash of the code the collective kernels are compiled from: a counter
    summary is valid only for the kernels it was taken on."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(HERE, rel), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def pmc_per_dispatch(path, counter, kernel=KERNEL):
    """Values of `counter` for every dispatch of kernels whose name holds
    `kernel`, in dispatch order (rocprofv3 counter_collection.csv)."""
    vals = {}
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            if kernel in row["Kernel_Name"] and row["Counter_Name"] == counter:
                d = int(row["Dispatch_Id"])
                vals[d] = vals.get(d, 0.0) + float(row["Counter_Value"])
    return [vals[d] for d in sorted(vals)]


def stats_rows(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def stats_markdown(path, command):
    rows = stats_rows(path)
    out = [f"Command (repository root, MI355X):\n\n    {command}\n",
           "| kernel | calls | avg (us) | min (us) | max (us) | share |", "|---|---:|---:|---:|---:|---:|"]
    for r in rows:
        name = r["Name"]
        if len(name) > 90:
            name = name[:87] + "..."
        out.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                   f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                   f"{float(r['Percentage']):.1f}% |")
    return "\n".join(out) + "\n"


def traffic(name, fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, copy_bytes, plan_bytes, command):
    """Counter-measured HBM bytes per launch of workload `name`.

    Every dispatch of the collective kernel in a run moves the same bytes, so
    the median over dispatches is taken (the first, cold, one included)."""
    kib = 1024.0
    fetch = statistics.median(pmc_per_dispatch(fetch_csv, "FETCH_SIZE")) * kib
    write = statistics.median(pmc_per_dispatch(write_csv, "WRITE_SIZE")) * kib
    cf = statistics.median(pmc_per_dispatch(copy_fetch_csv, "FETCH_SIZE")) * kib
    cw = statistics.median(pmc_per_dispatch(copy_write_csv, "WRITE_SIZE")) * kib
    f_scale, w_scale = copy_bytes / cf, copy_bytes / cw
    hbm = fetch * f_scale + write * w_scale
    return {
        "name": name,
        "kernel_hash": kernel_hash(),
        "fetch_bytes_raw": round(fetch),
        "write_bytes_raw": round(write),
        "copy_kernel_bytes_each_way": copy_bytes,
        "copy_fetch_raw": round(cf),
        "copy_write_raw": round(cw),
        "fetch_scale": round(f_scale, 4),
        "write_scale": round(w_scale, 4),
        "hbm_bytes_per_call": round(hbm),
        "plan_bytes_per_call": plan_bytes,
        "measured_over_plan": round(hbm / plan_bytes, 4) if plan_bytes else None,
        "command": command,
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="what", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--command", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--name", required=True)
    for k in ("fetch", "write", "copy-fetch", "copy-write"):
        t.add_argument(f"--{k}", required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--plan-bytes", type=int, required=True)
    t.add_argument("--command", required=True)
    t.add_argument("--out", required=True)
    args = ap.parse_args()
    if args.what == "stats":
        print(stats_markdown(args.csv, args.command))
    else:
        rec = traffic(args.name, args.fetch, args.write, args.copy_fetch, args.copy_write, args.copy_bytes,
                      args.plan_bytes, args.command)
        with open(args.out, "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")
        print(json.dumps(rec))


if __name__ == "__main__":
    main()
