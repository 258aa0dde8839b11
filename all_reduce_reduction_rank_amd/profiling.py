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
    python -m all_reduce_reduction_rank_amd.profiling survey --root RUNS --specs SPECS --out-dir profiles

``survey`` summarizes many workloads at once: per workload a bench JSON
line, a kernel trace and four counter runs (FETCH_SIZE, WRITE_SIZE, and the
raw read and write request counters).
"""

import argparse
import csv
import hashlib
import json
import os
import re
import statistics

HERE = os.path.dirname(os.path.abspath(__file__))
# Every collective kernel (ticketed or one workgroup per tile and rank) takes
# ar::KArgs; the fused and the ceiling kernels take other argument blocks.
KERNEL = "(ar::KArgs)"
KERNEL_SOURCES = ("csrc/kernels.hip", "csrc/device.hpp", "csrc/schedule.hpp", "csrc/plan.hpp", "csrc/rmsnorm.hip",
                  "csrc/rmsnorm.hpp", "csrc/ceiling.hip")


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


# Raw request counters behind FETCH_SIZE and WRITE_SIZE (rocprofv3 -L on
# gfx950).  FETCH_SIZE counts TCC_BUBBLE as 128-byte reads and every other
# read request as 64 bytes, but gfx950 reports its 128-byte reads in
# TCC_EA0_RDREQ_128B (TCC_BUBBLE stays near zero), so FETCH_SIZE reads half
# the bytes of a stream of 128-byte reads: the copy calibration's factor of
# 2.  Counted by request size the bytes are exact: no calibration needed.
RAW_READ = ("TCC_EA0_RDREQ_sum", "TCC_EA0_RDREQ_32B_sum", "TCC_EA0_RDREQ_64B_sum", "TCC_EA0_RDREQ_128B_sum")
RAW_WRITE = ("TCC_EA0_WRREQ_sum", "TCC_EA0_WRREQ_64B_sum")


def raw_bytes(read_csv, write_csv, kernel=KERNEL):
    """(read bytes, write bytes) per dispatch from the request counters:
    128/64/32-byte read requests, 64-byte and (the rest) 32-byte writes;
    medians over the dispatches."""
    med = lambda path, c: statistics.median(pmc_per_dispatch(path, c, kernel))  # noqa: E731
    rd = 128 * med(read_csv, "TCC_EA0_RDREQ_128B_sum") + 64 * med(read_csv, "TCC_EA0_RDREQ_64B_sum") + \
        32 * med(read_csv, "TCC_EA0_RDREQ_32B_sum")
    w64 = med(write_csv, "TCC_EA0_WRREQ_64B_sum")
    wr = 64 * w64 + 32 * (med(write_csv, "TCC_EA0_WRREQ_sum") - w64)
    return rd, wr


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


def traffic(name, fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, copy_bytes, plan_bytes, command,
            raw_read_csv=None, raw_write_csv=None, kernel=KERNEL):
    """Counter-measured HBM bytes per launch of workload `name`.

    Every dispatch of the collective kernel in a run moves the same bytes, so
    the median over dispatches is taken (the first, cold, one included).
    With the raw request-counter runs, their exact bytes are recorded too."""
    kib = 1024.0
    fetch = statistics.median(pmc_per_dispatch(fetch_csv, "FETCH_SIZE", kernel)) * kib
    write = statistics.median(pmc_per_dispatch(write_csv, "WRITE_SIZE", kernel)) * kib
    cf = statistics.median(pmc_per_dispatch(copy_fetch_csv, "FETCH_SIZE")) * kib
    cw = statistics.median(pmc_per_dispatch(copy_write_csv, "WRITE_SIZE")) * kib
    f_scale, w_scale = copy_bytes / cf, copy_bytes / cw
    hbm = fetch * f_scale + write * w_scale
    extra = {}
    if raw_read_csv and raw_write_csv:
        rd, wr = raw_bytes(raw_read_csv, raw_write_csv, kernel)
        extra = {"raw_read_bytes": round(rd), "raw_write_bytes": round(wr), "raw_hbm_bytes": round(rd + wr),
                 "raw_over_scaled": round((rd + wr) / hbm, 4) if hbm else None}
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
        **extra,
    }


PASS_COUNTERS = {  # the rocprofv3 --pmc pass of each run directory of a survey
    "fetch": "FETCH_SIZE",
    "write": "WRITE_SIZE",
    "rawr": " ".join(RAW_READ),
    "raww": " ".join(RAW_WRITE),
}


def _find(root, pattern):
    import glob
    hits = sorted(glob.glob(os.path.join(root, "**", pattern), recursive=True))
    return hits[0] if hits else None


def kernel_avg_us(stats_csv, kernel):
    for r in stats_rows(stats_csv):
        if kernel in r["Name"]:
            return float(r["AverageNs"]) / 1e3
    return None


def survey(root, specs, out_dir, copy_name="copy"):
    """Summaries of a survey: `root`/<name>/ holds, for each (name, bench
    arguments) of `specs`, the bench's JSON line (bench.json), a kernel trace
    (kt/) and four counter runs (fetch/, write/, rawr/, raww/).  Writes
    traffic_<workload>_<algo>_<proto>.json for every collective, and returns
    (counter table, kernel-trace table) as markdown."""
    cdir = os.path.join(root, copy_name)
    copy_fetch, copy_write = _find(os.path.join(cdir, "fetch"), "*counter_collection.csv"), \
        _find(os.path.join(cdir, "write"), "*counter_collection.csv")
    copy_bytes = json.load(open(os.path.join(cdir, "bench.json")))["config"]["bytes_per_rank"]
    rows, trows = [], []
    for name, args in specs:
        d = os.path.join(root, name)
        b = json.load(open(os.path.join(d, "bench.json")))
        cfg = b["config"]
        ceiling = cfg.get("reads") is not None
        kernel = "stream_kernel" if ceiling else ("rmsnorm_kernel" if cfg.get("op") == "allreduce_rmsnorm" else KERNEL)
        kt = _find(os.path.join(d, "kt"), "*kernel_stats.csv")
        avg = kernel_avg_us(kt, kernel) if kt else None
        csvs = {k: _find(os.path.join(d, k), "*counter_collection.csv") for k in PASS_COUNTERS}
        if ceiling:
            s_bytes = cfg["bytes_per_stream"]
            plan = (cfg["reads"] + cfg["writes"]) * s_bytes
            label = f"{cfg['reads']} read / {cfg['writes']} write streams"
        else:
            s_bytes = cfg["bytes_per_rank"]
            plan = b["hbm_bytes_per_call"]
            label = "fused RMSNorm (one-shot)" if cfg.get("op") == "allreduce_rmsnorm" else f"{cfg['algo']}/{cfg['proto']}"
        cmd = (f"rocprofv3 --pmc <counters> -f csv -d <dir> -o pmc -- python3 -u bench.py {args} "
               f"--steps 3 --warmup 1 --cpu-seconds 0 --no-ceiling")
        rec = traffic(name, csvs["fetch"], csvs["write"], copy_fetch, copy_write, copy_bytes, plan, cmd,
                      csvs["rawr"], csvs["raww"], kernel)
        if avg:
            rec["kernel_avg_us"] = round(avg, 2)
        if not ceiling and cfg.get("nranks", 0) > 1:
            wl = cfg["workload"]
            with open(os.path.join(out_dir, f"traffic_{wl}_{cfg['algo']}_{cfg['proto']}.json"), "w") as f:
                json.dump(rec, f, indent=1)
                f.write("\n")
        t = (avg or b["ms_per_step"] * 1e3) * 1e-6
        ceil = b.get("ceiling", {})
        rows.append(
            f"| {cfg.get('workload')} | {label} | {t * 1e6:.1f} | {plan / s_bytes:.2f} | "
            f"{rec['hbm_bytes_per_call'] / s_bytes:.2f} | {rec['raw_hbm_bytes'] / s_bytes:.2f} | "
            f"{rec['raw_read_bytes'] / s_bytes:.2f} / {rec['raw_write_bytes'] / s_bytes:.2f} | "
            f"{rec['raw_hbm_bytes'] / plan:.3f} | {plan / t / 1e12:.2f} | {rec['raw_hbm_bytes'] / t / 1e12:.2f} | "
            f"{(str(round(ceil['GBps'] / 1e3, 2)) + ' (' + str(ceil['reads']) + ':' + str(ceil['writes']) + ')') if ceil else ''} | "
            f"{b.get('ceiling_frac', '')} |")
        trows.append(f"| {cfg.get('workload')} | {label} | {avg:.2f} | {b.get('us_median', '')} | "
                     f"`rocprofv3 --kernel-trace --stats -f csv -d <dir> -o kt -- python3 -u bench.py {args} "
                     f"--steps 20 --warmup 2 --cpu-seconds 0 --no-ceiling` |" if avg else "")
    head = ("| workload | schedule | kernel us | model bytes (S) | FETCH+WRITE scaled (S) | requests (S) | "
            "read / write (S) | requests / model | model TB/s | requests TB/s | mix ceiling TB/s (r:w) | "
            "model / ceiling |\n|---|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|")
    thead = "| workload | schedule | trace avg (us) | bench median (us) | command |\n|---|---|---:|---:|---|"
    return head + "\n" + "\n".join(rows) + "\n", thead + "\n" + "\n".join(r for r in trows if r) + "\n"


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
    v = sub.add_parser("survey")
    v.add_argument("--root", required=True)
    v.add_argument("--specs", required=True, help="file of 'name|bench arguments' lines")
    v.add_argument("--out-dir", required=True)
    args = ap.parse_args()
    if args.what == "stats":
        print(stats_markdown(args.csv, args.command))
    elif args.what == "survey":
        specs = [tuple(x.strip().split("|", 1)) for x in open(args.specs) if x.strip()]
        table, traces = survey(args.root, specs, args.out_dir)
        print(table)
        print(traces)
    else:
        rec = traffic(args.name, args.fetch, args.write, args.copy_fetch, args.copy_write, args.copy_bytes,
                      args.plan_bytes, args.command)
        with open(args.out, "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")
        print(json.dumps(rec))


if __name__ == "__main__":
    main()
