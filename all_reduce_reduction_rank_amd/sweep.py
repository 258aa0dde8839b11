"""Message-size sweep of the all-reduce: every algorithm x protocol, per N and
dtype, timed with HIP events on the launch stream.

Sizes are 8 B * 4^k (k = 0..13) plus 1 GiB per rank, the range nccl-tests'
``-b 8 -e 1G`` covers.  Inputs are N(0, 1) drawn on the GPU once per (N,
dtype) at the largest size; smaller sizes use prefixes of the same buffers.
Each point is timed over at least 20 calls and 200 ms after 2 warm-up calls
(one event per call: median and minimum), and below 1 MiB also as a replay
of a HIP graph of 100 captured calls, which removes the host's launch cost.

    python -m all_reduce_reduction_rank_amd.sweep run --out sweep.jsonl [--op allreduce] [--n 2 4 8] [--dtype bf16 f32]
    python -m all_reduce_reduction_rank_amd.sweep summary sweep.jsonl

``run`` writes one JSON object per point as it goes; ``summary`` prints the
fastest schedule per size and the crossover sizes as markdown (host only).
"""

import argparse
import json
import math
import sys
import time

SIZES = [8 * 4 ** k for k in range(14)] + [1 << 30]
ALGOS = ("oneshot", "twoshot", "ring", "tree")
PROTOS = ("simple", "ll", "ll128")


def combos(op):
    """(algorithm, protocol) pairs a sweep of `op` times.  For reduce-scatter
    and all-gather one-shot and two-shot name the same direct schedule; the
    tree is an all-reduce schedule with Simple only."""
    if op != "allreduce":
        return [(a, p) for a in ("oneshot", "ring") for p in PROTOS]
    return [(a, p) for a in ("oneshot", "twoshot", "ring") for p in PROTOS] + [("tree", "simple")]
ESIZE = {"f32": 4, "bf16": 2, "i32": 4}
MALL_BYTES = 256 << 20


def _time_calls(call, stream, min_calls=20, min_seconds=0.2):
    import torch

    for _ in range(2):
        call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    call()
    torch.cuda.synchronize()
    est = max(time.perf_counter() - t0, 1e-6)
    k = int(min(5000, max(min_calls, math.ceil(min_seconds / est))))
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(k + 1)]
    for i in range(k):
        evs[i].record(stream)
        call()
    evs[-1].record(stream)
    torch.cuda.synchronize()
    per = sorted(evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(k))
    mean = evs[0].elapsed_time(evs[-1]) * 1e3 / k
    return {"calls": k, "us_mean": mean, "us_median": per[k // 2], "us_min": per[0]}


def _time_graph(call, stream, reps=100):
    import torch

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for _ in range(reps):
            call()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    del g
    return e0.elapsed_time(e1) * 1e3 / reps


def run(out_path, ns, dtypes, sizes=SIZES, graphs=True, op="allreduce"):
    """Time every (algorithm, protocol) at every size.  S = `bytes` is the
    full per-rank buffer: a reduce-scatter sends S and keeps S/N, an
    all-gather sends S/N and receives S (sizes whose shard is under one
    element are skipped).  For reduce-scatter and all-gather one-shot and
    two-shot name the same direct schedule, so only one-shot is timed."""
    import torch

    from . import Comm, inputs

    torch.cuda.set_device(0)
    with open(out_path, "a") as out:
        for n in ns:
            for dt in dtypes:
                es = ESIZE[dt]
                top = max(sizes)
                send = inputs.device_rank_inputs(n, top // es, dt, "normal", seed=0, cfg=5)
                recv = [torch.empty_like(t) for t in send]
                comm = Comm(n, top, top)
                side = torch.cuda.Stream()
                for nbytes in sizes:
                    full = nbytes // es
                    shard = full // n
                    if op == "allreduce":
                        count, s_in, s_out = full, [t[:full] for t in send], [t[:full] for t in recv]
                    elif shard == 0:
                        continue
                    elif op == "reduce_scatter":
                        count, s_in, s_out = shard, [t[:n * shard] for t in send], [t[:shard] for t in recv]
                    else:
                        count, s_in, s_out = shard, [t[:shard] for t in send], [t[:n * shard] for t in recv]
                    fn = getattr(comm, op)
                    for algo, proto in combos(op):
                        def call():
                            fn(s_in, s_out, algo=algo, proto=proto, stream=side)

                        with torch.cuda.stream(side):
                            rec = _time_calls(call, side)
                            if graphs and nbytes < (1 << 20):
                                rec["us_graph"] = _time_graph(call, side)
                        st = comm.check(side)
                        if st[0] != "AR_OK":
                            raise SystemExit(f"device error at {op} N={n} {dt} {nbytes} B {algo}/{proto}: {st}")
                        rec.update(op=op, n=n, dtype=dt, bytes=nbytes, algo=algo, proto=proto,
                                   cache_resident=2 * n * nbytes < 2 * MALL_BYTES)
                        out.write(json.dumps(rec) + "\n")
                        out.flush()
                    print(f"[sweep] {op} N={n} {dt} {nbytes} B done", file=sys.stderr, flush=True)
                comm.close()
                del send, recv, s_in, s_out
                torch.cuda.empty_cache()


def load(path):
    with open(path) as f:
        return [json.loads(line) for line in f if line.strip()]


def best_time(rec):
    """Time of one call: the graph replay below 1 MiB (no host launch cost),
    else the median of the eager calls."""
    return rec.get("us_graph", rec["us_median"])


def summary(recs, table_ranks=None):
    """Markdown: per (operation, N, dtype) the crossover sizes, and the full
    timing table where N is in `table_ranks` (None: every N)."""
    lines = []
    keys = sorted({(r.get("op", "allreduce"), r["n"], r["dtype"]) for r in recs})
    for op, n, dt in keys:
        rows = [r for r in recs if r.get("op", "allreduce") == op and r["n"] == n and r["dtype"] == dt]
        sizes = sorted({r["bytes"] for r in rows})
        cols = [c for c in combos(op) if any((r["algo"], r["proto"]) == c for r in rows)]
        lines.append(f"\n### {op}, N={n}, {dt} (µs per call)\n")
        if table_ranks is None or n in table_ranks:
            lines.append("(MALL: yes when the call's inputs and outputs, 2 N S, fit in twice the 256 MB "
                         "last-level cache, so repeated calls run largely from it; those rows are not HBM-bound.)\n")
            lines.append("| bytes/rank | MALL | " + " | ".join(f"{a}/{p}" for a, p in cols) + " | fastest |")
            lines.append("|---:|---|" + "---:|" * len(cols) + "---|")
        for s in sizes:
            if table_ranks is not None and n not in table_ranks:
                break
            t = {(r["algo"], r["proto"]): best_time(r) for r in rows if r["bytes"] == s}
            resident = any(r.get("cache_resident") for r in rows if r["bytes"] == s)
            fast = min(t, key=t.get)
            cells = [f"{t[c]:.1f}" if c in t else "" for c in cols]
            lines.append(f"| {s} | {'yes' if resident else 'no'} | " + " | ".join(cells) + f" | {fast[0]}/{fast[1]} |")
        lines.append("")
        t_all = {}
        for r in rows:
            t_all.setdefault(r["bytes"], {})[(r["algo"], r["proto"])] = best_time(r)
        prev, cross = None, []
        for s in sizes:
            k = min(t_all[s], key=t_all[s].get)
            if k != prev:
                cross.append(f"{k[0]}/{k[1]} from {s} B")
                prev = k
        lines.append("- fastest overall: " + ", ".join(cross))
        for p in PROTOS:
            prev, cross = None, []
            for s in sizes:
                t = {r["algo"]: best_time(r) for r in rows if r["bytes"] == s and r["proto"] == p}
                a = min(t, key=t.get)
                if a != prev:
                    cross.append(f"{a} from {s} B")
                    prev = a
            lines.append(f"- {p}: " + ", ".join(cross))
    return "\n".join(lines) + "\n"


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="what", required=True)
    r = sub.add_parser("run")
    r.add_argument("--out", required=True)
    r.add_argument("--n", type=int, nargs="+", default=[2, 4, 8])
    r.add_argument("--dtype", nargs="+", default=["bf16", "f32"])
    r.add_argument("--max-bytes", type=int, default=1 << 30)
    r.add_argument("--no-graphs", action="store_true")
    r.add_argument("--op", default="allreduce", choices=("allreduce", "reduce_scatter", "allgather"))
    s = sub.add_parser("summary")
    s.add_argument("path")
    s.add_argument("--tables", type=int, nargs="*", help="rank counts that get a full table (default: all)")
    args = ap.parse_args()
    if args.what == "run":
        run(args.out, args.n, args.dtype, [x for x in SIZES if x <= args.max_bytes], graphs=not args.no_graphs,
            op=args.op)
    else:
        print(summary(load(args.path), args.tables))


if __name__ == "__main__":
    main()
