#!/usr/bin/env python3
"""Benchmark of the all-reduce family on one MI355X.

A step is one call of the collective (one kernel: every rank program of the
call) over N simulated rank buffers already resident in HBM.  The default
workload is the gradient-bucket all-reduce: N=8 ranks, 256 MiB of fp32
N(0, 1e-3) per rank, ring, Simple protocol, 512 KiB chunks.

Prints ONE JSON line:
  value       algbw = S / t in GB/s (S = bytes per rank, t = time per call)
  busbw       algbw * 2(N-1)/N (all-reduce) or (N-1)/N (reduce-scatter,
              all-gather), the nccl-tests convention
  roofline    the call's kernel against MI355X's 8 TB/s HBM peak: achieved =
              the schedule's algorithmic HBM bytes per call / the kernel's
              average duration measured with HIP events on its stream
  cpu_baseline  the CPU oracle timed on a bounded sample of the same workload

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published

WORKLOADS = {
    # gradient buckets (N=8 fp32 N(0, 1e-3), ring, 512 KiB chunks, Simple)
    "grad-bucket-256MiB": dict(op="allreduce", nranks=8, bytes=256 << 20, dtype="f32", dist="normal_1e-3",
                               algo="ring", proto="simple", chunk=512 << 10),
    "grad-bucket-25MiB": dict(op="allreduce", nranks=8, bytes=25 << 20, dtype="f32", dist="normal_1e-3",
                              algo="ring", proto="simple", chunk=512 << 10),
    # TP activations: N=8 bf16 [tokens, 5120]
    "tp-decode-t1": dict(op="allreduce", nranks=8, bytes=1 * 5120 * 2, dtype="bf16", dist="normal",
                         algo="oneshot", proto="ll", chunk=0),
    "tp-decode-t8": dict(op="allreduce", nranks=8, bytes=8 * 5120 * 2, dtype="bf16", dist="normal",
                         algo="oneshot", proto="ll", chunk=0),
    "tp-decode-t64": dict(op="allreduce", nranks=8, bytes=64 * 5120 * 2, dtype="bf16", dist="normal",
                          algo="oneshot", proto="ll128", chunk=0),
    "tp-prefill-t512": dict(op="allreduce", nranks=8, bytes=512 * 5120 * 2, dtype="bf16", dist="normal",
                            algo="twoshot", proto="ll128", chunk=0),
    # bf16 of the same size as the fp32 bucket (N=8 N(0,1), fp32 accumulate,
    # rounded once per hop on the ring): the >= 64 MiB bandwidth target in bf16
    "bf16-256MiB": dict(op="allreduce", nranks=8, bytes=256 << 20, dtype="bf16", dist="normal",
                        algo="ring", proto="simple", chunk=512 << 10),
    # integer path: N=8 int32, 64 MiB per rank
    "int32-64MiB-ring": dict(op="allreduce", nranks=8, bytes=64 << 20, dtype="i32", dist="int20",
                             algo="ring", proto="simple", chunk=512 << 10),
    # reduce-scatter and all-gather of 256 MiB per rank (the full per-rank
    # buffer: RS sends it and keeps 1/N, AG receives it), N=8 fp32, direct
    "rs-256MiB": dict(op="reduce_scatter", nranks=8, bytes=256 << 20, dtype="f32", dist="normal",
                      algo="oneshot", proto="simple", chunk=512 << 10),
    "ag-256MiB": dict(op="allgather", nranks=8, bytes=256 << 20, dtype="f32", dist="normal",
                      algo="oneshot", proto="simple", chunk=512 << 10),
    # the same TP activations with the fused RMSNorm epilogue (residual add,
    # weight [5120]); one-shot sum
    "tp-decode-t1-rmsnorm": dict(op="allreduce_rmsnorm", nranks=8, bytes=1 * 5120 * 2, rows=1, hidden=5120,
                                 dtype="bf16", dist="normal", algo="oneshot", proto="simple", chunk=0),
    "tp-prefill-t512-rmsnorm": dict(op="allreduce_rmsnorm", nranks=8, bytes=512 * 5120 * 2, rows=512, hidden=5120,
                                    dtype="bf16", dist="normal", algo="oneshot", proto="simple", chunk=0),
    # calibration: one rank, whose all-reduce is a copy of 256 MiB (read S,
    # write S); its counter readings scale the others' to bytes
    "copy-256MiB": dict(op="allreduce", nranks=1, bytes=256 << 20, dtype="f32", dist="normal",
                        algo="ring", proto="simple", chunk=0),
    # streaming ceilings (ar_stream_ceiling): `reads` source and `writes`
    # destination streams of `bytes` each, far larger than the 256 MB MALL
    "ceiling-read": dict(op="ceiling", reads=1, writes=0, bytes=2 << 30),
    "ceiling-write": dict(op="ceiling", reads=0, writes=1, bytes=2 << 30),
    "ceiling-copy": dict(op="ceiling", reads=1, writes=1, bytes=1 << 30),
    "ceiling-add8": dict(op="ceiling", reads=8, writes=1, bytes=512 << 20),
    "ceiling-read3-write2": dict(op="ceiling", reads=3, writes=2, bytes=512 << 20),
}
CEILING_STREAM_BYTES = 512 << 20  # per stream of the ceiling run beside a collective: twice the MALL
MALL_BYTES = 256 << 20
DEFAULT_WORKLOAD = "grad-bucket-256MiB"

from all_reduce_reduction_rank_amd.profiling import kernel_hash  # noqa: E402


def mix_streams(read_bytes, write_bytes):
    """(reads, writes) streams of a ceiling run whose read:write ratio is the
    closest one to a schedule's (at most 8 reads and 2 writes)."""
    if write_bytes == 0:
        return 1, 0
    ratio = read_bytes / write_bytes
    best = None
    for wr in (1, 2):
        for rd in range(0, 9):
            err = abs(rd / wr - ratio)
            if best is None or err < best[0] - 1e-12:
                best = (err, rd, wr)
    return best[1], best[2]


def run_ceiling(reads, writes, nbytes, steps, warmup):
    """Time ar_stream_ceiling over `reads` + `writes` streams of `nbytes` in
    every configuration it offers -- plain or non-temporal loads and stores,
    4, 8 or 16 vectors per thread in flight, 1, 2, 4 or every workgroup per
    CU -- and keep the fastest: (microseconds per call, GB/s over every
    stream's bytes, the configuration)."""
    import torch

    from all_reduce_reduction_rank_amd import stream_ceiling

    src = [torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(i + 1) for i in range(reads)]
    dst = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(writes)]
    sink = torch.zeros(4, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    best = None
    for nt_l in ((False, True) if reads else (False,)):
        for nt_s in ((False, True) if writes else (False,)):
            for unroll in (4, 8, 16):
                for per_cu in (1, 2, 4, 0):
                    def once():
                        stream_ceiling(src, dst, sink, nt_l, nt_s, unroll, per_cu, stream=stream)
                    for _ in range(warmup):
                        once()
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    torch.cuda.synchronize()
                    e0.record(stream)
                    for _ in range(steps):
                        once()
                    e1.record(stream)
                    torch.cuda.synchronize()
                    us = e0.elapsed_time(e1) * 1e3 / steps
                    conf = (f"{'nt' if nt_l else 'plain'} loads, {'nt' if nt_s else 'plain'} stores, "
                            f"{unroll} in flight, {per_cu or 'all'} per CU")
                    if best is None or us < best[0]:
                        best = (us, conf)
    del src, dst
    torch.cuda.empty_cache()
    return best[0], (reads + writes) * nbytes / (best[0] * 1e-6) / 1e9, best[1]


def ceiling_main(args, w):
    """One JSON line for a streaming-ceiling workload."""
    us, gbps, hints = run_ceiling(w["reads"], w["writes"], w["bytes"], args.steps, args.warmup)
    out = {
        "metric": "all-reduce algbw/busbw GB/s and % of HBM peak vs message size, N=8",
        "value": round(gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us / 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u32",
        "data": "synthetic (constant bytes)",
        "config": {"workload": args.workload, "reads": w["reads"], "writes": w["writes"],
                   "bytes_per_stream": w["bytes"], "best_of": hints,
                   "note": "streaming-ceiling measurement aid, not a collective"},
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None},
        "kernel_hash": kernel_hash(),
    }
    print(json.dumps(out))


def busbw_factor(op, n):
    return 2 * (n - 1) / n if op in ("allreduce", "allreduce_rmsnorm") else (n - 1) / n


def fused_hbm_bytes(w):
    """Algorithmic HBM bytes of one fused all-reduce + RMSNorm call.  Each of
    the N rank programs, for each row, reads the row of the N inputs, its
    residual and the weight, and writes its residual and its output: N (N + 4) S
    with S = rows * hidden * esize per rank."""
    n, s = w["nranks"], w["bytes"]
    return n * (n + 4) * s


def counts(w):
    """(count argument of the call, input elements, output elements) per rank."""
    es = {"f32": 4, "bf16": 2, "i32": 4}[w["dtype"]]
    n = w["nranks"]
    if w["op"] in ("allreduce", "allreduce_rmsnorm"):
        return w["bytes"] // es, w["bytes"] // es, w["bytes"] // es
    per = w["bytes"] // es // n
    if w["op"] == "reduce_scatter":
        return per, n * per, per
    return per, per, n * per


def traffic_name(workload, w):
    return f"{workload}_{w['algo']}_{w['proto']}"


def traffic_from_profile(name):
    """Counter-measured HBM bytes per call from a committed rocprofv3 PMC
    summary of this workload, or None if absent or taken on other kernels."""
    path = os.path.join(ROOT, "profiles", f"traffic_{name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_hash") != kernel_hash():
        return None
    return rec.get("hbm_bytes_per_call")


def cpu_threads():
    """Host threads the threaded oracle run uses: the cores this process may
    run on, within the CPU share the environment grants (OMP_NUM_THREADS,
    when set: a shared GPU host gives each GPU's jobs a share of its cores)."""
    try:
        cores = max(1, len(os.sched_getaffinity(0)))
    except AttributeError:
        cores = max(1, os.cpu_count() or 1)
    share = os.environ.get("OMP_NUM_THREADS", "")
    return max(1, min(cores, int(share))) if share.isdigit() and int(share) > 0 else cores


def host_ram_bytes():
    try:
        return os.sysconf("SC_PAGE_SIZE") * os.sysconf("SC_PHYS_PAGES")
    except (ValueError, OSError, AttributeError):
        return 0


def split_parts(w, host, parts, blocks):
    """`parts` disjoint reduced problems that together are the whole call:
    part t holds the t-th piece of every block (all-reduce: the N blocks, the
    tree's two halves; reduce-scatter: every rank's N slices; all-gather:
    every rank's shard), so every element keeps its block and its summation
    order.  None when the blocks are not all of one length (then the call is
    not split).  Pieces are whole 16-byte vectors."""
    import numpy as np

    es = {"f32": 4, "bf16": 2, "i32": 4}[w["dtype"]]
    vec = 16 // es
    lens = {hi - lo for lo, hi in blocks}
    if len(lens) != 1:
        return None
    blen = lens.pop()
    piece = max(vec, -(-blen // parts // vec) * vec)
    out = []
    for a in range(0, blen, piece):
        b = min(blen, a + piece)
        if (b - a) % vec and w["op"] == "allreduce":
            return None  # all-reduce blocks are whole vectors: a reduced problem must keep them so
        idx = np.concatenate([np.arange(lo + a, lo + b) for lo, _ in blocks])
        out.append([x[idx] for x in host])
    return out


def cpu_baseline_threaded(w, threads, runs=3):
    """One oracle call split over `threads` host threads: each thread runs the
    oracle as it stands on its own disjoint piece of every block (NumPy
    releases the GIL in its loops), so together they compute the whole call
    once.  The workload's full size when its inputs and outputs fit in a
    quarter of host memory, else 256 MiB per rank.  Median of `runs`; the
    split itself is done before the clock starts."""
    from concurrent.futures import ThreadPoolExecutor

    from all_reduce_reduction_rank_amd import inputs
    from oracle import collectives, fused, geometry

    es = {"f32": 4, "bf16": 2, "i32": 4}[w["dtype"]]
    n = w["nranks"]
    size = w["bytes"]
    ram = host_ram_bytes()
    if ram and 3 * n * size > ram // 4:
        size = min(size, 256 << 20)
    if w["op"] == "allreduce_rmsnorm":
        rows, hidden = size // (w["hidden"] * es), w["hidden"]
        host = inputs.rank_inputs(n, rows * hidden, w["dtype"], w["dist"], seed=1, cfg=9)
        res = inputs.rank_inputs(n, rows * hidden, w["dtype"], w["dist"], seed=1001, cfg=9)
        weight = inputs.rank_inputs(1, hidden, w["dtype"], w["dist"], seed=3, cfg=9)[0]
        per = -(-rows // threads)
        jobs = []
        for r0 in range(0, rows, per):
            r1 = min(rows, r0 + per)
            sl = slice(r0 * hidden, r1 * hidden)
            jobs.append(lambda sl=sl, k=r1 - r0: fused.allreduce_rmsnorm(
                [x[sl] for x in host], [x[sl].copy() for x in res], weight, k, hidden, 1e-5, w["dtype"]))
    else:
        count = size // es
        if w["op"] == "allreduce":
            host = inputs.rank_inputs(n, count, w["dtype"], w["dist"], seed=1, cfg=9)
            halves = w["algo"] == "tree"
            blocks = geometry.ar_blocks(count, 2 if halves else n, w["dtype"])
            fn = collectives.allreduce
        elif w["op"] == "reduce_scatter":
            rc = count // n
            host = inputs.rank_inputs(n, n * rc, w["dtype"], w["dist"], seed=1, cfg=9)
            blocks = [(j * rc, (j + 1) * rc) for j in range(n)]
            fn = collectives.reduce_scatter
        else:
            sc = count // n
            host = inputs.rank_inputs(n, sc, w["dtype"], w["dist"], seed=1, cfg=9)
            blocks = [(0, sc)]
            fn = collectives.allgather
        parts = split_parts(w, host, threads, blocks) or [host]
        chunk = w["chunk"] or collectives.DEFAULT_CHUNK_BYTES
        jobs = [lambda p=p: fn(p, w["dtype"], w["algo"], chunk_bytes=chunk) for p in parts]
    times = []
    with ThreadPoolExecutor(threads) as pool:
        for _ in range(runs):
            t0 = time.perf_counter()
            list(pool.map(lambda job: job(), jobs))
            times.append(time.perf_counter() - t0)
    t = sorted(times)[len(times) // 2]
    return {
        "value": round(size / t / 1e9, 4),
        "unit": "GB/s",
        "cores": min(threads, len(jobs)),
        "kind": "oracle",
        "sample": f"{w['op']} {w['algo']} N={n} {w['dtype']} {w['dist']}, {size / 2**20:.4g} MiB per rank, "
                  f"one call split over {len(jobs)} disjoint piece(s) of every block on {min(threads, len(jobs))} "
                  f"threads, median of {runs} runs ({', '.join(f'{x:.3f}' for x in times)} s)",
    }


def cpu_baseline(w, min_seconds, seed=1):
    """The oracle as it stands, on a bounded sample: the same collective on
    the same N and distribution, 32 MiB per rank (or the workload's size if
    smaller), repeated until `min_seconds` have passed."""
    from all_reduce_reduction_rank_amd import inputs
    from oracle import collectives

    es = {"f32": 4, "bf16": 2, "i32": 4}[w["dtype"]]
    n = w["nranks"]
    if w["op"] == "allreduce_rmsnorm":
        from oracle import fused

        rows = max(1, min(w["rows"], 64))  # a bounded sample of the rows
        sample_bytes = rows * w["hidden"] * es
        host = inputs.rank_inputs(n, rows * w["hidden"], w["dtype"], w["dist"], seed=seed, cfg=9)
        res = inputs.rank_inputs(n, rows * w["hidden"], w["dtype"], w["dist"], seed=seed + 1000, cfg=9)
        weight = inputs.rank_inputs(1, w["hidden"], w["dtype"], w["dist"], seed=3, cfg=9)[0]

        def fn(x, dt, algo, chunk_bytes=0):
            fused.allreduce_rmsnorm(x, res, weight, rows, w["hidden"], 1e-5, dt)
    else:
        sample_bytes = min(w["bytes"], 32 << 20)
        per = sample_bytes // es
        if w["op"] != "allreduce":
            per //= n
        host = inputs.rank_inputs(n, per if w["op"] != "reduce_scatter" else n * per, w["dtype"], w["dist"],
                                  seed=seed, cfg=9)
        fn = {"allreduce": collectives.allreduce, "reduce_scatter": collectives.reduce_scatter,
              "allgather": collectives.allgather}[w["op"]]
    reps, t0 = 0, time.perf_counter()
    while True:
        fn(host, w["dtype"], w["algo"], chunk_bytes=w["chunk"] or collectives.DEFAULT_CHUNK_BYTES)
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds:
            break
    return {
        "_bytes": sample_bytes * reps,
        "value": round(sample_bytes * reps / el / 1e9, 4),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{w['op']} {w['algo']} N={n} {w['dtype']} {w['dist']}, {sample_bytes / 2**20:.3g} MiB per rank, "
                  f"{reps} calls in {el:.1f} s (NumPy, single thread)",
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(WORKLOADS))
    ap.add_argument("--algo", choices=("oneshot", "twoshot", "ring", "tree", "auto"))
    ap.add_argument("--proto", choices=("simple", "ll", "ll128", "auto"))
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="oracle sample length; 0 skips it")
    ap.add_argument("--no-ceiling", dest="ceiling", action="store_false",
                    help="skip the streaming-ceiling run beside the collective")
    ap.add_argument("--max-workgroups", type=int, default=0,
                    help="workgroup budget of the collective's kernel (0: the default, up to 3 per CU)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU: the N ranks are simulated inside one MI355X "
              f"(--gpus {args.gpus} is not supported).", file=sys.stderr)
        sys.exit(2)

    import torch

    from all_reduce_reduction_rank_amd import Comm, inputs, plan_bytes, select

    w = dict(WORKLOADS[args.workload])
    if w["op"] == "ceiling":
        torch.cuda.set_device(0)
        ceiling_main(args, w)
        return
    if args.algo:
        w["algo"] = args.algo
    if args.proto:
        w["proto"] = args.proto
    n, dt, op = w["nranks"], w["dtype"], w["op"]
    torch.cuda.set_device(0)
    count, n_in, n_out = counts(w)
    auto = "auto" in (w["algo"], w["proto"])
    line_cap = w["bytes"] if w["proto"] != "simple" else 0
    req_algo, req_proto = w["algo"], w["proto"]  # what each timed call asks for
    if auto:  # the library's choice (ar_select), resolved here for the report
        w["algo"], w["proto"], _ = select(n, op, count, dt, w["algo"], w["proto"], line_cap)
    send = inputs.device_rank_inputs(n, n_in, dt, w["dist"], seed=0, cfg=4)
    recv = [torch.empty(n_out, dtype=send[0].dtype, device="cuda") for _ in range(n)]
    comm = Comm(n, w["bytes"], line_cap if op != "allreduce_rmsnorm" else 0)
    if args.max_workgroups:
        comm.set_max_workgroups(args.max_workgroups)
    stream = torch.cuda.current_stream()
    if op == "allreduce_rmsnorm":
        rows, hidden = w["rows"], w["hidden"]
        send = [t.view(rows, hidden) for t in send]
        recv = [t.view(rows, hidden) for t in recv]
        residual = [t.view(rows, hidden) for t in inputs.device_rank_inputs(n, n_in, dt, w["dist"], seed=1, cfg=4)]
        weight = inputs.device_rank_inputs(1, hidden, dt, w["dist"], seed=2, cfg=4)[0]

        def call(s_, r_, algo=None, proto=None, chunk_bytes=0, stream=None):
            comm.allreduce_rmsnorm(s_, r_, weight, eps=1e-5, residual=residual, stream=stream)
    else:
        call = getattr(comm, op)

    def step():
        call(send, recv, algo=req_algo, proto=req_proto, chunk_bytes=w["chunk"], stream=stream)

    for _ in range(args.warmup):
        step()
    status = comm.check()
    if status[0] != "AR_OK":
        raise SystemExit(f"device error during warm-up: {status}")
    print(f"[bench] {args.workload}: warmup {args.warmup} done", file=sys.stderr, flush=True)
    # one HIP event before every call and one after the last, all on the
    # stream the kernels run on: the total gives the mean, the gaps each call
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for i in range(args.steps):
        evs[i].record(stream)
        step()
    evs[-1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    status = comm.check()
    if status[0] != "AR_OK":
        raise SystemExit(f"device error during the timed region: {status}")
    ms = evs[0].elapsed_time(evs[-1]) / args.steps
    per_call = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
    print(f"[bench] timed {args.steps} steps: {ms:.4f} ms per call (wall {wall:.3f} s)", file=sys.stderr, flush=True)

    us_graph = None
    if w["bytes"] < (1 << 20):
        # Small calls are latency-bound: a HIP graph of 100 captured calls,
        # replayed, times the device side without the host's launch cost.
        side = torch.cuda.Stream()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            for _ in range(100):
                call(send, recv, algo=req_algo, proto=req_proto, chunk_bytes=w["chunk"], stream=side)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(side):  # replay() launches on the current stream
            g.replay()
            torch.cuda.synchronize()
            e0.record(side)
            g.replay()
            e1.record(side)
        torch.cuda.synchronize()
        us_graph = round(e0.elapsed_time(e1) * 1e3 / 100, 2)
        status = comm.check()
        if status[0] != "AR_OK":
            raise SystemExit(f"device error during the graph replays: {status}")

    s = w["bytes"]
    t = ms / 1e3
    if op == "allreduce_rmsnorm":
        plan = {"hbm": fused_hbm_bytes(w), "read": n * (n + 2) * w["bytes"], "write": 2 * n * w["bytes"]}
    else:
        plan = plan_bytes(n, op, count, dt, w["algo"], w["proto"], chunk_bytes=w["chunk"])
    algbw = s / t / 1e9
    achieved = plan["hbm"] / t / 1e9
    traffic = traffic_from_profile(traffic_name(args.workload, w))
    out = {
        "metric": "all-reduce algbw/busbw GB/s and % of HBM peak vs message size, N=8",
        "value": round(algbw, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dt,
        "data": "synthetic (seeded, generated on the GPU)",
        "config": {
            "workload": args.workload, "op": op, "nranks": n, "bytes_per_rank": s, "dtype": dt,
            "dist": w["dist"], "algo": w["algo"], "proto": w["proto"], "chunk_bytes": w["chunk"],
            "selection": "auto" if auto else "fixed",
            "max_workgroups": args.max_workgroups or "default",
            "parallelism": f"{n} simulated ranks on 1 GPU",
        },
        "us_median": round(per_call[len(per_call) // 2] * 1e3, 2),
        "us_min": round(per_call[0] * 1e3, 2),
        "us_graph": us_graph,
        "cache_resident": 2 * n * s < 2 * MALL_BYTES,
        "algbw_GBps": round(algbw, 3),
        "busbw_GBps": round(algbw * busbw_factor(op, n), 3),
        "hbm_bytes_per_call": plan["hbm"],
        # HBM bytes per byte of payload (N ranks x S): the schedule's model
        "hbm_bytes_per_payload_byte": round(plan["hbm"] / (n * s), 4),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
        },
        "kernel_hash": kernel_hash(),
        # what the counters behind `traffic` count: requests from the XCDs' L2
        # caches to the data fabric; the 256 MB MALL sits behind them, so a
        # hit there counts like an HBM access (no memory-side counter is
        # exposed on gfx950)
        "traffic_level": "L2-to-fabric requests (TCC_EA), MALL hits included",
    }
    if args.ceiling:
        # the practical ceiling for this schedule's mix of reads and writes:
        # a pure streaming kernel with the closest read:write ratio, on
        # streams of twice the MALL, timed in the same run
        rd, wrs = mix_streams(plan["read"], plan["write"])
        c_us, c_gbps, c_hints = run_ceiling(rd, wrs, CEILING_STREAM_BYTES, 5, 1)
        out["ceiling"] = {"reads": rd, "writes": wrs, "bytes_per_stream": CEILING_STREAM_BYTES, "best_of": c_hints,
                          "schedule_read_write_ratio": round(plan["read"] / max(1, plan["write"]), 3),
                          "GBps": round(c_gbps, 1), "frac_of_peak": round(c_gbps / HBM_PEAK_GBPS, 4)}
        out["ceiling_frac"] = round(achieved / c_gbps, 4)
    if traffic:
        out["hbm_measured_GBps"] = round(traffic / t / 1e9, 1)
        out["hbm_measured_frac"] = round(traffic / t / 1e9 / HBM_PEAK_GBPS, 4)
        out["hbm_measured_bytes_per_payload_byte"] = round(traffic / (n * s), 4)
    if args.cpu_seconds > 0:
        # the oracle as it stands on one thread, then one call split over
        # every usable core
        base = cpu_baseline(w, args.cpu_seconds / 2)
        base.pop("_bytes")
        out["cpu_baseline"] = base
        out["cpu_baseline_threads"] = cpu_baseline_threaded(w, cpu_threads())
    comm.close()
    print(json.dumps(out))


if __name__ == "__main__":
    main()
