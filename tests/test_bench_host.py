"""Host logic of bench.py (no GPU): workload sizes, byte models and the
one-GPU contract."""

import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_counts_per_operation():
    w = dict(op="allreduce", nranks=8, bytes=1 << 20, dtype="f32")
    assert bench.counts(w) == (1 << 18, 1 << 18, 1 << 18)
    w = dict(op="reduce_scatter", nranks=8, bytes=1 << 20, dtype="bf16")
    assert bench.counts(w) == (1 << 16, 1 << 19, 1 << 16)
    w = dict(op="allgather", nranks=4, bytes=1 << 20, dtype="i32")
    assert bench.counts(w) == (1 << 16, 1 << 16, 1 << 18)


def test_every_workload_is_well_formed():
    for name, w in bench.WORKLOADS.items():
        if w["op"] == "ceiling":
            assert 0 <= w["reads"] <= 8 and 0 <= w["writes"] <= 2 and w["reads"] + w["writes"] > 0, name
            assert w["bytes"] % 16 == 0 and w["bytes"] >= 2 * bench.MALL_BYTES, name
            continue
        count, n_in, n_out = bench.counts(w)
        assert count > 0 and n_in > 0 and n_out > 0, name
        if w["op"] == "allreduce_rmsnorm":
            assert w["rows"] * w["hidden"] * 2 == w["bytes"], name
            assert bench.fused_hbm_bytes(w) == w["nranks"] * (w["nranks"] + 4) * w["bytes"]


def test_busbw_factors():
    assert bench.busbw_factor("allreduce", 8) == 2 * 7 / 8
    assert bench.busbw_factor("allgather", 8) == 7 / 8


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode == 2 and "one GPU" in res.stderr


def test_kernel_hash_is_stable():
    assert bench.kernel_hash() == bench.kernel_hash() and len(bench.kernel_hash()) == 16


def test_kernel_hash_ignores_comments_and_layout():
    from all_reduce_reduction_rank_amd import profiling
    code = "int f(int x) {\n  return x + 1;  // one more\n}\n"
    edited = "/* a note */\nint f(int x)   {\n  return x + 1;  // one more, said again\n}\n"
    changed = "int f(int x) {\n  return x + 2;\n}\n"
    assert profiling._code_only(code) == profiling._code_only(edited)
    assert profiling._code_only(code) != profiling._code_only(changed)


def test_threaded_baseline_split_is_the_whole_call():
    # The pieces the threaded baseline hands to its threads, put back in
    # place, give exactly the oracle's result on the whole call.
    import numpy as np

    from all_reduce_reduction_rank_amd import inputs
    from oracle import collectives, geometry

    for algo in ("ring", "twoshot", "oneshot", "tree"):
        w = dict(op="allreduce", nranks=4, bytes=4 * 4 * 8 * 25, dtype="f32", algo=algo, chunk=0)
        count = w["bytes"] // 4
        host = inputs.rank_inputs(4, count, "f32", "normal", seed=2, cfg=9)
        blocks = geometry.ar_blocks(count, 2 if algo == "tree" else 4, "f32")
        parts = bench.split_parts(w, host, 3, blocks)
        assert parts is not None and len(parts) == 3
        whole = collectives.allreduce(host, "f32", algo)
        blen = blocks[0][1] - blocks[0][0]
        piece = -(-blen // 3 // 4) * 4
        for t, p in enumerate(parts):
            got = collectives.allreduce(p, "f32", algo)
            a, b = t * piece, min(blen, (t + 1) * piece)
            idx = np.concatenate([np.arange(lo + a, lo + b) for lo, _ in blocks])
            for r in range(4):
                assert np.array_equal(got[r].view(np.uint32), whole[r][idx].view(np.uint32)), (algo, t, r)


def test_threaded_baseline_runs_small():
    w = dict(op="reduce_scatter", nranks=4, bytes=1 << 16, dtype="bf16", dist="normal", algo="ring", chunk=0)
    rec = bench.cpu_baseline_threaded(w, 4, runs=1)
    assert rec["kind"] == "oracle" and rec["cores"] == 4 and rec["value"] > 0


def test_mix_streams_matches_schedule_ratios():
    assert bench.mix_streams(21, 14) == (3, 2)      # ring: 21 S read, 14 S written
    assert bench.mix_streams(8, 1) == (8, 1)        # direct reduce-scatter
    assert bench.mix_streams(1, 1) == (1, 1)
    assert bench.mix_streams(5, 0) == (1, 0)        # nothing written: a read stream
    r, w = bench.mix_streams(15, 8)                 # two-shot: 15 S read, 8 S written
    assert abs(r / w - 15 / 8) <= 0.125
