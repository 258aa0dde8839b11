"""Automatic choice of algorithm and protocol (host only, no GPU).

The choice minimizes a fitted latency-plus-bandwidth time ("Collective
communication: NCCL's algorithms and protocols, and custom all-reduce",
section "Algorithms").  The fits come from the message-size sweep committed
next to the package; these tests check the fitting, the generated table,
that the library's choice is the measured fastest schedule at every swept
point, and that a fit on half of the sizes chooses well at the other half.
"""

import os

import numpy as np
import pytest

from all_reduce_reduction_rank_amd import select, tuning

ALGOS = ("oneshot", "twoshot", "ring")
PROTOS = ("simple", "ll", "ll128")


def test_fit_line_recovers_exact_alpha_and_gamma():
    b = np.array([8, 1 << 10, 1 << 20, 1 << 26, 1 << 30], dtype=np.float64)
    t = 7.5 + 2.5e-6 * b
    alpha, gamma = tuning.fit_line(b, t)
    assert alpha == pytest.approx(7.5, rel=1e-9)
    assert gamma == pytest.approx(2.5e-6, rel=1e-9)


def test_fit_line_never_negative():
    b = np.array([1e6, 2e6, 4e6])
    alpha, gamma = tuning.fit_line(b, 1e-6 * b - 0.5)  # would fit a negative latency
    assert alpha >= 0 and gamma > 0


def test_generated_table_matches_the_committed_sweep():
    fits = tuning.fit(tuning.load())
    want = tuning.header_text(fits, os.path.basename(tuning.SWEEP))
    with open(tuning.HEADER) as f:
        assert f.read() == want, "regenerate: python -m all_reduce_reduction_rank_amd.tuning header"


def test_choice_is_the_measured_fastest_at_every_swept_point():
    recs = tuning.load()
    points = {}
    for r in recs:
        key = (r.get("op", "allreduce"), r["n"], r["dtype"], r["bytes"])
        points.setdefault(key, {})[(r["algo"], r["proto"])] = tuning.device_time_us(r)
    worst, ratios = 1.0, []
    for (op, n, dt, nbytes), times in points.items():
        count = nbytes // tuning.ESIZE[dt]
        if op != "allreduce":
            count //= n  # recvcount / sendcount: the shard
        a, p, _ = select(n, op, count, dt, max_line_bytes_per_rank=1 << 40)
        if op != "allreduce" and a == "twoshot":
            a = "oneshot"  # the same direct schedule
        best = min(times.values())
        ratios.append(times[(a, p)] / best)
        worst = max(worst, ratios[-1])
    # A two-parameter line per cache band: on the committed sweep 99.2 % of
    # the 264 points pick the measured fastest and 99.6 % are within 5 %
    # (worst 1.10x, N=8 fp32 at 32 MiB, where one-shot and two-shot cross).
    assert worst <= 1.10, f"auto choice up to {worst:.2f}x the fastest measured"
    assert sum(r <= 1.05 for r in ratios) >= 0.97 * len(ratios)


def test_no_line_capacity_means_simple():
    for n in (2, 4, 8):
        for count in (2, 1 << 10, 1 << 20, 1 << 28):
            assert select(n, "allreduce", count, "bf16", max_line_bytes_per_rank=0)[1] == "simple"


def test_fixed_choices_are_kept():
    for a in ALGOS:
        for p in PROTOS:
            got = select(8, "allreduce", 1 << 20, "f32", algo=a, proto=p, max_line_bytes_per_rank=1 << 40)
            assert got[:2] == (a, p)
    assert select(8, "allreduce", 1 << 20, "f32", algo="ring")[0] == "ring"
    assert select(8, "allreduce", 1 << 20, "f32", proto="ll", max_line_bytes_per_rank=1 << 40)[1] == "ll"


def test_rank_counts_between_the_measured_ones_interpolate():
    for count in (1 << 10, 1 << 22):
        t2 = select(2, "allreduce", count, "f32", algo="twoshot", proto="simple")[2]
        t3 = select(3, "allreduce", count, "f32", algo="twoshot", proto="simple")[2]
        t4 = select(4, "allreduce", count, "f32", algo="twoshot", proto="simple")[2]
        assert min(t2, t4) <= t3 <= max(t2, t4)


@pytest.mark.parametrize("op", ["reduce_scatter", "allgather"])
def test_reduce_scatter_and_all_gather_get_a_choice(op):
    a, p, t = select(8, op, 1 << 20, "f32")
    assert a in ALGOS and p in PROTOS and t > 0


def test_int32_uses_the_four_byte_fits():
    assert select(8, "allreduce", 1 << 20, "i32")[:2] == select(8, "allreduce", 1 << 20, "f32")[:2]


def test_bad_arguments():
    from all_reduce_reduction_rank_amd.binding import ARError
    with pytest.raises(ARError):
        select(9, "allreduce", 10, "f32")


def test_choice_generalizes_to_sizes_left_out_of_the_fit():
    # Fit on the sizes 8 * 4^k with k even (and 1 GiB), then choose at the
    # sizes with k odd, which the fit never saw, and compare with what was
    # measured there ("Algorithms": the crossover points must be measured on
    # one's own machine; here the model must also predict between them).
    recs = tuning.load()
    def k_of(b):
        k = 0
        while 8 * 4 ** k < b:
            k += 1
        return k if 8 * 4 ** k == b else None
    train = [r for r in recs if k_of(r["bytes"]) is None or k_of(r["bytes"]) % 2 == 0]
    test = [r for r in recs if k_of(r["bytes"]) is not None and k_of(r["bytes"]) % 2 == 1]
    fits = tuning.fit(train)
    points = {}
    for r in test:
        key = (r.get("op", "allreduce"), r["n"], r["dtype"], r["bytes"])
        points.setdefault(key, {})[(r["algo"], r["proto"])] = tuning.device_time_us(r)
    ratios = []
    for (op, n, dt, nbytes), times in points.items():
        pick = tuning.choose(fits, op, n, tuning.ESIZE[dt], nbytes)
        assert pick is not None
        ratios.append(times[pick] / min(times.values()))
    ratios.sort()
    exact = sum(r <= 1.0 for r in ratios) / len(ratios)
    within = sum(r <= 1.10 for r in ratios) / len(ratios)
    # Measured on the committed sweep (126 held-out points): the held-out
    # choice is the fastest at 99.2 % of them (worst 1.10x, N=8 fp32 at
    # 32 MiB, where one-shot and two-shot cross).
    assert len(ratios) >= 100
    assert exact >= 0.90 and within >= 0.95 and ratios[-1] <= 1.3, (exact, within, ratios[-5:])
