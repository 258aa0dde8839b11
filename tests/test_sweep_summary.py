"""Host logic of the message-size sweep: picking the fastest schedule per
size and the crossover sizes (synthetic timings, no GPU)."""

from all_reduce_reduction_rank_amd import sweep


def _rec(nbytes, algo, proto, us, graph=None):
    r = {"n": 8, "dtype": "f32", "bytes": nbytes, "algo": algo, "proto": proto, "us_median": us}
    if graph is not None:
        r["us_graph"] = graph
    return r


def test_fastest_and_crossovers():
    recs = []
    for s, times in [(8, (5, 9, 20)), (1 << 20, (30, 25, 40)), (1 << 28, (2000, 1000, 900))]:
        for a, t in zip(sweep.ALGOS, times):
            for k, p in enumerate(sweep.PROTOS):
                recs.append(_rec(s, a, p, t + k))
    text = sweep.summary(recs)
    assert "| 8 | " in text and "oneshot/simple |" in text.split("| 8 | ")[1].split("\n")[0]
    assert "| 268435456 | " in text and text.split("| 268435456 | ")[1].split("\n")[0].endswith("ring/simple |")
    assert "- simple: oneshot from 8 B, twoshot from 1048576 B, ring from 268435456 B" in text


def test_graph_time_preferred_when_present():
    assert sweep.best_time(_rec(8, "ring", "ll", 30.0, graph=7.5)) == 7.5
    assert sweep.best_time(_rec(8, "ring", "ll", 30.0)) == 30.0


def test_sizes_cover_8_bytes_to_1_gib():
    assert sweep.SIZES[0] == 8 and sweep.SIZES[-1] == 1 << 30
    assert all(b == 4 * a for a, b in zip(sweep.SIZES[:-2], sweep.SIZES[1:-1]))
