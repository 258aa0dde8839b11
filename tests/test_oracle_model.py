"""Pins of the oracle's bf16 conversion, line codecs, cost model, byte tallies
and signal graph against what the pages print and what arithmetic fixes."""

import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import bf16, cost, proto, sim, traffic

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------ bf16
def test_bf16_narrow_matches_torch_on_random_values():
    # An independent library routine: torch's CPU float32 -> bfloat16 cast
    # (round to nearest even).
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 2 ** 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    finite = np.isfinite(f)
    ours = bf16.narrow_rne(f[finite])
    theirs = torch.from_numpy(f[finite].copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)


def test_bf16_narrow_matches_torch_on_every_tie():
    # Every high half with the low half exactly 0x8000 (a tie), plus the
    # neighbours 0x7FFF and 0x8001.
    hi = np.arange(0, 2 ** 16, dtype=np.uint32) << np.uint32(16)
    for low in (0x7FFF, 0x8000, 0x8001):
        f = (hi | np.uint32(low)).view(np.float32)
        keep = np.isfinite(f)
        ours = bf16.narrow_rne(f[keep])
        theirs = torch.from_numpy(f[keep].copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(ours, theirs), hex(low)


def test_bf16_specials():
    f = np.array([np.inf, -np.inf, 0.0, -0.0, np.nan, 0.0, 1e-40], dtype=np.float32)
    f[5] = np.array([0x7F7F8000], dtype=np.uint32).view(np.float32)[0]  # tie above max bf16
    out = bf16.narrow_rne(f)
    assert out[0] == 0x7F80 and out[1] == 0xFF80
    assert out[2] == 0x0000 and out[3] == 0x8000
    assert (out[4] & 0x7F80) == 0x7F80 and (out[4] & 0x0040)  # quiet NaN
    assert out[5] == 0x7F80  # rounds past the largest finite bf16
    assert out[6] != 0       # subnormal kept
    neg_nan = np.array([0xFFC00001], dtype=np.uint32).view(np.float32)
    assert bf16.narrow_rne(neg_nan)[0] == 0xFFC0


def test_bf16_widen_is_exact():
    bits = np.arange(0, 2 ** 16, dtype=np.uint32).astype(np.uint16)
    ours = bf16.widen(bits)
    theirs = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    same = (ours == theirs) | (np.isnan(ours) & np.isnan(theirs))
    assert same.all()


def test_ulp_distance():
    assert bf16.ulp_distance(np.array([0x3F80]), np.array([0x3F81]))[0] == 1
    assert bf16.ulp_distance(np.array([0x0000]), np.array([0x8000]))[0] == 0
    assert bf16.ulp_distance(np.array([0x0001]), np.array([0x8001]))[0] == 2


# ---------------------------------------------------------------- codecs
@pytest.mark.parametrize("nbytes", [0, 1, 4, 7, 119, 120, 121, 240, 1000, 4096])
def test_ll_round_trip_and_size(nbytes):
    rng = np.random.default_rng(nbytes)
    payload = rng.integers(0, 256, nbytes, dtype=np.uint8)
    lines = proto.ll_pack(payload, 0xABCD1234)
    assert len(lines) == 8 * -(-nbytes // 4)
    assert np.array_equal(proto.ll_unpack(lines, 0xABCD1234, nbytes), payload)
    l128 = proto.ll128_pack(payload, 0x1122334455667788)
    assert len(l128) == 128 * -(-nbytes // 120)
    assert np.array_equal(proto.ll128_unpack(l128, 0x1122334455667788, nbytes), payload)


def test_line_layout():
    payload = np.arange(1, 9, dtype=np.uint8)
    ll = proto.ll_pack(payload, 0x01020304)
    assert list(ll[:8]) == [1, 2, 3, 4, 4, 3, 2, 1]  # data then little-endian flag
    l128 = proto.ll128_pack(np.arange(120, dtype=np.uint8), 7)
    assert list(l128[:120]) == list(range(120)) and list(l128[120:]) == [7, 0, 0, 0, 0, 0, 0, 0]


def test_stale_line_is_detected():
    lines = proto.ll_pack(np.zeros(16, np.uint8), 5)
    lines[8 * 2 + 4] = 4  # line 2 carries the previous call's flag
    with pytest.raises(ValueError, match="line 2"):
        proto.ll_unpack(lines, 5, 16)
    with pytest.raises(ValueError):
        proto.ll_pack(np.zeros(4, np.uint8), 0)


def test_protocol_efficiencies_match_page():
    # "Protocols" table: LL about 50 %, LL128 about 94 %, Simple close to 100 %.
    big = 120 * 4 * 1000
    assert proto.efficiency(big, "ll") == 0.5
    assert proto.efficiency(big, "ll128") == 120 / 128 and round(100 * 120 / 128) == 94
    assert proto.efficiency(big, "simple") == 1.0


# ------------------------------------------------------------ cost model
def _golden_table():
    rows, ring = [], None
    with open(os.path.join(GOLDEN, "alphabeta_table_n8.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            parts = line.split()
            if parts[0] == "RING1GIB":
                ring = tuple(float(p) for p in parts[1:])
            else:
                rows.append((int(parts[0]), [float(p) for p in parts[1:6]], parts[6]))
    return rows, ring


def test_alpha_beta_table_reproduces_printed_values():
    rows, _ = _golden_table()
    assert len(rows) == 5
    for nbytes, printed, fastest in rows:
        for algo, want in zip(cost.MODEL_ALGOS, printed):
            us = cost.model_time(algo, nbytes, cost.N_PAGE, cost.ALPHA_PAGE, cost.BETA_PAGE) * 1e6
            assert f"{us:.1f}" == f"{want:.1f}", (nbytes, algo, us, want)
        assert cost.fastest_without_nvls(nbytes, cost.N_PAGE, cost.ALPHA_PAGE, cost.BETA_PAGE) == fastest


def test_one_gib_ring_line():
    _, (ms, alg, bus) = _golden_table()
    s = 1 << 30
    t = cost.model_time("ring", s, 8, cost.ALPHA_PAGE, cost.BETA_PAGE)
    assert f"{t * 1e3:.2f}" == f"{ms:.2f}"
    assert round(cost.algbw(s, t) / 1e9) == alg
    assert round(cost.busbw("allreduce", s, t, 8) / 1e9) == bus


def test_exercise_one_time_from_busbw():
    # 360 GB/s busbw at n=8: 256 MiB all-reduce ~1.3 ms, all-gather ~0.65 ms.
    s = 256 * 2 ** 20
    ar = cost.seconds_from_busbw("allreduce", s, 360e9, 8)
    ag = cost.seconds_from_busbw("allgather", s, 360e9, 8)
    assert round(ar * 1e3, 1) == 1.3
    assert round(ag * 1e3, 2) == 0.65
    assert round(360 / (2 * 7 / 8), 1) == 205.7 and round(360 / (7 / 8)) == 411


def test_exercise_two_crossover():
    s = cost.oneshot_twoshot_crossover(8, cost.ALPHA_PAGE, cost.BETA_PAGE)
    assert round(s / 1e3) == 257
    t1 = cost.model_time("one-shot", s, 8, cost.ALPHA_PAGE, cost.BETA_PAGE)
    t2 = cost.model_time("two-shot", s, 8, cost.ALPHA_PAGE, cost.BETA_PAGE)
    assert abs(t1 - t2) < 1e-15
    assert cost.oneshot_twoshot_crossover(2, cost.ALPHA_PAGE, cost.BETA_PAGE) is None
    for nbytes in (1, 1 << 20, 1 << 30):  # n=2: one-shot never slower
        assert cost.model_time("one-shot", nbytes, 2, 1.5e-6, 450e9) <= \
            cost.model_time("two-shot", nbytes, 2, 1.5e-6, 450e9)


def test_busbw_factors():
    assert cost.busbw_factor("allreduce", 8) == 2 * 7 / 8
    assert cost.busbw_factor("allgather", 8) == 7 / 8
    assert cost.busbw_factor("reduce_scatter", 4) == 3 / 4
    assert cost.busbw_factor("broadcast", 8) == 1


# --------------------------------------------------------------- traffic
@pytest.mark.parametrize("n", [2, 4, 8])
@pytest.mark.parametrize("dt,esize", [("f32", 4), ("bf16", 2), ("i32", 4)])
def test_link_bytes_match_page_closed_forms(n, dt, esize):
    count = n * (16 // esize) * 37      # N * A divides count: equal blocks
    s = count * esize
    for p in ("simple", "ll", "ll128"):
        ring = traffic.tally("allreduce", "ring", p, n, count, dt)
        assert ring.link == [2 * (n - 1) * s // n] * n           # ring: 2(n-1)/n S
        one = traffic.tally("allreduce", "oneshot", p, n, count, dt)
        assert one.link == [(n - 1) * s] * n                    # one-shot: (n-1) S
        two = traffic.tally("allreduce", "twoshot", p, n, count, dt)
        assert two.link == [2 * (n - 1) * s // n] * n           # two-shot: 2(n-1)/n S
        rc = count // n
        for algo in ("twoshot", "ring"):
            rs = traffic.tally("reduce_scatter", algo, p, n, rc, dt)
            ag = traffic.tally("allgather", algo, p, n, rc, dt)
            # (n-1)/n of the full per-rank buffer S = n * recvcount
            assert rs.link == [(n - 1) * rc * esize] * n
            assert ag.link == [(n - 1) * rc * esize] * n


def test_hbm_bytes_simple_schedules():
    n, count = 8, 8 * 4 * 1000
    s = count * 4
    assert traffic.tally("allreduce", "ring", "simple", n, count, "f32").hbm == 5 * (n - 1) * s
    assert traffic.tally("allreduce", "twoshot", "simple", n, count, "f32").hbm == (3 * n - 1) * s
    assert traffic.tally("allreduce", "oneshot", "simple", n, count, "f32").hbm == n * (n + 1) * s
    rc = count // n
    assert traffic.tally("reduce_scatter", "ring", "simple", n, rc, "f32").hbm == 3 * (n - 1) * s
    assert traffic.tally("reduce_scatter", "twoshot", "simple", n, rc, "f32").hbm == (n + 1) * s
    assert traffic.tally("allgather", "ring", "simple", n, rc, "f32").hbm == 2 * n * s
    assert traffic.tally("allgather", "twoshot", "simple", n, rc, "f32").hbm == 2 * n * s


def test_hbm_bytes_ll_is_wire_expansion():
    # LL doubles every byte that travels as lines; LL128 adds 128/120.
    n, count = 8, 8 * 4 * 120
    s = count * 4
    ring_ll = traffic.tally("allreduce", "ring", "ll", n, count, "f32").hbm
    assert ring_ll == 2 * n * s + 4 * (n - 1) * 2 * s
    ring_128 = traffic.tally("allreduce", "ring", "ll128", n, count, "f32").hbm
    assert ring_128 * 15 == (2 * n * s) * 15 + 4 * (n - 1) * 16 * s


@pytest.mark.parametrize("n", [2, 3, 4, 5, 8])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("proto,e", [("ll", Fraction(2)), ("ll128", Fraction(16, 15))])
def test_hbm_bytes_line_protocols_closed_forms(n, dt, proto, e):
    # Closed forms derived by hand from the schedules ("Algorithms": one-shot
    # reads every rank's input, two-shot reduces a slice per rank and gathers
    # the slice sums back, the ring does N-1 reduce hops and N-1 copy hops;
    # "Protocols": a line-protocol transfer is the sender writing e bytes of
    # lines per payload byte and the receiver reading them), with the staging
    # rules of this design: a rank puts its own input on the wire once, a rank
    # that just produced a value forwards it from registers, the own input is
    # read directly except in place.  e = 2 (LL) and 128/120 = 16/15 (LL128);
    # every block is a whole number of 120-byte lines, so e is exact.  S is
    # the per-rank buffer (all-reduce: count bytes; RS/AG: N shards).
    es = 4 if dt == "f32" else 2
    c = 240 * 3                       # block / shard bytes: 6 LL128 lines, a multiple of 16
    cnt = c // es
    s = n * c
    ar = lambda algo, **kw: traffic.tally("allreduce", algo, proto, n, n * cnt, dt, **kw).hbm  # noqa: E731
    rs = lambda algo: traffic.tally("reduce_scatter", algo, proto, n, cnt, dt).hbm  # noqa: E731
    ag = lambda algo: traffic.tally("allgather", algo, proto, n, cnt, dt).hbm  # noqa: E731
    # one-shot: every rank publishes its input (S read, eS written), then each
    # rank reads its own input and N-1 peers' lines and writes S
    assert ar("oneshot") == n * (3 + n * e) * s
    # ... in place: each rank reads all N ranks' lines, its own included
    assert ar("oneshot", in_place=True) == n * (2 + (n + 1) * e) * s
    # two-shot, per slice c = S/N: N-1 senders (c read, ec written); the owner
    # reads c and (N-1) ec, writes c and publishes ec; N-1 readers (ec read,
    # c written): 2N c + (3N-2) e c
    assert ar("twoshot") == 2 * n * s + (3 * n - 2) * e * s
    assert ar("ring") == 2 * n * s + 4 * (n - 1) * e * s
    # reduce-scatter, per slice: N-1 senders put it on the wire; the owner
    # reads its own slice and N-1 lines and writes c.  The ring: the first
    # sender (c, ec), N-1 hops reading ec + c, all but the last forwarding ec,
    # the last writing c.  Both come to (N+1) c + 2(N-1) e c.
    assert rs("twoshot") == rs("oneshot") == (n + 1) * s + 2 * (n - 1) * e * s
    assert rs("ring") == (n + 1) * s + 2 * (n - 1) * e * s
    # all-gather, per shard: the owner reads it, keeps a copy and publishes it
    # once (c read, c + ec written); N-1 receivers read ec and write c
    assert ag("twoshot") == ag("oneshot") == (n + 1) * s + n * e * s
    # ... ring: the owner's copy and first send, N-1 hops (ec read, c
    # written), all but the last forwarding ec
    assert ag("ring") == (n + 1) * s + 2 * (n - 1) * e * s


def test_hbm_bytes_simple_in_place_one_shot():
    # In place, each rank program still reads all N inputs and writes one
    # output: N(N+1) S, the same as out of place.
    n, count = 8, 8 * 4 * 100
    s = count * 4
    assert traffic.tally("allreduce", "oneshot", "simple", n, count, "f32", in_place=True).hbm == n * (n + 1) * s


# --------------------------------------------------------------- signals
@pytest.mark.parametrize("n", [2, 3, 4, 8])
def test_ring_withheld_signal_blocks_rest_of_one_chain(n):
    steps = 2 * (n - 1)
    for r in range(n):
        for s in range(steps - 1):
            stuck, first = sim.blocked("allreduce", "ring", n, withheld=(r, s))
            assert first == ((r + 1) % n, s + 1)
            assert len(stuck) == steps - 1 - s
    assert sim.blocked("allreduce", "ring", 4)[0] == []


def test_twoshot_withheld_signal_blocks_every_other_rank():
    n = 4
    stuck, first = sim.blocked("allreduce", "twoshot", n, withheld=(2, 0))
    assert stuck == [(0, 1), (1, 1), (3, 1)] and first == (0, 1)


def test_oneshot_has_nothing_to_wait_on_out_of_place():
    assert sim.blocked("allreduce", "oneshot", 8, withheld=(3, 0))[0] == []
    stuck, first = sim.blocked("allreduce", "oneshot", 8, withheld=(3, 0), in_place=True)
    assert len(stuck) == 8 and first == (0, 1)


@pytest.mark.parametrize("n", [2, 3, 5, 8])
def test_tree_bytes(n):
    # Per half of c bytes: going up, every node reads its input and each
    # child's partial (N + (N-1) reads of c) and writes its partial (N);
    # going down, N-1 nodes read their parent's sum and write it: (5N-3) c in
    # all, so (5N-3) S for the two halves.  Each rank-to-rank transfer (N-1
    # up, N-1 down per half) moves c: 2(N-1)/N S per rank on average, the
    # ring's figure ("Algorithms": the tree's bandwidth is close to optimal).
    count = 8 * 1000
    s = count * 4
    t = traffic.tally("allreduce", "tree", "simple", n, count, "f32")
    assert t.hbm == (5 * n - 3) * s
    assert sum(t.link) == 2 * (n - 1) * s
    with pytest.raises(ValueError):
        traffic.tally("allreduce", "tree", "ll", n, count, "f32")


# ------------------------------------------- signals of the line protocols
@pytest.mark.parametrize("proto", ["ll", "ll128"])
@pytest.mark.parametrize("n", [2, 3, 4, 8])
def test_line_ring_withheld_flags_block_the_rest_of_one_chain(n, proto):
    # 2N-1 steps per block (a first send, N-1 reduce receives, N-1 copy
    # receives); withholding the flags of step s blocks steps s+1 .. 2N-2 of
    # that block only, the first of them on the next rank around the ring.
    steps = 2 * n - 1
    for r in range(n):
        for s in range(steps - 1):
            stuck, first = sim.blocked("allreduce", "ring", n, withheld=(r, s), proto=proto)
            assert first == ((r + 1) % n, s + 1)
            assert len(stuck) == steps - 1 - s
        # the last step writes no lines: nothing waits on it
        assert sim.blocked("allreduce", "ring", n, withheld=(r, steps - 1), proto=proto)[0] == []
    for op in ("reduce_scatter", "allgather"):  # N steps per block
        stuck, first = sim.blocked(op, "ring", n, withheld=(0, 0), proto=proto)
        assert first == (1, 1) and len(stuck) == n - 1


@pytest.mark.parametrize("proto", ["ll", "ll128"])
def test_line_two_shot_withheld_flags(proto):
    n = 4
    # a sender that withholds its slices blocks every other owner's sum, then
    # every rank's receive of those sums
    stuck, first = sim.blocked("allreduce", "twoshot", n, withheld=(1, 0), proto=proto)
    assert first == (0, 1)
    assert stuck == [(0, 1), (2, 1), (3, 1), (0, 2), (1, 2), (2, 2), (3, 2)]
    # an owner that withholds its published sum blocks every other rank's step 2
    stuck, first = sim.blocked("allreduce", "twoshot", n, withheld=(2, 1), proto=proto)
    assert stuck == [(0, 2), (1, 2), (3, 2)] and first == (0, 2)


@pytest.mark.parametrize("proto", ["ll", "ll128"])
def test_line_one_shot_and_direct_withheld_flags(proto):
    n = 8
    stuck, first = sim.blocked("allreduce", "oneshot", n, withheld=(0, 0), proto=proto)
    assert stuck == [(r, 1) for r in range(1, n)] and first == (1, 1)
    stuck, _ = sim.blocked("allreduce", "oneshot", n, withheld=(0, 0), in_place=True, proto=proto)
    assert stuck == [(r, 1) for r in range(n)]  # in place the rank reads its own lines too
    for op in ("reduce_scatter", "allgather"):
        stuck, first = sim.blocked(op, "twoshot", n, withheld=(5, 0), proto=proto)
        assert stuck == [(r, 1) for r in range(n) if r != 5] and first == (0, 1)
