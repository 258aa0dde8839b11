"""Bytes each schedule moves (test infrastructure only).

Two tallies, both made by walking the schedule transfer by transfer rather
than from a closed form:

* link bytes per rank -- payload bytes each rank receives from its peers, the
  quantity the pages reason about ("Collective communication: NCCL's
  algorithms and protocols, and custom all-reduce", section "Algorithms":
  ring sends and receives 2(n-1)/n S per GPU, one-shot reads (n-1) S, two-shot
  reads 2(n-1)/n S; section "Reading nccl-tests": the reduce-scatter and the
  all-gather move (n-1)/n S);
* HBM bytes per call -- what the single-GPU simulation of all N rank
  programs reads and writes in device memory.  Ranks share one HBM, so a
  "link transfer" is the receiver reading the sender's buffer (Simple) or
  the sender writing LL / LL128 lines that the receiver then reads.  The rules
  (one per rank program, per block):

  Simple   the payload already sits in the sender's own buffer; the receiver
           reads it after the sender's flag.
  LL/LL128 the sender writes the payload as lines (wire bytes, see
           ``oracle.proto.wire_bytes``) into staging memory and the receiver
           reads those lines; a rank that just produced a value forwards it
           from registers, so it is not read again.

  Flags are a few bytes per tile and are left out of both tallies.

Blocks of two-shot and ring follow ``oracle.geometry``; the tree's two halves
are the N=2 blocks, and each node keeps its partial in its own output; LL / LL128 lines are
cut per block, so a block's wire bytes are ``wire_bytes(block bytes)``.
"""

from . import geometry, proto as protomod
from .dtypes import ESIZE


class Tally:
    def __init__(self, nranks: int):
        self.read = 0
        self.write = 0
        self.link = [0] * nranks

    def rd(self, n):
        self.read += n

    def wr(self, n):
        self.write += n

    def recv(self, rank, n):
        self.link[rank] += n

    @property
    def hbm(self):
        return self.read + self.write


def _tree_rank(n, tree, pos):
    return pos if tree == 0 else n - 1 - pos


def _blocks_bytes(op, nranks, count, dt):
    e = ESIZE[dt]
    if op == "allreduce":
        return [(hi - lo) * e for lo, hi in geometry.ar_blocks(count, nranks, dt)]
    return [count * e] * nranks  # reduce-scatter / all-gather: exact per-rank slices


def tally(op: str, algo: str, proto: str, nranks: int, count: int, dt: str,
          in_place: bool = False) -> Tally:
    """Walk one call.  `count` is elements per rank for all-reduce, recvcount
    for reduce-scatter and sendcount for all-gather."""
    n = nranks
    t = Tally(n)
    w = lambda c: protomod.wire_bytes(c, proto)  # noqa: E731
    enc = proto != "simple"
    if algo not in ("oneshot", "twoshot", "ring", "tree"):
        raise ValueError(algo)
    if algo == "tree" and (op != "allreduce" or enc):
        raise ValueError("the tree is an all-reduce schedule, run with Simple")
    if n == 1:  # a single rank: the result is its own input
        size = count * ESIZE[dt]
        if not in_place:
            t.rd(size)
            t.wr(size)
        return t
    cb = _blocks_bytes(op, n, count, dt)
    size = sum(cb) if op == "allreduce" else count * ESIZE[dt]

    if op == "allreduce" and algo == "oneshot":
        if enc:
            for i in range(n):  # every rank publishes its input as lines once
                t.rd(size)
                t.wr(w(size))
        for r in range(n):
            for i in range(n):
                if i != r:
                    t.recv(r, size)
                if not enc:
                    t.rd(size)
                elif i == r and not in_place:
                    t.rd(size)          # own input read directly
                else:
                    t.rd(w(size))       # peer lines (and own lines when in place)
            t.wr(size)
        return t

    if algo == "tree":
        e = ESIZE[dt]
        for tree, (lo, hi) in enumerate(geometry.ar_blocks(count, 2, dt)):
            c = (hi - lo) * e
            for pos in range(n):  # up: own input and the children's partials
                children = [ch for ch in (2 * pos + 1, 2 * pos + 2) if ch < n]
                t.rd(c * (1 + len(children)))
                t.wr(c)  # the partial (the root: the sum) in the rank's own output
                for _ in children:
                    t.recv(_tree_rank(n, tree, pos), c)
            for pos in range(1, n):  # down: copy the parent's sum
                t.rd(c)
                t.wr(c)
                t.recv(_tree_rank(n, tree, pos), c)
        return t

    if op == "allreduce" and algo == "twoshot":
        for j, c in enumerate(cb):
            # shot 1: owner j gathers slice j of every rank
            for i in range(n):
                if i == j:
                    continue
                t.recv(j, c)
                if enc:  # sender i encodes its slice j for owner j
                    t.rd(c)
                    t.wr(w(c))
            if enc:
                t.rd(c)                  # owner's own slice
                t.rd((n - 1) * w(c))     # peers' lines
                t.wr(c)                  # owner's output block
                t.wr(w(c))               # publish the sum as lines
            else:
                t.rd(n * c)
                t.wr(c)
            # shot 2: every other rank reads the sum back
            for r in range(n):
                if r == j:
                    continue
                t.recv(r, c)
                t.rd(w(c) if enc else c)
                t.wr(c)
        return t

    if algo == "ring":
        reduce_steps = op in ("allreduce", "reduce_scatter")
        gather_steps = op in ("allreduce", "allgather")
        for j, c in enumerate(cb):
            if reduce_steps:
                if enc:  # rank j+1 puts its input block j on the wire
                    t.rd(c)
                    t.wr(w(c))
                for s in range(n - 1):
                    q = (j + 2 + s) % n            # receiver of step s
                    t.recv(q, c)
                    last = s == n - 2
                    if enc:
                        t.rd(w(c))
                        t.rd(c)                    # own input block
                        if not last:
                            t.wr(w(c))             # forward the new partial
                        else:
                            t.wr(c)                # rank j keeps the sum
                            if gather_steps:
                                t.wr(w(c))         # and starts the copy steps
                    else:
                        t.rd(2 * c)                # sender's partial + own input
                        t.wr(c)
            if gather_steps:
                if not reduce_steps:               # all-gather: rank j's own copy
                    t.rd(c)
                    t.wr(c)
                    if enc:
                        t.wr(w(c))                 # and its first send
                for s in range(n - 1):
                    q = (j + 1 + s) % n
                    t.recv(q, c)
                    t.rd(w(c) if enc else c)
                    t.wr(c)
                    if enc and s < n - 2:
                        t.wr(w(c))
        return t

    if op == "reduce_scatter":  # direct
        for j, c in enumerate(cb):
            for i in range(n):
                if i == j:
                    continue
                t.recv(j, c)
                if enc:
                    t.rd(c)
                    t.wr(w(c))
            if enc:
                t.rd(c)
                t.rd((n - 1) * w(c))
            else:
                t.rd(n * c)
            t.wr(c)
        return t

    if op == "allgather":  # direct
        for j, c in enumerate(cb):
            if enc:  # rank j publishes its shard once and copies it locally
                t.rd(c)
                t.wr(w(c))
                t.wr(c)
            for r in range(n):
                if enc and r == j:
                    continue
                if r != j:
                    t.recv(r, c)
                t.rd(w(c) if (enc and r != j) else c)
                t.wr(c)
        return t

    raise ValueError(f"unknown collective {op!r}")
