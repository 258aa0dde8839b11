"""Signal graph of the Simple-protocol schedules, with a withheld signal
(test infrastructure only).

A collective hangs when one rank never sends what a peer waits for
("Collective communication: NCCL's algorithms and protocols, and custom
all-reduce", section "Common environment variables and debugging": a rank
that made one call fewer, or crashed, leaves its peers waiting forever).
This module builds, for one call, the graph of (rank, step) nodes in which a
node runs once every node it waits on has signalled, and reports which nodes
can never run when one (rank, step) withholds its signal.

Step numbering (one node per rank per step; a node is the receiving side):
  ring       step s of block j runs on rank j+2+s (reduce steps, s < N-1) and
             on rank j+1+(s-(N-1)) (copy steps); it waits on step s-1 of the
             same block, which ran on the previous rank.
  two-shot   step 0: owner j reduces block j; step 1: rank r copies every
             block j != r, waiting on (j, 0).
  one-shot   out of place: one step, nothing to wait on; in place: step 0
             reads, step 1 writes after every rank's step 0.
  direct reduce-scatter / all-gather: one step, nothing to wait on.

With LL or LL128 ("Protocols": the receiver polls the flags of lines the
sender writes) every transfer is a write of lines by its sender and a poll by
its receiver, so the graph has a node per sending and per receiving side:
  ring       step 0 of block j: rank j+1 puts its block on the wire; step s
             (s >= 1): rank j+1+s (all-reduce, reduce-scatter) or j+s
             (all-gather) receives what step s-1 wrote; the last step only
             receives.
  two-shot   step 0: rank r puts its slice of every block j != r on the
             wire; step 1: owner j sums block j, waiting on every other
             rank's step 0, and puts the sum on the wire; step 2: rank r
             receives every block j != r, waiting on (j, 1).
  one-shot   step 0: rank r puts its input on the wire; step 1: rank r sums,
             waiting on every other rank's step 0 (in place: on every
             rank's, its own lines included).
  direct reduce-scatter: step 0 sends, step 1 owner j waits on every other
             rank's step 0.  Direct all-gather: step 0 rank j publishes its
             shard, step 1 rank r waits on every other rank's step 0.
"""


def _line_deps(op: str, algo: str, n: int, in_place: bool):
    deps = {}
    if algo == "ring":
        steps = 2 * n - 1 if op == "allreduce" else n
        for j in range(n):
            prev = None
            for s in range(steps):
                rank = (j + s) % n if op == "allgather" else (j + 1 + s) % n
                node = (rank, s)
                deps.setdefault(node, [])
                if prev is not None:
                    deps[node].append(prev)
                prev = node
        return deps
    if op == "allreduce" and algo == "twoshot":
        for r in range(n):
            deps[(r, 0)] = []
        for j in range(n):
            deps[(j, 1)] = [(i, 0) for i in range(n) if i != j]
        for r in range(n):
            deps[(r, 2)] = [(j, 1) for j in range(n) if j != r]
        return deps
    for r in range(n):  # one-shot, direct reduce-scatter and all-gather
        deps[(r, 0)] = []
    for r in range(n):
        deps[(r, 1)] = [(i, 0) for i in range(n) if i != r or (in_place and op == "allreduce")]
    return deps


def nodes_and_deps(op: str, algo: str, n: int, in_place: bool = False, proto: str = "simple"):
    """Return {node: [nodes it waits on]} with node = (rank, step)."""
    deps = {}
    if n == 1:
        deps[(0, 0)] = []
        return deps
    if proto != "simple":
        return _line_deps(op, algo, n, in_place)
    if algo == "ring":
        red = n - 1 if op in ("allreduce", "reduce_scatter") else 0
        cop = n - 1 if op in ("allreduce", "allgather") else 0
        steps = red + cop
        for j in range(n):
            prev = None
            for s in range(steps):
                rank = (j + 2 + s) % n if s < red else (j + 1 + (s - red)) % n
                node = (rank, s)
                deps.setdefault(node, [])
                if prev is not None:
                    deps[node].append(prev)
                prev = node
        return deps
    if op == "allreduce" and algo == "twoshot":
        for j in range(n):
            deps[(j, 0)] = []
        for r in range(n):
            deps[(r, 1)] = [(j, 0) for j in range(n) if j != r]
        return deps
    if op == "allreduce" and algo == "oneshot" and in_place:
        for r in range(n):
            deps[(r, 0)] = []
        for r in range(n):
            deps[(r, 1)] = [(i, 0) for i in range(n)]
        return deps
    for r in range(n):
        deps[(r, 0)] = []
    return deps


def blocked(op: str, algo: str, n: int, withheld=None, in_place: bool = False, proto: str = "simple"):
    """Nodes that never run when node `withheld` = (rank, step) runs but
    never signals (with LL / LL128: writes its lines without their flags).
    Returns (sorted blocked nodes, first blocked or None), "first" being the
    smallest (step, rank)."""
    deps = nodes_and_deps(op, algo, n, in_place, proto)
    signalled = set()
    ran = set()
    progress = True
    while progress:
        progress = False
        for node, waits in deps.items():
            if node in ran:
                continue
            if all(w in signalled for w in waits):
                ran.add(node)
                if node != withheld:
                    signalled.add(node)
                progress = True
    stuck = sorted((node for node in deps if node not in ran), key=lambda x: (x[1], x[0]))
    return stuck, (stuck[0] if stuck else None)
