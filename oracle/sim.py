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
"""


def nodes_and_deps(op: str, algo: str, n: int, in_place: bool = False):
    """Return {node: [nodes it waits on]} with node = (rank, step)."""
    deps = {}
    if n == 1:
        deps[(0, 0)] = []
        return deps
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


def blocked(op: str, algo: str, n: int, withheld=None, in_place: bool = False):
    """Nodes that never run when node `withheld` = (rank, step) runs but
    never signals.  Returns (sorted blocked nodes, first blocked or None),
    "first" being the smallest (step, rank)."""
    deps = nodes_and_deps(op, algo, n, in_place)
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
