"""Alpha-beta cost model and the nccl-tests bandwidth figures
(test infrastructure only).

"Collective communication: NCCL's algorithms and protocols, and custom
all-reduce":

* section "Algorithms": the time of one all-reduce of S bytes per GPU on n
  GPUs with a per-step fixed cost alpha and a one-way per-GPU bandwidth beta:
  ring 2(n-1) alpha + 2(n-1)/n S/beta; double binary tree 2 log2(n) alpha +
  2 S/beta; one-shot 2 alpha + (n-1) S/beta; two-shot 4 alpha + 2(n-1)/n
  S/beta; NVLS 2 alpha + S/beta.  The page evaluates these at n=8,
  alpha=1.5 us, beta=450 GB/s.
* section "Reading nccl-tests": algbw = S/t; busbw = algbw times 2(n-1)/n for
  all-reduce, (n-1)/n for the reduce-scatter and the all-gather, and 1 for a
  broadcast.
* section "Exercises", exercise 2: the one-shot / two-shot crossover
  S* = 2 alpha beta / ((n-1)(1 - 2/n)); no crossover at n=2.
"""

import math

ALPHA_PAGE = 1.5e-6  # seconds per step, "only illustrative"
BETA_PAGE = 450e9    # bytes per second, one way, per GPU
N_PAGE = 8

MODEL_ALGOS = ("ring", "tree", "one-shot", "two-shot", "NVLS")


def model_time(algo: str, nbytes: float, n: int, alpha: float, beta: float) -> float:
    """Seconds for one all-reduce of `nbytes` per GPU under the page's model."""
    frac = (n - 1) / n
    if algo == "ring":
        return 2 * (n - 1) * alpha + 2 * frac * nbytes / beta
    if algo == "tree":
        return 2 * math.log2(n) * alpha + 2 * nbytes / beta
    if algo == "one-shot":
        return 2 * alpha + (n - 1) * nbytes / beta
    if algo == "two-shot":
        return 4 * alpha + 2 * frac * nbytes / beta
    if algo == "NVLS":
        return 2 * alpha + nbytes / beta
    raise ValueError(f"unknown model algorithm {algo!r}")


def fastest_without_nvls(nbytes: float, n: int, alpha: float, beta: float) -> str:
    times = {a: model_time(a, nbytes, n, alpha, beta) for a in MODEL_ALGOS if a != "NVLS"}
    return min(times, key=times.get)


def busbw_factor(op: str, n: int) -> float:
    """nccl-tests correction factor from algbw to busbw."""
    if op == "allreduce":
        return 2 * (n - 1) / n
    if op in ("allgather", "reduce_scatter"):
        return (n - 1) / n
    if op == "broadcast":
        return 1.0
    raise ValueError(f"unknown collective {op!r}")


def algbw(nbytes: float, seconds: float) -> float:
    return nbytes / seconds


def busbw(op: str, nbytes: float, seconds: float, n: int) -> float:
    return algbw(nbytes, seconds) * busbw_factor(op, n)


def seconds_from_busbw(op: str, nbytes: float, bus: float, n: int) -> float:
    """Exercise 1 worked backwards: the time a collective of `nbytes` per GPU
    takes at bus bandwidth `bus`."""
    return nbytes / (bus / busbw_factor(op, n))


def oneshot_twoshot_crossover(n: int, alpha: float, beta: float):
    """S* where one-shot and two-shot take equal model time; None when the
    two never cross (n <= 2: one-shot is never slower)."""
    denom = (n - 1) * (1 - 2 / n)
    if denom <= 0:
        return None
    return 2 * alpha * beta / denom
