"""All-reduce with a fused RMSNorm epilogue, written out plainly (test
infrastructure only).

"Collective communication: NCCL's algorithms and protocols, and custom
all-reduce", section "Source code", names FlashInfer's fused all-reduce +
RMSNorm kernel (integrated by SGLang) as the operation that follows tensor
parallelism's all-reduce.  The page gives no formula.  Reading taken (the
common decoder-layer form):

  for every rank r and row i of a [rows, hidden] buffer:
    a   = the one-shot all-reduce of row i (ascending rank order, fp32
          accumulate, rounded to the payload type once)
    h   = a + residual[r][i]   (fp32 add of the widened values; skipped when
          there is no residual, h = a)
    residual[r][i] <- h rounded to the payload type
    out[r][i] = h / sqrt(mean(h^2) + eps) * weight   (rounded once)

The all-reduce part and the residual update are exact definitions (the GPU
must match them bit for bit); the normalization is computed here in fp64,
so the GPU's fp32 result is compared within a tolerance derived from its
arithmetic.
"""

import numpy as np

from . import bf16, collectives, dtypes


def _widen64(x, dt):
    return dtypes.to_acc(x, dt).astype(np.float64)


def _round64(x, dt):
    """fp64 -> payload type, one rounding to nearest even (bf16 directly,
    not through fp32, whose own rounding could land on a bf16 tie)."""
    if dt == "bf16":
        return bf16.narrow_rne_f64(x)
    return x.astype(np.float32)


def allreduce_rmsnorm(inputs, residuals, weight, rows, hidden, eps, dt):
    """Returns (outs, residual_outs); residual_outs is None without residuals.
    `inputs` / `residuals` are N flat arrays of rows*hidden elements, `weight`
    one array of hidden elements, all in the payload type (f32 or bf16)."""
    if dt not in ("f32", "bf16"):
        raise ValueError("the fused RMSNorm runs on floating-point payloads")
    n = len(inputs)
    a = collectives.allreduce_oneshot(inputs, dt)[0]  # every rank holds the same sum
    w = _widen64(weight, dt)
    outs, res_outs = [], [] if residuals is not None else None
    for r in range(n):
        if residuals is not None:
            h32 = dtypes.add(dtypes.to_acc(a, dt), dtypes.to_acc(residuals[r], dt), dt)
            res_outs.append(dtypes.from_acc(h32, dt))
        else:
            h32 = dtypes.to_acc(a, dt)
        h = h32.astype(np.float64).reshape(rows, hidden)
        inv = 1.0 / np.sqrt(np.mean(h * h, axis=1, keepdims=True) + float(eps))
        outs.append(_round64((h * inv * w[None, :]).reshape(-1), dt))
    return outs, res_outs
