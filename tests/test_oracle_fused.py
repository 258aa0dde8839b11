"""Pins of the fused all-reduce + RMSNorm oracle (host only).

Each checks the oracle against an independent fact: torch's own RMSNorm on
the CPU in fp64, closed forms, exact integer arithmetic, scale invariance,
or the exact fp64 -> bf16 rounding against the fp32 one where no double
rounding can occur.
"""

import numpy as np
import pytest
import torch

from all_reduce_reduction_rank_amd import inputs
from oracle import bf16, collectives as C, fused


def _rows(n, rows, hidden, dt, seed, dist="normal"):
    return inputs.rank_inputs(n, rows * hidden, dt, dist, seed=seed, cfg=60)


def test_bf16_f64_rounding_agrees_with_f32_rounding_on_f32_values():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(200000) * 10.0 ** rng.integers(-40, 38, 200000)).astype(np.float32)
    assert np.array_equal(bf16.narrow_rne_f64(x.astype(np.float64)), bf16.narrow_rne(x))


def test_bf16_f64_rounding_ties_and_specials():
    t = np.array([1 + 2 ** -8 + 2 ** -40, 1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8 + 2 ** -40),
                  3.4e38, 1e-45, np.inf, -np.inf])
    want = [0x3F81, 0x3F80, 0x3F82, 0xBF81, 0x7F80, 0x0000, 0x7F80, 0xFF80]
    assert list(bf16.narrow_rne_f64(t)) == want
    assert (int(bf16.narrow_rne_f64(np.array([np.nan]))[0]) & 0x7FC0) == 0x7FC0


@pytest.mark.parametrize("n", [1, 2, 8])
def test_f32_matches_torch_rms_norm_in_fp64(n):
    rows, hidden, eps = 3, 320, 1e-6
    x = _rows(n, rows, hidden, "f32", seed=n)
    w = inputs.rank_inputs(1, hidden, "f32", "normal", seed=99, cfg=61)[0]
    out, res = fused.allreduce_rmsnorm(x, None, w, rows, hidden, eps, "f32")
    assert res is None
    a = torch.from_numpy(C.allreduce_oneshot(x, "f32")[0].astype(np.float64)).view(rows, hidden)
    want = torch.nn.functional.rms_norm(a, (hidden,), torch.from_numpy(w.astype(np.float64)), eps)
    want = want.to(torch.float32).numpy().reshape(-1)
    for r in range(n):
        ulps = np.abs(out[r].view(np.int32).astype(np.int64) - want.view(np.int32).astype(np.int64))
        assert ulps.max() <= 1


def test_unit_weight_rows_have_unit_rms():
    rows, hidden = 4, 1000
    x = _rows(4, rows, hidden, "f32", seed=5)
    out, _ = fused.allreduce_rmsnorm(x, None, np.ones(hidden, np.float32), rows, hidden, 0.0, "f32")
    ms = (out[0].astype(np.float64).reshape(rows, hidden) ** 2).mean(axis=1)
    assert np.allclose(ms, 1.0, rtol=1e-6)


def test_scale_invariance_without_eps():
    # RMSNorm(2^k v) == RMSNorm(v) exactly: scaling by a power of two is exact
    # in every step, and the norm cancels it.
    rows, hidden = 2, 256
    x = _rows(2, rows, hidden, "f32", seed=6)
    w = inputs.rank_inputs(1, hidden, "f32", "normal", seed=7, cfg=61)[0]
    base, _ = fused.allreduce_rmsnorm(x, None, w, rows, hidden, 0.0, "f32")
    scaled, _ = fused.allreduce_rmsnorm([v * np.float32(8.0) for v in x], None, w, rows, hidden, 0.0, "f32")
    assert np.array_equal(base[0], scaled[0])


def test_constant_row_closed_form():
    # every element c, unit weight: c / sqrt(c^2 + eps)
    rows, hidden, eps = 1, 64, 0.25
    x = [np.full(hidden, 0.5, np.float32), np.full(hidden, 0.25, np.float32)]  # sum 0.75
    out, _ = fused.allreduce_rmsnorm(x, None, np.ones(hidden, np.float32), rows, hidden, eps, "f32")
    assert np.all(out[0] == np.float32(0.75 / np.sqrt(0.75 ** 2 + eps)))


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_residual_update_is_the_exact_sum_on_integers(dt):
    # small integers: every sum is exact, so residual_out = sum + residual
    n, rows, hidden = 4, 2, 128
    rng = np.random.default_rng(3)
    ints = [rng.integers(-50, 50, rows * hidden) for _ in range(n)]
    res_ints = [rng.integers(-50, 50, rows * hidden) for _ in range(n)]

    def enc(v):
        f = v.astype(np.float32)
        return bf16.narrow_rne(f) if dt == "bf16" else f

    x = [enc(v) for v in ints]
    res = [enc(v) for v in res_ints]
    w = enc(np.ones(hidden, dtype=np.int64))
    _, res_out = fused.allreduce_rmsnorm(x, res, w, rows, hidden, 1e-6, dt)
    total = sum(ints)
    for r in range(n):
        got = bf16.widen(res_out[r]) if dt == "bf16" else res_out[r]
        assert np.array_equal(got.astype(np.int64), total + res_ints[r])


def test_integer_payload_is_rejected():
    with pytest.raises(ValueError):
        fused.allreduce_rmsnorm([np.zeros(8, np.int32)], None, np.ones(8, np.int32), 1, 8, 0.0, "i32")
