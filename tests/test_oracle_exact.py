"""Pins for the oracle's plain-fp64 decision mode (``exact=True``; CPU only).

By default the oracle takes every integer decision (range, scale, zero-point,
code) in fp32, the precision of the device kernels; with ``exact`` it takes
them in plain fp64.  These pins fix the fp64 mode against the printed INT8
example (its scale exactly (3.7 + 2.5) / 255 with no fp32 rounding), the
invariants of the quantizer, brute-force nearest grid points, and the
special cases of the GPTQ loop that reduce to RTN or to the literal OBS
route; and show that the two modes differ only at rounding ties.
"""
import json
import os

import numpy as np
import pytest

import oracle
from oracle.quantizer import f32


def test_worked_example_exact(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "worked_example_minmax_int8.json")))
    lo, hi = g["range"]
    row = np.array([[lo, 0.3, -1.0, hi]])
    scale, zero = oracle.group_params(row, g["bits"], exact=True)
    assert float(scale[0]) == (hi - lo) / g["levels_minus_one"]  # no fp32 rounding
    assert round(float(scale[0]), g["scale_printed_decimals"]) == g["scale_printed"]
    s32, _ = oracle.group_params(row, g["bits"])
    assert float(s32[0]) != float(scale[0])  # the two modes are distinct
    q = oracle.quantize_codes(row[0], scale[0], zero[0], g["bits"], exact=True)
    assert q[0] == 0 and q[-1] == 2 ** g["bits"] - 1
    assert zero[0] == np.rint(-lo * 255 / (hi - lo))


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_exact_codes_in_range_half_step_and_grid(bits):
    rng = np.random.default_rng(100 + bits)
    v = rng.standard_normal((300, 64)) * rng.uniform(0.001, 1, (300, 1)) + rng.uniform(-1, 1, (300, 1))
    scale, zero = oracle.group_params(v, bits, exact=True)
    maxq = 2 ** bits - 1
    assert np.all((zero >= 0) & (zero <= maxq)) and np.all(zero == np.rint(zero))
    q = oracle.quantize_codes(v, scale[:, None], zero[:, None], bits, exact=True)
    assert np.all((q >= 0) & (q <= maxq))
    dq = oracle.dequantize(q, scale[:, None], zero[:, None])
    lo = np.minimum(v.min(axis=1), 0)[:, None]
    hi = np.maximum(v.max(axis=1), 0)[:, None]
    inside = (v >= lo) & (v <= hi)
    assert np.all(np.abs(v - dq)[inside] <= (scale[:, None] * (0.5 + 1e-12) + 0 * v)[inside])
    codes = np.arange(maxq + 1, dtype=np.float64)[None, :]
    grid = oracle.dequantize(codes, scale[:, None], zero[:, None])
    back = oracle.quantize_codes(grid, scale[:, None], zero[:, None], bits, exact=True)
    assert np.array_equal(back, np.broadcast_to(codes, back.shape))


def test_exact_rtn_is_the_nearest_grid_point():
    rng = np.random.default_rng(7)
    W = rng.standard_normal((40, 64)) * 0.05
    codes, scales, zeros = oracle.rtn_minmax(W, 3, 32, exact=True)
    for r in range(W.shape[0]):
        for c in range(W.shape[1]):
            s, z = scales[r, c // 32], zeros[r, c // 32]
            dist = np.abs(W[r, c] - (np.arange(8) - z) * s)
            assert dist[int(codes[r, c])] == dist.min()


def test_exact_ties_round_half_even():
    q = oracle.quantize_codes(np.array([0.5, 1.5, 2.5, -0.5, -1.5]), np.array([1.0]),
                              np.array([8.0]), 4, exact=True)
    assert list(q) == [8, 10, 10, 8, 6]


def _layer(seed, m, n, t):
    rng = np.random.default_rng(seed)
    W = rng.standard_normal((m, n)) * 0.02
    X = rng.standard_normal((t, n))
    X[:, 3] *= 20.0
    return W, X


def test_exact_cholesky_route_equals_literal_obs_route():
    W, X = _layer(1, 24, 96, 400)
    S = oracle.hessian_S([X])
    P = oracle.prepare(S, 0.01, False)
    res = oracle.gptq_quantize(W, P.U, 4, 32, 64, exact=True)
    Hd = 2.0 * S + P.lam * np.eye(96)
    codes, scales, zeros = oracle.gptq_obs_literal(W, Hd, 4, 32, exact=True)
    assert np.array_equal(res.codes, codes)
    assert np.allclose(res.scales, scales, rtol=1e-12)


def test_exact_diagonal_hessian_and_single_column_reduce_to_rtn():
    rng = np.random.default_rng(3)
    W = rng.standard_normal((32, 64)) * 0.02
    U = np.diag(1.0 / np.sqrt(rng.uniform(0.5, 2.0, 64)))
    res = oracle.gptq_quantize(W, U, 4, 16, 64, exact=True)
    c, s, z = oracle.rtn_minmax(W, 4, 16, exact=True)
    assert np.array_equal(res.codes, c) and np.array_equal(res.scales, s)
    w1 = W[:, :1]
    r1 = oracle.gptq_quantize(w1, np.array([[0.7]]), 3, 1, 128, exact=True)
    c1, _, _ = oracle.rtn_minmax(w1, 3, 1, exact=True)
    assert np.array_equal(r1.codes, c1)


def test_fp32_and_fp64_decisions_differ_only_at_ties():
    """The fp32-decision loop's result, replayed against fp64 decisions, has no
    hard mismatch: wherever the two precisions take another code or zero-point,
    the fp64 value lies within 1e-3 of a step of the rounding boundary."""
    W, X = _layer(5, 64, 256, 2048)
    S = oracle.hessian_S([f32(X)])
    P = oracle.prepare(S, 0.01, True)
    r32 = oracle.gptq_quantize(W, P.U, 4, 64, 128, P.perm, P.dead)
    r64 = oracle.gptq_quantize(W, P.U, 4, 64, 128, P.perm, P.dead, exact=True)
    rate = float(np.mean(r32.codes == r64.codes))
    rep = oracle.replay_check(W, P.U, 4, 64, 128, P.perm, P.dead, r32.codes_proc, r32.scales,
                              r32.zeros, exact=True)
    assert rate >= 0.999
    assert rep.hard == 0 and rep.zero_hard == 0
    assert rep.scale_max_rel <= 2.0 ** -22  # the fp32 roundings of the range and the quotient
