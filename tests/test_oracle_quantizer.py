"""Pins for the oracle's quantizer (CPU only)."""
import itertools
import json
import os

import numpy as np
import pytest

import oracle
from oracle.quantizer import f32


def test_worked_example_minmax_int8(golden_dir):
    """Printed example: [-2.5, 3.7] onto 8-bit codes gives scale ~ 0.0243."""
    g = json.load(open(os.path.join(golden_dir, "worked_example_minmax_int8.json")))
    lo, hi = g["range"]
    row = np.array([[lo, 0.3, -1.0, hi]])
    scale, zero = oracle.group_params(row, g["bits"])
    assert round(float(scale[0]), g["scale_printed_decimals"]) == g["scale_printed"]
    assert abs(float(scale[0]) - (hi - lo) / g["levels_minus_one"]) < 1e-8
    # the range end points land on the ends of the code range
    q = oracle.quantize_codes(row[0], scale[0], zero[0], g["bits"])
    assert q[0] == 0 and q[-1] == 2 ** g["bits"] - 1
    # the zero-point is the code of 0.0 and lies inside the range
    assert zero[0] == np.rint(2.5 * 255 / 6.2)
    assert oracle.quantize_codes(np.array([0.0]), scale[0], zero[0], 8)[0] == zero[0]


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 8])
def test_codes_and_zero_in_range(bits):
    rng = np.random.default_rng(bits)
    v = rng.standard_normal((500, 64)) * rng.uniform(0.001, 10, (500, 1)) + rng.uniform(-3, 3, (500, 1))
    scale, zero = oracle.group_params(v, bits)
    maxq = 2 ** bits - 1
    assert np.all(scale > 0)
    assert np.all((zero >= 0) & (zero <= maxq)) and np.all(zero == np.rint(zero))
    q = oracle.quantize_codes(v, scale[:, None], zero[:, None], bits)
    assert np.all((q >= 0) & (q <= maxq)) and np.all(q == np.rint(q))


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_error_bounded_by_half_step_and_grid_roundtrip(bits):
    rng = np.random.default_rng(10 + bits)
    v = f32(rng.standard_normal((300, 128)) * 0.02)
    scale, zero = oracle.group_params(v, bits)
    q = oracle.quantize_codes(v, scale[:, None], zero[:, None], bits)
    dq = oracle.dequantize(q, scale[:, None], zero[:, None])
    # inside the range, |w - dq| <= scale/2, up to the fp32 rounding of the quotient
    # (relative 2^-24 of a value of at most maxq steps)
    maxq = 2 ** bits - 1
    assert np.all(np.abs(v - dq) <= scale[:, None] * (0.5 + maxq * 2.0 ** -23))
    # every grid point maps back to its own code
    maxq = 2 ** bits - 1
    codes = np.arange(maxq + 1, dtype=np.float64)[None, :]
    grid = oracle.dequantize(codes, scale[:, None], zero[:, None])
    back = oracle.quantize_codes(grid, scale[:, None], zero[:, None], bits)
    assert np.array_equal(back, np.broadcast_to(codes, back.shape))


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_rtn_equals_brute_force_nearest_grid_point(bits):
    rng = np.random.default_rng(20 + bits)
    W = f32(rng.standard_normal((64, 96)) * 0.05)
    codes, scales, zeros = oracle.rtn_minmax(W, bits, 32)
    maxq = 2 ** bits - 1
    for r in range(W.shape[0]):
        for c in range(W.shape[1]):
            g = c // 32
            s, z = scales[r, g], zeros[r, g]
            cand = np.arange(maxq + 1)
            dist = np.abs(W[r, c] - (cand - z) * s)
            best = np.flatnonzero(dist == dist.min())
            if len(best) == 1 and np.sort(dist)[1] - dist.min() > 1e-9 * s:
                assert codes[r, c] == best[0], (r, c)
            else:  # a tie: either neighbour is correct
                assert codes[r, c] in best or abs(np.sort(dist)[1] - dist.min()) <= 1e-9 * s


def test_all_zero_group_uses_unit_range():
    v = np.zeros((3, 16))
    scale, zero = oracle.group_params(v, 4)
    assert np.allclose(scale, f32(2.0 / 15))
    q = oracle.quantize_codes(v, scale[:, None], zero[:, None], 4)
    assert np.all(q == zero[:, None])
    assert np.all(oracle.dequantize(q, scale[:, None], zero[:, None]) == 0.0)


def test_one_signed_group_range_includes_zero():
    v = np.array([[0.5, 1.0, 2.0, 0.25]])  # all positive: xmin clamps to 0
    scale, zero = oracle.group_params(v, 4)
    assert zero[0] == 0 and np.isclose(scale[0], 2.0 / 15)
    v = -v
    scale, zero = oracle.group_params(v, 4)
    assert zero[0] == 15


def test_fp32_emulation_matches_native_fp32_arithmetic():
    """The decision precision is fp32; the emulation must be exact IEEE fp32."""
    rng = np.random.default_rng(7)
    a = rng.standard_normal(200000).astype(np.float32)
    b = (rng.uniform(0.001, 0.1, 200000)).astype(np.float32)
    assert np.array_equal(f32(a.astype(np.float64) / b.astype(np.float64)), (a / b).astype(np.float64))
    assert np.array_equal(f32(a.astype(np.float64) - b.astype(np.float64)), (a - b).astype(np.float64))
    assert np.array_equal(f32(a.astype(np.float64) * 15.0), (a * np.float32(15)).astype(np.float64))


def test_ties_round_half_even():
    scale = np.array([1.0])
    zero = np.array([8.0])
    w = np.array([0.5, 1.5, 2.5, -0.5, -1.5])
    q = oracle.quantize_codes(w, scale, zero, 4)
    assert list(q) == [8, 10, 10, 8, 6]


def test_symmetric_variant_matches_signed_range():
    """Symmetric codes minus the mid-point span the signed range [-2^(b-1), 2^(b-1)-1]."""
    rng = np.random.default_rng(3)
    v = rng.standard_normal((50, 32))
    for bits in (3, 4, 8):
        scale, zero = oracle.group_params(v, bits, sym=True)
        assert np.all(zero == 2 ** (bits - 1))
        q = oracle.quantize_codes(v, scale[:, None], zero[:, None], bits) - zero[:, None]
        assert q.min() >= -(2 ** (bits - 1)) and q.max() <= 2 ** (bits - 1) - 1
        # zero maps to zero exactly
        assert np.all(oracle.quantize_codes(np.zeros(50), scale, zero, bits) == zero)
