"""Pins for the oracle's dequantized-weight product (CPU only).

The product Y = X W_q^T with W_q[r, c] = scale[r, g(c)] * (q[r, c] - zero[r, g(c)])
("Quantized deployment, 1.5 TB to 250 GB" §2.1; "LLM quantization principles"
§5.2) is pinned here by what does not depend on the oracle's own code: a
brute-force loop that reads the bits out of the words by hand, closed forms
(codes at the zero-point give 0; unit scale and zero-point give the integer
product), the printed 8-bit worked example, the RTN error bound against the
unquantized product, and invariance under a consistent column permutation.
"""
import json
import os

import numpy as np
import pytest

import oracle


def _codes_bit_by_bit(words, n, bits):
    """Code c of a row: bits [c*b, c*b + b) of the little-endian word stream."""
    out = []
    for c in range(n):
        v = 0
        for k in range(bits):
            pos = c * bits + k
            v |= ((int(words[pos // 32]) >> (pos % 32)) & 1) << k
        out.append(v)
    return out


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_dequant_matmul_brute_force(bits):
    rng = np.random.default_rng(30 + bits)
    m, n, t, G = 3, 19, 2, 4
    codes = rng.integers(0, 2 ** bits, (m, n))
    perm = rng.permutation(n)
    pos = np.empty(n, dtype=np.int64)
    pos[perm] = np.arange(n)
    g_idx = pos // G  # groups follow a processing order, so g_idx is not monotone
    ng = (n + G - 1) // G
    scales = rng.uniform(0.01, 0.1, (m, ng))
    zeros = rng.integers(0, 2 ** bits, (m, ng)).astype(np.float64)
    X = rng.standard_normal((t, n))
    packed = oracle.pack_ref(codes, bits)
    Y = oracle.dequant_matmul(X, packed, n, bits, scales, zeros, g_idx)
    for r in range(m):
        q = _codes_bit_by_bit(packed[r], n, bits)
        for tt in range(t):
            acc = 0.0
            for c in range(n):
                g = int(g_idx[c])
                acc += X[tt, c] * scales[r, g] * (q[c] - zeros[r, g])
            assert abs(Y[tt, r] - acc) <= 1e-12 * max(1.0, abs(acc))


def test_codes_at_zero_point_give_zero():
    rng = np.random.default_rng(1)
    m, n, G, bits = 5, 40, 8, 4
    zeros = rng.integers(0, 16, (m, n // G)).astype(np.float64)
    codes = np.repeat(zeros, G, axis=1).astype(np.int64)
    packed = oracle.pack_ref(codes, bits)
    Y = oracle.dequant_matmul(rng.standard_normal((3, n)), packed, n, bits,
                              rng.uniform(0.1, 1.0, zeros.shape), zeros, np.arange(n) // G)
    assert np.all(Y == 0.0)


def test_unit_scale_zero_point_gives_integer_product():
    rng = np.random.default_rng(2)
    m, n, bits = 6, 33, 3
    codes = rng.integers(0, 8, (m, n))
    X = rng.integers(-50, 50, (4, n)).astype(np.float64)
    packed = oracle.pack_ref(codes, bits)
    Y = oracle.dequant_matmul(X, packed, n, bits, np.ones((m, 1)), np.zeros((m, 1)),
                              np.zeros(n, dtype=np.int64))
    expect = [[sum(int(X[t, c]) * int(codes[r, c]) for c in range(n)) for r in range(m)]
              for t in range(4)]
    assert np.array_equal(Y, np.array(expect, dtype=np.float64))


def test_constant_zero_point_subtracts_row_sums():
    """Y = s (X q^T - z rowsum(X)) for one scale s and zero-point z."""
    rng = np.random.default_rng(3)
    m, n, bits, s, z = 4, 24, 4, 0.125, 7.0
    codes = rng.integers(0, 16, (m, n))
    X = rng.integers(-9, 9, (5, n)).astype(np.float64)
    Y = oracle.dequant_matmul(X, oracle.pack_ref(codes, bits), n, bits, np.full((m, 1), s),
                              np.full((m, 1), z), np.zeros(n, dtype=np.int64))
    xq = np.array([[sum(int(X[t, c]) * int(codes[r, c]) for c in range(n)) for r in range(m)]
                   for t in range(5)], dtype=np.float64)
    rows = np.array([sum(X[t]) for t in range(5)])
    assert np.array_equal(Y, s * (xq - z * rows[:, None]))


def test_worked_example_end_codes_recover_range(golden_dir):
    """8-bit codes of [-2.5, 3.7]: codes 0 and 255 dequantize to the range ends,
    within half a quantization step."""
    g = json.load(open(os.path.join(golden_dir, "worked_example_minmax_int8.json")))
    lo, hi = g["range"]
    scale, zero = oracle.group_params(np.array([[lo, hi]]), g["bits"])
    packed = oracle.pack_ref(np.array([[0, 2 ** g["bits"] - 1]]), g["bits"])
    w = oracle.dequant_weights(packed, 2, g["bits"], scale[:, None], zero[:, None],
                               np.zeros(2, dtype=np.int64))
    assert abs(w[0, 0] - lo) <= 0.5 * scale[0] and abs(w[0, 1] - hi) <= 0.5 * scale[0]


@pytest.mark.parametrize("bits,G", [(8, 16), (4, 8), (3, 32)])
def test_rtn_product_within_step_bound(bits, G):
    """With RTN codes of W, each dequantized weight is within one step (scale) of
    the weight (half a step from rounding, at most one where the clamp binds), so
    |X W_q^T - X W^T| <= |X| scale elementwise."""
    rng = np.random.default_rng(4 + bits)
    m, n, t = 7, 96, 5
    W = rng.standard_normal((m, n)) * 0.02
    X = rng.standard_normal((t, n))
    codes, scales, zeros = oracle.rtn_minmax(W, bits, G)
    g_idx = np.arange(n) // G
    Y = oracle.dequant_matmul(X, oracle.pack_ref(codes.astype(np.int64), bits), n, bits, scales,
                              zeros, g_idx)
    bound = np.abs(X) @ scales[:, g_idx].T
    err = np.abs(Y - X @ W.T)
    assert np.all(err <= bound * (1 + 1e-9))
    # weight by weight: half a step wherever the code is not at the clamp ends, which
    # an off-by-one zero-point or another group's scale breaks
    Wq = oracle.dequant_weights(oracle.pack_ref(codes.astype(np.int64), bits), n, bits, scales,
                                zeros, g_idx)
    inner = (codes > 0) & (codes < 2 ** bits - 1)
    assert inner.mean() > 0.5
    assert np.all(np.abs(Wq - W)[inner] <= 0.5 * scales[:, g_idx][inner] * (1 + 1e-6))


def test_column_permutation_invariance():
    rng = np.random.default_rng(5)
    m, n, bits, G = 9, 64, 4, 16
    codes = rng.integers(0, 16, (m, n))
    scales = rng.uniform(0.01, 0.1, (m, n // G))
    zeros = rng.integers(0, 16, (m, n // G)).astype(np.float64)
    g_idx = np.arange(n) // G
    X = rng.standard_normal((3, n))
    Y = oracle.dequant_matmul(X, oracle.pack_ref(codes, bits), n, bits, scales, zeros, g_idx)
    p = rng.permutation(n)
    Yp = oracle.dequant_matmul(X[:, p], oracle.pack_ref(codes[:, p], bits), n, bits, scales,
                               zeros, g_idx[p])
    assert np.allclose(Y, Yp, rtol=0, atol=1e-12)
