"""Pins for the oracle's layer-sequential MLP stack (CPU only).

What does not come from the oracle's own code: bf16 rounding of hand-picked
values, silu at points with a closed form, the zero-weight block (the
residual passes the input through unchanged), a brute-force recomputation of
the activations that feed each block's Hessians from the quantized weights of
the blocks before it (and that the unquantized weights would give a
different Hessian), gate and up sharing one Hessian, and the quantized stack
approaching the unquantized one as the bit width grows.
"""
import numpy as np
import pytest

import oracle
from oracle.stack import float_stack, quantize_stack, silu, to_bf16

DAMP = float(np.float32(0.01))


def test_to_bf16_hand_values():
    cases = {
        1.0: 1.0,
        1.0 + 2.0 ** -8: 1.0,                       # tie -> even (last bit 0)
        1.0 + 3 * 2.0 ** -8: 1.0 + 2.0 ** -6,       # tie -> even (round up)
        1.0 + 2.0 ** -8 + 2.0 ** -20: 1.0 + 2.0 ** -7,  # above the tie
        -3.0: -3.0,
        0.1: 0.10009765625,                         # 0x3DCD
        1000.0: 1000.0,
        1001.0: 1000.0,                             # spacing 4 at 2^9..2^10: 1001 -> 1000
        0.0: 0.0,
    }
    for a, b in cases.items():
        assert to_bf16(np.array([a]))[0] == b, a


def test_silu_closed_forms():
    assert silu(np.array([0.0]))[0] == 0.0
    assert abs(silu(np.array([1.0]))[0] - 1.0 / (1.0 + np.exp(-1.0))) < 1e-15
    assert abs(silu(np.array([40.0]))[0] - 40.0) < 1e-12
    assert abs(silu(np.array([-40.0]))[0]) < 1e-15
    g = np.linspace(-5, 5, 11)
    assert np.allclose(silu(g) - silu(-g), g)  # g s(g) + g s(-g) = g


def _weights(rng, d, f, blocks, sigma=0.05):
    return [(to_bf16(rng.standard_normal((f, d)) * sigma), to_bf16(rng.standard_normal((f, d)) * sigma),
             to_bf16(rng.standard_normal((d, f)) * sigma)) for _ in range(blocks)]


def test_zero_weights_pass_the_input_through():
    rng = np.random.default_rng(0)
    d, f = 16, 24
    x0 = to_bf16(rng.standard_normal((40, d)))
    W = [(np.zeros((f, d)), np.zeros((f, d)), np.zeros((d, f)))] * 2
    res = quantize_stack(x0, W, 4, 8, 8, DAMP, False)
    for b in res:
        assert np.all(b.gate.Wq == 0) and np.all(b.h == 0)
        assert np.array_equal(b.x_out, x0)


@pytest.mark.parametrize("desc_act", [False, True])
def test_hessians_come_from_the_quantized_network(desc_act):
    rng = np.random.default_rng(1)
    d, f, t = 32, 48, 96
    x0 = rng.standard_normal((t, d))
    W = _weights(rng, d, f, 2)
    res = quantize_stack(x0, W, 3, 16, 16, DAMP, desc_act)
    x = to_bf16(x0)
    for k, b in enumerate(res):
        # brute force: the block's inputs and the hidden activations, from the
        # dequantized weights, by explicit loops over the products
        assert np.array_equal(b.x_in, x)
        Wg = oracle.dequant_layer(b.gate.codes, b.gate.scales, b.gate.zeros, b.gate.g_idx)
        Wu = oracle.dequant_layer(b.up.codes, b.up.scales, b.up.zeros, b.up.g_idx)
        Wd = oracle.dequant_layer(b.down.codes, b.down.scales, b.down.zeros, b.down.g_idx)
        h = np.empty((t, f))
        for i in range(t):
            for j in range(f):
                gg = sum(x[i, c] * Wg[j, c] for c in range(d))
                uu = sum(x[i, c] * Wu[j, c] for c in range(d))
                h[i, j] = gg / (1.0 + np.exp(-gg)) * uu
        h = to_bf16(h)
        # equal up to where the two summation orders straddle a bf16 rounding boundary
        assert np.mean(b.h == h) > 0.99
        assert np.all(np.abs(b.h - h) <= 2.0 ** -7 * np.abs(h))
        # gate and up were quantized with the Hessian of the block input
        assert np.allclose(b.S_x, x.T @ x, rtol=1e-12, atol=1e-9)
        assert np.allclose(b.S_h, b.h.T @ b.h, rtol=1e-12, atol=1e-9)
        x = to_bf16(x + b.h @ Wd.T)
        assert np.array_equal(b.x_out, x)
    # the second block's Hessian differs from the one the unquantized first block gives
    _, x1_float = oracle.stack.block_forward(to_bf16(x0), *[np.asarray(w, np.float64) for w in W[0]])
    assert not np.allclose(res[1].S_x, x1_float.T @ x1_float, rtol=1e-6)


def test_gate_and_up_share_one_prepare():
    rng = np.random.default_rng(2)
    d, f = 24, 40
    x0 = rng.standard_normal((64, d))
    W = _weights(rng, d, f, 1)
    b = quantize_stack(x0, W, 4, 8, 8, DAMP, True)[0]
    assert np.array_equal(b.gate.perm, b.up.perm)
    assert np.array_equal(b.gate.perm, oracle.prepare(b.S_x, DAMP, True).perm)


def test_error_shrinks_with_bits():
    rng = np.random.default_rng(3)
    d, f = 32, 64
    x0 = rng.standard_normal((128, d))
    W = _weights(rng, d, f, 2)
    ref = float_stack(x0, W)
    errs = []
    for bits in (2, 3, 4, 8):
        out = quantize_stack(x0, W, bits, 16, 16, DAMP, False)[-1].x_out
        errs.append(np.linalg.norm(out - ref) / np.linalg.norm(ref))
    assert errs[0] > errs[1] > errs[2] > errs[3]
    assert errs[3] < 0.01
