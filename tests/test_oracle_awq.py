"""Pins for the oracle's AWQ-lite scale search and awq_clip (CPU only).

Pinned by what does not come from the oracle's code: the scale formula at
hand-picked values and at alpha = 0 and 1; the rescaling leaving the layer's
output unchanged when nothing is rounded (8-bit codes in groups of 8 make the
rounding negligible), which fixes the direction of the rescaling; the error
through S against the error over the tokens, and the alpha search against a
brute-force loop; clip ratio 1 being plain group min-max and the search never
being worse than it; a planted outlier weight being clipped; and AWQ beating
plain min-max on a layer with outlier activation channels.
"""
import numpy as np
import pytest

import oracle
from oracle import awq
from oracle.quantizer import f32


def _layer(rng, m, n, t, outliers=()):
    W = rng.standard_normal((m, n)) * 0.02
    X = rng.standard_normal((t, n))
    for c in outliers:
        X[:, c] *= 30.0
    return W, X


def test_scale_formula_hand_values():
    xm, wm = np.array([1.0, 4.0]), np.array([2.0, 0.5])
    assert np.allclose(awq.awq_scales(xm, wm, 0.5), [1.0 / np.sqrt(2.0), 2.0 / np.sqrt(0.5)])
    assert np.allclose(awq.awq_scales(xm, wm, 0.0), 1.0 / wm)
    assert np.allclose(awq.awq_scales(xm, wm, 1.0), xm)
    assert np.all(np.isfinite(awq.awq_scales(np.array([0.0]), np.array([0.0]), 0.3)))


def test_rescaling_preserves_the_output_when_nothing_is_rounded():
    rng = np.random.default_rng(0)
    W, X = _layer(rng, 16, 64, 200, outliers=(3,))
    S = X.T @ X
    ref = np.linalg.norm(X @ W.T) ** 2
    lite = awq.awq_lite(W, S, awq.channel_absmean(X), 8, 8)
    assert np.all(lite.losses < 1e-4 * ref)
    # and with 3-bit codes the error is far from negligible: the pin has teeth
    lite3 = awq.awq_lite(W, S, awq.channel_absmean(X), 3, 8)
    assert np.all(lite3.losses > 1e-3 * ref)


def test_error_through_S_equals_error_over_tokens():
    rng = np.random.default_rng(1)
    W, X = _layer(rng, 8, 32, 100)
    D = rng.standard_normal(W.shape) * 1e-3
    direct = sum(float(np.dot(X[t] @ D.T, X[t] @ D.T)) for t in range(X.shape[0]))
    assert abs(awq.output_error(D, X.T @ X) - direct) <= 1e-12 * direct


def test_alpha_search_against_brute_force():
    rng = np.random.default_rng(2)
    m, n, G = 6, 16, 8
    W, X = _layer(rng, m, n, 64, outliers=(5,))
    S = X.T @ X
    xm = np.array([sum(abs(X[t, c]) for t in range(64)) / 64 for c in range(n)])
    wm = np.array([sum(abs(W[r, c]) for r in range(m)) / m for c in range(n)])
    lite = awq.awq_lite(W, S, xm, 3, G)
    losses = []
    for a in awq.ALPHAS:
        s = np.maximum(xm, 1e-8) ** a / np.maximum(wm, 1e-8) ** (1 - a)
        q, sc, z = awq.quantize_groups(W * s, 3, G)
        Weff = awq.dequant_groups(q, sc, z, G) / s
        err = 0.0
        for t in range(64):
            for r in range(m):
                err += (sum(X[t, c] * (Weff[r, c] - W[r, c]) for c in range(n))) ** 2
        losses.append(err)
    assert np.allclose(lite.losses, losses, rtol=1e-9)
    assert lite.alpha == awq.ALPHAS[int(np.argmin(losses))]


def test_clip_ratio_one_is_plain_minmax_and_the_search_never_worse():
    rng = np.random.default_rng(3)
    W, X = _layer(rng, 12, 64, 128, outliers=(7, 40))
    S = X.T @ X
    s = awq.awq_scales(awq.channel_absmean(X), awq.weight_absmean(W), 0.5)
    clip = awq.awq_clip(W, S, s, 4, 16)
    q, sc, z = awq.quantize_groups(W * s, 4, 16)
    c1, s1, z1 = oracle.rtn_minmax(W * s, 4, 16)
    assert np.array_equal(q, c1) and np.array_equal(sc, s1) and np.array_equal(z, z1)
    chosen = np.take_along_axis(clip.errors, clip.ratio_idx[:, :, None], axis=2)[:, :, 0]
    assert np.all(chosen <= clip.errors[:, :, 0])
    assert np.all(chosen == clip.errors.min(axis=2))


def test_clip_group_error_over_tokens_with_rescaled_inputs():
    """errors[r, g, k] is the group's share of the output error over the
    calibration tokens, with the activations divided by s: the sum over tokens
    of (X'[t, g] . d_g)^2, X' = X diag(1/s), d_g the candidate's rounding error
    in the rescaled space, summed here term by term."""
    rng = np.random.default_rng(6)
    m, n, t, G, bits = 3, 16, 40, 8, 3
    W, X = _layer(rng, m, n, t, outliers=(2,))
    s = rng.uniform(0.5, 2.0, n)
    clip = awq.awq_clip(W, X.T @ X, s, bits, G)
    Ws = f32(W * s)
    amax = np.stack([np.abs(Ws[:, g0:g0 + G]).max(axis=1) for g0 in range(0, n, G)], axis=1)
    for k, ratio in enumerate(awq.CLIP_RATIOS):
        bound = f32(amax * f32(ratio))
        q, sc, z = awq.quantize_groups(Ws, bits, G, ranges=bound)
        d = awq.dequant_groups(q, sc, z, G) - Ws
        for r in range(m):
            for gi, g0 in enumerate(range(0, n, G)):
                err = 0.0
                for tt in range(t):
                    acc = 0.0
                    for c in range(g0, g0 + G):
                        acc += (X[tt, c] / s[c]) * d[r, c]
                    err += acc * acc
                assert abs(clip.errors[r, gi, k] - err) <= 1e-10 * max(err, 1e-30), (r, gi, k)


def test_clip_parameters_come_from_the_clamped_range():
    """The chosen clip c bounds the range the group's parameters are computed
    from: scale = (min(c, max v) - max(-c, min v)) / maxq with 0 kept in the
    range (fp32, as every decision), while the values themselves are not
    clamped (a weight beyond c takes the end code)."""
    rng = np.random.default_rng(8)
    m, n, G, bits = 6, 32, 32, 3
    W = rng.standard_normal((m, n)) * 0.01
    W[:, 5] = 0.5
    clip = awq.awq_clip(W, np.eye(n) * 100.0, np.ones(n), bits, G)
    maxq = 2 ** bits - 1
    Ws = f32(W)
    for r in range(m):
        k = int(clip.ratio_idx[r, 0])
        assert k > 0
        c = f32(np.abs(Ws[r]).max() * f32(awq.CLIP_RATIOS[k]))
        hi = max(0.0, min(c, Ws[r].max()))
        lo = min(0.0, max(-c, Ws[r].min()))
        assert clip.scales[r, 0] == f32(f32(hi - lo) / maxq)
        assert clip.codes[r, 5] == maxq  # 0.5 lies beyond c: the top code
        # the unclamped value 0.5 alone decides its code: an in-range weight keeps
        # the code of its own value
        j = int(np.argmin(np.abs(Ws[r])))
        pre = f32(Ws[r, j] / clip.scales[r, 0])
        assert clip.codes[r, j] == np.clip(np.rint(pre) + clip.zeros[r, 0], 0, maxq)


def test_clip_cuts_a_planted_outlier():
    rng = np.random.default_rng(4)
    m, n, G = 4, 32, 32
    W = rng.standard_normal((m, n)) * 0.01
    W[:, 5] = 0.5  # one weight per row far outside the rest
    S = np.eye(n) * 100.0
    clip = awq.awq_clip(W, S, np.ones(n), 3, G)
    assert np.all(clip.ratio_idx[:, 0] > 0)


def test_awq_beats_plain_minmax_with_outlier_channels():
    rng = np.random.default_rng(5)
    m, n, G = 32, 256, 64
    W, X = _layer(rng, m, n, 512, outliers=(1, 17, 100, 200))
    S = X.T @ X
    lite = awq.awq_lite(W, S, awq.channel_absmean(X), 3, G)
    clip = awq.awq_clip(W, S, lite.s, 3, G)
    e_awq = awq.output_error(awq.awq_effective_weights(clip, lite.s, G) - W, S)
    c, sc, z = oracle.rtn_minmax(W, 3, G)
    e_rtn = awq.output_error(oracle.dequant_layer(c, sc, z, np.arange(n) // G) - W, S)
    assert lite.alpha > 0.0
    assert e_awq < 0.8 * e_rtn
