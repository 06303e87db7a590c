"""AWQ-lite channel scaling and awq_clip (oracle, test infrastructure only).

"AWQ, MinMax, GPTQ calibration in Model Optimizer" (gtnt.cn news 115337) §3:
  * awq_lite: input channels and weights are rescaled by per-channel factors
    in opposite directions, which leaves the layer's output unchanged but moves
    the rounding error; the factors are s = x^alpha / w^(1 - alpha), with x and w
    the per-channel mean absolute values of the activations and of the weights,
    and alpha is searched over [0, 1] in steps of 0.1 for the smallest error
    between the scaled, quantized layer's output and the true output;
  * awq_clip: after scaling, each quantization group's upper clip value is
    searched in [0.5 amax, amax] in steps of 0.05 amax (amax = the group's
    largest magnitude), cutting true outliers so they do not stretch the scale;
  * awq_full = awq_lite then awq_clip.
"LLM quantization principles" §3.2: the weights are multiplied by s and the
activations divided by s (important channels, those with large activations,
get larger weights and so a smaller relative rounding error).

Readings (the pages leave these open):
  * x[c] = mean over tokens of |X[t, c]|; w[c] = mean over output rows of
    |W[r, c]|; both floored at 1e-8 so that s is finite for dead channels;
  * W' = W diag(s), X' = X diag(1/s) (§3.2's direction; §3's sentence reads the
    other way round, but its formula for s only protects salient channels in
    this direction);
  * the quantizer is the group min-max quantizer of ``quantizer.py`` applied
    to W' (no compensation);
  * the error is the squared Frobenius norm ||X (W_eff - W)^T||^2 over the
    calibration tokens, W_eff = dequant(Q(W')) diag(1/s), computed through
    S = X^T X as sum((D S) * D) with D = W_eff - W (the same number);
  * clip: the candidate c_k = (1 - 0.05 k) amax, k = 0..10 (formed in fp32,
    like every value that decides a code), limits the range
    the group's parameters are computed from (values clamped to [-c_k, c_k]);
    the codes of the unclamped values are clamped to the code range as usual;
    the error of a candidate is that of the group alone, d S'_gg d^T with
    S' = diag(1/s) S diag(1/s) the scaled inputs' second moments and d the
    group's error in the scaled space;
  * ties (equal errors) keep the first candidate: the smallest alpha, the
    largest clip.
Everything is fp64 except the quantizer's decisions, which are fp32 as in
``quantizer.py``.
"""
from __future__ import annotations

import dataclasses

import numpy as np

from .quantizer import dequantize, f32, group_params, quantize_codes

ALPHAS = np.arange(11) / 10.0
CLIP_RATIOS = 1.0 - 0.05 * np.arange(11)
FLOOR = 1e-8


def channel_absmean(X: np.ndarray) -> np.ndarray:
    """Mean over tokens of |X[t, c]| per input channel c."""
    return np.abs(np.asarray(X, dtype=np.float64)).mean(axis=0)


def weight_absmean(W: np.ndarray) -> np.ndarray:
    """Mean over output rows of |W[r, c]| per input channel c."""
    return np.abs(np.asarray(W, dtype=np.float64)).mean(axis=0)


def awq_scales(x_mean: np.ndarray, w_mean: np.ndarray, alpha: float) -> np.ndarray:
    x = np.maximum(np.asarray(x_mean, np.float64), FLOOR)
    w = np.maximum(np.asarray(w_mean, np.float64), FLOOR)
    return x ** alpha / w ** (1.0 - alpha)


def _groups(n: int, G: int):
    G = n if G <= 0 else G
    return [(g0, min(n, g0 + G)) for g0 in range(0, n, G)]


def quantize_groups(Ws: np.ndarray, bits: int, G: int, sym: bool = False,
                    ranges: np.ndarray | None = None):
    """Group min-max quantization of Ws [m, n]; ``ranges`` [m, ngroups]: clip
    values c (parameters from the values clamped to [-c, c]), or None.
    Returns (codes, scales, zeros) with groups of consecutive columns."""
    Ws = np.asarray(Ws, np.float64)
    m, n = Ws.shape
    gs = _groups(n, G)
    codes = np.zeros((m, n))
    scales = np.zeros((m, len(gs)))
    zeros = np.zeros((m, len(gs)))
    for k, (g0, g1) in enumerate(gs):
        v = Ws[:, g0:g1]
        basis = v if ranges is None else np.clip(v, -ranges[:, k:k + 1], ranges[:, k:k + 1])
        scale, zero = group_params(basis, bits, sym)
        scales[:, k], zeros[:, k] = scale, zero
        codes[:, g0:g1] = quantize_codes(v, scale[:, None], zero[:, None], bits)
    return codes, scales, zeros


def dequant_groups(codes, scales, zeros, G):
    m, n = codes.shape
    out = np.zeros((m, n))
    for k, (g0, g1) in enumerate(_groups(n, G)):
        out[:, g0:g1] = dequantize(codes[:, g0:g1], scales[:, k:k + 1], zeros[:, k:k + 1])
    return out


def output_error(D: np.ndarray, S: np.ndarray) -> float:
    """||X D^T||_F^2 = sum((D S) * D) for S = X^T X (full, symmetric)."""
    D = np.asarray(D, np.float64)
    return float(np.sum((D @ S) * D))


@dataclasses.dataclass
class AWQLite:
    alpha: float
    s: np.ndarray          # [n] chosen scales
    losses: np.ndarray     # [len(ALPHAS)] output error of each alpha


def awq_lite(W: np.ndarray, S: np.ndarray, x_mean: np.ndarray, bits: int, G: int,
             sym: bool = False, alphas: np.ndarray = ALPHAS) -> AWQLite:
    """Search alpha; S = X^T X (full symmetric, fp64)."""
    W = np.asarray(W, np.float64)
    w_mean = weight_absmean(W)
    losses = np.zeros(len(alphas))
    for i, a in enumerate(alphas):
        s = awq_scales(x_mean, w_mean, a)
        q, sc, z = quantize_groups(W * s, bits, G, sym)
        D = dequant_groups(q, sc, z, G) / s - W
        losses[i] = output_error(D, S)
    best = int(np.argmin(losses))  # first minimum: the smallest alpha
    return AWQLite(float(alphas[best]), awq_scales(x_mean, w_mean, alphas[best]), losses)


@dataclasses.dataclass
class AWQClip:
    codes: np.ndarray     # [m, n] codes of W' = W diag(s)
    scales: np.ndarray    # [m, ngroups]
    zeros: np.ndarray
    ratio_idx: np.ndarray  # [m, ngroups] chosen k (clip = (1 - 0.05 k) amax)
    errors: np.ndarray     # [m, ngroups, len(ratios)] group errors d S'_gg d^T


def awq_clip(W: np.ndarray, S: np.ndarray, s: np.ndarray, bits: int, G: int, sym: bool = False,
             ratios: np.ndarray = CLIP_RATIOS) -> AWQClip:
    """Per (row, group) clip search on W' = W diag(s); S = X^T X (full)."""
    W = np.asarray(W, np.float64)
    s = np.asarray(s, np.float64)
    # W' in the quantizer's decision precision (fp32), and the clip bounds with it
    Ws = f32(W * s)
    Sp = S / np.outer(s, s)  # second moments of X' = X diag(1/s)
    m, n = Ws.shape
    gs = _groups(n, G)
    errs = np.zeros((m, len(gs), len(ratios)))
    amax = np.stack([np.abs(Ws[:, g0:g1]).max(axis=1) for g0, g1 in gs], axis=1)

    def bound(r):
        return f32(amax * f32(r))

    for k, ratio in enumerate(ratios):
        q, sc, z = quantize_groups(Ws, bits, G, sym, ranges=bound(ratio))
        d = dequant_groups(q, sc, z, G) - Ws
        for gi, (g0, g1) in enumerate(gs):
            dg = d[:, g0:g1]
            errs[:, gi, k] = np.einsum("ri,ij,rj->r", dg, Sp[g0:g1, g0:g1], dg)
    ridx = np.argmin(errs, axis=2)  # first minimum: the largest clip
    codes, scales, zeros = quantize_groups(Ws, bits, G, sym, ranges=bound(ratios[ridx]))
    return AWQClip(codes, scales, zeros, ridx, errs)


def awq_effective_weights(clip: AWQClip, s: np.ndarray, G: int) -> np.ndarray:
    """W_eff = dequant(Q(W')) diag(1/s): what the quantized layer multiplies X by."""
    return dequant_groups(clip.codes, clip.scales, clip.zeros, G) / np.asarray(s, np.float64)
