"""Group-wise asymmetric min-max quantizer (oracle, test infrastructure only).

Sources:
* "LLM quantization principles: GPTQ, AWQ, GGUF", §2.1: q = round(x / scale)
  + zero_point; the linear min-max mapping scale = (max - min) / (qmax - qmin).
* "Quantized deployment, 1.5 TB to 250 GB", §2.1: dequantization
  r = (q - zero_point) * scale.
* "Calibration algorithms guide", §2.2: each group of weights gets its own
  min/max, hence its own scale and zero-point.

Conventions the pages leave open (parity unpinned by the pages; fixed here and
followed by the device path):
* the range is widened to include 0: [min(0, min v), max(0, max v)], so the
  zero-point lies in [0, maxq] and 0 is exactly representable;
* an all-zero group uses the range [-1, 1];
* zero = round((-xmin * maxq) / (xmax - xmin)) rather than round(-xmin / scale),
  a form that is stable at exact ties for bf16 inputs;
* codes are unsigned in [0, 2^bits - 1], clamped after adding the zero-point;
* rounding is round-half-to-even (IEEE rint) and every division is a true
  division, never a multiplication by a reciprocal;
* the decision precision is fp32 (see the package docstring); with
  ``exact=True`` every step is plain fp64 instead (no rounding to fp32
  anywhere), the reference against which an fp32 decision is shown to differ
  only at rounding ties.
"""
from __future__ import annotations

import numpy as np


def f32(x) -> np.ndarray:
    """Round fp64 values to the nearest fp32 value, returned as fp64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def _rounder(exact: bool):
    """The rounding applied after each step: to fp32 (the kernels' decision
    precision), or none (plain fp64)."""
    if exact:
        return lambda x: np.asarray(x, dtype=np.float64)
    return f32


def group_params(v: np.ndarray, bits: int, sym: bool = False, exact: bool = False):
    """Scale and zero-point of each row of ``v`` ([rows, group_len] current values).

    Returns (scale, zero), both fp64 arrays holding fp32 values (fp64 values
    with ``exact``); zero is integral.  Asymmetric: min-max range with 0
    included.  Symmetric: zero-point fixed at the middle of the code range,
    scale = 2*max|v| / maxq (the symmetric variant of "LLM quantization
    principles" §2.3, expressed on unsigned codes).
    """
    r = _rounder(exact)
    maxq = float(2 ** bits - 1)
    v32 = r(v)
    if sym:
        amax = np.abs(v32).max(axis=1)
        amax = np.where(amax == 0.0, 1.0, amax)
        scale = r(r(2.0 * amax) / maxq)
        zero = np.full_like(scale, np.floor((maxq + 1.0) / 2.0))
        return scale, zero
    xmin = np.minimum(v32.min(axis=1), 0.0)
    xmax = np.maximum(v32.max(axis=1), 0.0)
    degenerate = xmin == xmax
    xmin = np.where(degenerate, -1.0, xmin)
    xmax = np.where(degenerate, 1.0, xmax)
    span = r(xmax - xmin)
    scale = r(span / maxq)
    zero = np.rint(r(r(-xmin * maxq) / span))
    return scale, zero


def pre_round_value(w: np.ndarray, scale: np.ndarray, exact: bool = False) -> np.ndarray:
    """w / scale in fp32 (fp64 with ``exact``): the value whose rounding gives
    the code before the offset."""
    r = _rounder(exact)
    return r(r(w) / scale)


def quantize_codes(w: np.ndarray, scale: np.ndarray, zero: np.ndarray, bits: int,
                   exact: bool = False) -> np.ndarray:
    """q = clamp(round(w / scale) + zero, 0, maxq), ties to even; fp64 integral values."""
    maxq = float(2 ** bits - 1)
    return np.clip(np.rint(pre_round_value(w, scale, exact)) + zero, 0.0, maxq)


def dequantize(q: np.ndarray, scale: np.ndarray, zero: np.ndarray) -> np.ndarray:
    """r = (q - zero) * scale, in fp64 (exact for fp32 scale and small integers)."""
    return (np.asarray(q, dtype=np.float64) - zero) * scale
