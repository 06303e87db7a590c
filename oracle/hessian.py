"""Layer Hessian from calibration activations (oracle, test infrastructure only).

"GPTQ deep dive", §3.1 step 1: with the layer input X (channels x tokens), the
layer Hessian is H = 2 X X^T (the damping term lambda*I is added by
``prepare``).  The activations arrive token-major, X_t [tokens, channels], so
X X^T = X_t^T X_t = sum over tokens t of x_t x_t^T.

S is the raw sum (no 1/N): accumulation stays additive over calibration
chunks and GPTQ's output is invariant to a positive scaling of H because the
damping scales with it.
"""
from __future__ import annotations

from typing import Iterable

import numpy as np


def hessian_S(chunks: Iterable[np.ndarray], n: int | None = None) -> np.ndarray:
    """S = sum over chunks of X_c^T X_c in fp64; each X_c is [tokens, n]."""
    S = None
    for X in chunks:
        X64 = np.asarray(X, dtype=np.float64)
        if S is None:
            S = np.zeros((X64.shape[1], X64.shape[1]), dtype=np.float64)
        S += X64.T @ X64
    if S is None:
        if n is None:
            raise ValueError("no calibration chunks and no n")
        S = np.zeros((n, n), dtype=np.float64)
    return S


def hessian(chunks: Iterable[np.ndarray]) -> np.ndarray:
    """H = 2 X X^T (undamped)."""
    return 2.0 * hessian_S(chunks)
