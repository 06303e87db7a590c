"""Dequantized-weight matrix product (oracle, test infrastructure only).

"Quantized deployment, 1.5 TB to 250 GB" (lmnt.cn news 123823) §2.1: a stored
code q is turned back into a real value as (q - zero_point) * scale.  "LLM
quantization principles: GPTQ, AWQ, GGUF" (0539edu.com news 6111416) §5.2: at
inference the 4-bit weights are dequantized before the matrix product, and
fusing the two is what keeps the dequantization from costing more than the
low-bit weights save.  This is that product, written as its definition:

    Y[t, r] = sum_c X[t, c] * scale[r, g(c)] * (q[r, c] - zero[r, g(c)])

with q read from the packed layout of ``pack.py`` and g(c) = g_idx[c], the
group of original column c (with desc_act the groups follow the processing
order, so g_idx is not monotone).  fp64 throughout.
"""
from __future__ import annotations

import numpy as np

from .pack import unpack_ref


def dequant_weights(packed: np.ndarray, n: int, bits: int, scales: np.ndarray,
                    zeros: np.ndarray, g_idx: np.ndarray) -> np.ndarray:
    """W_q [m, n] in fp64 from packed codes and per-group scale / zero-point."""
    q = unpack_ref(packed, n, bits).astype(np.float64)
    g = np.asarray(g_idx, dtype=np.int64)
    s = np.asarray(scales, dtype=np.float64)[:, g]
    z = np.asarray(zeros, dtype=np.float64)[:, g]
    return s * (q - z)


def dequant_matmul(X: np.ndarray, packed: np.ndarray, n: int, bits: int, scales: np.ndarray,
                   zeros: np.ndarray, g_idx: np.ndarray) -> np.ndarray:
    """Y [tokens, m] = X [tokens, n] @ W_q^T, fp64."""
    Wq = dequant_weights(packed, n, bits, scales, zeros, g_idx)
    return np.asarray(X, dtype=np.float64) @ Wq.T
