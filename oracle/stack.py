"""Layer-sequential GPTQ over a stack of MLP blocks (oracle, test infrastructure only).

"GPTQ deep dive" (hncyxsy.com news 243429) §3.1 step 4 and "AWQ, MinMax, GPTQ
calibration in Model Optimizer" (gtnt.cn news 115337) §4: the layers of a model
are quantized one after another, and the calibration inputs of a layer are the
outputs of the network whose earlier layers are already quantized, so each
layer's Hessian sees the error of the layers before it.  Layers that read the
same input (gate and up) share one Hessian.

The stack here is a synthetic Llama-style MLP block with a residual, repeated
(this project's stand-in for a model; the pages name the layers, not the block):

    g = x Wg_q^T,  u = x Wu_q^T            gate, up: Hessian of x
    h = bf16(silu(g) * u)                   silu(g) = g / (1 + e^-g)
    y = h Wd_q^T                            down: Hessian of h
    x' = bf16(x + y)

Activations are bf16 between layers (the workloads' activation type), rounded
once from the exact value here (``to_bf16``).  Everything else is fp64.  The
products use the dequantized weights W_q = scale * (q - zero) ("Quantized
deployment, 1.5 TB to 250 GB" §2.1) of the layers already quantized.
"""
from __future__ import annotations

import dataclasses
from typing import List, Sequence, Tuple

import numpy as np

from .gptq import dequant_layer, gptq_quantize
from .hessian import hessian_S
from .prepare import prepare


def to_bf16(a: np.ndarray) -> np.ndarray:
    """Round to the nearest bf16 value (8 significant bits), ties to even; fp64 out."""
    a = np.asarray(a, dtype=np.float64)
    m, e = np.frexp(a)  # a = m 2^e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)


def silu(g: np.ndarray) -> np.ndarray:
    g = np.asarray(g, dtype=np.float64)
    return g / (1.0 + np.exp(-g))


@dataclasses.dataclass
class LayerQuant:
    codes: np.ndarray
    scales: np.ndarray
    zeros: np.ndarray
    g_idx: np.ndarray
    perm: np.ndarray
    Wq: np.ndarray  # dequantized, original column order


@dataclasses.dataclass
class BlockResult:
    x_in: np.ndarray  # bf16 values (fp64 array)
    S_x: np.ndarray   # Hessian sum of x_in (shared by gate and up)
    gate: LayerQuant
    up: LayerQuant
    h: np.ndarray
    S_h: np.ndarray
    down: LayerQuant
    x_out: np.ndarray


def quantize_with(S: np.ndarray, W: np.ndarray, bits: int, group_size: int, block_size: int,
                  perc_damp: float, desc_act: bool, sym: bool = False) -> LayerQuant:
    """One layer's GPTQ given the Hessian sum S of its calibration inputs."""
    P = prepare(S, perc_damp, desc_act)
    r = gptq_quantize(W, P.U, bits, group_size, block_size, P.perm, P.dead, sym)
    return LayerQuant(r.codes, r.scales, r.zeros, r.g_idx, P.perm,
                      dequant_layer(r.codes, r.scales, r.zeros, r.g_idx))


def block_forward(x: np.ndarray, Wg_q: np.ndarray, Wu_q: np.ndarray,
                  Wd_q: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """(h, x') of one block with the given (dequantized) weights."""
    h = to_bf16(silu(x @ Wg_q.T) * (x @ Wu_q.T))
    return h, to_bf16(x + h @ Wd_q.T)


def quantize_stack(x0: np.ndarray, weights: Sequence[Tuple[np.ndarray, np.ndarray, np.ndarray]],
                   bits: int, group_size: int, block_size: int, perc_damp: float,
                   desc_act: bool, sym: bool = False) -> List[BlockResult]:
    """Quantize every block in order, each from the quantized network's activations."""
    x = to_bf16(x0)
    out = []
    for Wg, Wu, Wd in weights:
        S_x = hessian_S([x])
        gate = quantize_with(S_x, Wg, bits, group_size, block_size, perc_damp, desc_act, sym)
        up = quantize_with(S_x, Wu, bits, group_size, block_size, perc_damp, desc_act, sym)
        h = to_bf16(silu(x @ gate.Wq.T) * (x @ up.Wq.T))
        S_h = hessian_S([h])
        down = quantize_with(S_h, Wd, bits, group_size, block_size, perc_damp, desc_act, sym)
        x_next = to_bf16(x + h @ down.Wq.T)
        out.append(BlockResult(x, S_x, gate, up, h, S_h, down, x_next))
        x = x_next
    return out


def float_stack(x0: np.ndarray, weights) -> np.ndarray:
    """The unquantized stack's output (same bf16 rounding points)."""
    x = to_bf16(x0)
    for Wg, Wu, Wd in weights:
        _, x = block_forward(x, np.asarray(Wg, np.float64), np.asarray(Wu, np.float64),
                             np.asarray(Wd, np.float64))
    return x
