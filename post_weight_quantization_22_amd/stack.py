"""Layer-sequential GPTQ over a stack of MLP blocks, as a sequence of C-ABI calls.

"GPTQ deep dive" (hncyxsy.com news 243429) §3.1 step 4 and "AWQ, MinMax, GPTQ
calibration in Model Optimizer" (gtnt.cn news 115337) §4: layers are quantized
in order, each on the calibration activations produced by the network whose
earlier layers are already quantized; layers that read the same input share its
Hessian.  The block is a Llama-style MLP with a residual:

    g = x Wg_q^T, u = x Wu_q^T       gate, up: one Hessian of x, one prepare
    h = bf16(silu(g) * u)            gptq_swiglu
    y = h Wd_q^T                     down: Hessian of h
    x' = bf16(x + y)                 gptq_residual_add

Every step runs in libgptq_mi355x.so (Hessian, prepare, quantize, processing-
order packing, the products, the elementwise steps); this module allocates the
caller-owned buffers and issues the calls on one stream.  Activations stay
resident in HBM (x and h of the current block); the products run over token
chunks so their fp32 outputs stay small.  The products multiply by the
quantized weights either as a dense bf16 matrix dequantized once per layer
(gptq_dequantize + gptq_gemm_bf16, the default: the calibration set is large,
so no tile should dequantize again) or straight from the packed codes
(gptq_dequant_gemm); both form the same weights, bf16(fma(q, s, -(z s))).
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence, Tuple

import torch

from . import _lib, pipeline


@dataclasses.dataclass
class QuantizedLayer:
    buf: pipeline.LayerBuffers  # codes, scales, zeros, g_idx (original order), U, perm
    packed: torch.Tensor        # processing-order packing, the product's input
    perm: Optional[torch.Tensor]  # None when the processing order is the identity
    wq: Optional[torch.Tensor] = None  # dense bf16 weights, processing order (dense products)


@dataclasses.dataclass
class QuantizedBlock:
    gate: QuantizedLayer
    up: QuantizedLayer
    down: QuantizedLayer
    x_in: Optional[torch.Tensor] = None  # kept on request (tests)
    h: Optional[torch.Tensor] = None


class _Products:
    """Preallocated outputs and workspaces of the chunked products."""

    def __init__(self, device):
        self.device = device
        self.ws = {}
        self.out = {}
        self.xp = {}

    def get(self, tokens: int, m: int, n: int, has_perm: bool, slot: str, need_ws: bool = True):
        key = (tokens, m, n, has_perm)
        if need_ws and key not in self.ws:
            nb = _lib.gptq_dequant_gemm_workspace_size(tokens, m, n, has_perm)
            self.ws[key] = torch.empty(max(nb, 1), dtype=torch.uint8, device=self.device)
        okey = (tokens, m, slot)
        if okey not in self.out:
            self.out[okey] = torch.empty((tokens, m), dtype=torch.float32, device=self.device)
        return self.ws.get(key), self.out[okey]


def _packed(buf: pipeline.LayerBuffers, desc_act: bool, dense: bool, stream) -> QuantizedLayer:
    nw = -(-(buf.n * buf.cfg.bits) // 32)
    packed = torch.empty((buf.m, nw), dtype=torch.int32, device=buf.codes.device)
    perm = buf.perm if desc_act else None
    _lib.gptq_pack_ordered(buf.codes, buf.cfg.bits, perm, packed, stream=stream)
    wq = None
    if dense:
        ldw = -(-buf.n // 8) * 8
        wq = torch.empty((buf.m, ldw), dtype=torch.bfloat16, device=packed.device)[:, :buf.n]
        _lib.gptq_dequantize(packed, buf.cfg.bits, buf.cfg.group_size, buf.scales, buf.zeros,
                             buf.n, wq, stream=stream)
    return QuantizedLayer(buf, packed, perm, wq)


def _gathered(prod: _Products, X: torch.Tensor, perm: Optional[torch.Tensor], slot: str,
              stream) -> torch.Tensor:
    """X in the layers' processing order (X itself without desc_act), formed
    once for every layer that reads it."""
    if perm is None:
        return X
    key = (X.shape[0], X.shape[1], slot)
    if key not in prod.xp:
        ldxp = -(-X.shape[1] // 8) * 8
        prod.xp[key] = torch.empty((X.shape[0], ldxp), dtype=torch.bfloat16,
                                   device=prod.device)[:, :X.shape[1]]
    Xp = prod.xp[key]
    _lib.gptq_gather_columns(X, perm, Xp, stream=stream)
    return Xp


def _product(prod: _Products, Xp: torch.Tensor, L: QuantizedLayer, slot: str,
             stream) -> torch.Tensor:
    """Y = X W_q^T from the activations already in L's processing order."""
    ws, Y = prod.get(Xp.shape[0], L.buf.m, L.buf.n, False, slot, need_ws=L.wq is None)
    if L.wq is not None:
        _lib.gptq_gemm_bf16(Xp, L.wq, Y, stream=stream)
    else:
        _lib.gptq_dequant_gemm(Xp, L.packed, L.buf.cfg.bits, L.buf.cfg.group_size, L.buf.scales,
                               L.buf.zeros, Y, perm=None, ws=ws, stream=stream)
    return Y


def quantize_stack(x0: torch.Tensor, weights: Sequence[Tuple[torch.Tensor, torch.Tensor,
                                                             torch.Tensor]],
                   cfg: _lib.GPTQConfig, chunk_tokens: int = 16384, keep: bool = False,
                   stream=None, marks: Optional[list] = None, dense: bool = True
                   ) -> Tuple[List[QuantizedBlock], torch.Tensor]:
    """Quantize every block of the stack in order; returns the blocks and the
    quantized network's output activations (bf16 [tokens, d]).

    x0: bf16 [tokens, d] calibration activations (device).  weights: per block
    (Wg [f, d], Wu [f, d], Wd [d, f]) bf16 or fp32 device tensors.  Enqueued on
    ``stream`` (default: the current stream); the data-error words of a block's
    three layers are checked (a synchronization) at the end of the block.  ``marks``: if a list,
    (phase, event) pairs are appended, each event recorded on ``stream`` at the
    end of the phase (timing only).  ``dense``: multiply by the dequantized bf16
    weights (gptq_gemm_bf16) instead of the packed codes (gptq_dequant_gemm)."""
    if stream is None:
        stream = torch.cuda.current_stream()
    dev = x0.device
    T, d = x0.shape
    desc = bool(cfg.desc_act)
    prod = _Products(dev)
    def mark(name):
        if marks is not None:
            ev = torch.cuda.Event(enable_timing=True)
            ev.record(stream)
            marks.append((name, ev))

    mark("start")
    x = x0
    blocks = []
    for Wg, Wu, Wd in weights:
        f = Wg.shape[0]
        # gate and up: one Hessian of x, one prepare, two quantizations
        bg = pipeline.allocate(f, d, cfg, T, device=dev)
        bu = pipeline.allocate(f, d, cfg, 0, device=dev)
        bg.S.zero_()
        pipeline.accumulate(bg, [x], stream)
        mark("hessian")
        pipeline.prepare(bg, T, stream)
        mark("prepare")
        bu.S, bu.U, bu.perm, bu.dead = bg.S, bg.U, bg.perm, bg.dead  # shared Hessian
        pipeline.quantize(bg, Wg, stream)
        pipeline.quantize(bu, Wu, stream)
        gate, up = _packed(bg, desc, dense, stream), _packed(bu, desc, dense, stream)
        mark("quantize")
        # h = silu(x Wg_q^T) * (x Wu_q^T), chunk by chunk
        h = torch.empty((T, f), dtype=torch.bfloat16, device=dev)
        for t0 in range(0, T, chunk_tokens):
            t1 = min(T, t0 + chunk_tokens)
            xp = _gathered(prod, x[t0:t1], gate.perm, "x", stream)  # gate and up: one order
            g = _product(prod, xp, gate, "g", stream)
            u = _product(prod, xp, up, "u", stream)
            _lib.gptq_swiglu(g, u, h[t0:t1], stream=stream)
        mark("forward")
        # down: Hessian of h
        bd = pipeline.allocate(d, f, cfg, T, device=dev)
        bd.S.zero_()
        pipeline.accumulate(bd, [h], stream)
        mark("hessian")
        pipeline.prepare(bd, T, stream)
        mark("prepare")
        pipeline.quantize(bd, Wd, stream)
        down = _packed(bd, desc, dense, stream)
        mark("quantize")
        # x' = x + h Wd_q^T
        x_next = torch.empty_like(x)
        for t0 in range(0, T, chunk_tokens):
            t1 = min(T, t0 + chunk_tokens)
            y = _product(prod, _gathered(prod, h[t0:t1], down.perm, "h", stream), down, "y",
                         stream)
            _lib.gptq_residual_add(x[t0:t1], y, x_next[t0:t1], stream=stream)
        mark("forward")
        for b in (bg, bu, bd):
            pipeline.check_info(b)
        blocks.append(QuantizedBlock(gate, up, down, x if keep else None, h if keep else None))
        x = x_next
    return blocks, x
