"""One linear layer through the whole GPTQ path, as a sequence of C-ABI calls.

"GPTQ deep dive" (hncyxsy.com news 243429) section 3.1: per layer, (1) the
Hessian from the layer's calibration inputs, (2) damping and the Cholesky
factorization, (3) the blocked column loop, (4) the integer weights with their
scales and zero-points.  Every step runs in libgptq_mi355x.so; this module only
allocates the caller-owned buffers once (torch device memory) and issues the
calls on one stream, so a timed run allocates nothing.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence

import torch

from . import _lib


@dataclasses.dataclass
class LayerBuffers:
    m: int
    n: int
    cfg: _lib.GPTQConfig
    S: torch.Tensor
    U: torch.Tensor
    perm: torch.Tensor
    dead: torch.Tensor
    lam: torch.Tensor
    info_prep: torch.Tensor
    info_quant: torch.Tensor
    codes: torch.Tensor
    scales: torch.Tensor
    zeros: torch.Tensor
    g_idx: torch.Tensor
    row_err: torch.Tensor
    packed: torch.Tensor
    ws_hess: Optional[torch.Tensor]
    ws_prep: torch.Tensor
    ws_quant: torch.Tensor


def ngroups(n: int, group_size: int) -> int:
    return 1 if group_size <= 0 else -(-n // group_size)


def allocate(m: int, n: int, cfg: _lib.GPTQConfig, hessian_tokens: int,
             device: str = "cuda") -> LayerBuffers:
    f32 = dict(dtype=torch.float32, device=device)
    ng = ngroups(n, cfg.group_size)
    nw = -(-(n * cfg.bits) // 32)
    hw = _lib.gptq_hessian_workspace_size(n, hessian_tokens) if hessian_tokens > 0 else 0
    return LayerBuffers(
        m=m, n=n, cfg=cfg,
        S=torch.zeros((n, n), **f32),
        U=torch.empty((n, n), **f32),
        perm=torch.empty(n, dtype=torch.int32, device=device),
        dead=torch.empty(n, dtype=torch.uint8, device=device),
        lam=torch.empty(1, **f32),
        info_prep=torch.zeros(1, dtype=torch.int32, device=device),
        info_quant=torch.zeros(1, dtype=torch.int32, device=device),
        codes=torch.empty((m, n), dtype=torch.uint8, device=device),
        scales=torch.empty((m, ng), **f32),
        zeros=torch.empty((m, ng), **f32),
        g_idx=torch.empty(n, dtype=torch.int32, device=device),
        row_err=torch.empty(m, **f32),
        packed=torch.empty((m, nw), dtype=torch.int32, device=device),
        ws_hess=torch.empty(hw, dtype=torch.uint8, device=device) if hw else None,
        ws_prep=torch.empty(_lib.gptq_prepare_workspace_size(n), dtype=torch.uint8,
                            device=device),
        ws_quant=torch.empty(max(1, _lib.gptq_quantize_workspace_size(m, n, cfg)),
                             dtype=torch.uint8, device=device),
    )


def accumulate(buf: LayerBuffers, X_chunks: Sequence[torch.Tensor], stream=None) -> int:
    """S += X^T X over the given device chunks; returns the number of tokens added."""
    tokens = 0
    for X in X_chunks:
        _lib.gptq_hessian_accumulate(buf.S, X, ws=buf.ws_hess, stream=stream)
        tokens += X.shape[0]
    return tokens


def prepare(buf: LayerBuffers, tokens: int, stream=None) -> None:
    _lib.gptq_prepare(buf.S, tokens, buf.cfg.perc_damp, bool(buf.cfg.desc_act), buf.U,
                      perm=buf.perm, dead=buf.dead, lambda_out=buf.lam, info=buf.info_prep,
                      ws=buf.ws_prep, stream=stream)


def quantize(buf: LayerBuffers, W: torch.Tensor, stream=None) -> None:
    _lib.gptq_quantize_layer(W, buf.U, buf.cfg, buf.codes, buf.scales, buf.zeros,
                             perm=buf.perm, dead=buf.dead, g_idx=buf.g_idx,
                             row_err=buf.row_err, info=buf.info_quant, ws=buf.ws_quant,
                             stream=stream)


def pack(buf: LayerBuffers, stream=None) -> None:
    _lib.gptq_pack(buf.codes, buf.cfg.bits, buf.packed, stream=stream)


def run_layer(buf: LayerBuffers, W: torch.Tensor, X_chunks: Sequence[torch.Tensor],
              stream=None) -> None:
    """Zero S, accumulate all chunks, prepare, quantize and pack (enqueued, not synced)."""
    buf.S.zero_()
    tokens = accumulate(buf, X_chunks, stream)
    prepare(buf, tokens, stream)
    quantize(buf, W, stream)
    pack(buf, stream)


def check_info(buf: LayerBuffers) -> None:
    """Raise if gptq_prepare or gptq_quantize_layer reported a data error (syncs)."""
    ip = int(buf.info_prep.item())
    iq = int(buf.info_quant.item())
    if ip > 0:
        raise _lib.GPTQError(_lib.GPTQ_ERR_NOT_PD, "gptq_prepare",
                             f"non-positive pivot at processing position {ip - 1}")
    if ip < 0 or iq < 0:
        raise _lib.GPTQError(_lib.GPTQ_ERR_NONFINITE, "gptq layer", "non-finite input")
