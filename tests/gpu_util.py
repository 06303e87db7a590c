"""Shared helpers for the GPU parity tests (device uploads, oracle runs, comparisons)."""
from __future__ import annotations

import dataclasses
import sys
from typing import Optional

import numpy as np
import pytest

import oracle
import synth
from oracle.quantizer import f32

torch = pytest.importorskip("torch")


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import post_weight_quantization_22_amd as q  # noqa: F401  (loads the HIP library)
    return q


def say(*a):
    """Name the case before a GPU step, flushed, so a fault leaves a trace."""
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray, dtype) -> "torch.Tensor":
    return torch.from_numpy(np.ascontiguousarray(a)).to(device="cuda").to(dtype)


def storage_dtype(name: str):
    return torch.bfloat16 if name == "bf16" else torch.float32


def host(t) -> np.ndarray:
    return t.detach().cpu().numpy()


@dataclasses.dataclass
class OracleLayer:
    W: np.ndarray
    X: np.ndarray
    S: np.ndarray
    P: oracle.Prepared
    res: oracle.GPTQResult


def oracle_layer(wl: synth.Workload, layer: Optional[str] = None) -> OracleLayer:
    ls = wl.layer(layer)
    W = synth.weight(wl, ls.name)
    X = synth.x_all(wl, ls.x)
    S = oracle.hessian_S([X])
    q = wl.quant
    P = oracle.prepare(S, q.perc_damp, q.desc_act)
    res = oracle.gptq_quantize(W, P.U, q.bits, q.group_size, q.block_size, P.perm, P.dead, q.sym)
    return OracleLayer(W=W, X=X, S=S, P=P, res=res)


def match_rate(a: np.ndarray, b: np.ndarray) -> float:
    return float(np.mean(np.asarray(a) == np.asarray(b))) if np.asarray(a).size else 1.0


def root_cascade(codes_a: np.ndarray, codes_b: np.ndarray, perm: np.ndarray):
    """Per row, the first mismatch in processing order is a root; the rest cascade."""
    A = np.asarray(codes_a)[:, perm]
    B = np.asarray(codes_b)[:, perm]
    bad = A != B
    rows = np.flatnonzero(bad.any(axis=1))
    return len(rows), int(bad.sum()) - len(rows)
