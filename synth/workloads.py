"""Workload definitions and seeded generators.

The five layer workloads stand in for the calibration setting the pages
describe (128-512 calibration sequences of 512-2048 tokens, activation
outlier channels around 1 %), with random weights of Llama-7B / 70B layer
shapes.  No dataset and no trained weights are used.

Random state: every tensor is drawn from its own
``Generator(PCG64(SeedSequence(seed, spawn_key=(workload_id, tensor_id, chunk))))``
so that any chunk can be regenerated alone, in any order, on any thread.

Recipe (identical for host and device consumers):
  * W: N(0, sigma^2) sampled in fp64, rounded to fp32, then to bf16 with
    round-to-nearest-even when the workload stores bf16.  Drawn in row blocks
    of 1024 rows (chunk = row block index).
  * X: one chunk per calibration sequence, [chunk_len, n] row-major
    (token-major).  Sampled in fp64 from the named distribution, outlier
    channels multiplied by their factor, rounded to fp32, then to bf16.
  * Outlier channels: k = round-half-even(frac * n) channels drawn without
    replacement from the workload's outlier stream, returned sorted.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List, Optional, Tuple

import numpy as np

W_ROW_BLOCK = 1024


# ----------------------------------------------------------------------------
# specs
# ----------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class XSpec:
    """One calibration activation stream X of shape [chunks * chunk_len, n]."""

    tensor_id: int
    n: int
    chunks: int
    chunk_len: int
    dist: str  # "normal" | "student_t4" | "laplace"
    outlier_frac: float
    outlier_mult: float
    dtype: str  # "f32" | "bf16"
    outlier_tensor_id: int = 3

    @property
    def tokens(self) -> int:
        return self.chunks * self.chunk_len


@dataclasses.dataclass(frozen=True)
class LayerSpec:
    name: str
    m: int  # d_out (rows of W)
    n: int  # d_in (columns of W)
    w_sigma: float
    w_dtype: str  # "f32" | "bf16"
    w_tensor_id: int
    x: str  # key into Workload.xs


@dataclasses.dataclass(frozen=True)
class QuantSpec:
    bits: int
    group_size: int
    block_size: int
    perc_damp: float
    desc_act: bool
    sym: bool = False


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    workload_id: int
    seed: int
    layers: Tuple[LayerSpec, ...]
    xs: Dict[str, XSpec]
    quant: QuantSpec
    description: str = ""

    def layer(self, name: Optional[str] = None) -> LayerSpec:
        if name is None:
            return self.layers[0]
        for l in self.layers:
            if l.name == name:
                return l
        raise KeyError(name)


def _wl(name, wid, layers, xs, quant, desc):
    return Workload(name=name, workload_id=wid, seed=0, layers=tuple(layers), xs=xs,
                    quant=quant, description=desc)


WORKLOADS: Dict[str, Workload] = {}


def _register(w: Workload) -> None:
    WORKLOADS[w.name] = w


# 256 x 256, fp32 W and X, one 1024-token sequence, 1 % outliers x20, 4-bit g128.
_register(_wl(
    "layer256", 1,
    [LayerSpec("proj", 256, 256, 0.02, "f32", 0, "x")],
    {"x": XSpec(2, 256, 1, 1024, "normal", 0.01, 20.0, "f32")},
    QuantSpec(4, 128, 128, 0.01, False),
    "single 256x256 linear layer, fp32, 1024 calibration tokens"))

# Llama-7B attention projection: 4096 x 4096 bf16, 128 x 2048 tokens,
# 0.5 % outliers x30, 4-bit g128, desc_act off.
_register(_wl(
    "llama7b_attn", 2,
    [LayerSpec("q_proj", 4096, 4096, 0.02, "bf16", 0, "x")],
    {"x": XSpec(2, 4096, 128, 2048, "normal", 0.005, 30.0, "bf16")},
    QuantSpec(4, 128, 128, 0.01, False),
    "Llama-7B-shaped attention projection 4096x4096, 262144 calibration tokens"))

# Llama-7B MLP: gate and up (11008 x 4096) share X; down (4096 x 11008) has its own X.
# Student-t (nu = 4) activations, 4-bit g128, desc_act on.
_register(_wl(
    "llama7b_mlp", 3,
    [LayerSpec("gate_proj", 11008, 4096, 0.02, "bf16", 0, "x_in"),
     LayerSpec("up_proj", 11008, 4096, 0.02, "bf16", 1, "x_in"),
     LayerSpec("down_proj", 4096, 11008, 0.02, "bf16", 5, "x_mid")],
    {"x_in": XSpec(2, 4096, 128, 2048, "student_t4", 0.0, 1.0, "bf16"),
     "x_mid": XSpec(4, 11008, 128, 2048, "student_t4", 0.0, 1.0, "bf16")},
    QuantSpec(4, 128, 128, 0.01, True),
    "Llama-7B-shaped MLP (gate/up share one Hessian, down has its own)"))

# 70B square projection: 8192 x 8192, 256 x 2048 tokens, 1 % outliers x50, 3-bit g128.
_register(_wl(
    "llama70b_square", 4,
    [LayerSpec("o_proj", 8192, 8192, 0.015, "bf16", 0, "x")],
    {"x": XSpec(2, 8192, 256, 2048, "normal", 0.01, 50.0, "bf16")},
    QuantSpec(3, 128, 128, 0.01, False),
    "70B-shaped square projection 8192x8192, 3-bit"))

# 70B down projection: 8192 x 28672, Laplace activations, 4-bit g64, desc_act on.
_register(_wl(
    "llama70b_down", 5,
    [LayerSpec("down_proj", 8192, 28672, 0.01, "bf16", 0, "x")],
    {"x": XSpec(2, 28672, 256, 2048, "laplace", 0.0, 1.0, "bf16")},
    QuantSpec(4, 64, 128, 0.01, True),
    "70B-shaped down projection 8192x28672 (28672^2 Hessian), 4-bit g64"))


def get_workload(name: str) -> Workload:
    return WORKLOADS[name]


def custom_workload(name: str, m: int, n: int, tokens: int, chunk_len: int, *,
                    w_sigma: float = 0.02, w_dtype: str = "bf16", x_dist: str = "normal",
                    outlier_frac: float = 0.01, outlier_mult: float = 20.0,
                    x_dtype: str = "bf16", bits: int = 4, group_size: int = 128,
                    block_size: int = 128, perc_damp: float = 0.01, desc_act: bool = False,
                    sym: bool = False, workload_id: int = 100, seed: int = 0) -> Workload:
    """A reduced-size workload of the same recipe, for parity tests."""
    if tokens % chunk_len:
        raise ValueError("tokens must be a multiple of chunk_len")
    return Workload(
        name=name, workload_id=workload_id, seed=seed,
        layers=(LayerSpec("layer", m, n, w_sigma, w_dtype, 0, "x"),),
        xs={"x": XSpec(2, n, tokens // chunk_len, chunk_len, x_dist, outlier_frac,
                       outlier_mult, x_dtype)},
        quant=QuantSpec(bits, group_size, block_size, perc_damp, desc_act, sym),
        description=f"custom {m}x{n}, {tokens} tokens")


def stack_workload(name: str, d: int, f: int, blocks: int, tokens: int, chunk_len: int, *,
                   w_sigma: float = 0.02, x_dist: str = "student_t4",
                   outlier_frac: float = 0.0, outlier_mult: float = 1.0, bits: int = 4,
                   group_size: int = 128, block_size: int = 128, perc_damp: float = 0.01,
                   desc_act: bool = True, sym: bool = False, workload_id: int = 200,
                   seed: int = 0) -> Workload:
    """A stack of Llama-style MLP blocks: per block k the layers gate_k, up_k
    ([f, d]) and down_k ([d, f]), bf16 N(0, w_sigma^2); the stack's input stream
    "x0" [tokens, d] bf16.  Only the input is drawn: the inputs of later layers
    are what the quantized layers before them produce."""
    if tokens % chunk_len:
        raise ValueError("tokens must be a multiple of chunk_len")
    layers = []
    for k in range(blocks):
        layers += [LayerSpec(f"gate_{k}", f, d, w_sigma, "bf16", 20 + 3 * k, "x0"),
                   LayerSpec(f"up_{k}", f, d, w_sigma, "bf16", 21 + 3 * k, "x0"),
                   LayerSpec(f"down_{k}", d, f, w_sigma, "bf16", 22 + 3 * k, "x0")]
    return Workload(
        name=name, workload_id=workload_id, seed=seed, layers=tuple(layers),
        xs={"x0": XSpec(2, d, tokens // chunk_len, chunk_len, x_dist, outlier_frac,
                        outlier_mult, "bf16")},
        quant=QuantSpec(bits, group_size, block_size, perc_damp, desc_act, sym),
        description=f"{blocks} MLP blocks d={d} f={f}, {tokens} tokens")


# A two-block stack of Llama-7B MLP blocks (d 4096, f 11008) on the MLP
# workload's activation recipe, 4-bit g128 desc_act: the layer-sequential case.
_register(stack_workload("llama7b_mlp_stack", 4096, 11008, 2, 128 * 2048, 2048, workload_id=6))


# ----------------------------------------------------------------------------
# generators
# ----------------------------------------------------------------------------
def _rng(wl: Workload, tensor_id: int, chunk: int) -> np.random.Generator:
    ss = np.random.SeedSequence(wl.seed, spawn_key=(wl.workload_id, tensor_id, chunk))
    return np.random.Generator(np.random.PCG64(ss))


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round an fp32 array to bf16 (nearest, ties to even); returned as fp32 values."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    u = (u + np.uint64(0x7FFF) + lsb) & np.uint64(0xFFFF0000)
    return u.astype(np.uint32).view(np.float32)


def _to_storage(a64: np.ndarray, dtype: str) -> np.ndarray:
    a32 = a64.astype(np.float32)
    if dtype == "f32":
        return a32
    if dtype == "bf16":
        return round_to_bf16(a32)
    raise ValueError(dtype)


def outlier_channels(wl: Workload, xname: str) -> np.ndarray:
    xs = wl.xs[xname]
    k = int(round(xs.outlier_frac * xs.n))  # Python round(): half to even
    if k == 0:
        return np.zeros(0, dtype=np.int64)
    r = _rng(wl, xs.outlier_tensor_id + 100 * xs.tensor_id, 0)
    return np.sort(r.choice(xs.n, size=k, replace=False)).astype(np.int64)


def x_chunk(wl: Workload, xname: str, idx: int,
            outliers: Optional[np.ndarray] = None) -> np.ndarray:
    """Calibration chunk ``idx``: [chunk_len, n] fp32 values (bf16-exact for bf16)."""
    xs = wl.xs[xname]
    if not 0 <= idx < xs.chunks:
        raise IndexError(idx)
    r = _rng(wl, xs.tensor_id, idx)
    shape = (xs.chunk_len, xs.n)
    if xs.dist == "normal":
        a = r.standard_normal(shape)
    elif xs.dist == "student_t4":
        a = r.standard_t(4.0, shape)
    elif xs.dist == "laplace":
        a = r.laplace(0.0, 1.0, shape)
    else:
        raise ValueError(xs.dist)
    if outliers is None:
        outliers = outlier_channels(wl, xname)
    if outliers.size:
        a[:, outliers] *= xs.outlier_mult
    return _to_storage(a, xs.dtype)


def _threads(threads: Optional[int]) -> int:
    if threads:
        return threads
    return max(1, min(16, os.cpu_count() or 1))


def x_all(wl: Workload, xname: str, chunks: Optional[List[int]] = None,
          threads: Optional[int] = None) -> np.ndarray:
    """Concatenate the selected chunks (default: all) into one [tokens, n] fp32 array."""
    xs = wl.xs[xname]
    idx = list(range(xs.chunks)) if chunks is None else list(chunks)
    out = np.empty((len(idx) * xs.chunk_len, xs.n), dtype=np.float32)
    outl = outlier_channels(wl, xname)

    def fill(j):
        out[j * xs.chunk_len:(j + 1) * xs.chunk_len] = x_chunk(wl, xname, idx[j], outl)

    with ThreadPoolExecutor(_threads(threads)) as ex:
        list(ex.map(fill, range(len(idx))))
    return out


def weight(wl: Workload, layer: Optional[str] = None, rows: Optional[slice] = None,
           threads: Optional[int] = None) -> np.ndarray:
    """W [m, n] fp32 values (bf16-exact for bf16 layers); ``rows`` selects a row range."""
    ls = wl.layer(layer)
    r0, r1 = 0, ls.m
    if rows is not None:
        r0, r1, _ = rows.indices(ls.m)
    out = np.empty((r1 - r0, ls.n), dtype=np.float32)
    blocks = range(r0 // W_ROW_BLOCK, (r1 + W_ROW_BLOCK - 1) // W_ROW_BLOCK) if r1 > r0 else []

    def fill(b):
        lo, hi = b * W_ROW_BLOCK, min((b + 1) * W_ROW_BLOCK, ls.m)
        r = _rng(wl, ls.w_tensor_id + 10, b)
        blk = _to_storage(r.normal(0.0, ls.w_sigma, (hi - lo, ls.n)), ls.w_dtype)
        s0, s1 = max(lo, r0), min(hi, r1)
        out[s0 - r0:s1 - r0] = blk[s0 - lo:s1 - lo]

    with ThreadPoolExecutor(_threads(threads)) as ex:
        list(ex.map(fill, blocks))
    return out
