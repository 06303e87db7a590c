"""ctypes binding of libgptq_mi355x.so (argument marshalling only).

Every computation happens in the library's HIP kernels; this module converts
torch tensors into device pointers, passes the current HIP stream and maps a
non-zero status to an exception.  It never computes a result itself, and it
fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgptq_mi355x.so")

GPTQ_OK = 0
GPTQ_ERR_INVALID_ARG = 1
GPTQ_ERR_NOT_PD = 2
GPTQ_ERR_NONFINITE = 3
GPTQ_ERR_EMPTY = 4
GPTQ_ERR_WORKSPACE = 5
GPTQ_ERR_HIP = 6
GPTQ_ERR_UNSUPPORTED = 7

GPTQ_F32 = 0
GPTQ_BF16 = 1

# every symbol the C header declares
EXPORTED = (
    "gptq_abi_version",
    "gptq_status_str",
    "gptq_hessian_workspace_size",
    "gptq_hessian_accumulate",
    "gptq_prepare_workspace_size",
    "gptq_prepare",
    "gptq_quantize_workspace_size",
    "gptq_quantize_layer",
    "gptq_quantize_layer_noalloc",
    "gptq_pack",
    "gptq_pack_ordered",
    "gptq_dequant_gemm_workspace_size",
    "gptq_dequant_gemm",
    "gptq_gather_columns",
    "gptq_dequantize",
    "gptq_gemm_bf16",
    "gptq_swiglu",
    "gptq_residual_add",
    "awq_absum_workspace_size",
    "awq_activation_absum",
    "awq_lite_workspace_size",
    "awq_lite",
    "awq_clip_quantize",
    "rtn_minmax",
    "gptq_layer_error_workspace_size",
    "gptq_layer_error",
)


class GPTQConfig(ctypes.Structure):
    _fields_ = [
        ("bits", ctypes.c_int32),
        ("group_size", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("perc_damp", ctypes.c_float),
        ("desc_act", ctypes.c_int32),
        ("sym", ctypes.c_int32),
        ("static_groups", ctypes.c_int32),
    ]


class GPTQError(RuntimeError):
    def __init__(self, status: int, where: str, msg: str):
        super().__init__(f"{where}: {msg} (status {status})")
        self.status = status


_lib = None

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_sz = ctypes.c_size_t


def load() -> ctypes.CDLL:
    """Load the HIP library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with "
            "`python post_weight_quantization_22_amd/build.py` (or __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    lib.gptq_abi_version.restype = ctypes.c_uint32
    lib.gptq_abi_version.argtypes = []
    lib.gptq_status_str.restype = ctypes.c_char_p
    lib.gptq_status_str.argtypes = [_i32]
    lib.gptq_hessian_workspace_size.restype = _i32
    lib.gptq_hessian_workspace_size.argtypes = [_i64, _i64, ctypes.POINTER(_sz)]
    lib.gptq_hessian_accumulate.restype = _i32
    lib.gptq_hessian_accumulate.argtypes = [_vp, _i64, _i64, _vp, _i32, _i64, _i64, _vp, _sz, _vp]
    lib.gptq_prepare_workspace_size.restype = _i32
    lib.gptq_prepare_workspace_size.argtypes = [_i64, ctypes.POINTER(_sz)]
    lib.gptq_prepare.restype = _i32
    lib.gptq_prepare.argtypes = [_vp, _i64, _i64, _i64, ctypes.c_float, _i32, _vp, _i64, _vp, _vp,
                                 _vp, _vp, _vp, _sz, _vp]
    lib.gptq_quantize_workspace_size.restype = _i32
    lib.gptq_quantize_workspace_size.argtypes = [_i64, _i64, ctypes.POINTER(GPTQConfig),
                                                 ctypes.POINTER(_sz)]
    lib.gptq_quantize_layer.restype = _i32
    lib.gptq_quantize_layer.argtypes = [_vp, _i32, _i64, _i64, _i64, _vp, _i64, _vp, _vp,
                                        ctypes.POINTER(GPTQConfig), _vp, _vp, _vp, _vp, _vp, _vp,
                                        _vp, _sz, _vp]
    lib.gptq_quantize_layer_noalloc.restype = _i32
    lib.gptq_quantize_layer_noalloc.argtypes = [_vp, _i32, _i64, _i64, _i64, _vp, _i64, _vp, _vp,
                                                ctypes.POINTER(GPTQConfig), _vp, _vp, _vp, _vp,
                                                _vp, _vp, _vp]
    lib.gptq_pack.restype = _i32
    lib.gptq_pack.argtypes = [_vp, _i64, _i64, _i32, _vp, _vp]
    lib.gptq_pack_ordered.restype = _i32
    lib.gptq_pack_ordered.argtypes = [_vp, _i64, _i64, _i32, _vp, _vp, _vp]
    lib.gptq_dequant_gemm_workspace_size.restype = _i32
    lib.gptq_dequant_gemm_workspace_size.argtypes = [_i64, _i64, _i64, _i32, ctypes.POINTER(_sz)]
    lib.gptq_dequant_gemm.restype = _i32
    lib.gptq_dequant_gemm.argtypes = [_vp, _i32, _i64, _i64, _i64, _vp, _i64, _i32, _i32, _vp,
                                      _vp, _vp, _i64, _vp, _i32, _i64, _vp, _sz, _vp]
    lib.gptq_dequantize.restype = _i32
    lib.gptq_dequantize.argtypes = [_vp, _i64, _i32, _i32, _vp, _vp, _i64, _i64, _vp, _i64, _vp]
    lib.gptq_gemm_bf16.restype = _i32
    lib.gptq_gemm_bf16.argtypes = [_vp, _i64, _i64, _i64, _vp, _i64, _i64, _vp, _i32, _i64, _vp]
    lib.gptq_gather_columns.restype = _i32
    lib.gptq_gather_columns.argtypes = [_vp, _i32, _i64, _i64, _i64, _vp, _vp, _i64, _vp]
    lib.gptq_swiglu.restype = _i32
    lib.gptq_swiglu.argtypes = [_vp, _i64, _vp, _i64, _i64, _i64, _vp, _i64, _vp]
    lib.gptq_residual_add.restype = _i32
    lib.gptq_residual_add.argtypes = [_vp, _i64, _vp, _i64, _i64, _i64, _vp, _i64, _vp]
    lib.awq_absum_workspace_size.restype = _i32
    lib.awq_absum_workspace_size.argtypes = [_i64, _i64, ctypes.POINTER(_sz)]
    lib.awq_activation_absum.restype = _i32
    lib.awq_activation_absum.argtypes = [_vp, _i32, _i64, _i64, _i64, _vp, _vp, _sz, _vp]
    lib.awq_lite_workspace_size.restype = _i32
    lib.awq_lite_workspace_size.argtypes = [_i64, _i64, ctypes.POINTER(_sz)]
    lib.awq_lite.restype = _i32
    lib.awq_lite.argtypes = [_vp, _i32, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _i32, _i32, _i32,
                             _i32, _vp, _vp, _vp, _vp, _sz, _vp]
    lib.awq_clip_quantize.restype = _i32
    lib.awq_clip_quantize.argtypes = [_vp, _i32, _i64, _i64, _i64, _vp, _i64, _vp, _i32, _i32,
                                      _i32, _i32, _vp, _vp, _vp, _vp, _vp]
    lib.rtn_minmax.restype = _i32
    lib.rtn_minmax.argtypes = [_vp, _i32, _i64, _i64, _i64, _i32, _i32, _i32, _vp, _vp, _vp, _vp]
    lib.gptq_layer_error_workspace_size.restype = _i32
    lib.gptq_layer_error_workspace_size.argtypes = [_i64, _i64, ctypes.POINTER(_sz)]
    lib.gptq_layer_error.restype = _i32
    lib.gptq_layer_error.argtypes = [_vp, _i32, _i64, _i64, _i64, _vp, _vp, _vp, _i64, _vp, _vp,
                                     _i64, _vp, _vp, _sz, _vp]
    _lib = lib
    return lib


def status_str(status: int) -> str:
    return load().gptq_status_str(status).decode()


def _check(status: int, where: str) -> None:
    if status != GPTQ_OK:
        raise GPTQError(status, where, status_str(status))


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _dtype_code(t) -> int:
    import torch

    if t.dtype == torch.bfloat16:
        return GPTQ_BF16
    if t.dtype == torch.float32:
        return GPTQ_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ld(t) -> int:
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError("expected a 2-D tensor with unit column stride")
    return t.stride(0)


def _workspace(nbytes: int, device, stream=None):
    """A per-call workspace allocated on the stream the call is enqueued on, so
    that torch's caching allocator does not hand the memory to other work
    before the library's kernels on that stream are done with it."""
    import torch

    if nbytes == 0:
        return None
    if stream is None:
        return torch.empty(nbytes, dtype=torch.uint8, device=device)
    with torch.cuda.stream(stream):
        return torch.empty(nbytes, dtype=torch.uint8, device=device)


_INT32_LIKE = ("int32", "uint32")


def _buf(t, name: str, shape, dtypes, device, optional: bool = True, min_rows=None):
    """Check an output or index buffer before its pointer goes to the library:
    the kernels write ``shape`` elements with the row stride the ABI states, so
    a smaller, strided, mistyped or foreign-device tensor would be written out
    of bounds.  ``shape`` entries of None are not checked; ``dtypes`` are torch
    dtype names."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if str(t.dtype).replace("torch.", "") not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype}, expected one of {dtypes}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if len(shape) == 1:
        if t.numel() < shape[0]:
            raise ValueError(f"{name}: {t.numel()} elements, need {shape[0]}")
        return
    if t.dim() != len(shape) or any(s is not None and d != s for d, s in zip(t.shape, shape)):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")


def _mat(t, name: str, rows: int, cols: int, dtypes, device):
    """A 2-D operand read or written with an explicit row stride: unit column
    stride, at least ``rows`` x ``cols``, on ``device``."""
    if t is None:
        raise ValueError(f"{name} is required")
    if str(t.dtype).replace("torch.", "") not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype}, expected one of {dtypes}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dim() != 2 or t.stride(1) != 1 or t.shape[0] < rows or t.shape[1] < cols:
        raise ValueError(f"{name}: expected a 2-D tensor of at least {rows} x {cols} with unit "
                         f"column stride, got shape {tuple(t.shape)} strides {t.stride()}")


def _ngroups(n: int, group_size: int) -> int:
    return 1 if group_size <= 0 else -(-n // group_size)


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------
def gptq_abi_version() -> int:
    return int(load().gptq_abi_version())


def gptq_status_str(status: int) -> str:
    return status_str(status)


def gptq_hessian_workspace_size(n: int, tokens: int) -> int:
    out = _sz(0)
    _check(load().gptq_hessian_workspace_size(n, tokens, ctypes.byref(out)),
           "gptq_hessian_workspace_size")
    return out.value


def gptq_hessian_accumulate(S, X, ws=None, stream=None) -> None:
    """S[n, n] (fp32, lower triangle) += X^T X for X[tokens, n] (bf16 or fp32)."""
    n = S.shape[0]
    tokens = X.shape[0]
    _mat(S, "S", n, n, ("float32",), S.device)
    _mat(X, "X", tokens, n, ("bfloat16", "float32"), S.device)
    need = gptq_hessian_workspace_size(n, tokens) if _dtype_code(X) == GPTQ_BF16 else 0
    if ws is None:
        ws = _workspace(need, S.device, stream)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(load().gptq_hessian_accumulate(_ptr(S), n, _ld(S), _ptr(X), _dtype_code(X), tokens,
                                          _ld(X), _ptr(ws), nbytes, _stream(stream)),
           "gptq_hessian_accumulate")


def gptq_prepare_workspace_size(n: int) -> int:
    out = _sz(0)
    _check(load().gptq_prepare_workspace_size(n, ctypes.byref(out)), "gptq_prepare_workspace_size")
    return out.value


def gptq_prepare(S, tokens: int, perc_damp: float, desc_act: bool, U, perm=None, dead=None,
                 lambda_out=None, info=None, ws=None, stream=None) -> None:
    n = S.shape[0]
    d = S.device
    _mat(S, "S", n, n, ("float32",), d)
    _mat(U, "U", n, n, ("float32",), d)
    _buf(perm, "perm", (n,), _INT32_LIKE, d)
    _buf(dead, "dead", (n,), ("uint8", "bool"), d)
    _buf(lambda_out, "lambda_out", (1,), ("float32",), d)
    _buf(info, "info", (1,), ("int32",), d, optional=False)
    if ws is None:
        ws = _workspace(gptq_prepare_workspace_size(n), S.device, stream)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(load().gptq_prepare(_ptr(S), n, _ld(S), int(tokens), float(perc_damp), int(desc_act),
                               _ptr(U), _ld(U), _ptr(perm), _ptr(dead), _ptr(lambda_out),
                               _ptr(info), _ptr(ws), nbytes, _stream(stream)),
           "gptq_prepare")


def make_config(bits: int, group_size: int, block_size: int = 128, perc_damp: float = 0.01,
                desc_act: bool = False, sym: bool = False,
                static_groups: bool = False) -> GPTQConfig:
    return GPTQConfig(bits, group_size, block_size, perc_damp, int(desc_act), int(sym),
                      int(static_groups))


def gptq_quantize_workspace_size(m: int, n: int, cfg: GPTQConfig) -> int:
    out = _sz(0)
    _check(load().gptq_quantize_workspace_size(m, n, ctypes.byref(cfg), ctypes.byref(out)),
           "gptq_quantize_workspace_size")
    return out.value


def gptq_quantize_layer(W, U, cfg: GPTQConfig, codes, scales, zeros, perm=None, dead=None,
                        g_idx=None, row_err=None, info=None, ws=None, stream=None) -> None:
    m, n = W.shape
    d = W.device
    ng = _ngroups(n, cfg.group_size)
    _mat(W, "W", m, n, ("bfloat16", "float32"), d)
    _mat(U, "U", n, n, ("float32",), d)
    _buf(codes, "codes", (m, n), ("uint8",), d, optional=False)
    _buf(scales, "scales", (m, ng), ("float32",), d, optional=False)
    _buf(zeros, "zeros", (m, ng), ("float32",), d, optional=False)
    _buf(perm, "perm", (n,), _INT32_LIKE, d)
    _buf(dead, "dead", (n,), ("uint8", "bool"), d)
    _buf(g_idx, "g_idx", (n,), _INT32_LIKE, d)
    _buf(row_err, "row_err", (m,), ("float32",), d)
    _buf(info, "info", (1,), ("int32",), d)
    if ws is None:
        ws = _workspace(gptq_quantize_workspace_size(m, n, cfg), W.device, stream)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(load().gptq_quantize_layer(_ptr(W), _dtype_code(W), m, n, _ld(W), _ptr(U), _ld(U),
                                      _ptr(perm), _ptr(dead), ctypes.byref(cfg), _ptr(codes),
                                      _ptr(scales), _ptr(zeros), _ptr(g_idx), _ptr(row_err),
                                      _ptr(info), _ptr(ws), nbytes, _stream(stream)),
           "gptq_quantize_layer")


GPTQ_NOALLOC_SCRATCH_BYTES = 64 << 20


def gptq_quantize_layer_noalloc(W, U, cfg: GPTQConfig, codes, scales, zeros, perm=None,
                                dead=None, g_idx=None, row_err=None, info=None,
                                stream=None) -> None:
    """gptq_quantize_layer on the library's fixed per-GPU scratch: allocates
    nothing (GPTQ_ERR_WORKSPACE for layers whose workspace exceeds it)."""
    m, n = W.shape
    d = W.device
    ng = _ngroups(n, cfg.group_size)
    _mat(W, "W", m, n, ("bfloat16", "float32"), d)
    _mat(U, "U", n, n, ("float32",), d)
    _buf(codes, "codes", (m, n), ("uint8",), d, optional=False)
    _buf(scales, "scales", (m, ng), ("float32",), d, optional=False)
    _buf(zeros, "zeros", (m, ng), ("float32",), d, optional=False)
    _buf(perm, "perm", (n,), _INT32_LIKE, d)
    _buf(dead, "dead", (n,), ("uint8", "bool"), d)
    _buf(g_idx, "g_idx", (n,), _INT32_LIKE, d)
    _buf(row_err, "row_err", (m,), ("float32",), d)
    _buf(info, "info", (1,), ("int32",), d)
    _check(load().gptq_quantize_layer_noalloc(_ptr(W), _dtype_code(W), m, n, _ld(W), _ptr(U),
                                              _ld(U), _ptr(perm), _ptr(dead), ctypes.byref(cfg),
                                              _ptr(codes), _ptr(scales), _ptr(zeros),
                                              _ptr(g_idx), _ptr(row_err), _ptr(info),
                                              _stream(stream)),
           "gptq_quantize_layer_noalloc")


def gptq_pack(codes, bits: int, packed, stream=None) -> None:
    m, n = codes.shape
    _buf(codes, "codes", (m, n), ("uint8",), codes.device, optional=False)
    _buf(packed, "packed", (m, -(-(n * int(bits)) // 32)), _INT32_LIKE, codes.device,
         optional=False)
    _check(load().gptq_pack(_ptr(codes), m, n, int(bits), _ptr(packed), _stream(stream)),
           "gptq_pack")


def gptq_pack_ordered(codes, bits: int, perm, packed, stream=None) -> None:
    """packed[r] = codes[r, perm[0]], codes[r, perm[1]], ... in the gptq_pack layout."""
    m, n = codes.shape
    _buf(codes, "codes", (m, n), ("uint8",), codes.device, optional=False)
    _buf(perm, "perm", (n,), _INT32_LIKE, codes.device)
    _buf(packed, "packed", (m, -(-(n * int(bits)) // 32)), _INT32_LIKE, codes.device,
         optional=False)
    _check(load().gptq_pack_ordered(_ptr(codes), m, n, int(bits), _ptr(perm), _ptr(packed),
                                    _stream(stream)),
           "gptq_pack_ordered")


def gptq_dequant_gemm_workspace_size(tokens: int, m: int, n: int, has_perm: bool) -> int:
    out = _sz(0)
    _check(load().gptq_dequant_gemm_workspace_size(tokens, m, n, int(bool(has_perm)),
                                                   ctypes.byref(out)),
           "gptq_dequant_gemm_workspace_size")
    return out.value


def gptq_dequant_gemm(X, packed, bits: int, group_size: int, scales, zeros, Y, perm=None,
                      ws=None, stream=None) -> None:
    """Y[tokens, m] = X[tokens, n] W_q^T with W_q from processing-order packed codes."""
    tokens, n = X.shape
    m = packed.shape[0]
    d = X.device
    ng = _ngroups(n, group_size)
    _mat(packed, "packed", m, -(-(n * int(bits)) // 32), _INT32_LIKE, d)
    _buf(scales, "scales", (m, ng), ("float32",), d, optional=False)
    _buf(zeros, "zeros", (m, ng), ("float32",), d, optional=False)
    _buf(perm, "perm", (n,), _INT32_LIKE, d)
    _mat(Y, "Y", tokens, m, ("float32", "bfloat16"), d)
    if ws is None:
        ws = _workspace(gptq_dequant_gemm_workspace_size(tokens, m, n, perm is not None),
                        X.device, stream)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(load().gptq_dequant_gemm(_ptr(X), _dtype_code(X), tokens, n, _ld(X), _ptr(packed),
                                    _ld(packed), int(bits), int(group_size), _ptr(scales),
                                    _ptr(zeros), _ptr(perm), m, _ptr(Y), _dtype_code(Y), _ld(Y),
                                    _ptr(ws), nbytes, _stream(stream)),
           "gptq_dequant_gemm")


def gptq_dequantize(packed, bits: int, group_size: int, scales, zeros, n: int, W,
                    stream=None) -> None:
    """W[m, n] (bf16) = the product's weights from processing-order packed codes."""
    m = packed.shape[0]
    d = packed.device
    ng = _ngroups(int(n), group_size)
    _mat(packed, "packed", m, -(-(int(n) * int(bits)) // 32), _INT32_LIKE, d)
    _buf(scales, "scales", (m, ng), ("float32",), d, optional=False)
    _buf(zeros, "zeros", (m, ng), ("float32",), d, optional=False)
    _mat(W, "W", m, int(n), ("bfloat16",), d)
    _check(load().gptq_dequantize(_ptr(packed), _ld(packed), int(bits), int(group_size),
                                  _ptr(scales), _ptr(zeros), m, int(n), _ptr(W), _ld(W),
                                  _stream(stream)),
           "gptq_dequantize")


def gptq_gemm_bf16(X, W, Y, stream=None) -> None:
    """Y[tokens, m] = X[tokens, n] W[m, n]^T (bf16 operands, Y fp32 or bf16)."""
    tokens, n = X.shape
    m = W.shape[0]
    _mat(W, "W", m, n, ("bfloat16",), X.device)
    _mat(Y, "Y", tokens, m, ("float32", "bfloat16"), X.device)
    _check(load().gptq_gemm_bf16(_ptr(X), tokens, n, _ld(X), _ptr(W), m, _ld(W), _ptr(Y),
                                 _dtype_code(Y), _ld(Y), _stream(stream)),
           "gptq_gemm_bf16")


def gptq_gather_columns(X, perm, Xp, stream=None) -> None:
    """Xp[t, p] = X[t, perm[p]] (bf16; Xp's columns past n are zeroed)."""
    tokens, n = X.shape
    _buf(perm, "perm", (n,), _INT32_LIKE, X.device, optional=False)
    _mat(Xp, "Xp", tokens, n, ("bfloat16",), X.device)
    _check(load().gptq_gather_columns(_ptr(X), _dtype_code(X), tokens, n, _ld(X), _ptr(perm),
                                      _ptr(Xp), _ld(Xp), _stream(stream)),
           "gptq_gather_columns")


def gptq_swiglu(gate, up, h, stream=None) -> None:
    """h[tokens, n] (bf16) = silu(gate) * up for fp32 gate, up."""
    tokens, n = gate.shape
    _mat(up, "up", tokens, n, ("float32",), gate.device)
    _mat(h, "h", tokens, n, ("bfloat16",), gate.device)
    _check(load().gptq_swiglu(_ptr(gate), _ld(gate), _ptr(up), _ld(up), tokens, n, _ptr(h),
                              _ld(h), _stream(stream)),
           "gptq_swiglu")


def gptq_residual_add(x, y, out, stream=None) -> None:
    """out[tokens, n] (bf16) = x (bf16) + y (fp32); out may be x."""
    tokens, n = x.shape
    _mat(y, "y", tokens, n, ("float32",), x.device)
    _mat(out, "out", tokens, n, ("bfloat16",), x.device)
    _check(load().gptq_residual_add(_ptr(x), _ld(x), _ptr(y), _ld(y), tokens, n, _ptr(out),
                                    _ld(out), _stream(stream)),
           "gptq_residual_add")


def awq_absum_workspace_size(n: int, tokens: int) -> int:
    out = _sz(0)
    _check(load().awq_absum_workspace_size(n, tokens, ctypes.byref(out)),
           "awq_absum_workspace_size")
    return out.value


def awq_lite_workspace_size(m: int, n: int) -> int:
    out = _sz(0)
    _check(load().awq_lite_workspace_size(m, n, ctypes.byref(out)), "awq_lite_workspace_size")
    return out.value


def awq_activation_absum(X, absum, ws=None, stream=None) -> None:
    """absum[n] += sum over tokens of |X[t, c]|."""
    tokens, n = X.shape
    _buf(absum, "absum", (n,), ("float32",), X.device, optional=False)
    if ws is None:
        ws = _workspace(awq_absum_workspace_size(n, tokens), X.device, stream)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(load().awq_activation_absum(_ptr(X), _dtype_code(X), tokens, n, _ld(X), _ptr(absum),
                                       _ptr(ws), nbytes, _stream(stream)),
           "awq_activation_absum")


def awq_lite(W, S, absum, tokens: int, bits: int, group_size: int, s_out, alpha_out, losses,
             sym: bool = False, ws=None, stream=None) -> None:
    """alpha search; s_out[n], alpha_out[1], losses[n_alpha] fp32 device tensors."""
    m, n = W.shape
    d = W.device
    _mat(S, "S", n, n, ("float32",), d)
    _buf(absum, "absum", (n,), ("float32",), d, optional=False)
    _buf(s_out, "s_out", (n,), ("float32",), d, optional=False)
    _buf(alpha_out, "alpha_out", (1,), ("float32",), d, optional=False)
    _buf(losses, "losses", (1,), ("float32",), d, optional=False)
    if ws is None:
        ws = _workspace(awq_lite_workspace_size(m, n), W.device, stream)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(load().awq_lite(_ptr(W), _dtype_code(W), m, n, _ld(W), _ptr(S), _ld(S), _ptr(absum),
                           int(tokens), int(bits), int(group_size), int(sym), losses.numel(),
                           _ptr(s_out), _ptr(alpha_out), _ptr(losses), _ptr(ws), nbytes,
                           _stream(stream)),
           "awq_lite")


def awq_clip_quantize(W, S, s, bits: int, group_size: int, codes, scales, zeros, clip_idx=None,
                      sym: bool = False, n_steps: int = 11, stream=None) -> None:
    m, n = W.shape
    d = W.device
    ng = _ngroups(n, group_size)
    _mat(S, "S", n, n, ("float32",), d)
    _buf(s, "s", (n,), ("float32",), d)
    _buf(codes, "codes", (m, n), ("uint8",), d, optional=False)
    _buf(scales, "scales", (m, ng), ("float32",), d, optional=False)
    _buf(zeros, "zeros", (m, ng), ("float32",), d, optional=False)
    _buf(clip_idx, "clip_idx", (m, ng), ("uint8",), d)
    _check(load().awq_clip_quantize(_ptr(W), _dtype_code(W), m, n, _ld(W), _ptr(S), _ld(S),
                                    _ptr(s), int(bits), int(group_size), int(sym), int(n_steps),
                                    _ptr(codes), _ptr(scales), _ptr(zeros), _ptr(clip_idx),
                                    _stream(stream)),
           "awq_clip_quantize")


def rtn_minmax(W, bits: int, group_size: int, codes, scales, zeros, sym: bool = False,
               stream=None) -> None:
    m, n = W.shape
    d = W.device
    ng = _ngroups(n, group_size)
    _buf(codes, "codes", (m, n), ("uint8",), d, optional=False)
    _buf(scales, "scales", (m, ng), ("float32",), d, optional=False)
    _buf(zeros, "zeros", (m, ng), ("float32",), d, optional=False)
    _check(load().rtn_minmax(_ptr(W), _dtype_code(W), m, n, _ld(W), int(bits), int(group_size),
                             int(sym), _ptr(codes), _ptr(scales), _ptr(zeros), _stream(stream)),
           "rtn_minmax")


def gptq_layer_error_workspace_size(m: int, n: int) -> int:
    out = _sz()
    _check(load().gptq_layer_error_workspace_size(int(m), int(n), ctypes.byref(out)),
           "gptq_layer_error_workspace_size")
    return int(out.value)


def gptq_layer_error(W, codes, scales, zeros, g_idx, S, err, ws=None, stream=None) -> None:
    """err[m] (float64) = per-row output error delta_r S delta_r^T of the quantized layer."""
    m, n = W.shape
    d = W.device
    ng = scales.shape[1] if scales.dim() == 2 else 0
    _buf(codes, "codes", (m, n), ("uint8",), d, optional=False)
    _buf(scales, "scales", (m, ng), ("float32",), d, optional=False)
    _buf(zeros, "zeros", (m, ng), ("float32",), d, optional=False)
    _buf(g_idx, "g_idx", (n,), _INT32_LIKE, d, optional=False)
    _mat(S, "S", n, n, ("float32",), d)
    _buf(err, "err", (m,), ("float64",), d, optional=False)
    if ws is None:
        ws = _workspace(gptq_layer_error_workspace_size(m, n), d, stream)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(load().gptq_layer_error(_ptr(W), _dtype_code(W), m, n, _ld(W), _ptr(codes),
                                   _ptr(scales), _ptr(zeros), int(ng), _ptr(g_idx), _ptr(S),
                                   _ld(S), _ptr(err), _ptr(ws), nbytes, _stream(stream)),
           "gptq_layer_error")
