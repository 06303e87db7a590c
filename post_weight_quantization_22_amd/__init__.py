"""GPTQ layer-wise weight quantization for AMD Instinct MI355X (gfx950).

The computation lives in ``libgptq_mi355x.so`` (hand-written HIP kernels
behind a C ABI, declared in ``include/gptq_mi355x.h``).  This package is its
Python binding: ``_lib`` mirrors the C entry points one to one and
``pipeline`` chains them for one layer.  Importing the package loads the
library and raises ImportError when it has not been built; there is no
fallback implementation.
"""
from . import _lib
from ._lib import (  # noqa: F401
    EXPORTED,
    awq_absum_workspace_size,
    awq_activation_absum,
    awq_clip_quantize,
    awq_lite,
    awq_lite_workspace_size,
    GPTQConfig,
    GPTQError,
    GPTQ_ERR_WORKSPACE,
    GPTQ_NOALLOC_SCRATCH_BYTES,
    gptq_abi_version,
    gptq_dequant_gemm,
    gptq_dequant_gemm_workspace_size,
    gptq_dequantize,
    gptq_gather_columns,
    gptq_gemm_bf16,
    gptq_hessian_accumulate,
    gptq_hessian_workspace_size,
    gptq_layer_error,
    gptq_layer_error_workspace_size,
    gptq_pack,
    gptq_pack_ordered,
    gptq_prepare,
    gptq_prepare_workspace_size,
    gptq_quantize_layer,
    gptq_quantize_layer_noalloc,
    gptq_quantize_workspace_size,
    gptq_residual_add,
    gptq_status_str,
    gptq_swiglu,
    make_config,
    rtn_minmax,
)

_lib.load()
