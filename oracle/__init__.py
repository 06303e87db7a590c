"""fp64 CPU oracle for GPTQ layer-wise weight quantization.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the package
``post_weight_quantization_22_amd`` and its HIP library) imports, links or
calls this package; only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may.  It shares no code with the HIP
path: the two meet only at the seeded input generators in ``synth/``.

It is a plain, slow, obviously-correct restatement of the method on these pages:

* "GPTQ deep dive" (hncyxsy.com news 243429): §2.1 (second-order Taylor
  model), §2.2 (OBS compensation with the inverse Hessian), §2.4 (fixed
  column order, lazy batched updates, Cholesky), §3.1 (the four-step
  per-layer algorithm, H = 2XX^T + lambda*I, block size 128), §3.3
  (group size, desc_act, damp_percent 0.01).
* "LLM quantization principles: GPTQ, AWQ, GGUF" (0539edu.com news 6111416):
  §2.1 (q = round(x/scale) + zero_point and the [-2.5, 3.7] INT8 example),
  §3.1 (objective ||WX - W_qX||^2), §4.2 (bits per weight 4 + 32/G).
* "Calibration algorithms guide" (bhfrc.com news 5741): §2.2 (group-wise
  min-max), §2.3 (GPTQ order by descending Hessian diagonal, block size).
* "Quantized deployment, 1.5 TB to 250 GB" (lmnt.cn news 123823): §2.1
  (dequantization r = (q - zero_point) * scale), used by the dequantized-weight
  product of "LLM quantization principles" §5.2.
* "AWQ, MinMax, GPTQ calibration in Model Optimizer" (gtnt.cn news 115337):
  §4 (block_size a multiple of group_size, perc_damp 0.01; layers quantized in
  order on the quantized network's activations, in ``stack.py``).

Floating point is fp64 throughout, except where a floating value decides an
integer (a code, a zero-point): there the decision is taken in fp32, the
precision of the device kernels, emulated exactly (each fp32 operation is the
fp64 result rounded once to fp32, which is the correctly rounded fp32 result
for +, -, *, / of fp32 operands).  The quantizer, the GPTQ loop, RTN and the
replay also take ``exact=True``: every decision in plain fp64, the reference
against which the fp32 decisions are shown to differ only at rounding ties.

Every function below is pinned by ``tests/test_oracle_*.py`` against values
the pages print, closed forms, special cases and brute force; the module
docstrings name any part whose convention the pages do not fix.
"""
from .quantizer import (  # noqa: F401
    f32,
    group_params,
    quantize_codes,
    dequantize,
    pre_round_value,
)
from .hessian import hessian_S, hessian  # noqa: F401
from .prepare import prepare, Prepared, check_descending_order  # noqa: F401
from .gptq import (  # noqa: F401
    GPTQResult,
    gptq_quantize,
    gptq_obs_literal,
    rtn_minmax,
    dequant_layer,
    recon_error_from_H,
    recon_error_direct,
    replay_check,
)
from .pack import pack_ref, unpack_ref  # noqa: F401
from .dequant import dequant_weights, dequant_matmul  # noqa: F401
from . import stack  # noqa: F401,E402  (layer-sequential MLP stack)
from . import awq  # noqa: F401,E402  (AWQ-lite scale search and clip)
