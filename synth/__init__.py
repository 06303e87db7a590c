"""Seeded synthetic inputs for the GPTQ layer workloads.

This package draws the weights W and the calibration activations X that both
the HIP path and the fp64 oracle consume.  It holds none of the method's
arithmetic: it only samples, scales outlier channels and rounds to the storage
dtype (fp32 or bf16).  Nothing here quantizes, accumulates or factors.
"""
from .workloads import (  # noqa: F401
    WORKLOADS,
    LayerSpec,
    QuantSpec,
    Workload,
    XSpec,
    custom_workload,
    get_workload,
    outlier_channels,
    round_to_bf16,
    stack_workload,
    weight,
    x_all,
    x_chunk,
)
