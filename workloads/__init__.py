"""Seeded synthetic workloads shared by the tests, the bench and the smoke check.

This package draws inputs only.  It holds none of the arithmetic of the MLA
prolog or of the fused qkv RmsNorm-RoPE-cache op: no matmul, no norm, no
rotation, no quantisation of results.  Floats are drawn in float64 with
NumPy's PCG64 and rounded to their storage dtype (bf16, fp16) by
round-to-nearest-even; the rounded values are the inputs both the oracle and
the HIP library consume.
"""

from .configs import CONFIGS, MlaConfig, PreConfig, QkvConfig, get_config
from .gen import (
    Workload,
    make_workload,
    make_mla_workload,
    make_preprocess_workload,
    make_qkv_workload,
    bf16_bits_from_f64,
    sub_workload,
)

__all__ = [
    "CONFIGS",
    "MlaConfig",
    "PreConfig",
    "QkvConfig",
    "get_config",
    "Workload",
    "make_workload",
    "make_mla_workload",
    "make_preprocess_workload",
    "make_qkv_workload",
    "bf16_bits_from_f64",
    "sub_workload",
]
