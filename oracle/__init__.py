"""Plain float64 CPU oracle for the MLA prolog and the fused qkv op.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
CPU-baseline leg may import this package.  The HIP library never calls it and
shares no code with it: decoding of storage dtypes, norms, rotations,
quantisation and scatter are all written again here, in NumPy float64, so a
reader can check each step against the pages by eye.

Sources (each function cites the section it follows):

* "MlaPrologV2" README (ops-transformer, attention/mla_prolog_v2): the
  function description and formulas section, the parameter table, and the
  constraints section (shape rules, quantisation-scenario table, dtype and
  shape table).
* "aclnnQkvRmsNormRopeCache" (CANN API reference): formulas (1) SplitVD,
  (2) RmsNorm, (3) RoPE half-and-half, (4) Quant, and the input-shape and
  other restrictions.
* "aclnnMlaPreprocessV2" (CANN API reference): the interface function
  bullets (the order of the steps) and the RmsNormQuant formula block.

Parity status: every function here is pinned by the CPU tests (closed forms,
library special cases, brute force on tiny inputs, invariants).  End-to-end
values are unpinned by the pages themselves: they print no worked example.
"""

from .common import (
    decode,
    rmsnorm,
    rope_half,
    quant_int8,
    dynamic_quant_int8,
    int_matmul_exact,
    scatter_slots,
    check_index,
)
from .mla_prolog_v2 import mla_prolog_v2, mla_query_from_quantized
from .mla_prolog_v2 import quant_query_per_head as mla_prolog_v2_quant_query
from .qkv_rmsnorm_rope_cache import qkv_rmsnorm_rope_cache
from .mla_preprocess_v2 import (
    mla_preprocess_v2,
    preprocess_query_from_codes,
    rmsnorm_quant,
    rmsnorm_quant_values,
)

__all__ = [
    "decode",
    "rmsnorm",
    "rope_half",
    "quant_int8",
    "dynamic_quant_int8",
    "int_matmul_exact",
    "scatter_slots",
    "check_index",
    "mla_prolog_v2",
    "mla_query_from_quantized",
    "mla_prolog_v2_quant_query",
    "qkv_rmsnorm_rope_cache",
    "mla_preprocess_v2",
    "preprocess_query_from_codes",
    "rmsnorm_quant",
    "rmsnorm_quant_values",
]
