"""MI355X (gfx950) MLA prolog and fused qkv RmsNorm-RoPE-cache library.

Python names mirror the C ABI in include/qkvnr.h:

* :func:`mla_prolog_v2` - the MlaPrologV2 prolog (c^Q, q^N, q^R, c^KV and
  k^R with paged-cache scatter), non-quantised and partially quantised;
* :func:`mla_pack_weight` / :func:`mla_pack_weight_uq_qr` /
  :func:`mla_pack_weight_uk` - one-time
  packing of a (K, N) weight into the MFMA-native K16 blocked layout the
  prolog streams;
* :func:`qkv_rmsnorm_rope_cache` - the fused qkv split / RmsNorm / RoPE /
  quant / scatter op;
* :func:`mla_preprocess_v2` - MlaPreprocessV2 (RmsNormQuant of x, int8
  W^DQKV, RmsNormQuant of the query latent, int8 W^UQ, W^UK, RoPE, caches).

All work runs in the HIP library ``lib/libqkvnr.so``; build it with
``python -m qkv_norm_rope_amd.build``.
"""

from ._binding import (  # noqa: F401
    EXPORTS,
    LIB_PATH,
    MLA_FLAG_CHECK_INDEX,
    MLA_KERNELS,
    MLA_NO_ALLOC_SCRATCH_BYTES,
    MLA_PHASES,
    MLA_QUANT,
    MLA_WEIGHT_ND,
    MLA_WEIGHT_PACKED_K16,
    QKV_FLAG_CHECK_INPUTS,
    QKV_QUANT,
    MlaPreprocessV2Args,
    MlaPrologV2Args,
    PreparedMlaPrologV2,
    QkvRmsNormRopeCacheArgs,
    QkvnrError,
    load_library,
    mla_check_cache_index,
    mla_pack_weight,
    mla_probe_mfma_bf16,
    mla_probe_read,
    mla_pack_weight_uk,
    mla_pack_weight_uq_qr,
    mla_preprocess_v2,
    mla_prolog_v2,
    mla_prolog_v2_args,
    mla_prolog_v2_kernels,
    mla_prolog_v2_no_alloc,
    mla_prolog_v2_workspace_size,
    qkv_rmsnorm_rope_cache,
    qkv_rmsnorm_rope_cache_args,
    status_string,
    version,
)
