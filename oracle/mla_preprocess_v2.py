"""MlaPreprocessV2 in float64 (test infrastructure only).

Follows the "aclnnMlaPreprocessV2" page (CANN API reference): the interface
function bullets give the order of the steps, the formula block defines
RmsNormQuant.  Per token:

    x8  = RmsNormQuant(x)                 over He, gamma_x, bias_x
    [h | g_kv | g_r] = x8 . W^DQKV        int8 product, dequantised
    path 1: c8 = RmsNormQuant(h)          over Hcq, gamma_cq, bias_cq
            y  = c8 . W^UQ                int8 product, dequantised
            path 3: q^N = q^C . W^UK      per head (q^C = y's first N*D)
            path 4: q^R = RoPE(y's last N*Dr)
    path 2: path 5: k^N = RmsNorm(g_kv)   -> kv_cache at cache_index
            path 6: k^R = RoPE(g_r)       -> kr_cache at cache_index

Readings where the page is garbled or silent (each also listed in the
design notes as P-1 to P-12):

* The step order is the bullets'; the printed formulas for q^N, k^N and k^R
  drop steps (the second RmsNormQuant and W^UQ; W^DQKV and the split) and
  are read as shorthand for that chain.
* RmsNormQuant(v) = (RmsNorm(v) + bias) * deqScale, as the formula block
  prints it (multiply), then rounded half to even and saturated to the int8
  range [-128, 127]: the name's "Quant".  deqScale is one value per tensor
  (a per-channel activation scale could not be folded into the per-output-
  channel dequantisation of the following int8 product); bias is per
  channel.  The formula's RMS uses one epsilon, shared by all three norms.
* W^DQKV is int8 (He, Hcq+Hckv+Dr) = [W^DQ | W^DKV | W^KR] in name order;
  W^UQ is int8 (Hcq, N*(D+Dr)) = [W^UQ | W^QR], head n of each block at
  n*D and N*D + n*Dr.  Each int8 product is the exact integer sum times a
  per-output-channel fp32 dequant scale (the page's parameter table is
  lost; the scale folds the activation's step and the weight's scale).
* W^UK is bf16 (N, D, Hckv); RoPE is the half-and-half form with the
  token's (cos, sin) of width Dr; the caches are bf16 paged
  (BlockNum, BlockSize, 1, H) updated at cache_index (-1 skips).
"""

from __future__ import annotations

import numpy as np

from .common import decode, int_matmul_exact, rmsnorm, rope_half, scatter_slots
from .mla_prolog_v2 import _per_head_uk, _split_query


def rmsnorm_quant_values(v, gamma, bias, scale, eps):
    """The value RmsNormQuant rounds: (RmsNorm(v) + bias) * deqScale
    (aclnnMlaPreprocessV2, formula block)."""
    return (rmsnorm(v, gamma, eps) + np.asarray(bias, np.float64)) * float(scale)


def rmsnorm_quant(v, gamma, bias, scale, eps):
    """RmsNormQuant as int8 codes: round half to even, saturate to
    [-128, 127]."""
    return np.clip(np.rint(rmsnorm_quant_values(v, gamma, bias, scale, eps)),
                   -128, 127).astype(np.int64)


def preprocess_query_from_codes(c8, w8_uqqr, dq_uqqr, wuk, cos, sin, N, D, Dr):
    """Paths 3 and 4 from given c^Q codes: y = (c8 . W8) * dq per channel,
    q^N = q^C . W^UK per head, q^R = RoPE(y's rope block)."""
    y = int_matmul_exact(c8, w8_uqqr).astype(np.float64) \
        * np.asarray(dq_uqqr, np.float64)[None, :]
    qc, qr_pre = _split_query(y, N, D, Dr)
    return _per_head_uk(qc, wuk), rope_half(qr_pre, cos[:, None, :],
                                            sin[:, None, :])


def mla_preprocess_v2(arrays: dict, dtypes: dict, dims: dict,
                      eps: float = 1e-6, x_int8=None, cq_int8=None) -> dict:
    """Run the whole operator on stored inputs (named as in the library's
    MlaPreprocessV2Args).  dims: He, Hcq, N, D, Hckv, Dr.

    Returns float64 query (T, N, Hckv) and query_rope (T, N, Dr), the full
    updated kv_cache / kr_cache, the per-token cache rows, the int8 codes of
    both RmsNormQuant steps (x_int8, cq_int8) and the values they round
    (x_q, cq_q).

    x_int8 / cq_int8, when given, replace the codes of the corresponding
    RmsNormQuant step (the values it rounds are still computed and
    returned), and the rest of the chain runs from them.  A code whose value
    sits within rounding error of a .5 tie can legitimately round either
    way in a lower precision; the GPU parity check re-runs the chain from
    the GPU's own codes after checking that they differ only there.
    """
    He, Hcq, N, D, Hckv, Dr = (dims[k] for k in ("He", "Hcq", "N", "D",
                                                  "Hckv", "Dr"))
    ntot = Hcq + Hckv + Dr
    X = decode(arrays["token_x"], dtypes["token_x"]).reshape(-1, He)
    T = X.shape[0]
    W1 = decode(arrays["weight_dqkv"], dtypes["weight_dqkv"]).reshape(He, ntot)
    W2 = decode(arrays["weight_uq_qr"],
                dtypes["weight_uq_qr"]).reshape(Hcq, N * (D + Dr))
    Wuk = decode(arrays["weight_uk"], dtypes["weight_uk"]).reshape(N, D, Hckv)
    g_x = decode(arrays["gamma_x"], dtypes["gamma_x"])
    g_cq = decode(arrays["gamma_cq"], dtypes["gamma_cq"])
    g_ckv = decode(arrays["gamma_ckv"], dtypes["gamma_ckv"])
    b_x = decode(arrays["bias_x"], dtypes["bias_x"])
    b_cq = decode(arrays["bias_cq"], dtypes["bias_cq"])
    s_x = float(decode(arrays["quant_scale_x"], dtypes["quant_scale_x"]).reshape(-1)[0])
    s_cq = float(decode(arrays["quant_scale_cq"], dtypes["quant_scale_cq"]).reshape(-1)[0])
    d1 = decode(arrays["dequant_scale_dqkv"], dtypes["dequant_scale_dqkv"])
    d2 = decode(arrays["dequant_scale_uq_qr"], dtypes["dequant_scale_uq_qr"])
    cos = decode(arrays["rope_cos"], dtypes["rope_cos"]).reshape(T, Dr)
    sin = decode(arrays["rope_sin"], dtypes["rope_sin"]).reshape(T, Dr)
    index = np.asarray(arrays["cache_index"], np.int64).reshape(T)

    out = {}
    # x -> RmsNormQuant -> x W^DQKV (downsampling)
    out["x_q"] = rmsnorm_quant_values(X, g_x, b_x, s_x, eps)
    x8 = rmsnorm_quant(X, g_x, b_x, s_x, eps) if x_int8 is None \
        else np.asarray(x_int8, np.int64).reshape(T, He)
    out["x_int8"] = x8
    Y1 = int_matmul_exact(x8, W1).astype(np.float64) * d1[None, :]
    # split into path 1 (query latent) and path 2 (key latent)
    h = Y1[:, :Hcq]
    g_kv, g_r = Y1[:, Hcq:Hcq + Hckv], Y1[:, Hcq + Hckv:]
    # path 1: RmsNormQuant -> W^UQ -> paths 3 (W^UK) and 4 (RoPE)
    out["cq_q"] = rmsnorm_quant_values(h, g_cq, b_cq, s_cq, eps)
    c8 = rmsnorm_quant(h, g_cq, b_cq, s_cq, eps) if cq_int8 is None \
        else np.asarray(cq_int8, np.int64).reshape(T, Hcq)
    out["cq_int8"] = c8
    out["query"], out["query_rope"] = preprocess_query_from_codes(
        c8, W2, d2, Wuk, cos, sin, N, D, Dr)
    # path 2: path 5 (RmsNorm -> cache), path 6 (RoPE -> another cache)
    kv_rows = rmsnorm(g_kv, g_ckv, eps)
    kr_rows = rope_half(g_r, cos, sin)
    out["kv_rows"], out["kr_rows"] = kv_rows, kr_rows
    out["kv_cache"] = scatter_slots(decode(arrays["kv_cache"], dtypes["kv_cache"]),
                                    index, kv_rows[:, None, :])
    out["kr_cache"] = scatter_slots(decode(arrays["kr_cache"], dtypes["kr_cache"]),
                                    index, kr_rows[:, None, :])
    return out
