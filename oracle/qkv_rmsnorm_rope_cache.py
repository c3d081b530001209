"""QkvRmsNormRopeCache in float64 (test infrastructure only).

Follows "aclnnQkvRmsNormRopeCache" (CANN API reference): the API function
description (outputs qOut, kCache, vCache and the optional BeforeQuant
tensors) and formulas (1) SplitVD, (2) RmsNorm, (3) RoPE half-and-half and
(4) Quant; the cache-index rule comes from its other restrictions.

Readings where the page is silent or its tables were lost:

* qkv is (T, Nq+Nk+Nv, D); gamma_q and gamma_k are (D,) shared by heads;
  cos and sin are (T, D) shared by heads (the requireMemory sum counts 2*D
  gamma values and 2*B*S*D RoPE values).
* v is only split, quantised and scattered (formulas (2) and (3) name q and
  k only); q is normalised and rotated but never quantised.
* Scales and offsets are per channel over (head, dim): k_scale (Nk*D),
  v_scale (Nv*D), likewise the offsets.
* Caches are (BlockNum, BlockSize, Nk|Nv, D), slot s at [s // BlockSize,
  s % BlockSize]; int8 when quantised, else the input dtype.
* The optional BeforeQuant outputs are the per-token values just before the
  quant step: qRoPE, kRoPE and v.
"""

from __future__ import annotations

import numpy as np

from .common import decode, quant_int8, rmsnorm, rope_half, scatter_slots

QUANT_MODES = ("none", "symmetric", "asymmetric")


def qkv_rmsnorm_rope_cache(arrays: dict, dtypes: dict, dims: dict,
                           quant_mode: str = "symmetric",
                           eps: float = 1e-6) -> dict:
    if quant_mode not in QUANT_MODES:
        raise ValueError(f"quant_mode {quant_mode!r}")
    Nq, Nk, Nv, D = (dims[k] for k in ("Nq", "Nk", "Nv", "D"))
    if Nk != Nv:
        raise ValueError("SplitVD requires Nk == Nv")
    qkv = decode(arrays["qkv"], dtypes["qkv"]).reshape(-1, Nq + Nk + Nv, D)
    T = qkv.shape[0]
    gq = decode(arrays["gamma_q"], dtypes["gamma_q"]).reshape(D)
    gk = decode(arrays["gamma_k"], dtypes["gamma_k"]).reshape(D)
    cos = decode(arrays["cos"], dtypes["cos"]).reshape(T, 1, D)
    sin = decode(arrays["sin"], dtypes["sin"]).reshape(T, 1, D)
    index = np.asarray(arrays["index"], np.int64).reshape(T)

    # (1) SplitVD: q = first Nq heads, k = the middle Nk, v = the last Nv.
    q = qkv[:, :Nq]
    k = qkv[:, Nq:Nq + Nk]
    v = qkv[:, Nq + Nk:]
    # (2) RmsNorm of q and k over D, (3) half-and-half RoPE.
    q_rope = rope_half(rmsnorm(q, gq, eps), cos, sin)
    k_rope = rope_half(rmsnorm(k, gk, eps), cos, sin)
    # (4) Quant of k and v.
    if quant_mode == "none":
        k_rows, v_rows = k_rope, v
    else:
        ks = decode(arrays["k_scale"], dtypes["k_scale"]).reshape(Nk, D)
        vs = decode(arrays["v_scale"], dtypes["v_scale"]).reshape(Nv, D)
        ko = vo = None
        if quant_mode == "asymmetric":
            ko = decode(arrays["k_offset"], dtypes["k_offset"]).reshape(Nk, D)
            vo = decode(arrays["v_offset"], dtypes["v_offset"]).reshape(Nv, D)
        k_rows = quant_int8(k_rope, ks, ko)
        v_rows = quant_int8(v, vs, vo)

    out = {
        "q_out": q_rope,
        "k_rows": k_rows,
        "v_rows": v_rows,
        "q_before_quant": q_rope,
        "k_before_quant": k_rope,
        "v_before_quant": v,
    }
    kc = decode(arrays["k_cache"], dtypes["k_cache"])
    vc = decode(arrays["v_cache"], dtypes["v_cache"])
    out["k_cache"] = scatter_slots(kc, index, k_rows)
    out["v_cache"] = scatter_slots(vc, index, v_rows)
    return out
