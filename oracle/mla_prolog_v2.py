"""MlaPrologV2 in float64 (test infrastructure only).

Follows the "MlaPrologV2" README (ops-transformer), function description and
formulas section:

    c^Q  = RmsNorm(x . W^DQ)
    q^C  = c^Q . W^UQ
    q^N  = q^C . W^UK              (per head)
    q^R  = RoPE(c^Q . W^QR)
    c^KV = RmsNorm(x . W^DKV)      -> kv_cache   (k^C)
    k^R  = RoPE(x . W^KR)          -> kr_cache

Quantisation modes follow the constraints section's scenario table:
"none" (everything bf16), "partial_kv_bf16" (int8 weight_uq_qr with a
per-channel dequant scale and a dynamically quantised c^Q; bf16 caches),
"partial_kv_int8" (the same plus int8 caches with per-channel quant scales),
and the two full-quantisation rows: "full_kv_bf16" (also int8 token_x with
a per-token dequant scale and int8 weight_dq / weight_dkv_kr with
per-channel dequant scales; bf16 caches and outputs) and "full_kv_int8" (the
same with an int8 kv_cache, a bf16 kr_cache and an int8 query quantised per
(token, head), its scales returned as dequant_scale_q_nope), per the
dtype/shape table of the constraints section.

Readings where the page is silent (each also listed in the design notes):

* weight_uq_qr (Hcq, N*(D+Dr)) is the block concatenation [W^UQ | W^QR]:
  columns [0, N*D) are W^UQ with head n at n*D, columns [N*D, N*(D+Dr)) are
  W^QR with head n at N*D + n*Dr.  dequant_scale_w_uq_qr uses the same order.
* weight_dkv_kr (He, Hckv+Dr) is [W^DKV | W^KR].
* RoPE is the half-and-half form of aclnnQkvRmsNormRopeCache formula (3),
  with the token's (cos, sin) of width Dr shared by all heads.
* int8 GEMM dequant: y = (sum_k c8 * w8) * s_token * dq_channel.
* Cache quantisation divides by the per-channel scale (as formula (4) of
  aclnnQkvRmsNormRopeCache does), rounds half to even and saturates.
* Full quantisation dequantises the down projections the same way as the
  up projection: h = (sum_k x8 * w8) * dequant_scale_x[t] *
  dequant_scale_w[j].  Its int8 kv_cache scale is taken per channel,
  shape (1, Hckv), as the dtype/shape table gives it (the scenario table
  calls it per-tensor; a per-tensor scale is the case of equal entries).
  The int8 query is quantised per (token, head) like c^Q: scale =
  max|q^N| / 127 over the head's Hckv values, codes round half to even in
  [-127, 127]; dequant_scale_q_nope holds the scale (query ~ code * scale).
"""

from __future__ import annotations

import numpy as np

from .common import (
    decode,
    dynamic_quant_int8,
    int_matmul_exact,
    quant_int8,
    rmsnorm,
    rope_half,
    scatter_slots,
)

QUANT_MODES = ("none", "partial_kv_bf16", "partial_kv_int8", "full_kv_bf16",
               "full_kv_int8")


def _split_query(Y: np.ndarray, N: int, D: int, Dr: int):
    """Split y = c^Q . [W^UQ | W^QR] into q^C (T,N,D) and the pre-RoPE q^R."""
    T = Y.shape[0]
    qc = Y[:, : N * D].reshape(T, N, D)
    qr_pre = Y[:, N * D : N * (D + Dr)].reshape(T, N, Dr)
    return qc, qr_pre


def _per_head_uk(qc: np.ndarray, wuk: np.ndarray) -> np.ndarray:
    """q^N[t, n, :] = q^C[t, n, :] . W^UK[n]  (W^UK is (N, D, Hckv))."""
    # (N, T, D) @ (N, D, Hckv) -> (N, T, Hckv) -> (T, N, Hckv)
    return np.matmul(qc.transpose(1, 0, 2), wuk).transpose(1, 0, 2)


def mla_query_from_quantized(c8, s, w8, dq, wuk, cos, sin, N, D, Dr):
    """Query outputs from an already quantised c^Q (partial-quant modes).

    Used both by :func:`mla_prolog_v2` and to re-run the query path from a
    given (codes, scale) pair.  Inputs are decoded values: c8 (T, Hcq) and w8
    (Hcq, N*(D+Dr)) integers, s (T,), dq (N*(D+Dr),), wuk (N, D, Hckv),
    cos/sin (T, Dr) float64.
    """
    acc = int_matmul_exact(c8, w8)                       # exact int64
    Y = acc.astype(np.float64) * np.asarray(s, np.float64)[:, None] \
        * np.asarray(dq, np.float64)[None, :]
    qc, qr_pre = _split_query(Y, N, D, Dr)
    query = _per_head_uk(qc, wuk)
    query_rope = rope_half(qr_pre, cos[:, None, :], sin[:, None, :])
    return query, query_rope


def quant_query_per_head(query: np.ndarray):
    """int8 query per (token, head), the full_kv_int8 output.

    MlaPrologV2 README, scenario table: the query is returned quantised per
    token and head; dtype/shape table: dequant_scale_q_nope is (T, N, 1).
    Each head's Hckv values are quantised like c^Q's dynamic quantisation
    (without a smooth factor): scale = max|q| / 127, codes round half to
    even in [-127, 127], an all-zero row gets scale 0 and zero codes.
    Returns the codes (T, N, Hckv) and the scales (T, N).
    """
    q = np.asarray(query, np.float64)
    return dynamic_quant_int8(q, np.ones(q.shape[-1]))


def mla_prolog_v2(arrays: dict, dtypes: dict, dims: dict,
                  quant_mode: str = "none", eps_cq: float = 1e-5,
                  eps_ckv: float = 1e-5) -> dict:
    """Run the whole prolog on stored inputs.

    arrays/dtypes: the named tensors of the README's parameter table, as
    stored (bf16 as raw bits).  dims: He, Hcq, N, D, Hckv, Dr.
    Returns float64 query (T,N,Hckv), query_rope (T,N,Dr), the full updated
    kv_cache / kr_cache (float64 values, or int64 codes for int8 caches), the
    unscattered per-token cache rows, and in the partial-quant modes the
    c^Q codes and per-token scales.
    """
    if quant_mode not in QUANT_MODES:
        raise ValueError(f"quant_mode {quant_mode!r}")
    He, Hcq, N, D, Hckv, Dr = (dims[k] for k in ("He", "Hcq", "N", "D",
                                                  "Hckv", "Dr"))
    X = decode(arrays["token_x"], dtypes["token_x"]).reshape(-1, He)
    T = X.shape[0]
    Wdq = decode(arrays["weight_dq"], dtypes["weight_dq"]).reshape(He, Hcq)
    Wdkvkr = decode(arrays["weight_dkv_kr"],
                    dtypes["weight_dkv_kr"]).reshape(He, Hckv + Dr)
    Wuqqr = decode(arrays["weight_uq_qr"],
                   dtypes["weight_uq_qr"]).reshape(Hcq, N * (D + Dr))
    Wuk = decode(arrays["weight_uk"], dtypes["weight_uk"]).reshape(N, D, Hckv)
    g_cq = decode(arrays["rmsnorm_gamma_cq"], dtypes["rmsnorm_gamma_cq"])
    g_ckv = decode(arrays["rmsnorm_gamma_ckv"], dtypes["rmsnorm_gamma_ckv"])
    cos = decode(arrays["rope_cos"], dtypes["rope_cos"]).reshape(T, Dr)
    sin = decode(arrays["rope_sin"], dtypes["rope_sin"]).reshape(T, Dr)
    index = np.asarray(arrays["cache_index"], np.int64).reshape(T)
    kv_dt, kr_dt = dtypes["kv_cache"], dtypes["kr_cache"]
    kv_cache = decode(arrays["kv_cache"], kv_dt)
    kr_cache = decode(arrays["kr_cache"], kr_dt)

    out = {}
    full = quant_mode.startswith("full")
    if full:
        # int8 x (per token) and int8 down-projection weights (per channel):
        # the exact integer products, dequantised per token and per channel.
        sx = decode(arrays["dequant_scale_x"], dtypes["dequant_scale_x"]).reshape(T)
        sw_dq = decode(arrays["dequant_scale_w_dq"], dtypes["dequant_scale_w_dq"])
        sw_dkv = decode(arrays["dequant_scale_w_dkv_kr"],
                        dtypes["dequant_scale_w_dkv_kr"])
        H = int_matmul_exact(X, Wdq).astype(np.float64) * sx[:, None] * sw_dq[None, :]
        G = int_matmul_exact(X, Wdkvkr).astype(np.float64) * sx[:, None] \
            * sw_dkv[None, :]
    else:
        H = X @ Wdq
        G = X @ Wdkvkr
    # Query path.  c^Q = RmsNorm(x . W^DQ).
    cq = rmsnorm(H, g_cq, eps_cq)
    out["cq"] = cq
    if quant_mode == "none":
        # q^C = c^Q . W^UQ and the pre-RoPE q^R = c^Q . W^QR, in one product
        # over the concatenated weight.
        Y = cq @ Wuqqr
        qc, qr_pre = _split_query(Y, N, D, Dr)
        query = _per_head_uk(qc, Wuk)
        query_rope = rope_half(qr_pre, cos[:, None, :], sin[:, None, :])
    else:
        smooth = decode(arrays["smooth_scales_cq"], dtypes["smooth_scales_cq"])
        dq = decode(arrays["dequant_scale_w_uq_qr"],
                    dtypes["dequant_scale_w_uq_qr"])
        c8, s = dynamic_quant_int8(cq, smooth)
        out["cq_int8"], out["cq_scale"] = c8, s
        query, query_rope = mla_query_from_quantized(
            c8, s, Wuqqr.astype(np.int64), dq, Wuk, cos, sin, N, D, Dr)
    if quant_mode == "full_kv_int8":
        out["query_f64"] = query
        query, out["dequant_scale_q_nope"] = quant_query_per_head(query)
    out["query"] = query
    out["query_rope"] = query_rope

    # Key path.  c^KV = RmsNorm(x . W^DKV) and k^R = RoPE(x . W^KR).
    ckv = rmsnorm(G[:, :Hckv], g_ckv, eps_ckv)
    kr = rope_half(G[:, Hckv:], cos, sin)
    out["ckv"], out["kr"] = ckv, kr
    if quant_mode == "partial_kv_int8":
        qs_ckv = decode(arrays["quant_scale_ckv"], dtypes["quant_scale_ckv"])
        qs_ckr = decode(arrays["quant_scale_ckr"], dtypes["quant_scale_ckr"])
        kv_rows = quant_int8(ckv, qs_ckv)
        kr_rows = quant_int8(kr, qs_ckr)
    elif quant_mode == "full_kv_int8":
        qs_ckv = decode(arrays["quant_scale_ckv"], dtypes["quant_scale_ckv"])
        kv_rows = quant_int8(ckv, qs_ckv)
        kr_rows = kr
    else:
        kv_rows, kr_rows = ckv, kr
    out["kv_rows"], out["kr_rows"] = kv_rows, kr_rows
    # k^C = Cache(c^KV), k^R = Cache(RoPE(x . W^KR)): rows go to their slots.
    out["kv_cache"] = scatter_slots(kv_cache, index, kv_rows[:, None, :])
    out["kr_cache"] = scatter_slots(kr_cache, index, kr_rows[:, None, :])
    return out
