"""Shared helpers of the GPU parity tests: device upload of seeded workloads,
calls through the library's binding, and the acceptance checks.

Acceptance (per output kind):
* bf16 / fp16 values: |gpu - ref| <= 0.02 * max(1, |ref|) elementwise;
* int8 cache codes: within +/-1 of the oracle's code;
* cache slots no valid index names: bit-identical to their bytes before the
  call; the set of changed slots equals the set of valid indexes.
"""

from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import qkv_norm_rope_amd as qn
from oracle.common import decode
from workloads import device as _dev
from workloads import sub_workload  # noqa: F401  (re-exported for the tests)

TOL_REL = 0.02


def announce(msg: str):
    print(f"[gpu] {msg}", file=sys.stderr, flush=True)


to_dev = _dev.to_device
upload = _dev.upload


def dev_to_f64(t: torch.Tensor) -> np.ndarray:
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.float().cpu().numpy().astype(np.float64)
    if t.dtype == torch.int8:
        return t.cpu().numpy().astype(np.int64)
    return t.cpu().numpy().astype(np.float64)


def raw_bits(t: torch.Tensor) -> np.ndarray:
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).cpu().numpy()
    return t.cpu().numpy()


def assert_close(gpu: np.ndarray, ref: np.ndarray, what: str,
                 tol_rel: float = TOL_REL):
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    if gpu.size == 0:
        return 0.0
    bound = tol_rel * np.maximum(1.0, np.abs(ref))
    err = np.abs(gpu - ref)
    bad = err > bound
    ratio = float((err / bound).max())
    if bad.any():
        i = np.argwhere(bad)[:5]
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {gpu.size} elements outside "
            f"0.02*max(1,|ref|); worst err/tol {ratio:.3g}; first at "
            f"{i.tolist()}: gpu={gpu[tuple(i[0])]!r} ref={ref[tuple(i[0])]!r}")
    return ratio


def assert_codes(gpu: np.ndarray, ref: np.ndarray, what: str):
    d = np.abs(gpu.astype(np.int64) - ref.astype(np.int64))
    if (d > 1).any():
        i = np.argwhere(d > 1)[:5]
        raise AssertionError(f"{what}: {int((d > 1).sum())} codes off by >1, "
                             f"first at {i.tolist()}")
    return int((d == 1).sum())


def check_cache(before_bits: np.ndarray, after: torch.Tensor, index: np.ndarray,
                ref_rows: np.ndarray, is_int8: bool, what: str,
                token_rows=None):
    """before_bits: raw cache bits before the call; after: device cache.

    ref_rows[i] is the oracle row of token token_rows[i] (all tokens when
    token_rows is None).
    """
    bn, bs = after.shape[0], after.shape[1]
    slots = bn * bs
    after_bits = raw_bits(after).reshape(slots, -1)
    before_bits = before_bits.reshape(slots, -1)
    changed = np.nonzero((after_bits != before_bits).any(axis=1))[0]
    valid = index[index >= 0]
    # every changed slot is a valid index (a written row may equal its old
    # bytes by chance, so valid slots need not all differ)
    extra = np.setdiff1d(changed, valid)
    assert extra.size == 0, f"{what}: slots written without an index: {extra[:8]}"
    toks = np.arange(index.size) if token_rows is None else token_rows
    # An indexed slot whose bytes did not change must belong to a token whose
    # row is compared below: it passes only if its old bytes already hold
    # that token's row (a missed write fails the comparison).
    unchanged = np.setdiff1d(valid, changed)
    checked = index[toks][index[toks] >= 0]
    missed = np.setdiff1d(unchanged, checked)
    assert missed.size == 0, \
        f"{what}: indexed slots left unchanged: {missed[:8]}"
    vals = dev_to_f64(after).reshape(slots, -1)
    worst = 0.0
    for i, t in enumerate(toks):
        s = index[t]
        if s < 0:
            continue
        if is_int8:
            assert_codes(vals[s], ref_rows[i].reshape(-1), f"{what} slot {s}")
        else:
            worst = max(worst, assert_close(vals[s], ref_rows[i].reshape(-1),
                                            f"{what} slot {s}"))
    return worst


# ---------------------------------------------------------------------------
# MLA prolog
# ---------------------------------------------------------------------------

def mla_dims(cfg):
    return dict(He=cfg.He, Hcq=cfg.Hcq, N=cfg.N, D=cfg.D, Hckv=cfg.Hckv,
                Dr=cfg.Dr)


def run_mla_gpu(w, dev=None, layout="packed", bsh=False, workspace=None):
    """Run the library on workload w.  Returns dict of device tensors."""
    cfg = w.cfg
    d = dev if dev is not None else upload(w)
    quant = cfg.quant_mode
    if layout == "packed":
        wdq = qn.mla_pack_weight(d["weight_dq"])
        wdkvkr = qn.mla_pack_weight(d["weight_dkv_kr"])
        wuqqr = qn.mla_pack_weight_uq_qr(d["weight_uq_qr"], cfg.N, cfg.D,
                                         cfg.Dr)
        wuk = qn.mla_pack_weight_uk(d["weight_uk"])
        lay = qn.MLA_WEIGHT_PACKED_K16
    else:
        wdq, wdkvkr, wuqqr, wuk = (d["weight_dq"], d["weight_dkv_kr"],
                                   d["weight_uq_qr"], d["weight_uk"])
        lay = qn.MLA_WEIGHT_ND
    x = d["token_x"]
    if bsh:
        x = x.view(cfg.B, cfg.S, cfg.He)
    res = qn.mla_prolog_v2(
        x, wdq, wuqqr, wuk, wdkvkr, d["rmsnorm_gamma_cq"],
        d["rmsnorm_gamma_ckv"], d["rope_sin"], d["rope_cos"],
        d["cache_index"], d["kv_cache"], d["kr_cache"], quant_mode=quant,
        weight_layout=lay, rmsnorm_epsilon_cq=cfg.eps_cq,
        rmsnorm_epsilon_ckv=cfg.eps_ckv,
        dequant_scale_w_uq_qr=d.get("dequant_scale_w_uq_qr"),
        quant_scale_ckv=d.get("quant_scale_ckv"),
        quant_scale_ckr=d.get("quant_scale_ckr"),
        smooth_scales_cq=d.get("smooth_scales_cq"),
        dequant_scale_x=d.get("dequant_scale_x"),
        dequant_scale_w_dq=d.get("dequant_scale_w_dq"),
        dequant_scale_w_dkv_kr=d.get("dequant_scale_w_dkv_kr"),
        return_cq_quant=quant != "none", workspace=workspace)
    out = {"query": res[0], "query_rope": res[1], "kv_cache": d["kv_cache"],
           "kr_cache": d["kr_cache"]}
    if quant == "full_kv_int8":
        out["dequant_scale_q_nope"] = res[2]
    if quant != "none":
        out["cq_int8"], out["cq_scale"] = res[-2], res[-1]
    return out


def check_mla(w, out, before, tokens=None, chunk=None):
    """Compare GPU outputs against the oracle (on `tokens` only if given).

    chunk: run the oracle on consecutive pieces of at most `chunk` of the
    checked tokens (tokens are independent, so each piece is the same
    workload restricted to its tokens); every checked token is still
    compared, and the caches are checked over all of them at once.
    Returns the worst err/tol ratio per output (and the quantised paths'
    counters, summed).
    """
    cfg = w.cfg
    toks = np.arange(cfg.T) if tokens is None else np.asarray(tokens)
    step = max(1, toks.size if not chunk else int(chunk))
    T = cfg.T
    q_all = out["query"].reshape(T, cfg.N, cfg.Hckv)
    qr_all = out["query_rope"].reshape(T, cfg.N, cfg.Dr)
    stats = {}
    kv_rows, kr_rows = [], []
    for c0 in range(0, max(toks.size, 1), step):
        sel = toks[c0:c0 + step]
        whole = tokens is None and sel.size == T
        ww = w if whole else sub_workload(w, sel)
        ref = oracle.mla_prolog_v2(ww.arrays, ww.dtypes, mla_dims(cfg),
                                   cfg.quant_mode, cfg.eps_cq, cfg.eps_ckv)
        if whole:
            q, qr = q_all, qr_all
        else:
            idx_t = torch.as_tensor(sel, device=q_all.device)
            q, qr = q_all[idx_t], qr_all[idx_t]
        if cfg.quant_mode == "none":
            part = {"query": assert_close(dev_to_f64(q), ref["query"], "query"),
                    "query_rope": assert_close(dev_to_f64(qr),
                                               ref["query_rope"],
                                               "query_rope")}
        else:
            part = check_quant_conditioned(ww, ref, out, q, qr,
                                           None if whole else sel)
        for k, v in part.items():
            if isinstance(v, int):
                stats[k] = stats.get(k, 0) + v
            else:
                stats[k] = max(stats.get(k, 0.0), v)
        kv_rows.append(ref["kv_rows"])
        kr_rows.append(ref["kr_rows"])
    kv8 = cfg.quant_mode in ("partial_kv_int8", "full_kv_int8")
    kr8 = cfg.quant_mode == "partial_kv_int8"
    index = w.arrays["cache_index"].reshape(-1)
    if cfg.slots > 0:
        tok = None if tokens is None else toks
        stats["kv_cache"] = check_cache(before["kv_cache"], out["kv_cache"],
                                        index, np.concatenate(kv_rows), kv8,
                                        "kv_cache", tok)
        stats["kr_cache"] = check_cache(before["kr_cache"], out["kr_cache"],
                                        index, np.concatenate(kr_rows), kr8,
                                        "kr_cache", tok)
    return stats


def check_quant_conditioned(ww, ref, out, q, qr, tokens):
    """Partial-quant parity, conditioned on the GPU's own c^Q codes.

    (i) per-token scales agree to 1e-5 relative; (ii) every code is within
    +/-1 of the oracle's and differs only where the oracle's value sits
    within 1e-2 of a rounding tie; (iii) query and query_rope match the
    oracle's up-projection re-run from the GPU's codes and scales.
    """
    cfg = ww.cfg
    c8 = out["cq_int8"].cpu().numpy().astype(np.int64)
    s = out["cq_scale"].cpu().numpy().astype(np.float64)
    if tokens is not None:
        c8, s = c8[tokens], s[tokens]
    np.testing.assert_allclose(s, ref["cq_scale"], rtol=1e-5, atol=0)
    smooth = decode(ww.arrays["smooth_scales_cq"], "fp32")
    u_over_s = ref["cq"] * smooth / np.where(ref["cq_scale"] > 0,
                                             ref["cq_scale"], 1.0)[:, None]
    diff = c8 != ref["cq_int8"]
    assert np.abs(c8 - ref["cq_int8"]).max() <= 1
    frac = np.abs(u_over_s) - np.floor(np.abs(u_over_s))
    tie_dist = np.abs(frac - 0.5)
    assert (tie_dist[diff] < 1e-2).all(), "code flips away from a tie"
    W8 = decode(ww.arrays["weight_uq_qr"], "int8")
    dq = decode(ww.arrays["dequant_scale_w_uq_qr"], "fp32")
    Wuk = decode(ww.arrays["weight_uk"], "bf16").reshape(cfg.N, cfg.D, cfg.Hckv)
    cos = decode(ww.arrays["rope_cos"], "bf16").reshape(-1, cfg.Dr)
    sin = decode(ww.arrays["rope_sin"], "bf16").reshape(-1, cfg.Dr)
    rq, rqr = oracle.mla_query_from_quantized(c8, s, W8, dq, Wuk, cos, sin,
                                              cfg.N, cfg.D, cfg.Dr)
    stats = {"code_flips": int(diff.sum()),
             "query_rope": assert_close(dev_to_f64(qr), rqr, "query_rope")}
    if cfg.quant_mode != "full_kv_int8":
        stats["query"] = assert_close(dev_to_f64(q), rq, "query")
        return stats
    # int8 query per (token, head): the oracle's quantisation of the re-run
    # q^N; scales to 1e-3 relative, codes within +/-1
    codes, scale = oracle.mla_prolog_v2_quant_query(rq)
    sg = out["dequant_scale_q_nope"].reshape(-1, cfg.N).cpu().numpy().astype(np.float64)
    if tokens is not None:
        sg = sg[tokens]
    np.testing.assert_allclose(sg, scale, rtol=1e-3, atol=1e-12)
    qg = q.cpu().numpy().astype(np.int64)
    assert_codes(qg, codes, "query")
    stats["query_code_mismatch"] = int((qg != codes).sum())
    return stats


# ---------------------------------------------------------------------------
# qkv op
# ---------------------------------------------------------------------------

def run_qkv_gpu(w, dev=None):
    cfg = w.cfg
    d = dev if dev is not None else upload(w)
    res = qn.qkv_rmsnorm_rope_cache(
        d["qkv"], d["gamma_q"], d["gamma_k"], d["cos"], d["sin"], d["index"],
        d["k_cache"], d["v_cache"], Nq=cfg.Nq, Nk=cfg.Nk, Nv=cfg.Nv,
        quant_mode=cfg.quant_mode, epsilon=cfg.eps,
        k_scale=d.get("k_scale"), v_scale=d.get("v_scale"),
        k_offset=d.get("k_offset"), v_offset=d.get("v_offset"),
        before_quant=cfg.before_quant, B=cfg.B, S=cfg.S)
    out = {"k_cache": d["k_cache"], "v_cache": d["v_cache"]}
    if cfg.before_quant:
        out["q_out"], out["q_bq"], out["k_bq"], out["v_bq"] = res
    else:
        out["q_out"] = res
    return out


def check_qkv(w, out, before):
    cfg = w.cfg
    ref = oracle.qkv_rmsnorm_rope_cache(
        w.arrays, w.dtypes, dict(Nq=cfg.Nq, Nk=cfg.Nk, Nv=cfg.Nv, D=cfg.D),
        cfg.quant_mode, cfg.eps)
    stats = {"q_out": assert_close(dev_to_f64(out["q_out"]), ref["q_out"],
                                   "q_out")}
    if cfg.before_quant:
        stats["q_bq"] = assert_close(dev_to_f64(out["q_bq"]),
                                     ref["q_before_quant"], "q_before_quant")
        stats["k_bq"] = assert_close(dev_to_f64(out["k_bq"]),
                                     ref["k_before_quant"], "k_before_quant")
        # v passes through unchanged: bit-exact
        np.testing.assert_array_equal(raw_bits(out["v_bq"]).reshape(-1),
                                      w.arrays["qkv"].reshape(
                                          cfg.T, -1, cfg.D)[:, cfg.Nq + cfg.Nk:]
                                      .view(np.int16).reshape(-1))
    int8 = cfg.quant_mode != "none"
    index = w.arrays["index"].reshape(-1)
    stats["k_cache"] = check_cache(before["k_cache"], out["k_cache"], index,
                                   ref["k_rows"], int8, "k_cache")
    stats["v_cache"] = check_cache(before["v_cache"], out["v_cache"], index,
                                   ref["v_rows"], int8, "v_cache")
    return stats


# ---------------------------------------------------------------------------
# MlaPreprocessV2
# ---------------------------------------------------------------------------

def run_preprocess_gpu(w, dev=None, layout="packed", bsh=False):
    """Run MlaPreprocessV2 on workload w; returns dict of device tensors
    (query, query_rope, caches, and the two steps' int8 codes)."""
    cfg = w.cfg
    d = dev if dev is not None else upload(w)
    if layout == "packed":
        w1 = qn.mla_pack_weight(d["weight_dqkv"])
        w2 = qn.mla_pack_weight_uq_qr(d["weight_uq_qr"], cfg.N, cfg.D, cfg.Dr)
        wuk = qn.mla_pack_weight_uk(d["weight_uk"])
        lay = qn.MLA_WEIGHT_PACKED_K16
    else:
        w1, w2, wuk = d["weight_dqkv"], d["weight_uq_qr"], d["weight_uk"]
        lay = qn.MLA_WEIGHT_ND
    x = d["token_x"]
    if bsh:
        x = x.view(cfg.B, cfg.S, cfg.He)
    q, qr, x8, c8 = qn.mla_preprocess_v2(
        x, d["gamma_x"], d["bias_x"], float(w.arrays["quant_scale_x"][0]), w1,
        d["dequant_scale_dqkv"], d["gamma_cq"], d["bias_cq"],
        float(w.arrays["quant_scale_cq"][0]), w2, d["dequant_scale_uq_qr"],
        wuk, d["gamma_ckv"], d["rope_sin"], d["rope_cos"], d["cache_index"],
        d["kv_cache"], d["kr_cache"], epsilon=cfg.eps, weight_layout=lay,
        return_codes=True)
    return {"query": q, "query_rope": qr, "kv_cache": d["kv_cache"],
            "kr_cache": d["kr_cache"], "x_int8": x8, "cq_int8": c8}


def _codes_near_ties(gpu, ref_codes, values, what, window=1e-2):
    """GPU int8 codes within +/-1 of the oracle's, differing only where the
    oracle's unrounded value sits within `window` of a .5 tie."""
    diff = gpu != ref_codes
    assert np.abs(gpu - ref_codes).max(initial=0) <= 1, f"{what}: code off by >1"
    v = np.abs(values)
    tie = np.abs(v - np.floor(v) - 0.5)
    assert (tie[diff] < window).all(), f"{what}: a code flips away from a tie"
    return int(diff.sum())


def check_preprocess(w, out, before):
    """MlaPreprocessV2 parity, conditioned on the GPU's own int8 codes (the
    A-9 rule of the prolog, applied to both RmsNormQuant steps): (i) x's
    codes within +/-1 of the oracle's, differing only near a rounding tie;
    (ii) the query latent's codes likewise against the oracle re-run from
    the GPU's x codes; (iii) query, query_rope and every cache row against
    the oracle re-run from both of the GPU's code sets, under the
    0.02 * max(1, |ref|) rule; placement as for the prolog."""
    cfg = w.cfg
    dims = mla_dims(cfg)
    ref = oracle.mla_preprocess_v2(w.arrays, w.dtypes, dims, cfg.eps)
    x8 = out["x_int8"].cpu().numpy().astype(np.int64)
    stats = {"x_code_flips": _codes_near_ties(x8, ref["x_int8"], ref["x_q"],
                                              "x codes")}
    if stats["x_code_flips"]:
        ref = oracle.mla_preprocess_v2(w.arrays, w.dtypes, dims, cfg.eps,
                                       x_int8=x8)
    c8 = out["cq_int8"].cpu().numpy().astype(np.int64)
    stats["cq_code_flips"] = _codes_near_ties(c8, ref["cq_int8"], ref["cq_q"],
                                              "c^Q codes")
    if stats["cq_code_flips"]:
        ref = oracle.mla_preprocess_v2(w.arrays, w.dtypes, dims, cfg.eps,
                                       x_int8=x8, cq_int8=c8)
    T = cfg.T
    stats["query"] = assert_close(
        dev_to_f64(out["query"].reshape(T, cfg.N, cfg.Hckv)), ref["query"],
        "query")
    stats["query_rope"] = assert_close(
        dev_to_f64(out["query_rope"].reshape(T, cfg.N, cfg.Dr)),
        ref["query_rope"], "query_rope")
    index = w.arrays["cache_index"].reshape(-1)
    if cfg.slots > 0:
        stats["kv_cache"] = check_cache(before["kv_cache"], out["kv_cache"],
                                        index, ref["kv_rows"], False,
                                        "kv_cache")
        stats["kr_cache"] = check_cache(before["kr_cache"], out["kr_cache"],
                                        index, ref["kr_rows"], False,
                                        "kr_cache")
    return stats
