"""Pure-Python loop versions of both ops, for tiny inputs only.

Written independently of the oracle (no NumPy arithmetic: explicit loops over
Python floats and ints) so that a transposed operand, a wrong index or a
dropped term in the vectorised oracle shows up as a mismatch.  Values come in
as nested Python lists of exact floats (decoded from storage by the test).
"""

from __future__ import annotations

import math


def _dot(a, b):
    s = 0.0
    for x, y in zip(a, b):
        s += x * y
    return s


def _matvec_rows(x_row, W, ncols):
    # x_row (K) times W (K x ncols), W as a list of rows
    out = [0.0] * ncols
    for k, xv in enumerate(x_row):
        wr = W[k]
        for j in range(ncols):
            out[j] += xv * wr[j]
    return out


def _rms_norm(row, gamma, eps):
    ms = sum(v * v for v in row) / len(row)
    r = math.sqrt(ms + eps)
    return [gamma[i] * row[i] / r for i in range(len(row))]


def _rope(row, cos_row, sin_row):
    h = len(row) // 2
    out = []
    for i in range(len(row)):
        partner = -row[i + h] if i < h else row[i - h]
        out.append(row[i] * cos_row[i] + partner * sin_row[i])
    return out


def _q8(v, scale, offset=0.0):
    q = v / scale + offset
    r = round(q)  # Python rounds half to even
    return max(-128, min(127, int(r)))


def mla_prolog_brute(x, Wdq, Wdkvkr, Wuqqr, Wuk, g_cq, g_ckv, cos, sin,
                     dims, eps_cq, eps_ckv, quant=None):
    """Per-token loops.  quant: None or dict(smooth, dq[, qs_ckv, qs_ckr,
    query_int8]).

    Returns per-token lists: query[t][n][j], query_rope[t][n][j], kv_row[t],
    kr_row[t] (codes when qs_ckv / qs_ckr is given), and c8/s when
    quantised.  With query_int8 the query rows are int8 codes of a per-row
    scale max|row| / 127 (returned in q_scale[t][n]).
    """
    He, Hcq, N, D, Hckv, Dr = (dims[k] for k in ("He", "Hcq", "N", "D",
                                                  "Hckv", "Dr"))
    res = {"query": [], "query_rope": [], "kv_row": [], "kr_row": [],
           "c8": [], "s": [], "q_scale": []}
    for t in range(len(x)):
        h = _matvec_rows(x[t], Wdq, Hcq)
        cq = _rms_norm(h, g_cq, eps_cq)
        if quant is None:
            y = _matvec_rows(cq, Wuqqr, N * (D + Dr))
        else:
            u = [cq[i] * quant["smooth"][i] for i in range(Hcq)]
            amax = max(abs(v) for v in u)
            s = amax / 127.0
            c8 = [max(-127, min(127, int(round(v / s)))) if s > 0 else 0
                  for v in u]
            res["c8"].append(c8)
            res["s"].append(s)
            y = []
            for j in range(N * (D + Dr)):
                acc = 0
                for k in range(Hcq):
                    acc += c8[k] * int(Wuqqr[k][j])
                y.append(acc * s * quant["dq"][j])
        qn, qr = [], []
        for n in range(N):
            qc = y[n * D:(n + 1) * D]
            row = []
            for j in range(Hckv):
                row.append(_dot(qc, [Wuk[n][d][j] for d in range(D)]))
            qn.append(row)
            pre = y[N * D + n * Dr: N * D + (n + 1) * Dr]
            qr.append(_rope(pre, cos[t], sin[t]))
        if quant is not None and quant.get("query_int8"):
            scales = []
            for n in range(N):
                amax = max(abs(v) for v in qn[n])
                sc = amax / 127.0
                qn[n] = [max(-127, min(127, int(round(v / sc)))) if sc > 0 else 0
                         for v in qn[n]]
                scales.append(sc)
            res["q_scale"].append(scales)
        res["query"].append(qn)
        res["query_rope"].append(qr)
        g = _matvec_rows(x[t], Wdkvkr, Hckv + Dr)
        ckv = _rms_norm(g[:Hckv], g_ckv, eps_ckv)
        kr = _rope(g[Hckv:], cos[t], sin[t])
        if quant is not None and quant.get("qs_ckv") is not None:
            ckv = [_q8(ckv[j], quant["qs_ckv"][j]) for j in range(Hckv)]
        if quant is not None and quant.get("qs_ckr") is not None:
            kr = [_q8(kr[j], quant["qs_ckr"][j]) for j in range(Dr)]
        res["kv_row"].append(ckv)
        res["kr_row"].append(kr)
    return res


def qkv_brute(qkv, gq, gk, cos, sin, dims, eps, scales=None):
    """qkv[t][head][d].  scales: None or dict(ks, vs[, ko, vo]) per (h, d)."""
    Nq, Nk, Nv, D = (dims[k] for k in ("Nq", "Nk", "Nv", "D"))
    q_out, k_rows, v_rows = [], [], []
    for t in range(len(qkv)):
        qt, kt, vt = [], [], []
        for hh in range(Nq + Nk + Nv):
            row = qkv[t][hh]
            if hh < Nq:
                qt.append(_rope(_rms_norm(row, gq, eps), cos[t], sin[t]))
            elif hh < Nq + Nk:
                kr = _rope(_rms_norm(row, gk, eps), cos[t], sin[t])
                if scales is not None:
                    i = hh - Nq
                    kr = [_q8(kr[d], scales["ks"][i][d],
                              scales.get("ko", [[0.0] * D] * Nk)[i][d])
                          for d in range(D)]
                kt.append(kr)
            else:
                vr = list(row)
                if scales is not None:
                    i = hh - Nq - Nk
                    vr = [_q8(vr[d], scales["vs"][i][d],
                              scales.get("vo", [[0.0] * D] * Nv)[i][d])
                          for d in range(D)]
                vt.append(vr)
        q_out.append(qt)
        k_rows.append(kt)
        v_rows.append(vt)
    return q_out, k_rows, v_rows


def _rmsnorm_quant(row, gamma, bias, scale, eps):
    v = _rms_norm(row, gamma, eps)
    out = []
    for i in range(len(v)):
        q = round((v[i] + bias[i]) * scale)  # half to even
        out.append(max(-128, min(127, int(q))))
    return out


def preprocess_brute(x, W1, W2, Wuk, g_x, g_cq, g_ckv, b_x, b_cq, s_x, s_cq,
                     d1, d2, cos, sin, dims, eps):
    """MlaPreprocessV2 per token, in the bullets' order: RmsNormQuant of x,
    the int8 product with W^DQKV (exact Python ints) and its per-channel
    dequant, the split, RmsNormQuant of the query latent, the int8 product
    with [W^UQ | W^QR], W^UK per head, RoPE, and the key latent's RmsNorm
    and RoPE.  Returns per-token lists: query[t][n][j], query_rope[t][n][j],
    kv_row[t], kr_row[t], x8[t], c8[t]."""
    He, Hcq, N, D, Hckv, Dr = (dims[k] for k in ("He", "Hcq", "N", "D",
                                                  "Hckv", "Dr"))
    ntot = Hcq + Hckv + Dr
    res = {"query": [], "query_rope": [], "kv_row": [], "kr_row": [],
           "x8": [], "c8": []}
    for t in range(len(x)):
        x8 = _rmsnorm_quant(x[t], g_x, b_x, s_x, eps)
        y1 = []
        for j in range(ntot):
            acc = 0
            for k in range(He):
                acc += x8[k] * W1[k][j]
            y1.append(acc * d1[j])
        h, gkv, gr = y1[:Hcq], y1[Hcq:Hcq + Hckv], y1[Hcq + Hckv:]
        c8 = _rmsnorm_quant(h, g_cq, b_cq, s_cq, eps)
        ncol = N * (D + Dr)
        y2 = []
        for j in range(ncol):
            acc = 0
            for k in range(Hcq):
                acc += c8[k] * W2[k][j]
            y2.append(acc * d2[j])
        q_t, qr_t = [], []
        for n in range(N):
            qc = y2[n * D:(n + 1) * D]
            row = []
            for j in range(Hckv):
                s = 0.0
                for d in range(D):
                    s += qc[d] * Wuk[n][d][j]
                row.append(s)
            q_t.append(row)
            qr_t.append(_rope(y2[N * D + n * Dr:N * D + (n + 1) * Dr],
                              cos[t], sin[t]))
        res["query"].append(q_t)
        res["query_rope"].append(qr_t)
        res["kv_row"].append(_rms_norm(gkv, g_ckv, eps))
        res["kr_row"].append(_rope(gr, cos[t], sin[t]))
        res["x8"].append(x8)
        res["c8"].append(c8)
    return res
