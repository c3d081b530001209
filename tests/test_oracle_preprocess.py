"""Pins for the MlaPreprocessV2 part of the float64 oracle.

RmsNormQuant is pinned by hand-derived worked examples
(tests/golden/worked_examples.txt), closed forms and invariants; the whole
operator by pure-Python brute-force loops on tiny inputs and by reductions
to the already-pinned MlaPrologV2 oracle functions (its key path is the
full-quantisation key path of the prolog fed the RmsNormQuant codes, its
query path the prolog's query path from given codes).  Mutants of
RmsNormQuant (the readings turned around) must fail a pin.
"""

from __future__ import annotations

import importlib

import numpy as np
import pytest

import oracle
from tests import brute_force as bf
from tests.test_oracle_pins import _golden, _kv, _vec
from workloads import make_workload

op = importlib.import_module("oracle.mla_preprocess_v2")
DIMS = ("He", "Hcq", "N", "D", "Hckv", "Dr")


def _dims(cfg):
    return {k: getattr(cfg, k) for k in DIMS}


# ---------------------------------------------------------------- pins ----

def pin_rmsnorm_quant_golden(rq):
    for spec, want in _golden("rmsnormquant"):
        a = _kv(spec)
        got = rq(a["v"], a["gamma"], a["bias"], float(a["scale"][0]),
                 float(a["eps"][0]))
        np.testing.assert_array_equal(got, _vec(want).astype(np.int64))


def pin_rmsnorm_quant_closed_forms(rq, rng):
    # a constant row with gamma = 1, bias = 0, eps = 0 normalises to its
    # sign, so every code is round(scale) with that sign
    for c in (-3.7, 0.01, 250.0):
        row = np.full((1, 40), c)
        got = rq(row, np.ones(40), np.zeros(40), 17.0, 0.0)
        np.testing.assert_array_equal(got, np.full((1, 40), 17 * np.sign(c)))
    # the bias shifts before the scale: (1 + b) * s with b = 0.5, s = 9
    got = rq(np.ones((1, 8)), np.ones(8), np.full(8, 0.5), 9.0, 0.0)
    np.testing.assert_array_equal(got, np.full((1, 8), 14))  # 13.5 -> 14
    # scale invariance of the norm: codes of alpha * v equal codes of v
    v = rng.standard_normal((6, 96))
    g, b = rng.uniform(0.5, 1.5, 96), rng.uniform(-0.1, 0.1, 96)
    np.testing.assert_array_equal(rq(3.25 * v, g, b, 23.0, 0.0),
                                  rq(v, g, b, 23.0, 0.0))
    # rows built so that every value is an exact integer + 1/4: codes are
    # the integers (no tie), within the int8 range
    k = rng.integers(-100, 100, (4, 16)).astype(np.float64)
    vals = k + 0.25
    # RmsNorm of a row of +-1 with eps = 0 is gamma * row: put the wanted
    # value into gamma (scale 1, bias 0)
    ones = np.ones((4, 16))
    for r in range(4):
        got = rq(ones[r:r + 1], vals[r], np.zeros(16), 1.0, 0.0)
        np.testing.assert_array_equal(got[0], k[r])
    # saturation on both sides
    got = rq(np.array([[1.0, -1.0]]), np.ones(2), np.zeros(2), 1e4, 0.0)
    np.testing.assert_array_equal(got, [[127, -128]])


def test_rmsnorm_quant_golden():
    pin_rmsnorm_quant_golden(oracle.rmsnorm_quant)


def test_rmsnorm_quant_closed_forms(rng):
    pin_rmsnorm_quant_closed_forms(oracle.rmsnorm_quant, rng)


# ---------------------------------------------------------- brute force ----

def _decoded(w):
    a, t = w.arrays, w.dtypes
    d = {k: oracle.decode(v, t[k]) for k, v in a.items()}
    return d


@pytest.mark.parametrize("key", ["pre_tiny", "pre_ragged"])
def test_preprocess_matches_brute_force(key):
    w = make_workload(key)
    c = w.cfg
    if key == "pre_ragged":  # keep the pure-Python loops to a few seconds
        from workloads import sub_workload
        w = sub_workload(w, np.arange(5))
    ref = oracle.mla_preprocess_v2(w.arrays, w.dtypes, _dims(c), c.eps)
    d = _decoded(w)
    T = w.cfg.T
    ntot = c.Hcq + c.Hckv + c.Dr
    res = bf.preprocess_brute(
        d["token_x"].reshape(T, c.He).tolist(),
        d["weight_dqkv"].reshape(c.He, ntot).tolist(),
        d["weight_uq_qr"].reshape(c.Hcq, -1).tolist(),
        d["weight_uk"].reshape(c.N, c.D, c.Hckv).tolist(),
        d["gamma_x"].tolist(), d["gamma_cq"].tolist(), d["gamma_ckv"].tolist(),
        d["bias_x"].tolist(), d["bias_cq"].tolist(),
        float(d["quant_scale_x"][0]), float(d["quant_scale_cq"][0]),
        d["dequant_scale_dqkv"].tolist(), d["dequant_scale_uq_qr"].tolist(),
        d["rope_cos"].reshape(T, c.Dr).tolist(),
        d["rope_sin"].reshape(T, c.Dr).tolist(), _dims(c), c.eps)
    np.testing.assert_array_equal(np.array(res["x8"]), ref["x_int8"])
    np.testing.assert_array_equal(np.array(res["c8"]), ref["cq_int8"])
    np.testing.assert_allclose(np.array(res["query"]), ref["query"],
                               rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(np.array(res["query_rope"]), ref["query_rope"],
                               rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(np.array(res["kv_row"]), ref["kv_rows"],
                               rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(np.array(res["kr_row"]), ref["kr_rows"],
                               rtol=1e-11, atol=1e-12)
    # no code sits on a rounding tie, so the exact comparison above is fair
    for q in (ref["x_q"], ref["cq_q"]):
        assert np.min(np.abs(np.abs(q - np.floor(q)) - 0.5)) > 1e-9


# --------------------------------------- reductions to the pinned prolog ----

def test_preprocess_key_path_is_the_prolog_full_quant_key_path():
    # MlaPrologV2 in full quantisation computes c^KV = RmsNorm(x8 . W^DKV *
    # sx * sw) and k^R = RoPE(x8 . W^KR * sx * sw).  Fed the RmsNormQuant
    # codes as token_x, sx = 1 and the split of W^DQKV and its dequant
    # scales, it must give the preprocess key rows.
    w = make_workload("pre_ragged")
    c = w.cfg
    ref = oracle.mla_preprocess_v2(w.arrays, w.dtypes, _dims(c), c.eps)
    A = w.arrays
    W1 = A["weight_dqkv"]
    d1 = A["dequant_scale_dqkv"]
    T = c.T
    arr = {
        "token_x": ref["x_int8"].astype(np.int8),
        "weight_dq": W1[:, :c.Hcq], "weight_dkv_kr": W1[:, c.Hcq:],
        "weight_uq_qr": A["weight_uq_qr"], "weight_uk": A["weight_uk"],
        "rmsnorm_gamma_cq": A["gamma_cq"], "rmsnorm_gamma_ckv": A["gamma_ckv"],
        "rope_cos": A["rope_cos"], "rope_sin": A["rope_sin"],
        "cache_index": A["cache_index"], "kv_cache": A["kv_cache"],
        "kr_cache": A["kr_cache"],
        "dequant_scale_x": np.ones(T, np.float32),
        "dequant_scale_w_dq": d1[:c.Hcq], "dequant_scale_w_dkv_kr": d1[c.Hcq:],
        "dequant_scale_w_uq_qr": A["dequant_scale_uq_qr"],
        "smooth_scales_cq": np.ones(c.Hcq, np.float32),
    }
    typ = {k: ("int8" if arr[k].dtype == np.int8 else
               "fp32" if arr[k].dtype == np.float32 else
               "int64" if arr[k].dtype == np.int64 else "bf16") for k in arr}
    pro = oracle.mla_prolog_v2(arr, typ, _dims(c), "full_kv_bf16", c.eps, c.eps)
    np.testing.assert_allclose(pro["kv_rows"], ref["kv_rows"], rtol=1e-13,
                               atol=1e-14)
    np.testing.assert_allclose(pro["kr_rows"], ref["kr_rows"], rtol=1e-13,
                               atol=1e-14)
    np.testing.assert_array_equal(pro["kv_cache"], ref["kv_cache"])


def test_preprocess_query_path_is_the_prolog_query_path_from_codes():
    # The prolog's query path from given c^Q codes and per-token scale 1 is
    # the preprocess paths 3 and 4.
    w = make_workload("pre_ragged")
    c = w.cfg
    ref = oracle.mla_preprocess_v2(w.arrays, w.dtypes, _dims(c), c.eps)
    d = _decoded(w)
    q, qr = oracle.mla_query_from_quantized(
        ref["cq_int8"], np.ones(c.T), d["weight_uq_qr"].reshape(c.Hcq, -1),
        d["dequant_scale_uq_qr"], d["weight_uk"].reshape(c.N, c.D, c.Hckv),
        d["rope_cos"].reshape(c.T, c.Dr), d["rope_sin"].reshape(c.T, c.Dr),
        c.N, c.D, c.Dr)
    np.testing.assert_allclose(q, ref["query"], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(qr, ref["query_rope"], rtol=1e-13, atol=1e-13)


def test_preprocess_scatter_and_empty():
    w = make_workload("pre_tiny")
    c = w.cfg
    ref = oracle.mla_preprocess_v2(w.arrays, w.dtypes, _dims(c), c.eps)
    idx = w.arrays["cache_index"]
    before = oracle.decode(w.arrays["kv_cache"], "bf16").reshape(c.slots, -1)
    after = ref["kv_cache"].reshape(c.slots, -1)
    changed = np.nonzero((before != after).any(axis=1))[0]
    np.testing.assert_array_equal(np.sort(changed), np.sort(idx[idx >= 0]))
    # no tokens: empty outputs, caches untouched
    from workloads import sub_workload
    e = sub_workload(w, np.arange(0))
    r0 = oracle.mla_preprocess_v2(e.arrays, e.dtypes, _dims(c), c.eps)
    assert r0["query"].shape == (0, c.N, c.Hckv)
    np.testing.assert_array_equal(r0["kv_cache"].reshape(c.slots, -1), before)


# ------------------------------------------------------------- mutants ----

def _mutant_divide(v, g, b, s, eps):
    return np.clip(np.rint((oracle.rmsnorm(v, g, eps) + b) / s), -128,
                   127).astype(np.int64)


def _mutant_bias_after_scale(v, g, b, s, eps):
    return np.clip(np.rint(oracle.rmsnorm(v, g, eps) * s + b), -128,
                   127).astype(np.int64)


def _mutant_no_bias(v, g, b, s, eps):
    return np.clip(np.rint(oracle.rmsnorm(v, g, eps) * s), -128,
                   127).astype(np.int64)


def _mutant_truncate(v, g, b, s, eps):
    return np.clip(np.trunc((oracle.rmsnorm(v, g, eps) + b) * s), -128,
                   127).astype(np.int64)


def _mutant_half_up(v, g, b, s, eps):
    return np.clip(np.floor((oracle.rmsnorm(v, g, eps) + b) * s + 0.5), -128,
                   127).astype(np.int64)


def _mutant_sym127(v, g, b, s, eps):
    return np.clip(np.rint((oracle.rmsnorm(v, g, eps) + b) * s), -127,
                   127).astype(np.int64)


@pytest.mark.parametrize("mutant", [_mutant_divide, _mutant_bias_after_scale,
                                    _mutant_no_bias, _mutant_truncate,
                                    _mutant_half_up, _mutant_sym127])
def test_pins_reject_rmsnorm_quant_mutants(mutant, rng):
    with pytest.raises(AssertionError):
        pin_rmsnorm_quant_golden(mutant)
        pin_rmsnorm_quant_closed_forms(mutant, rng)


def test_brute_force_rejects_a_dropped_second_quant(monkeypatch):
    # a plausible slip: path 1 multiplying the unquantised RmsNorm (no
    # second RmsNormQuant) -- the brute-force pin must catch it
    real = op.rmsnorm_quant
    calls = []

    def second_unquantised(v, g, b, s, eps):
        calls.append(1)
        if len(calls) == 2:  # the query-latent step
            return oracle.rmsnorm(v, g, eps)
        return real(v, g, b, s, eps)
    monkeypatch.setattr(op, "rmsnorm_quant", second_unquantised)
    with pytest.raises(AssertionError):
        test_preprocess_matches_brute_force("pre_tiny")
