"""Pins for the float64 oracle, independent of the oracle's own formulas.

Each pin ties a step to something other than its own code: a hand-derived
worked example (tests/golden/worked_examples.txt), a closed form, a library
routine for a special case, an invariant, or brute-force loops on tiny
inputs.  The last group plants plausible mistakes into copies of the oracle's
steps and checks that some pin rejects each one.
"""

from __future__ import annotations

import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import common as oc
from tests import brute_force as bf
from workloads import make_workload, get_config
from workloads.gen import bf16_bits_from_f64

GOLDEN = os.path.join(os.path.dirname(__file__), "golden",
                      "worked_examples.txt")

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")


def _vec(s):
    return np.array([float(v) for v in s.split(",")], dtype=np.float64)


def _golden(op):
    cases = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = [p.strip() for p in line.split("|")]
            if parts[0] == op:
                cases.append(parts[1:])
    assert cases, op
    return cases


def _kv(spec):
    out = {}
    for item in spec.split(";"):
        k, v = item.strip().split("=")
        out[k.strip()] = _vec(v)
    return out


# ---------------------------------------------------------------- pins ----
# Each pin takes the implementation under test so that the mutation tests at
# the bottom can feed it deliberately broken variants.

def pin_decode_golden(decode):
    for bits, val in _golden("bf16"):
        got = decode(np.array([int(bits, 16)], dtype=np.uint16), "bf16")[0]
        want = float(val)
        assert got == want and math.copysign(1, got) == math.copysign(1, want)


def pin_rmsnorm_golden(rmsnorm):
    for spec, want in _golden("rmsnorm"):
        a = _kv(spec)
        got = rmsnorm(a["x"], a["gamma"], float(a["eps"][0]))
        np.testing.assert_allclose(got, _vec(want), rtol=1e-15, atol=0)


def pin_rmsnorm_library(rmsnorm, rng):
    # torch.nn.functional.rms_norm is the textbook RMSNorm
    # (x / sqrt(mean(x^2) + eps) * weight); in float64 on the CPU it is an
    # independent implementation of the same definition.
    x = rng.standard_normal((7, 96)) * 3.0
    g = rng.uniform(0.5, 1.5, 96)
    for eps in (1e-6, 1e-5, 0.7):
        ref = torch.nn.functional.rms_norm(
            torch.from_numpy(x), (96,), torch.from_numpy(g), eps).numpy()
        np.testing.assert_allclose(rmsnorm(x, g, eps), ref, rtol=1e-13,
                                   atol=1e-15)


def pin_rmsnorm_invariants(rmsnorm, rng):
    x = rng.standard_normal((5, 64))
    ones = np.ones(64)
    eps = 1e-3
    y = rmsnorm(x, ones, eps)
    ms = np.mean(x * x, axis=1)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=1)),
                               np.sqrt(ms / (ms + eps)), rtol=1e-13)
    # scale invariance with eps = 0
    np.testing.assert_allclose(rmsnorm(37.5 * x, ones, 0.0),
                               rmsnorm(x, ones, 0.0), rtol=1e-13)
    # a constant row c maps to gamma * sign(c) when eps = 0
    g = rng.uniform(0.5, 1.5, 64)
    np.testing.assert_allclose(rmsnorm(np.full((1, 64), -4.0), g, 0.0)[0],
                               -g, rtol=1e-15)


def pin_rope_golden(rope):
    for spec, want in _golden("rope"):
        a = _kv(spec)
        got = rope(a["y"], a["cos"], a["sin"])
        np.testing.assert_allclose(got, _vec(want), rtol=0, atol=2e-16)


def pin_rope_complex(rope, rng):
    # With duplicated half angles, half-and-half RoPE is the complex product
    # (y_i + j*y_{i+h}) * exp(j*theta_i) for each i < h.
    d, h = 64, 32
    y = rng.standard_normal((9, d))
    th = rng.uniform(-7, 7, (9, h))
    cos = np.concatenate([np.cos(th), np.cos(th)], axis=1)
    sin = np.concatenate([np.sin(th), np.sin(th)], axis=1)
    z = (y[:, :h] + 1j * y[:, h:]) * np.exp(1j * th)
    want = np.concatenate([z.real, z.imag], axis=1)
    np.testing.assert_allclose(rope(y, cos, sin), want, rtol=0, atol=1e-13)


def pin_rope_invariants(rope, rng):
    d, h = 16, 8
    y = rng.standard_normal((4, d))
    np.testing.assert_array_equal(rope(y, np.ones(d), np.zeros(d)), y)
    t1, t2 = rng.uniform(-3, 3, h), rng.uniform(-3, 3, h)

    def tab(t):
        return (np.concatenate([np.cos(t), np.cos(t)]),
                np.concatenate([np.sin(t), np.sin(t)]))

    c1, s1 = tab(t1)
    c2, s2 = tab(t2)
    c12, s12 = tab(t1 + t2)
    np.testing.assert_allclose(rope(rope(y, c1, s1), c2, s2),
                               rope(y, c12, s12), atol=1e-14)
    out = rope(y, c1, s1)
    np.testing.assert_allclose(out[:, :h] ** 2 + out[:, h:] ** 2,
                               y[:, :h] ** 2 + y[:, h:] ** 2, rtol=1e-13)


def pin_quant_golden(quant):
    for spec, want in _golden("quant"):
        a = _kv(spec)
        got = quant(a["v"], a["scale"][0], a.get("offset"))
        np.testing.assert_array_equal(got, _vec(want).astype(np.int64))


def pin_quant_exact_multiples(quant, rng):
    scale = rng.uniform(0.01, 0.05, 128)
    codes = rng.integers(-128, 128, (20, 128))
    np.testing.assert_array_equal(quant(codes * scale, scale), codes)
    big = np.where(rng.random((20, 128)) < 0.5, -1.0, 1.0) * \
        rng.uniform(128.6, 900.0, (20, 128))
    got = quant(big * scale, scale)
    np.testing.assert_array_equal(got, np.where(big > 0, 127, -128))


def pin_dynamic_quant(dq, rng):
    cq = rng.standard_normal((6, 200))
    smooth = rng.uniform(0.5, 1.5, 200)
    c8, s = dq(cq, smooth)
    u = cq * smooth
    j = np.argmax(np.abs(u), axis=1)
    np.testing.assert_array_equal(np.abs(c8[np.arange(6), j]), 127)
    np.testing.assert_allclose(s, np.max(np.abs(u), axis=1) / 127, rtol=1e-15)
    # every code reconstructs within half a step
    assert np.all(np.abs(c8 * s[:, None] - u) <= 0.5 * s[:, None] * (1 + 1e-12))
    assert c8.min() >= -127 and c8.max() <= 127
    # rows built as exact multiples of a step give exact codes
    codes = rng.integers(-126, 127, (3, 50))
    codes[:, 7] = 127
    step = 0.03125
    c8b, sb = dq(codes * step, np.ones(50))
    np.testing.assert_array_equal(c8b, codes)
    np.testing.assert_allclose(sb, step, rtol=1e-15)
    z8, zs = dq(np.zeros((1, 50)), np.ones(50))
    assert zs[0] == 0 and not z8.any()


# ------------------------------------------------------- the pin tests ----

def test_decode_golden():
    pin_decode_golden(oc.decode)


def test_decode_fp16_and_ints():
    h = np.array([1.5, -0.000061035156, 65504.0], dtype=np.float16)
    np.testing.assert_array_equal(oc.decode(h, "fp16"),
                                  [1.5, -2.0 ** -14, 65504.0])
    assert oc.decode(np.array([-128, 127], np.int8), "int8").tolist() == \
        [-128, 127]


def test_generator_bf16_rounding_is_rne():
    # ties go to the even neighbour; halfway points between bf16 values at 1.0
    # are 1 + k*2^-8 for odd k.
    vals = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -30,
                     -(1 + 2 ** -8), 3.14159265358979])
    bits = bf16_bits_from_f64(vals)
    assert bits.tolist() == [0x3F80, 0x3F82, 0x3F81, 0xBF80, 0x4049]
    # agreement with torch's own fp32 -> bf16 rounding where fp32 is exact
    r = np.random.default_rng(3).standard_normal(4096).astype(np.float32)
    tb = torch.from_numpy(r).to(torch.bfloat16).view(torch.int16).numpy()
    np.testing.assert_array_equal(bf16_bits_from_f64(r.astype(np.float64)),
                                  tb.view(np.uint16))


def test_rmsnorm_golden():
    pin_rmsnorm_golden(oc.rmsnorm)


def test_rmsnorm_matches_library(rng):
    pin_rmsnorm_library(oc.rmsnorm, rng)


def test_rmsnorm_invariants(rng):
    pin_rmsnorm_invariants(oc.rmsnorm, rng)


def test_rope_golden():
    pin_rope_golden(oc.rope_half)


def test_rope_is_complex_rotation(rng):
    pin_rope_complex(oc.rope_half, rng)


def test_rope_invariants(rng):
    pin_rope_invariants(oc.rope_half, rng)


def test_quant_golden():
    pin_quant_golden(oc.quant_int8)


def test_quant_exact_multiples_and_saturation(rng):
    pin_quant_exact_multiples(oc.quant_int8, rng)


def test_dynamic_quant(rng):
    pin_dynamic_quant(oc.dynamic_quant_int8, rng)


def test_int_matmul_exact(rng):
    a = rng.integers(-127, 128, (3, 300))
    b = rng.integers(-127, 128, (300, 5))
    got = oc.int_matmul_exact(a, b)
    for i in range(3):
        for j in range(5):
            assert got[i, j] == sum(int(a[i, k]) * int(b[k, j])
                                    for k in range(300))


def test_scatter_touches_only_indexed_slots(rng):
    cache = rng.standard_normal((3, 4, 2, 5))
    rows = rng.standard_normal((6, 2, 5))
    idx = np.array([5, -1, 0, 11, -1, 7])
    out = oc.scatter_slots(cache, idx, rows)
    flat_in = cache.reshape(12, 2, 5)
    flat_out = out.reshape(12, 2, 5)
    for s in range(12):
        hits = [t for t in range(6) if idx[t] == s]
        if hits:
            np.testing.assert_array_equal(flat_out[s], rows[hits[0]])
        else:
            np.testing.assert_array_equal(flat_out[s], flat_in[s])
    np.testing.assert_array_equal(cache.reshape(12, 2, 5), flat_in)  # no alias


def test_scatter_rejects_bad_index(rng):
    cache = np.zeros((2, 4, 1, 3))
    rows = np.ones((3, 1, 3))
    with pytest.raises(ValueError):
        oc.scatter_slots(cache, np.array([1, 1, -1]), rows)
    with pytest.raises(ValueError):
        oc.scatter_slots(cache, np.array([8, 0, -1]), rows)
    with pytest.raises(ValueError):
        oc.scatter_slots(cache, np.array([-2, 0, 1]), rows)
    # repeated -1 is fine, and zero slots means nothing is written
    oc.scatter_slots(cache, np.array([-1, -1, 3]), rows)
    empty = np.zeros((0, 4, 1, 3))
    assert oc.scatter_slots(empty, np.array([5, 6, 7]), rows).shape == \
        empty.shape


# ------------------------------------------- whole-op pins: MLA prolog ----

def _dims(cfg):
    return dict(He=cfg.He, Hcq=cfg.Hcq, N=cfg.N, D=cfg.D, Hckv=cfg.Hckv,
                Dr=cfg.Dr)


def _run_mla(w, **kw):
    cfg = w.cfg
    return oracle.mla_prolog_v2(w.arrays, w.dtypes, _dims(cfg),
                                kw.get("quant_mode", cfg.quant_mode),
                                cfg.eps_cq, cfg.eps_ckv)


def _dec(w, name):
    return oc.decode(w.arrays[name], w.dtypes[name])


@pytest.mark.parametrize("key", [0, "mla_ragged_qb"])
def test_mla_matches_brute_force(key):
    w = make_workload(key)
    cfg = w.cfg
    if cfg.T > 8:  # keep the Python loops short
        cfg = cfg.replace(B=6, S=1, n_skip=1)
        w = make_workload(cfg)
    d = _dims(cfg)
    ref = _run_mla(w)
    quant = None
    if cfg.quant_mode != "none":
        quant = dict(smooth=_dec(w, "smooth_scales_cq").tolist(),
                     dq=_dec(w, "dequant_scale_w_uq_qr").tolist())
    bres = bf.mla_prolog_brute(
        _dec(w, "token_x").tolist(), _dec(w, "weight_dq").tolist(),
        _dec(w, "weight_dkv_kr").tolist(), _dec(w, "weight_uq_qr").tolist(),
        _dec(w, "weight_uk").tolist(), _dec(w, "rmsnorm_gamma_cq").tolist(),
        _dec(w, "rmsnorm_gamma_ckv").tolist(), _dec(w, "rope_cos").tolist(),
        _dec(w, "rope_sin").tolist(), d, cfg.eps_cq, cfg.eps_ckv, quant)
    np.testing.assert_allclose(ref["query"], np.array(bres["query"]),
                               rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(ref["query_rope"],
                               np.array(bres["query_rope"]),
                               rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(ref["kv_rows"], np.array(bres["kv_row"]),
                               rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(ref["kr_rows"], np.array(bres["kr_row"]),
                               rtol=1e-12, atol=1e-13)
    if quant is not None:
        np.testing.assert_array_equal(ref["cq_int8"], np.array(bres["c8"]))


def test_mla_quant_matches_brute_force_with_int8_caches():
    cfg = get_config("mla_ragged_q").replace(B=4, He=128, Hcq=64, N=2,
                                            D=32, Hckv=64, Dr=16, n_skip=1)
    w = make_workload(cfg)
    ref = _run_mla(w)
    quant = dict(smooth=_dec(w, "smooth_scales_cq").tolist(),
                 dq=_dec(w, "dequant_scale_w_uq_qr").tolist(),
                 qs_ckv=_dec(w, "quant_scale_ckv").tolist(),
                 qs_ckr=_dec(w, "quant_scale_ckr").tolist())
    bres = bf.mla_prolog_brute(
        _dec(w, "token_x").tolist(), _dec(w, "weight_dq").tolist(),
        _dec(w, "weight_dkv_kr").tolist(), _dec(w, "weight_uq_qr").tolist(),
        _dec(w, "weight_uk").tolist(), _dec(w, "rmsnorm_gamma_cq").tolist(),
        _dec(w, "rmsnorm_gamma_ckv").tolist(), _dec(w, "rope_cos").tolist(),
        _dec(w, "rope_sin").tolist(), _dims(cfg), cfg.eps_cq, cfg.eps_ckv,
        quant)
    np.testing.assert_array_equal(ref["cq_int8"], np.array(bres["c8"]))
    np.testing.assert_allclose(ref["query"], np.array(bres["query"]),
                               rtol=1e-11, atol=1e-11)
    np.testing.assert_array_equal(ref["kv_rows"], np.array(bres["kv_row"]))
    np.testing.assert_array_equal(ref["kr_rows"], np.array(bres["kr_row"]))


@pytest.mark.parametrize("mode", ["full_kv_bf16", "full_kv_int8"])
def test_mla_full_quant_matches_brute_force_on_dequantised_inputs(mode):
    """Full quantisation against the brute-force loops fed the dequantised
    int8 inputs: x8[t, k] * dequant_scale_x[t] and w8[k, j] *
    dequant_scale_w[j] (exact in float64: 8-bit times 24-bit mantissas).
    Equality pins where each scale multiplies (per token, per channel, which
    weight's scale), the rest of the partial-quant path, the int8 kv_cache
    with a bf16 kr_cache, and the per-(token, head) int8 query."""
    cfg = get_config("mla_full_kvbf16").replace(
        B=3, He=128, Hcq=64, N=2, D=32, Hckv=64, Dr=16, n_skip=1,
        quant_mode=mode)
    w = make_workload(cfg)
    ref = _run_mla(w)
    x8, sx = _dec(w, "token_x"), _dec(w, "dequant_scale_x")
    wdq8, swdq = _dec(w, "weight_dq"), _dec(w, "dequant_scale_w_dq")
    wkv8, swkv = _dec(w, "weight_dkv_kr"), _dec(w, "dequant_scale_w_dkv_kr")
    x = [[float(x8[t, k]) * float(sx[t]) for k in range(cfg.He)]
         for t in range(cfg.T)]
    wdq = [[float(wdq8[k, j]) * float(swdq[j]) for j in range(cfg.Hcq)]
           for k in range(cfg.He)]
    wkv = [[float(wkv8[k, j]) * float(swkv[j])
            for j in range(cfg.Hckv + cfg.Dr)] for k in range(cfg.He)]
    quant = dict(smooth=_dec(w, "smooth_scales_cq").tolist(),
                 dq=_dec(w, "dequant_scale_w_uq_qr").tolist())
    if mode == "full_kv_int8":
        quant.update(qs_ckv=_dec(w, "quant_scale_ckv").tolist(),
                     query_int8=True)
    bres = bf.mla_prolog_brute(
        x, wdq, wkv, _dec(w, "weight_uq_qr").tolist(),
        _dec(w, "weight_uk").tolist(), _dec(w, "rmsnorm_gamma_cq").tolist(),
        _dec(w, "rmsnorm_gamma_ckv").tolist(), _dec(w, "rope_cos").tolist(),
        _dec(w, "rope_sin").tolist(), _dims(cfg), cfg.eps_cq, cfg.eps_ckv,
        quant)
    np.testing.assert_array_equal(ref["cq_int8"], np.array(bres["c8"]))
    np.testing.assert_allclose(ref["query_rope"], np.array(bres["query_rope"]),
                               rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(ref["kr_rows"], np.array(bres["kr_row"]),
                               rtol=1e-12, atol=1e-12)
    if mode == "full_kv_bf16":
        np.testing.assert_allclose(ref["query"], np.array(bres["query"]),
                                   rtol=1e-11, atol=1e-11)
        np.testing.assert_allclose(ref["kv_rows"], np.array(bres["kv_row"]),
                                   rtol=1e-12, atol=1e-12)
        assert "dequant_scale_q_nope" not in ref
    else:
        np.testing.assert_array_equal(ref["query"], np.array(bres["query"]))
        np.testing.assert_allclose(ref["dequant_scale_q_nope"],
                                   np.array(bres["q_scale"]), rtol=1e-12)
        np.testing.assert_array_equal(ref["kv_rows"], np.array(bres["kv_row"]))
        assert ref["query"].dtype == np.int64


def test_query_quant_per_head_worked_example():
    """Per-(token, head) int8 query, by hand: the row (0.5, -1.0, 0.25, 0)
    has max |q| = 1, scale 1/127; 0.5 * 127 = 63.5 rounds half to even to
    64, 0.25 * 127 = 31.75 to 32; a zero row gets scale 0 and zero codes;
    the largest magnitude always maps to +/-127."""
    q = np.zeros((1, 2, 4))
    q[0, 0] = [0.5, -1.0, 0.25, 0.0]
    codes, scale = oracle.mla_prolog_v2_quant_query(q)
    np.testing.assert_array_equal(codes[0, 0], [64, -127, 32, 0])
    np.testing.assert_array_equal(codes[0, 1], [0, 0, 0, 0])
    assert scale[0, 0] == 1.0 / 127.0 and scale[0, 1] == 0.0
    r = np.random.default_rng(7).standard_normal((3, 4, 64))
    c, s = oracle.mla_prolog_v2_quant_query(r)
    assert np.all(np.abs(c).max(axis=-1) == 127)
    assert np.all(np.abs(c * s[..., None] - r) <= s[..., None] / 2 + 1e-15)


def test_mla_associativity():
    # c^Q . (W^UQ_n . W^UK_n) equals the staged (c^Q . W^UQ_n) . W^UK_n
    w = make_workload("mla_ragged")
    cfg = w.cfg
    ref = _run_mla(w)
    Wuq = _dec(w, "weight_uq_qr").reshape(cfg.Hcq, -1)[:, :cfg.N * cfg.D]
    Wuk = _dec(w, "weight_uk").reshape(cfg.N, cfg.D, cfg.Hckv)
    for n in range(cfg.N):
        fused = Wuq[:, n * cfg.D:(n + 1) * cfg.D] @ Wuk[n]
        np.testing.assert_allclose(ref["cq"] @ fused, ref["query"][:, n],
                                   rtol=1e-10, atol=1e-10)


def test_mla_column_blocks_of_fused_weights():
    # Reading: weight_uq_qr = [W^UQ (N*D cols) | W^QR (N*Dr cols)] and
    # weight_dkv_kr = [W^DKV (Hckv) | W^KR (Dr)].  Zeroing one block must zero
    # exactly the outputs that block feeds.
    w = make_workload(0)
    cfg = w.cfg
    base = _run_mla(w)
    zero = bf16_bits_from_f64(np.zeros(1))[0]
    w1 = make_workload(0)
    w1.arrays["weight_uq_qr"] = w1.arrays["weight_uq_qr"].copy()
    w1.arrays["weight_uq_qr"][:, cfg.N * cfg.D:] = zero
    r1 = _run_mla(w1)
    assert not r1["query_rope"].any()
    np.testing.assert_array_equal(r1["query"], base["query"])
    w2 = make_workload(0)
    w2.arrays["weight_uq_qr"] = w2.arrays["weight_uq_qr"].copy()
    w2.arrays["weight_uq_qr"][:, :cfg.N * cfg.D] = zero
    r2 = _run_mla(w2)
    assert not r2["query"].any()
    np.testing.assert_array_equal(r2["query_rope"], base["query_rope"])
    w3 = make_workload(0)
    w3.arrays["weight_dkv_kr"] = w3.arrays["weight_dkv_kr"].copy()
    w3.arrays["weight_dkv_kr"][:, cfg.Hckv:] = zero
    r3 = _run_mla(w3)
    assert not r3["kr_rows"].any()
    np.testing.assert_array_equal(r3["kv_rows"], base["kv_rows"])


def test_mla_identity_weights_closed_form():
    # W^DQ = I (He == Hcq), gamma = 1, eps = 0, W^UQ_n = I, W^UK_n = [I | 0],
    # cos = 1, sin = 0: query[t, n, :D] = x_t / rms(x_t), rest 0, and
    # query_rope = c^Q . W^QR exactly.
    rng = np.random.default_rng(7)
    T, H, N, D, Hckv, Dr = 3, 16, 2, 8, 12, 4
    x = rng.standard_normal((T, H))
    one = np.eye(H)
    wuq = np.zeros((H, N * (D + Dr)))
    for n in range(N):
        wuq[n * D:(n + 1) * D, n * D:(n + 1) * D] = np.eye(D)
    wqr = rng.standard_normal((H, N * Dr))
    wuq[:, N * D:] = wqr
    wuk = np.zeros((N, D, Hckv))
    for n in range(N):
        wuk[n, :, :D] = np.eye(D)
    arrays = dict(token_x=x, weight_dq=one,
                  weight_dkv_kr=rng.standard_normal((H, Hckv + Dr)),
                  weight_uq_qr=wuq, weight_uk=wuk,
                  rmsnorm_gamma_cq=np.ones(H), rmsnorm_gamma_ckv=np.ones(Hckv),
                  rope_cos=np.ones((T, Dr)), rope_sin=np.zeros((T, Dr)),
                  cache_index=np.array([0, -1, 2]),
                  kv_cache=np.zeros((1, 4, 1, Hckv)),
                  kr_cache=np.zeros((1, 4, 1, Dr)))
    dtypes = {k: "fp64" for k in arrays}
    dtypes["cache_index"] = "int64"
    dims = dict(He=H, Hcq=H, N=N, D=D, Hckv=Hckv, Dr=Dr)
    r = oracle.mla_prolog_v2(arrays, dtypes, dims, "none", 0.0, 0.0)
    cq = x / np.sqrt(np.mean(x * x, axis=1, keepdims=True))
    for n in range(N):
        np.testing.assert_allclose(r["query"][:, n, :D],
                                   cq[:, n * D:(n + 1) * D], rtol=1e-14)
        assert not r["query"][:, n, D:].any()
        np.testing.assert_allclose(r["query_rope"][:, n],
                                   cq @ wqr[:, n * Dr:(n + 1) * Dr],
                                   rtol=1e-13)
    np.testing.assert_allclose(r["kr_rows"],
                               x @ arrays["weight_dkv_kr"][:, Hckv:],
                               rtol=1e-13)
    np.testing.assert_array_equal(r["kv_cache"][0, 1], 0)
    np.testing.assert_array_equal(r["kv_cache"][0, 3], 0)
    np.testing.assert_allclose(r["kv_cache"][0, 2, 0], r["kv_rows"][2])


def test_mla_partial_quant_within_quantisation_bound():
    # The int8 path is the bf16 product up to c^Q's rounding error: each code
    # is within half a step s of c^Q * smooth, so with smooth = 1 and dq = 1
    # |y_q - c^Q . W8| <= (s/2) * sum_k |W8[k, j]| for every output column.
    w = make_workload("mla_ragged_q")
    cfg = w.cfg
    w.arrays["smooth_scales_cq"] = np.ones(cfg.Hcq, np.float32)
    w.arrays["dequant_scale_w_uq_qr"] = np.ones(cfg.n_uqqr, np.float32)
    r = _run_mla(w)
    W8 = _dec(w, "weight_uq_qr").astype(np.float64)
    exact = r["cq"] @ W8
    Wuk = _dec(w, "weight_uk")
    T, N, D, Dr = cfg.T, cfg.N, cfg.D, cfg.Dr
    bound_y = 0.5 * r["cq_scale"][:, None] * np.abs(W8).sum(0)[None, :] \
        * (1 + 1e-9)
    qc_exact = exact[:, :N * D].reshape(T, N, D)
    q_exact = np.matmul(qc_exact.transpose(1, 0, 2), Wuk).transpose(1, 0, 2)
    # the error propagates through W^UK: |dq^N| <= sum_d |dq^C_d| |W^UK[d]|
    err_qc = bound_y[:, :N * D].reshape(T, N, D)
    bound_q = np.matmul(err_qc.transpose(1, 0, 2), np.abs(Wuk)).transpose(
        1, 0, 2)
    assert np.all(np.abs(r["query"] - q_exact) <= bound_q + 1e-12)
    assert np.abs(r["query"] - q_exact).max() > 0  # the bound is not vacuous


def test_mla_empty_and_zero_slot_cases():
    w = make_workload(0)
    cfg = w.cfg
    # T = 0: empty queries, caches unchanged
    w0 = make_workload(0)
    for k in ("token_x", "rope_cos", "rope_sin", "cache_index"):
        w0.arrays[k] = w0.arrays[k][:0]
    r0 = _run_mla(w0)
    assert r0["query"].shape == (0, cfg.N, cfg.Hckv)
    assert r0["query_rope"].shape == (0, cfg.N, cfg.Dr)
    np.testing.assert_array_equal(r0["kv_cache"], _dec(w, "kv_cache"))
    # no cache slots: queries as usual, nothing written
    wz = make_workload(0)
    wz.arrays["kv_cache"] = wz.arrays["kv_cache"][:0]
    wz.arrays["kr_cache"] = wz.arrays["kr_cache"][:0]
    rz = _run_mla(wz)
    base = _run_mla(w)
    np.testing.assert_array_equal(rz["query"], base["query"])
    assert rz["kv_cache"].shape[0] == 0


def test_mla_scatter_bit_identical_elsewhere():
    w = make_workload("mla_ragged")
    r = _run_mla(w)
    cfg = w.cfg
    idx = w.arrays["cache_index"]
    before = _dec(w, "kv_cache").reshape(cfg.slots, -1)
    after = r["kv_cache"].reshape(cfg.slots, -1)
    changed = set(np.nonzero((before != after).any(1))[0].tolist())
    assert changed == set(idx[idx >= 0].tolist())
    assert (idx == -1).sum() == cfg.n_skip


# ------------------------------------------- whole-op pins: qkv op -------

def _qkv_dims(cfg):
    return dict(Nq=cfg.Nq, Nk=cfg.Nk, Nv=cfg.Nv, D=cfg.D)


@pytest.mark.parametrize("key", ["qkv_ragged", "qkv_ragged_none",
                                 "qkv_ragged_asym"])
def test_qkv_matches_brute_force(key):
    cfg = get_config(key).replace(B=1, S=5)
    cfg = cfg.replace(block_num=1, block_size=64)
    w = make_workload(cfg)
    ref = oracle.qkv_rmsnorm_rope_cache(w.arrays, w.dtypes, _qkv_dims(cfg),
                                        cfg.quant_mode, cfg.eps)
    Nk, Nv, D = cfg.Nk, cfg.Nv, cfg.D
    scales = None
    if cfg.quant_mode != "none":
        scales = dict(ks=_dec(w, "k_scale").reshape(Nk, D).tolist(),
                      vs=_dec(w, "v_scale").reshape(Nv, D).tolist())
        if cfg.quant_mode == "asymmetric":
            scales["ko"] = _dec(w, "k_offset").reshape(Nk, D).tolist()
            scales["vo"] = _dec(w, "v_offset").reshape(Nv, D).tolist()
    q, k, v = bf.qkv_brute(_dec(w, "qkv").tolist(), _dec(w, "gamma_q").tolist(),
                           _dec(w, "gamma_k").tolist(), _dec(w, "cos").tolist(),
                           _dec(w, "sin").tolist(), _qkv_dims(cfg), cfg.eps,
                           scales)
    np.testing.assert_allclose(ref["q_out"], np.array(q), rtol=1e-12,
                               atol=1e-13)
    if scales is None:
        np.testing.assert_allclose(ref["k_rows"], np.array(k), rtol=1e-12,
                                   atol=1e-13)
        np.testing.assert_array_equal(ref["v_rows"], np.array(v))
    else:
        np.testing.assert_array_equal(ref["k_rows"], np.array(k))
        np.testing.assert_array_equal(ref["v_rows"], np.array(v))


def test_qkv_split_order_and_v_passthrough():
    # Head h of the token carries the constant value h+1: q gets heads
    # [0, Nq), k the next Nk, v the last Nv.  With gamma = 1, cos = 1 and
    # sin = 0, a constant row normalises to 1 (eps = 0) and v passes
    # through untouched.
    Nq, Nk, Nv, D, T = 3, 2, 2, 8, 2
    qkv = np.zeros((T, Nq + Nk + Nv, D))
    for h in range(Nq + Nk + Nv):
        qkv[:, h, :] = h + 1
    arrays = dict(qkv=qkv, gamma_q=np.ones(D), gamma_k=np.full(D, 2.0),
                  cos=np.ones((T, D)), sin=np.zeros((T, D)),
                  index=np.array([1, 0]),
                  k_cache=np.zeros((1, 2, Nk, D)),
                  v_cache=np.zeros((1, 2, Nv, D)))
    dtypes = {k: "fp64" for k in arrays}
    dtypes["index"] = "int64"
    r = oracle.qkv_rmsnorm_rope_cache(arrays, dtypes,
                                      dict(Nq=Nq, Nk=Nk, Nv=Nv, D=D),
                                      "none", 0.0)
    np.testing.assert_array_equal(r["q_out"], np.ones((T, Nq, D)))
    np.testing.assert_array_equal(r["k_cache"][0, 1], np.full((Nk, D), 2.0))
    np.testing.assert_array_equal(r["v_cache"][0, 0, 0], np.full(D, 6.0))
    np.testing.assert_array_equal(r["v_cache"][0, 0, 1], np.full(D, 7.0))


# ------------------------------------------------ planted mistakes --------
# Each mutant is a plausible slip in one oracle step; at least one pin must
# reject it, or the pins would not protect the oracle.

def _rope_wrong_sign(y, cos, sin):
    h = y.shape[-1] // 2
    return y * cos + np.concatenate([y[..., h:], -y[..., :h]], -1) * sin


def _rope_interleaved(y, cos, sin):
    rot = np.empty_like(y)
    rot[..., 0::2] = -y[..., 1::2]
    rot[..., 1::2] = y[..., 0::2]
    return y * cos + rot * sin


def _rms_no_eps(x, g, eps):
    return oc.rmsnorm(x, g, 0.0)


def _rms_eps_outside(x, g, eps):
    x = np.asarray(x, np.float64)
    return x / (np.sqrt(np.mean(x * x, -1, keepdims=True)) + eps) * g


def _rms_sum_not_mean(x, g, eps):
    x = np.asarray(x, np.float64)
    return x / np.sqrt(np.sum(x * x, -1, keepdims=True) + eps) * g


def _quant_multiply(v, s, o=None):
    return oc.quant_int8(np.asarray(v) * np.asarray(s) ** 2, s, o)


def _quant_truncate(v, s, o=None):
    q = np.asarray(v, np.float64) / s + (0 if o is None else o)
    return np.clip(np.trunc(q), -128, 127).astype(np.int64)


def _quant_no_saturation(v, s, o=None):
    q = np.asarray(v, np.float64) / s + (0 if o is None else o)
    return np.rint(q).astype(np.int64)


def _dq_scale_255(cq, smooth):
    c8, s = oc.dynamic_quant_int8(cq, smooth)
    return c8, s * 127 / 255


def _dq_no_smooth(cq, smooth):
    return oc.dynamic_quant_int8(cq, np.ones_like(smooth))


def _decode_wrong_shift(arr, dt):
    if dt == "bf16":
        bits = np.asarray(arr, np.uint16).astype(np.uint32) << np.uint32(15)
        return bits.view(np.float32).astype(np.float64)
    return oc.decode(arr, dt)


def _raises_somewhere(checks):
    failed = 0
    for fn in checks:
        try:
            fn()
        except AssertionError:
            failed += 1
    return failed


@pytest.mark.parametrize("mutant", [_rope_wrong_sign, _rope_interleaved])
def test_pins_reject_rope_mutants(mutant, rng):
    assert _raises_somewhere([
        lambda: pin_rope_golden(mutant),
        lambda: pin_rope_complex(mutant, rng),
        lambda: pin_rope_invariants(mutant, rng)]) >= 1


@pytest.mark.parametrize("mutant", [_rms_no_eps, _rms_eps_outside,
                                    _rms_sum_not_mean])
def test_pins_reject_rmsnorm_mutants(mutant, rng):
    assert _raises_somewhere([
        lambda: pin_rmsnorm_golden(mutant),
        lambda: pin_rmsnorm_library(mutant, rng),
        lambda: pin_rmsnorm_invariants(mutant, rng)]) >= 1


@pytest.mark.parametrize("mutant", [_quant_multiply, _quant_truncate,
                                    _quant_no_saturation])
def test_pins_reject_quant_mutants(mutant, rng):
    assert _raises_somewhere([
        lambda: pin_quant_golden(mutant),
        lambda: pin_quant_exact_multiples(mutant, rng)]) >= 1


@pytest.mark.parametrize("mutant", [_dq_scale_255, _dq_no_smooth])
def test_pins_reject_dynamic_quant_mutants(mutant, rng):
    assert _raises_somewhere([lambda: pin_dynamic_quant(mutant, rng)]) >= 1


def test_pins_reject_decode_mutant():
    assert _raises_somewhere([lambda: pin_decode_golden(
        _decode_wrong_shift)]) >= 1


def test_brute_force_rejects_transposed_uk(monkeypatch):
    # A transposed W^UK (or swapped head split) in the vectorised oracle is
    # caught by the loop version.
    import importlib
    mod = importlib.import_module("oracle.mla_prolog_v2")

    def bad_uk(qc, wuk):
        return np.matmul(qc.transpose(1, 0, 2),
                         wuk[::-1]).transpose(1, 0, 2)  # wrong head order

    monkeypatch.setattr(mod, "_per_head_uk", bad_uk)
    with pytest.raises(AssertionError):
        test_mla_matches_brute_force(0)
