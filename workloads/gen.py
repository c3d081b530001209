"""Seeded input generators.

Every draw uses ``numpy.random.default_rng(cfg.seed)`` (PCG64) in a fixed
order, so the same config always yields bit-identical inputs on any host.

MLA prolog draw order: x, W^DQ, W^DKV_KR, W^UQ_QR, W^UK, gamma_cq, gamma_ckv,
positions, cache_index, kv/kr cache pre-fill, scales.

Distributions (per workload description):

* x ~ N(0, 1); every weight ~ N(0, 1/sqrt(k)) with k its fan-in (He for
  W^DQ and W^DKV_KR, Hcq for W^UQ_QR, D for W^UK);
* gamma ~ U(0.5, 1.5);
* RoPE tables: for i < Dr/2, theta_i = pos * 10000^(-2i/Dr) with pos drawn
  uniformly from [0, 4096); cos = [cos(theta), cos(theta)] and
  sin = [sin(theta), sin(theta)] (halves duplicated), rounded to the storage
  dtype;
* cache_index: distinct slots drawn without replacement from
  [0, BlockNum*BlockSize), with ``n_skip`` tokens (random positions) set to -1;
* caches pre-filled with N(0,1) bf16 or uniform int8 so untouched slots are
  recognisable;
* partial-quant scales: W^UQ_QR int8 uniform on [-127, 127], its per-channel
  dequant scale ~ U(0.001, 0.01), smooth scale ~ U(0.5, 1.5), cache quant
  scales ~ U(0.01, 0.05).

Storage conventions of the returned arrays: bf16 tensors are ``np.uint16``
holding the raw bf16 bit patterns; fp16 tensors are ``np.float16``; int8 are
``np.int8``; fp32 scales ``np.float32``; indexes ``np.int64``.  ``dtypes``
names the logical dtype of each array.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from .configs import MlaConfig, PreConfig, QkvConfig, get_config


def bf16_bits_from_f64(a) -> np.ndarray:
    """Round float64 values to bf16 (nearest, ties to even); return the bits.

    Rounds the float64 significand directly at bf16 precision (7 stored
    bits), so there is no double rounding through float32.  Inputs here are
    finite and far from the bf16 overflow and subnormal ranges.
    """
    a = np.ascontiguousarray(a, dtype=np.float64)
    b = a.view(np.uint64)
    lsb = (b >> np.uint64(45)) & np.uint64(1)
    r = ((b + np.uint64((1 << 44) - 1) + lsb) >> np.uint64(45)) << np.uint64(45)
    f32 = r.view(np.float64).astype(np.float32)  # exact: 8-bit significand
    return (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _store(values: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_bits_from_f64(values)
    if dtype == "fp16":
        return np.asarray(values, dtype=np.float64).astype(np.float16)
    if dtype == "fp32":
        return np.asarray(values, dtype=np.float64).astype(np.float32)
    raise ValueError(dtype)


def _rope_tables(rng, T: int, width: int, dtype: str):
    pos = rng.integers(0, 4096, size=T).astype(np.float64)
    half = width // 2
    inv = 10000.0 ** (-2.0 * np.arange(half, dtype=np.float64) / width)
    theta = pos[:, None] * inv[None, :]
    theta = np.concatenate([theta, theta], axis=1)
    return pos, _store(np.cos(theta), dtype), _store(np.sin(theta), dtype)


def _index(rng, T: int, slots: int, n_skip: int) -> np.ndarray:
    n_valid = T - n_skip
    if n_valid > slots:
        raise ValueError("more valid tokens than cache slots")
    idx = np.full(T, -1, dtype=np.int64)
    valid_pos = np.sort(rng.permutation(T)[:n_valid])
    idx[valid_pos] = rng.choice(slots, size=n_valid, replace=False)
    return idx


@dataclass
class Workload:
    cfg: object
    arrays: dict = field(default_factory=dict)
    dtypes: dict = field(default_factory=dict)
    extra: dict = field(default_factory=dict)

    def __getitem__(self, k):
        return self.arrays[k]


def make_mla_workload(cfg: MlaConfig) -> Workload:
    rng = np.random.default_rng(cfg.seed)
    T, He, Hcq, N, D, Hckv, Dr = (cfg.T, cfg.He, cfg.Hcq, cfg.N, cfg.D,
                                  cfg.Hckv, cfg.Dr)
    quant = cfg.quant_mode
    w = Workload(cfg)
    A, Ty = w.arrays, w.dtypes

    def put(name, arr, dt):
        A[name] = arr
        Ty[name] = dt

    full = quant.startswith("full")
    if full:
        # int8 x and down-projection weights, uniform on [-127, 127]; their
        # dequant scales (drawn last) bring them to the bf16 workloads'
        # magnitudes
        put("token_x", rng.integers(-127, 128, size=(T, He)).astype(np.int8),
            "int8")
        put("weight_dq",
            rng.integers(-127, 128, size=(He, Hcq)).astype(np.int8), "int8")
        put("weight_dkv_kr",
            rng.integers(-127, 128, size=(He, Hckv + Dr)).astype(np.int8),
            "int8")
    else:
        put("token_x", _store(rng.standard_normal((T, He)), "bf16"), "bf16")
        put("weight_dq",
            _store(rng.standard_normal((He, Hcq)) / np.sqrt(He), "bf16"),
            "bf16")
        put("weight_dkv_kr",
            _store(rng.standard_normal((He, Hckv + Dr)) / np.sqrt(He), "bf16"),
            "bf16")
    if quant == "none":
        put("weight_uq_qr",
            _store(rng.standard_normal((Hcq, N * (D + Dr))) / np.sqrt(Hcq),
                   "bf16"), "bf16")
    else:
        put("weight_uq_qr",
            rng.integers(-127, 128, size=(Hcq, N * (D + Dr))).astype(np.int8),
            "int8")
    put("weight_uk",
        _store(rng.standard_normal((N, D, Hckv)) / np.sqrt(D), "bf16"), "bf16")
    put("rmsnorm_gamma_cq", _store(rng.uniform(0.5, 1.5, Hcq), "bf16"), "bf16")
    put("rmsnorm_gamma_ckv", _store(rng.uniform(0.5, 1.5, Hckv), "bf16"),
        "bf16")
    pos, cos, sin = _rope_tables(rng, T, Dr, "bf16")
    w.extra["positions"] = pos
    put("rope_cos", cos, "bf16")
    put("rope_sin", sin, "bf16")
    put("cache_index", _index(rng, T, cfg.slots, cfg.n_skip), "int64")

    kv_shape = (cfg.block_num, cfg.block_size, cfg.Nkv, Hckv)
    kr_shape = (cfg.block_num, cfg.block_size, cfg.Nkv, Dr)
    if quant == "partial_kv_int8":
        put("kv_cache", rng.integers(-128, 128, size=kv_shape).astype(np.int8),
            "int8")
        put("kr_cache", rng.integers(-128, 128, size=kr_shape).astype(np.int8),
            "int8")
    elif quant == "full_kv_int8":
        # the full-quantisation int8 row keeps kr_cache in bf16
        put("kv_cache", rng.integers(-128, 128, size=kv_shape).astype(np.int8),
            "int8")
        put("kr_cache", _store(rng.standard_normal(kr_shape), "bf16"), "bf16")
    else:
        put("kv_cache", _store(rng.standard_normal(kv_shape), "bf16"), "bf16")
        put("kr_cache", _store(rng.standard_normal(kr_shape), "bf16"), "bf16")

    if quant != "none":
        put("dequant_scale_w_uq_qr",
            _store(rng.uniform(0.001, 0.01, N * (D + Dr)), "fp32"), "fp32")
        put("smooth_scales_cq", _store(rng.uniform(0.5, 1.5, Hcq), "fp32"),
            "fp32")
    if quant in ("partial_kv_int8", "full_kv_int8"):
        put("quant_scale_ckv", _store(rng.uniform(0.01, 0.05, Hckv), "fp32"),
            "fp32")
    if quant == "partial_kv_int8":
        put("quant_scale_ckr", _store(rng.uniform(0.01, 0.05, Dr), "fp32"),
            "fp32")
    if full:
        # per-token x scale ~ U(0.01, 0.02): x8 * s has a standard deviation
        # near 1; per-channel weight scales U(0.5, 1.5) / (73 sqrt(He)): a
        # dequantised weight's standard deviation near 1/sqrt(He) (73 is
        # the standard deviation of the uniform int8 draw)
        put("dequant_scale_x", _store(rng.uniform(0.01, 0.02, T), "fp32"),
            "fp32")
        put("dequant_scale_w_dq",
            _store(rng.uniform(0.5, 1.5, Hcq) / (73.0 * np.sqrt(He)), "fp32"),
            "fp32")
        put("dequant_scale_w_dkv_kr",
            _store(rng.uniform(0.5, 1.5, Hckv + Dr) / (73.0 * np.sqrt(He)),
                   "fp32"), "fp32")
    return w


def make_qkv_workload(cfg: QkvConfig) -> Workload:
    rng = np.random.default_rng(cfg.seed)
    T, Nq, Nk, Nv, D = cfg.T, cfg.Nq, cfg.Nk, cfg.Nv, cfg.D
    w = Workload(cfg)
    A, Ty = w.arrays, w.dtypes

    def put(name, arr, dt):
        A[name] = arr
        Ty[name] = dt

    put("qkv", _store(rng.standard_normal((T, Nq + Nk + Nv, D)), "fp16"),
        "fp16")
    put("gamma_q", _store(rng.uniform(0.5, 1.5, D), "fp16"), "fp16")
    put("gamma_k", _store(rng.uniform(0.5, 1.5, D), "fp16"), "fp16")
    pos, cos, sin = _rope_tables(rng, T, D, "fp16")
    w.extra["positions"] = pos
    put("cos", cos, "fp16")
    put("sin", sin, "fp16")
    n_skip = int(round(cfg.skip_frac * T))
    put("index", _index(rng, T, cfg.slots, n_skip), "int64")
    k_shape = (cfg.block_num, cfg.block_size, Nk, D)
    v_shape = (cfg.block_num, cfg.block_size, Nv, D)
    if cfg.quant_mode == "none":
        put("k_cache", _store(rng.standard_normal(k_shape), "fp16"), "fp16")
        put("v_cache", _store(rng.standard_normal(v_shape), "fp16"), "fp16")
    else:
        put("k_cache", rng.integers(-128, 128, size=k_shape).astype(np.int8),
            "int8")
        put("v_cache", rng.integers(-128, 128, size=v_shape).astype(np.int8),
            "int8")
        put("k_scale", _store(rng.uniform(0.01, 0.05, Nk * D), "fp32"), "fp32")
        put("v_scale", _store(rng.uniform(0.01, 0.05, Nv * D), "fp32"), "fp32")
        if cfg.quant_mode == "asymmetric":
            put("k_offset", _store(rng.uniform(-8.0, 8.0, Nk * D), "fp32"),
                "fp32")
            put("v_offset", _store(rng.uniform(-8.0, 8.0, Nv * D), "fp32"),
                "fp32")
    return w


def make_preprocess_workload(cfg: PreConfig) -> Workload:
    """MlaPreprocessV2 inputs.  Draw order: x, W^DQKV, W^UQ_QR, W^UK, the
    three gammas, the two biases, the two quant scales, the two dequant
    scales, positions, index, cache pre-fill.

    x ~ N(0, 1) bf16; int8 weights uniform on [-127, 127]; gammas
    U(0.5, 1.5) bf16; biases U(-0.1, 0.1) fp32; each quant scale one fp32
    value U(20, 30), so the normalised rows (|v| up to ~5) span most of the
    int8 range and saturate only in the far tails; per-channel dequant
    scales U(0.5, 1.5) / (quant scale * 73 * sqrt(K)) (73 is the standard
    deviation of the uniform int8 draw), which brings the dequantised
    products to unit size; W^UK ~ N(0, 1/sqrt(D)) bf16; caches pre-filled
    N(0, 1) bf16.
    """
    rng = np.random.default_rng(cfg.seed)
    T, He, Hcq, N, D, Hckv, Dr = (cfg.T, cfg.He, cfg.Hcq, cfg.N, cfg.D,
                                  cfg.Hckv, cfg.Dr)
    w = Workload(cfg)
    A, Ty = w.arrays, w.dtypes

    def put(name, arr, dt):
        A[name] = arr
        Ty[name] = dt

    ntot = Hcq + Hckv + Dr
    put("token_x", _store(rng.standard_normal((T, He)), "bf16"), "bf16")
    put("weight_dqkv", rng.integers(-127, 128, size=(He, ntot)).astype(np.int8),
        "int8")
    put("weight_uq_qr",
        rng.integers(-127, 128, size=(Hcq, N * (D + Dr))).astype(np.int8),
        "int8")
    put("weight_uk",
        _store(rng.standard_normal((N, D, Hckv)) / np.sqrt(D), "bf16"), "bf16")
    put("gamma_x", _store(rng.uniform(0.5, 1.5, He), "bf16"), "bf16")
    put("gamma_cq", _store(rng.uniform(0.5, 1.5, Hcq), "bf16"), "bf16")
    put("gamma_ckv", _store(rng.uniform(0.5, 1.5, Hckv), "bf16"), "bf16")
    put("bias_x", _store(rng.uniform(-0.1, 0.1, He), "fp32"), "fp32")
    put("bias_cq", _store(rng.uniform(-0.1, 0.1, Hcq), "fp32"), "fp32")
    qsx = _store(rng.uniform(20.0, 30.0, 1), "fp32")
    qsc = _store(rng.uniform(20.0, 30.0, 1), "fp32")
    put("quant_scale_x", qsx, "fp32")
    put("quant_scale_cq", qsc, "fp32")
    put("dequant_scale_dqkv",
        _store(rng.uniform(0.5, 1.5, ntot)
               / (float(qsx[0]) * 73.0 * np.sqrt(He)), "fp32"), "fp32")
    put("dequant_scale_uq_qr",
        _store(rng.uniform(0.5, 1.5, N * (D + Dr))
               / (float(qsc[0]) * 73.0 * np.sqrt(Hcq)), "fp32"), "fp32")
    pos, cos, sin = _rope_tables(rng, T, Dr, "bf16")
    w.extra["positions"] = pos
    put("rope_cos", cos, "bf16")
    put("rope_sin", sin, "bf16")
    put("cache_index", _index(rng, T, cfg.slots, cfg.n_skip), "int64")
    put("kv_cache", _store(rng.standard_normal(
        (cfg.block_num, cfg.block_size, 1, Hckv)), "bf16"), "bf16")
    put("kr_cache", _store(rng.standard_normal(
        (cfg.block_num, cfg.block_size, 1, Dr)), "bf16"), "bf16")
    return w


def make_workload(key) -> Workload:
    cfg = key if isinstance(key, (MlaConfig, QkvConfig, PreConfig)) \
        else get_config(key)
    if isinstance(cfg, MlaConfig):
        return make_mla_workload(cfg)
    if isinstance(cfg, PreConfig):
        return make_preprocess_workload(cfg)
    return make_qkv_workload(cfg)


def sub_workload(w: Workload, tokens) -> Workload:
    """The same MLA workload restricted to some tokens (in the given
    order).  Tokens are independent: each output row depends only on its
    own x, RoPE row and index, so the restriction is a valid workload of
    len(tokens) tokens with the same weights and caches."""
    import copy
    tokens = np.asarray(tokens)
    s = copy.copy(w)
    s.arrays = dict(w.arrays)
    for k in ("token_x", "rope_cos", "rope_sin", "cache_index"):
        s.arrays[k] = w.arrays[k].reshape(w.cfg.T, -1)[tokens].reshape(
            (len(tokens),) + w.arrays[k].shape[1:])
    s.cfg = w.cfg.replace(B=len(tokens), S=1)
    return s
