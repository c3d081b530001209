"""CPU tests of the C ABI boundary: the library loads, exports every function
the public header declares, and its host-side validation returns the
documented status codes.  No kernel runs here (there is no GPU): every call
either is a pure validation entry point or fails validation / is empty before
any HIP call.
"""

from __future__ import annotations

import ctypes
import os
import re

import pytest

import qkv_norm_rope_amd as qn
from qkv_norm_rope_amd import _binding as b

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include",
                      "qkvnr.h")

pytestmark = pytest.mark.skipif(not os.path.exists(b.LIB_PATH),
                                reason="libqkvnr.so not built")


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\([^;{]*\)\s*;",
                       src, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_binding_exports():
    assert sorted(b.EXPORTS) == header_functions()


def test_library_exports_every_header_symbol():
    lib = ctypes.CDLL(b.LIB_PATH)
    for name in header_functions():
        assert hasattr(lib, name), name
    assert qn.version() == "0.1.0"
    assert qn.status_string(0) == "ok"
    assert qn.status_string(-4) == "unsupported configuration"
    assert qn.status_string(12345) == "unknown status"
    assert qn.status_string(-11) == "cache index out of range or repeated"
    assert qn.status_string(-12) == "a quant scale is zero"


# ---- host index check (both operators' index restriction) -----------------

@pytest.mark.parametrize("index,slots,code", [
    ([], 0, 0),
    ([-1, -1], 0, 0),                 # -1 skips; no slot needed
    ([0, 5, -1, 3], 6, 0),
    ([5, 0, 5], 6, -11),              # repeated slot
    ([-1, 2, -1, 2], 3, -11),
    ([0, 6], 6, -11),                 # past BlockNum * BlockSize
    ([0, -2], 6, -11),                # below -1
    ([2**62], 6, -11),
    ([0], -1, -2),                    # negative slot count
])
def test_check_cache_index(index, slots, code):
    assert qn.mla_check_cache_index(index, slots) == code


def test_check_cache_index_large_and_null():
    import numpy as np
    rng = np.random.default_rng(5)
    idx = rng.permutation(1 << 20).astype(np.int64)
    idx[rng.integers(0, idx.size, 1000)] = -1
    assert qn.mla_check_cache_index(idx, 1 << 20) == 0
    idx[7] = idx[9] = 1234567 % (1 << 20)
    assert qn.mla_check_cache_index(idx, 1 << 20) == -11
    lib = b.load_library()
    assert lib.mla_check_cache_index(None, 3, 10) == -1
    assert lib.mla_check_cache_index(None, -1, 10) == -2


# ---- fake device pointers: validation never dereferences them -------------
_FAKE = [0x10000000]


def fake(align=256):
    _FAKE[0] += 1 << 20
    return _FAKE[0] - (_FAKE[0] % align)


def mla_args(T=32, quant="none", He=7168, Hcq=1536, N=128, D=128, Hckv=512,
             Dr=64, bn=192, bs=128, layout=b.MLA_WEIGHT_PACKED_K16):
    a = b.MlaPrologV2Args()
    a.struct_size = ctypes.sizeof(b.MlaPrologV2Args)
    a.quant_mode = b.MLA_QUANT[quant]
    a.weight_layout = layout
    a.B, a.S = T, 1
    a.He, a.Hcq, a.N, a.D, a.Hckv, a.Dr, a.Nkv = He, Hcq, N, D, Hckv, Dr, 1
    a.block_num, a.block_size = bn, bs
    a.rmsnorm_epsilon_cq = a.rmsnorm_epsilon_ckv = 1e-5
    for f in ("token_x", "weight_dq", "weight_uq_qr", "weight_uk",
              "weight_dkv_kr", "rmsnorm_gamma_cq", "rmsnorm_gamma_ckv",
              "rope_sin", "rope_cos", "cache_index", "kv_cache", "kr_cache",
              "query", "query_rope"):
        setattr(a, f, fake())
    if quant != "none":
        a.dequant_scale_w_uq_qr = fake()
        a.smooth_scales_cq = fake()
    if quant == "partial_kv_int8":
        a.quant_scale_ckv = fake()
        a.quant_scale_ckr = fake()
    if quant.startswith("full"):
        a.dequant_scale_x = fake()
        a.dequant_scale_w_dq = fake()
        a.dequant_scale_w_dkv_kr = fake()
    if quant == "full_kv_int8":
        a.quant_scale_ckv = fake()
        a.dequant_scale_q_nope = fake()
    return a


def mla_validate(a):
    return b.load_library().mla_prolog_v2_validate(ctypes.byref(a))


def test_mla_valid_args_pass():
    for q in ("none", "partial_kv_bf16", "partial_kv_int8", "full_kv_bf16",
              "full_kv_int8"):
        assert mla_validate(mla_args(quant=q)) == 0
    assert mla_validate(mla_args(T=4, He=256, Hcq=128, N=4, D=32, Hckv=64,
                                 Dr=16, bn=4, bs=16)) == 0


def test_mla_kernels_mask():
    # every plan launches the four main kernels once when there are tokens,
    # except bf16 decode with one 32-row block (T <= 32), whose up
    # projection launch also runs the W^UK product, and above T = 128 with
    # D = 128 (except FULL_KV_INT8), whose fused launch also runs q^R
    merged = ("down", "norm", "uqqr")
    fused = ("down", "norm", "uk")
    for T in (1, 32, 33, 64, 128, 129, 4096):
        for q in ("none", "partial_kv_int8", "full_kv_int8"):
            want = merged if (q == "none" and T <= 32) else (
                fused if (T > 128 and q != "full_kv_int8") else qn.MLA_KERNELS)
            assert qn.mla_prolog_v2_kernels(mla_args(T=T, quant=q)) == want
    # with 32 heads the quantised modes with a bf16 query merge the W^UK
    # product into the up projection's launch up to T = 64 (two row blocks)
    for T in (1, 32, 33, 64, 65, 129):
        for q in ("partial_kv_bf16", "partial_kv_int8", "full_kv_bf16", "full_kv_int8"):
            want = merged if (T <= 64 and q != "full_kv_int8") else (
                fused if (T > 128 and q != "full_kv_int8") else qn.MLA_KERNELS)
            assert qn.mla_prolog_v2_kernels(mla_args(T=T, quant=q, N=32)) == want, (T, q)
    e = mla_args(T=0)
    assert qn.mla_prolog_v2_kernels(e) == ()
    bad = mla_args()
    bad.He = 7000
    with pytest.raises(qn.QkvnrError):
        qn.mla_prolog_v2_kernels(bad)
    lib = b.load_library()
    assert lib.mla_prolog_v2_kernels(ctypes.byref(mla_args()), None) == -1


@pytest.mark.parametrize("mutate,code", [
    (lambda a: setattr(a, "struct_size", 8), -8),
    (lambda a: setattr(a, "flags", 2), -3),        # unknown debug flag bit
    (lambda a: setattr(a, "flags", -1), -3),
    (lambda a: setattr(a, "quant_mode", 3), -1),   # full quant without its scales
    (lambda a: setattr(a, "quant_mode", 4), -1),
    (lambda a: setattr(a, "quant_mode", 9), -3),
    (lambda a: setattr(a, "weight_layout", 7), -3),
    (lambda a: setattr(a, "cache_mode", b"PA_NZ"), -4),
    (lambda a: setattr(a, "cache_mode", b"bogus"), -3),
    (lambda a: setattr(a, "B", -1), -2),
    (lambda a: setattr(a, "He", 0), -2),
    (lambda a: setattr(a, "Dr", 15), -2),
    (lambda a: setattr(a, "Nkv", 2), -4),
    (lambda a: setattr(a, "He", 7000), -4),        # not a multiple of 32
    (lambda a: setattr(a, "Dr", 48), -4),
    (lambda a: setattr(a, "rmsnorm_epsilon_cq", -1.0), -7),
    (lambda a: setattr(a, "rmsnorm_epsilon_ckv", float("nan")), -7),
    (lambda a: setattr(a, "dequant_scale_x", fake()), -5),
    (lambda a: setattr(a, "dequant_scale_w_dq", fake()), -5),
    (lambda a: setattr(a, "dequant_scale_w_dkv_kr", fake()), -5),
    (lambda a: setattr(a, "dequant_scale_q_nope", fake()), -5),
    (lambda a: setattr(a, "token_x", None), -1),
    (lambda a: setattr(a, "weight_uk", None), -1),
    (lambda a: setattr(a, "cache_index", None), -1),
    (lambda a: setattr(a, "kv_cache", None), -1),
    (lambda a: setattr(a, "query_rope", None), -1),
    (lambda a: setattr(a, "token_x", fake() + 2), -9),
    (lambda a: setattr(a, "cache_index", fake() + 4), -9),
])
def test_mla_validation_errors(mutate, code):
    a = mla_args()
    mutate(a)
    assert mla_validate(a) == code


def test_mla_quant_mode_needs_its_scales():
    a = mla_args(quant="partial_kv_int8")
    a.quant_scale_ckr = None
    assert mla_validate(a) == -1
    a = mla_args(quant="partial_kv_bf16")
    a.smooth_scales_cq = None
    assert mla_validate(a) == -1
    # Hcq must be a multiple of 64 for the int8 up-projection
    assert mla_validate(mla_args(quant="partial_kv_bf16", Hcq=1568)) == -4


def test_mla_full_quant_scales():
    """Full quantisation needs the x and down-projection dequant scales (and,
    with the int8 kv_cache, its quant scale and the query's output scale);
    scales its scenario does not use must be NULL; He must be a multiple of
    64 (int8 K steps of the tiled down projection)."""
    for q in ("full_kv_bf16", "full_kv_int8"):
        for f in ("dequant_scale_x", "dequant_scale_w_dq",
                  "dequant_scale_w_dkv_kr", "dequant_scale_w_uq_qr",
                  "smooth_scales_cq"):
            a = mla_args(quant=q)
            setattr(a, f, None)
            assert mla_validate(a) == -1, (q, f)
        a = mla_args(quant=q)
        a.quant_scale_ckr = fake()          # kr_cache stays bf16
        assert mla_validate(a) == -5
        assert mla_validate(mla_args(quant=q, He=7136)) == -4
    a = mla_args(quant="full_kv_int8")
    a.dequant_scale_q_nope = None
    assert mla_validate(a) == -1
    a = mla_args(quant="full_kv_int8")
    a.quant_scale_ckv = None
    assert mla_validate(a) == -1
    a = mla_args(quant="full_kv_bf16")
    a.dequant_scale_q_nope = fake()         # bf16 query: no output scale
    assert mla_validate(a) == -5
    a = mla_args(quant="full_kv_bf16")
    a.quant_scale_ckv = fake()              # bf16 kv_cache
    assert mla_validate(a) == -5
    a = mla_args(quant="partial_kv_bf16")
    a.dequant_scale_x = fake()              # x stays bf16
    assert mla_validate(a) == -5


def test_mla_empty_cases():
    lib = b.load_library()
    # T = 0: every per-token pointer may be NULL; nothing is launched.
    a = mla_args(T=0)
    for f in ("token_x", "rope_sin", "rope_cos", "cache_index", "query",
              "query_rope"):
        setattr(a, f, None)
    assert mla_validate(a) == 0
    n = ctypes.c_size_t(99)
    assert lib.mla_prolog_v2_workspace_size(ctypes.byref(a), ctypes.byref(n)) == 0
    assert n.value == 0
    assert lib.mla_prolog_v2(ctypes.byref(a), None, 0, None) == 0
    # no cache slots: caches may be NULL, queries are still required
    a = mla_args(bn=0)
    a.kv_cache = a.kr_cache = None
    assert mla_validate(a) == 0


def test_mla_workspace_size_and_too_small():
    lib = b.load_library()
    n = ctypes.c_size_t(0)
    a = mla_args()
    assert lib.mla_prolog_v2_workspace_size(ctypes.byref(a), ctypes.byref(n)) == 0
    packed = n.value
    # decode: split-K partials + c^Q + q^C, a few MB
    assert 1 << 20 < packed < 64 << 20
    a = mla_args(layout=b.MLA_WEIGHT_ND)
    assert lib.mla_prolog_v2_workspace_size(ctypes.byref(a), ctypes.byref(n)) == 0
    # ND weights are packed into the workspace on every call
    assert n.value >= packed + 122_552_320
    a = mla_args()
    assert lib.mla_prolog_v2(ctypes.byref(a), ctypes.c_void_p(fake()),
                             packed - 1, None) == -6
    assert lib.mla_prolog_v2_workspace_size(ctypes.byref(a), None) == -1
    bad = mla_args(He=0)
    n = ctypes.c_size_t(5)
    assert lib.mla_prolog_v2_workspace_size(ctypes.byref(bad), ctypes.byref(n)) == -2
    assert n.value == 0


def test_mla_row_width_limit():
    # the down projection's row (Hcq + Hckv + Dr fp32 values) is staged in
    # 64 KB of LDS: 16384 values pass, 16 more do not
    assert mla_validate(mla_args(T=13, He=64, Hcq=12288, N=2, D=32,
                                 Hckv=4032, Dr=64)) == 0
    assert mla_validate(mla_args(T=13, He=64, Hcq=12288, N=2, D=32,
                                 Hckv=4048, Dr=64)) == -4


def test_pack_weight_validation():
    lib = b.load_library()
    assert lib.mla_pack_weight(None, None, 1, 16, 8, 3, None) == -3
    assert lib.mla_pack_weight(None, None, 1, 12, 8, 2, None) == -2
    assert lib.mla_pack_weight(None, None, 1, 24, 8, 1, None) == -2
    assert lib.mla_pack_weight(None, None, 0, 16, 8, 2, None) == 0
    assert lib.mla_pack_weight(None, None, 1, 16, 8, 2, None) == -1
    # sizes whose products would overflow int64 are rejected before use
    big = 1 << 40
    assert lib.mla_pack_weight(None, None, big, big, big, 2, None) == -2
    assert lib.mla_pack_weight(None, None, 1, 1 << 30, 1 << 30, 2, None) == -2
    assert lib.mla_pack_weight(None, None, 65536, 16, 32, 2, None) == -2
    assert lib.mla_pack_weight(ctypes.c_void_p(fake()),
                               ctypes.c_void_p(fake() + 8), 1, 16, 8, 2,
                               None) == -9


def test_pack_weight_uk_validation():
    lib = b.load_library()
    f = lib.mla_pack_weight_uk
    assert f(None, None, 2, 24, 32, None) == -2        # D % 16
    assert f(None, None, -1, 32, 32, None) == -2
    assert f(None, None, 0, 32, 32, None) == 0         # empty: nothing
    assert f(None, None, 2, 32, 32, None) == -1
    assert f(None, None, 65535, 1 << 30, 1 << 30, None) == -2   # too large
    assert f(ctypes.c_void_p(fake()), ctypes.c_void_p(fake() + 8), 2, 32, 32,
             None) == -9


def test_pack_weight_uq_qr_validation():
    lib = b.load_library()
    f = lib.mla_pack_weight_uq_qr
    assert f(None, None, 64, 4, 32, 64, 3, None) == -3       # element size
    assert f(None, None, 12, 4, 32, 64, 2, None) == -2       # Hcq % 8
    assert f(None, None, 24, 4, 32, 64, 1, None) == -2       # Hcq % 16 (int8)
    assert f(None, None, 64, -1, 32, 64, 2, None) == -2
    assert f(None, None, 0, 4, 32, 64, 2, None) == 0         # empty: nothing
    assert f(None, None, 64, 4, 48, 64, 2, None) == -4       # D % 32
    assert f(None, None, 64, 4, 32, 48, 2, None) == -4       # Dr not 16/32/64
    assert f(None, None, 64, 4, 32, 64, 2, None) == -1
    assert f(None, None, 1 << 30, 65535, 1 << 30, 64, 2, None) == -2  # too large
    assert f(ctypes.c_void_p(fake()), ctypes.c_void_p(fake() + 8), 64, 4, 32,
             64, 2, None) == -9


# ---- QkvRmsNormRopeCache ---------------------------------------------------

def qkv_args(B=64, S=128, quant="symmetric", bn=64, bs=128, D=128):
    a = b.QkvRmsNormRopeCacheArgs()
    a.struct_size = ctypes.sizeof(b.QkvRmsNormRopeCacheArgs)
    a.quant_mode = b.QKV_QUANT[quant]
    a.dtype = 0
    a.B, a.S, a.Nq, a.Nk, a.Nv, a.D = B, S, 32, 8, 8, D
    a.block_num, a.block_size = bn, bs
    a.epsilon = 1e-6
    for f in ("qkv", "gamma_q", "gamma_k", "cos", "sin", "index", "k_cache",
              "v_cache", "q_out"):
        setattr(a, f, fake())
    if quant != "none":
        a.k_scale, a.v_scale = fake(), fake()
    if quant == "asymmetric":
        a.k_offset, a.v_offset = fake(), fake()
    return a


def qkv_validate(a):
    return b.load_library().qkv_rmsnorm_rope_cache_validate(ctypes.byref(a))


def test_qkv_valid_args_pass():
    for q in ("none", "symmetric", "asymmetric"):
        assert qkv_validate(qkv_args(quant=q)) == 0


@pytest.mark.parametrize("mutate,code", [
    (lambda a: setattr(a, "struct_size", 4), -8),
    (lambda a: setattr(a, "flags", 4), -3),        # unknown debug flag bit
    (lambda a: setattr(a, "quant_mode", 3), -3),
    (lambda a: setattr(a, "dtype", 2), -3),
    (lambda a: setattr(a, "cache_mode", b"PA_NZ"), -4),
    (lambda a: setattr(a, "Nv", 7), -2),           # Nk != Nv
    (lambda a: setattr(a, "D", 64), -4),           # only D = 128
    (lambda a: setattr(a, "D", 127), -2),          # D even
    (lambda a: setattr(a, "block_num", 63), -2),   # BlockNum >= ceil(S/BS)*B
    (lambda a: setattr(a, "block_size", 0), -2),
    (lambda a: setattr(a, "epsilon", -1e-6), -7),
    (lambda a: setattr(a, "k_scale", None), -1),
    (lambda a: setattr(a, "index", None), -1),
    (lambda a: setattr(a, "qkv", fake() + 8), -9),
    (lambda a: setattr(a, "q_before_quant", fake() + 2), -9),
])
def test_qkv_validation_errors(mutate, code):
    a = qkv_args()
    mutate(a)
    assert qkv_validate(a) == code


def test_qkv_asymmetric_needs_offsets_and_empty_is_noop():
    a = qkv_args(quant="asymmetric")
    a.v_offset = None
    assert qkv_validate(a) == -1
    lib = b.load_library()
    e = qkv_args(B=0)
    for f in ("qkv", "cos", "sin", "index", "q_out"):
        setattr(e, f, None)
    assert lib.qkv_rmsnorm_rope_cache(ctypes.byref(e), None) == 0


def test_binding_refuses_cpu_tensors():
    import torch
    w = torch.zeros(16, 8, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        qn.mla_pack_weight(w)


# ---- the binding's tensor checks (metadata only; CPU tensors) ------------

def _mla_tensors(T, He, Hcq, N, D, Hckv, Dr, bn, bs, quant, packed):
    import torch
    bf, i8, f32 = torch.bfloat16, torch.int8, torch.float32
    full, q = quant.startswith("full"), quant != "none"
    kv8, kr8 = quant in ("partial_kv_int8", "full_kv_int8"), quant == "partial_kv_int8"
    p = (lambda n: (n + 31) // 32 * 32) if packed else (lambda n: n)
    e = torch.empty
    t = dict(token_x=e(T, He, dtype=i8 if full else bf),
             weight_dq=e(He, p(Hcq), dtype=i8 if full else bf),
             weight_dkv_kr=e(He, p(Hckv + Dr), dtype=i8 if full else bf),
             weight_uq_qr=e(Hcq, p(N * (D + Dr)), dtype=i8 if q else bf),
             weight_uk=e(N, D, p(Hckv), dtype=bf),
             rmsnorm_gamma_cq=e(Hcq, dtype=bf), rmsnorm_gamma_ckv=e(Hckv, dtype=bf),
             rope_sin=e(T, Dr, dtype=bf), rope_cos=e(T, Dr, dtype=bf),
             cache_index=e(T, dtype=torch.int64),
             kv_cache=e(bn, bs, 1, Hckv, dtype=i8 if kv8 else bf),
             kr_cache=e(bn, bs, 1, Dr, dtype=i8 if kr8 else bf),
             query=e(T, N, Hckv, dtype=i8 if quant == "full_kv_int8" else bf),
             query_rope=e(T, N, Dr, dtype=bf))
    if q:
        t.update(dequant_scale_w_uq_qr=e(N * (D + Dr), dtype=f32),
                 smooth_scales_cq=e(Hcq, dtype=f32))
    if kv8:
        t["quant_scale_ckv"] = e(Hckv, dtype=f32)
    if kr8:
        t["quant_scale_ckr"] = e(Dr, dtype=f32)
    if full:
        t.update(dequant_scale_x=e(T, dtype=f32), dequant_scale_w_dq=e(Hcq, dtype=f32),
                 dequant_scale_w_dkv_kr=e(Hckv + Dr, dtype=f32))
    if quant == "full_kv_int8":
        t["dequant_scale_q_nope"] = e(T, N, 1, dtype=f32)
    return t


@pytest.mark.parametrize("quant", list(b.MLA_QUANT))
@pytest.mark.parametrize("packed", [True, False])
def test_binding_checks_mla_tensor_types_and_sizes(quant, packed):
    import torch
    dims = dict(T=5, He=256, Hcq=128, N=3, D=32, Hckv=80, Dr=16, bn=2, bs=16)
    lay = b.MLA_WEIGHT_PACKED_K16 if packed else b.MLA_WEIGHT_ND
    a = mla_args(T=5, quant=quant, He=256, Hcq=128, N=3, D=32, Hckv=80, Dr=16,
                 bn=2, bs=16, layout=lay)
    t = _mla_tensors(quant=quant, packed=packed, **dims)
    b._validate_mla(a, t)  # consistent tensors pass
    # a wrong element type, a short weight, an unpadded packed weight, a
    # cache of the other type, a short scale: each is refused
    with pytest.raises(TypeError):
        b._validate_mla(a, dict(t, rope_cos=t["rope_cos"].float()))
    with pytest.raises(ValueError):
        b._validate_mla(a, dict(t, weight_uk=t["weight_uk"][:, :, :16]))
    with pytest.raises(TypeError):
        b._validate_mla(a, dict(t, kv_cache=torch.empty(
            2, 16, 1, 80, dtype=torch.bfloat16 if t["kv_cache"].dtype == torch.int8
            else torch.int8)))
    with pytest.raises(ValueError):
        b._validate_mla(a, dict(t, cache_index=t["cache_index"][:4]))
    if packed:
        with pytest.raises(ValueError):  # Hckv = 80 packs to 96 columns
            b._validate_mla(a, dict(t, weight_uk=t["weight_uk"][:, :, :80].contiguous()))
    if quant != "none":
        with pytest.raises(ValueError):
            b._validate_mla(a, dict(t, smooth_scales_cq=t["smooth_scales_cq"][:64]))


@pytest.mark.parametrize("quant", list(b.QKV_QUANT))
def test_binding_checks_qkv_tensor_types_and_sizes(quant):
    import torch
    h, f32, i8 = torch.float16, torch.float32, torch.int8
    T, bn, bs = 6, 2, 16
    a = qkv_args(B=2, S=3, quant=quant, bn=bn, bs=bs)
    e = torch.empty
    cache = h if quant == "none" else i8
    t = dict(qkv=e(T, 48, 128, dtype=h), gamma_q=e(128, dtype=h),
             gamma_k=e(128, dtype=h), cos=e(T, 128, dtype=h), sin=e(T, 128, dtype=h),
             index=e(T, dtype=torch.int64), k_cache=e(bn, bs, 8, 128, dtype=cache),
             v_cache=e(bn, bs, 8, 128, dtype=cache), q_out=e(T, 32, 128, dtype=h))
    if quant != "none":
        t.update(k_scale=e(1024, dtype=f32), v_scale=e(1024, dtype=f32))
    if quant == "asymmetric":
        t.update(k_offset=e(1024, dtype=f32), v_offset=e(1024, dtype=f32))
    b._validate_qkv(a, t)
    with pytest.raises(TypeError):
        b._validate_qkv(a, dict(t, gamma_k=t["gamma_k"].to(torch.bfloat16)))
    with pytest.raises(ValueError):
        b._validate_qkv(a, dict(t, index=t["index"][:5]))
    with pytest.raises(ValueError):
        b._validate_qkv(a, dict(t, q_out=e(T, 8, 128, dtype=h)))
    if quant != "none":
        with pytest.raises(ValueError):
            b._validate_qkv(a, dict(t, v_scale=e(128, dtype=f32)))


def test_mla_fuzzed_args_validate_size_and_plan_consistently():
    # Random dims (up to and past the validator's caps), modes, layouts and
    # pointer patterns: validate, workspace sizing and the kernel mask must
    # agree and return documented codes.  Under the host sanitizer build
    # (tests/test_host_sanitizers.py) an overflow or bad access in the
    # validation or plan arithmetic aborts the run.
    import numpy as np
    rng = np.random.default_rng(2024)
    lib = b.load_library()
    codes = set(b.STATUS_NAMES)
    dims = ("B", "S", "He", "Hcq", "N", "D", "Hckv", "Dr", "Nkv", "block_num",
            "block_size")
    choices = [0, 1, 2, 15, 16, 32, 48, 64, 96, 128, 512, 1536, 7168, 16384,
               1 << 22, (1 << 22) + 32, 1 << 23, 1 << 30, (1 << 30) + 1,
               1 << 40, -1]
    for it in range(3000):
        q = list(b.MLA_QUANT)[int(rng.integers(0, 5))]
        a = mla_args(quant=q, layout=int(rng.integers(0, 2)))
        for d in dims:
            if rng.random() < 0.3:
                setattr(a, d, int(rng.choice(choices)))
        if rng.random() < 0.1:
            a.flags = int(rng.integers(0, 3))
        if rng.random() < 0.1:
            a.cache_index = None
        rc = mla_validate(a)
        assert rc in codes, (it, rc)
        n = ctypes.c_size_t(123)
        rs = lib.mla_prolog_v2_workspace_size(ctypes.byref(a), ctypes.byref(n))
        m = ctypes.c_uint32(7)
        rk = lib.mla_prolog_v2_kernels(ctypes.byref(a), ctypes.byref(m))
        assert rs == rc and rk == rc, (it, rc, rs, rk)
        if rc != 0:
            assert n.value == 0 and m.value == 0
        else:
            T = a.B * a.S
            # all four kernels, or all but the W^UK launch (merged into the
            # up projection's for bf16 decode with D <= 128 and T <= 32, and
            # for the quantised modes with a bf16 query, T <= 64, D <= 128
            # and fewer than 128 of the 96-column up-projection tiles)
            merged = ((q == "none" and 0 < T <= 32 and a.D <= 128) or
                      (q in ("partial_kv_bf16", "partial_kv_int8", "full_kv_bf16")
                       and 0 < T <= 64 and a.D <= 128
                       and (a.N * (a.D + a.Dr) + 95) // 96 < 128))
            fused = (T > 128 and q != "full_kv_int8" and a.D == 128
                     and (a.N * a.D) % 256 == 0)
            want = 0 if T == 0 else (7 if merged else (11 if fused else 15))
            assert (n.value > 0) == (T > 0) and m.value == want, (it, T, q)


def test_no_alloc_entry_point_host_checks():
    # refusals happen on the host before any launch (no GPU needed)
    lib = b.load_library()
    src = open(HEADER).read()
    m = re.search(r"#define MLA_NO_ALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", src)
    assert m and int(m.group(1)) << int(m.group(2)) == qn.MLA_NO_ALLOC_SCRATCH_BYTES
    big = mla_args(T=4096)
    assert qn.mla_prolog_v2_workspace_size(big) > qn.MLA_NO_ALLOC_SCRATCH_BYTES
    assert lib.mla_prolog_v2_no_alloc(ctypes.byref(big), None) == -13
    nd = mla_args(T=32, layout=b.MLA_WEIGHT_ND)  # packs weights into scratch
    assert lib.mla_prolog_v2_no_alloc(ctypes.byref(nd), None) == -13
    dbg = mla_args(T=32)
    dbg.flags = b.MLA_FLAG_CHECK_INDEX
    assert lib.mla_prolog_v2_no_alloc(ctypes.byref(dbg), None) == -3
    e = mla_args(T=0)
    assert lib.mla_prolog_v2_no_alloc(ctypes.byref(e), None) == 0
    bad = mla_args(T=32)
    bad.He = 7000
    assert lib.mla_prolog_v2_no_alloc(ctypes.byref(bad), None) == -4
    # the decode shapes it is for fit
    for q, T in (("none", 128), ("partial_kv_int8", 128), ("full_kv_bf16", 128),
                 ("full_kv_int8", 32)):
        assert qn.mla_prolog_v2_workspace_size(mla_args(T=T, quant=q)) <= \
            qn.MLA_NO_ALLOC_SCRATCH_BYTES, (q, T)
    assert qn.status_string(-13).startswith("the call needs more than")


# ---- MlaPreprocessV2 -------------------------------------------------------

def pre_args(T=32, He=7168, Hcq=1536, N=32, D=128, Hckv=512, Dr=64, bn=192,
             bs=128, layout=b.MLA_WEIGHT_PACKED_K16):
    a = b.MlaPreprocessV2Args()
    a.struct_size = ctypes.sizeof(b.MlaPreprocessV2Args)
    a.weight_layout = layout
    a.B, a.S = T, 1
    a.He, a.Hcq, a.N, a.D, a.Hckv, a.Dr = He, Hcq, N, D, Hckv, Dr
    a.block_num, a.block_size = bn, bs
    a.epsilon = 1e-6
    a.quant_scale_x, a.quant_scale_cq = 25.0, 21.0
    for f in ("token_x", "gamma_x", "bias_x", "weight_dqkv",
              "dequant_scale_dqkv", "gamma_cq", "bias_cq", "weight_uq_qr",
              "dequant_scale_uq_qr", "weight_uk", "gamma_ckv", "rope_sin",
              "rope_cos", "cache_index", "kv_cache", "kr_cache", "query",
              "query_rope"):
        setattr(a, f, fake())
    return a


def pre_validate(a):
    return b.load_library().mla_preprocess_v2_validate(ctypes.byref(a))


def test_preprocess_valid_args_pass():
    assert pre_validate(pre_args()) == 0
    assert pre_validate(pre_args(T=4, He=256, Hcq=128, N=4, D=32, Hckv=64,
                                 Dr=16, bn=4, bs=16)) == 0
    assert pre_validate(pre_args(T=4096)) == 0


@pytest.mark.parametrize("mutate,code", [
    (lambda a: setattr(a, "struct_size", 8), -8),
    (lambda a: setattr(a, "reserved0", 1), -8),
    (lambda a: setattr(a, "flags", 2), -3),
    (lambda a: setattr(a, "quant_scale_x", float("inf")), -12),
    (lambda a: setattr(a, "quant_scale_cq", float("nan")), -12),
    (lambda a: setattr(a, "He", 7168 + 32), -4),    # int8 K: multiple of 64
    (lambda a: setattr(a, "Hcq", 1536 + 32), -4),
    (lambda a: setattr(a, "Hcq", -64), -2),
    (lambda a: setattr(a, "Dr", 48), -4),
    (lambda a: setattr(a, "epsilon", -1.0), -7),
    (lambda a: setattr(a, "cache_mode", b"PA_NZ"), -4),
    (lambda a: setattr(a, "gamma_x", None), -1),
    (lambda a: setattr(a, "bias_x", None), -1),
    (lambda a: setattr(a, "bias_cq", None), -1),
    (lambda a: setattr(a, "dequant_scale_dqkv", None), -1),
    (lambda a: setattr(a, "dequant_scale_uq_qr", None), -1),
    (lambda a: setattr(a, "weight_dqkv", None), -1),
    (lambda a: setattr(a, "kv_cache", None), -1),
    (lambda a: setattr(a, "bias_x", fake() + 4), -9),
    (lambda a: setattr(a, "token_x", fake() + 2), -9),
])
def test_preprocess_validation_errors(mutate, code):
    a = pre_args()
    mutate(a)
    assert pre_validate(a) == code


def test_preprocess_workspace_and_empty():
    lib = b.load_library()
    n = ctypes.c_size_t(0)
    a = pre_args()
    assert lib.mla_preprocess_v2_workspace_size(ctypes.byref(a),
                                                ctypes.byref(n)) == 0
    # at least the prolog's full-quantisation workspace plus x's codes
    assert n.value >= 32 * 7168
    small = ctypes.c_size_t(0)
    a2 = pre_args(T=4, He=256, Hcq=128, N=4, D=32, Hckv=64, Dr=16, bn=4, bs=16)
    lib.mla_preprocess_v2_workspace_size(ctypes.byref(a2), ctypes.byref(small))
    assert 0 < small.value < n.value
    assert lib.mla_preprocess_v2(ctypes.byref(a), fake(), n.value - 256,
                                 None) == -6
    e = pre_args(T=0)
    for f in ("token_x", "rope_sin", "rope_cos", "cache_index", "query",
              "query_rope"):
        setattr(e, f, None)
    assert pre_validate(e) == 0
    assert lib.mla_preprocess_v2(ctypes.byref(e), None, 0, None) == 0
