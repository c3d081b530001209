"""ctypes binding over libqkvnr.so (argument marshalling only).

Every computation happens in the HIP library; this module checks tensor
metadata, allocates outputs and workspace through torch (device memory and
streams only), fills the C argument structs declared in include/qkvnr.h and
raises on a non-zero status.  There is no fallback: without the built
library every entry point raises.
"""

from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libqkvnr.so")

# ---- constants mirrored from include/qkvnr.h --------------------------------
QKVNR_OK = 0
STATUS_NAMES = {
    0: "QKVNR_OK", -1: "QKVNR_ERR_NULL_ARG", -2: "QKVNR_ERR_BAD_SHAPE",
    -3: "QKVNR_ERR_BAD_MODE", -4: "QKVNR_ERR_UNSUPPORTED",
    -5: "QKVNR_ERR_RESERVED_NONNULL", -6: "QKVNR_ERR_WORKSPACE_TOO_SMALL",
    -7: "QKVNR_ERR_BAD_EPS", -8: "QKVNR_ERR_BAD_STRUCT",
    -9: "QKVNR_ERR_BAD_ALIGNMENT", -10: "QKVNR_ERR_LAUNCH_FAILED",
    -11: "QKVNR_ERR_BAD_INDEX", -12: "QKVNR_ERR_BAD_SCALE",
    -13: "QKVNR_ERR_SCRATCH_TOO_SMALL",
}
MLA_NO_ALLOC_SCRATCH_BYTES = 16 << 20
MLA_FLAG_CHECK_INDEX = 1
QKV_FLAG_CHECK_INPUTS = 1
MLA_QUANT = {"none": 0, "partial_kv_bf16": 1, "partial_kv_int8": 2,
             "full_kv_bf16": 3, "full_kv_int8": 4}
MLA_WEIGHT_ND, MLA_WEIGHT_PACKED_K16 = 0, 1
MLA_PHASES = ("start", "after_down", "after_norm", "after_uqqr", "after_uk")
MLA_KERNELS = ("down", "norm", "uqqr", "uk")
QKV_QUANT = {"none": 0, "symmetric": 1, "asymmetric": 2}
QKV_DTYPE = {torch.float16: 0, torch.bfloat16: 1}

EXPORTS = (
    "mla_status_string", "mla_lib_version", "mla_check_cache_index",
    "mla_prolog_v2_workspace_size", "mla_prolog_v2_validate",
    "mla_prolog_v2_kernels", "mla_prolog_v2", "mla_prolog_v2_no_alloc",
    "mla_pack_weight",
    "mla_pack_weight_uq_qr", "mla_pack_weight_uk",
    "qkv_rmsnorm_rope_cache_validate", "qkv_rmsnorm_rope_cache",
    "mla_probe_read", "mla_probe_mfma_bf16",
    "mla_preprocess_v2_validate", "mla_preprocess_v2_workspace_size",
    "mla_preprocess_v2",
)

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64


class MlaPrologV2Args(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32), ("quant_mode", ctypes.c_int32),
        ("weight_layout", ctypes.c_int32), ("flags", ctypes.c_int32),
        ("B", _i64), ("S", _i64), ("He", _i64), ("Hcq", _i64), ("N", _i64),
        ("D", _i64), ("Hckv", _i64), ("Dr", _i64), ("Nkv", _i64),
        ("block_num", _i64), ("block_size", _i64),
        ("rmsnorm_epsilon_cq", ctypes.c_double),
        ("rmsnorm_epsilon_ckv", ctypes.c_double),
        ("cache_mode", ctypes.c_char_p),
        ("token_x", _vp), ("weight_dq", _vp), ("weight_uq_qr", _vp),
        ("weight_uk", _vp), ("weight_dkv_kr", _vp),
        ("rmsnorm_gamma_cq", _vp), ("rmsnorm_gamma_ckv", _vp),
        ("rope_sin", _vp), ("rope_cos", _vp), ("cache_index", _vp),
        ("dequant_scale_x", _vp), ("dequant_scale_w_dq", _vp),
        ("dequant_scale_w_uq_qr", _vp), ("dequant_scale_w_dkv_kr", _vp),
        ("quant_scale_ckv", _vp), ("quant_scale_ckr", _vp),
        ("smooth_scales_cq", _vp),
        ("kv_cache", _vp), ("kr_cache", _vp),
        ("query", _vp), ("query_rope", _vp), ("dequant_scale_q_nope", _vp),
        ("dbg_cq_int8", _vp), ("dbg_cq_scale", _vp),
        ("phase_events", ctypes.POINTER(_vp)), ("n_phase_events", ctypes.c_int32),
        ("kernel_events", ctypes.POINTER(_vp)), ("n_kernel_events", ctypes.c_int32),
    ]


class QkvRmsNormRopeCacheArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32), ("quant_mode", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("flags", ctypes.c_int32),
        ("B", _i64), ("S", _i64), ("Nq", _i64), ("Nk", _i64), ("Nv", _i64),
        ("D", _i64), ("block_num", _i64), ("block_size", _i64),
        ("epsilon", ctypes.c_double), ("cache_mode", ctypes.c_char_p),
        ("qkv", _vp), ("gamma_q", _vp), ("gamma_k", _vp), ("cos", _vp),
        ("sin", _vp), ("index", _vp), ("k_scale", _vp), ("v_scale", _vp),
        ("k_offset", _vp), ("v_offset", _vp), ("k_cache", _vp),
        ("v_cache", _vp), ("q_out", _vp), ("q_before_quant", _vp),
        ("k_before_quant", _vp), ("v_before_quant", _vp),
    ]


class MlaPreprocessV2Args(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32), ("weight_layout", ctypes.c_int32),
        ("flags", ctypes.c_int32), ("reserved0", ctypes.c_int32),
        ("B", _i64), ("S", _i64), ("He", _i64), ("Hcq", _i64), ("N", _i64),
        ("D", _i64), ("Hckv", _i64), ("Dr", _i64), ("block_num", _i64),
        ("block_size", _i64), ("epsilon", ctypes.c_double),
        ("quant_scale_x", ctypes.c_float), ("quant_scale_cq", ctypes.c_float),
        ("cache_mode", ctypes.c_char_p),
        ("token_x", _vp), ("gamma_x", _vp), ("bias_x", _vp),
        ("weight_dqkv", _vp), ("dequant_scale_dqkv", _vp),
        ("gamma_cq", _vp), ("bias_cq", _vp), ("weight_uq_qr", _vp),
        ("dequant_scale_uq_qr", _vp), ("weight_uk", _vp), ("gamma_ckv", _vp),
        ("rope_sin", _vp), ("rope_cos", _vp), ("cache_index", _vp),
        ("kv_cache", _vp), ("kr_cache", _vp), ("query", _vp),
        ("query_rope", _vp), ("dbg_x_int8", _vp), ("dbg_cq_int8", _vp),
    ]


class QkvnrError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS_NAMES.get(status, status)} "
                         f"({status_string(status)})")


_lib = None


def load_library(path: str = None) -> ctypes.CDLL:
    """Load libqkvnr.so once; raise if it has not been built.

    QKVNR_LIBRARY overrides the path (the host sanitizer test points it at
    an address/undefined-behaviour-sanitized build of the C ABI layer)."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or os.environ.get("QKVNR_LIBRARY") or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m qkv_norm_rope_amd.build`"
            " (there is no non-HIP fallback)")
    lib = ctypes.CDLL(path)
    lib.mla_status_string.restype = ctypes.c_char_p
    lib.mla_status_string.argtypes = [ctypes.c_int]
    lib.mla_lib_version.restype = ctypes.c_char_p
    lib.mla_lib_version.argtypes = []
    lib.mla_check_cache_index.restype = ctypes.c_int
    lib.mla_check_cache_index.argtypes = [_vp, _i64, _i64]
    lib.mla_probe_read.restype = ctypes.c_int
    lib.mla_probe_read.argtypes = [_vp, ctypes.c_size_t, _vp, _vp]
    lib.mla_probe_mfma_bf16.restype = ctypes.c_int
    lib.mla_probe_mfma_bf16.argtypes = [_i64, _vp, _vp]
    lib.mla_prolog_v2_kernels.restype = ctypes.c_int
    lib.mla_prolog_v2_kernels.argtypes = [
        ctypes.POINTER(MlaPrologV2Args), ctypes.POINTER(ctypes.c_uint32)]
    lib.mla_prolog_v2_workspace_size.restype = ctypes.c_int
    lib.mla_prolog_v2_workspace_size.argtypes = [
        ctypes.POINTER(MlaPrologV2Args), ctypes.POINTER(ctypes.c_size_t)]
    lib.mla_prolog_v2_validate.restype = ctypes.c_int
    lib.mla_prolog_v2_validate.argtypes = [ctypes.POINTER(MlaPrologV2Args)]
    lib.mla_preprocess_v2_validate.restype = ctypes.c_int
    lib.mla_preprocess_v2_validate.argtypes = [ctypes.POINTER(MlaPreprocessV2Args)]
    lib.mla_preprocess_v2_workspace_size.restype = ctypes.c_int
    lib.mla_preprocess_v2_workspace_size.argtypes = [
        ctypes.POINTER(MlaPreprocessV2Args), ctypes.POINTER(ctypes.c_size_t)]
    lib.mla_preprocess_v2.restype = ctypes.c_int
    lib.mla_preprocess_v2.argtypes = [ctypes.POINTER(MlaPreprocessV2Args), _vp,
                                      ctypes.c_size_t, _vp]
    lib.mla_prolog_v2_no_alloc.restype = ctypes.c_int
    lib.mla_prolog_v2_no_alloc.argtypes = [ctypes.POINTER(MlaPrologV2Args), _vp]
    lib.mla_prolog_v2.restype = ctypes.c_int
    lib.mla_prolog_v2.argtypes = [ctypes.POINTER(MlaPrologV2Args), _vp,
                                  ctypes.c_size_t, _vp]
    lib.mla_pack_weight.restype = ctypes.c_int
    lib.mla_pack_weight.argtypes = [_vp, _vp, _i64, _i64, _i64, ctypes.c_int32,
                                    _vp]
    lib.mla_pack_weight_uk.restype = ctypes.c_int
    lib.mla_pack_weight_uk.argtypes = [_vp, _vp, _i64, _i64, _i64, _vp]
    lib.mla_pack_weight_uq_qr.restype = ctypes.c_int
    lib.mla_pack_weight_uq_qr.argtypes = [_vp, _vp, _i64, _i64, _i64, _i64,
                                          ctypes.c_int32, _vp]
    lib.qkv_rmsnorm_rope_cache_validate.restype = ctypes.c_int
    lib.qkv_rmsnorm_rope_cache_validate.argtypes = [
        ctypes.POINTER(QkvRmsNormRopeCacheArgs)]
    lib.qkv_rmsnorm_rope_cache.restype = ctypes.c_int
    lib.qkv_rmsnorm_rope_cache.argtypes = [
        ctypes.POINTER(QkvRmsNormRopeCacheArgs), _vp]
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().mla_status_string(status).decode()


def version() -> str:
    return load_library().mla_lib_version().decode()


def mla_check_cache_index(index, slots: int) -> int:
    """The index restriction checked on the host: returns the library's
    status for `index` (a CPU int64 tensor or array) against `slots`
    (QKVNR_OK, or QKVNR_ERR_BAD_INDEX for an out-of-range or repeated
    index)."""
    import numpy as np
    a = np.ascontiguousarray(
        index.cpu().numpy() if isinstance(index, torch.Tensor) else index,
        dtype=np.int64).reshape(-1)
    return load_library().mla_check_cache_index(
        a.ctypes.data if a.size else None, a.size, int(slots))


def _check(status: int, what: str):
    if status != QKVNR_OK:
        raise QkvnrError(status, what)


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, dtype, name):
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def _pad32(n: int) -> int:
    return (n + 31) // 32 * 32


def _expect(t, dtype, numel: int, name: str):
    """The library takes raw pointers and cannot see tensor sizes, so each
    tensor's element type and element count are checked here, before a
    kernel could read or write past it.  An absent tensor is left to the
    library's own NULL checks."""
    if t is None:
        return
    _need(t, dtype, name)
    if t.numel() != numel:
        raise ValueError(f"{name} must hold {numel} elements for these "
                         f"dimensions, got {t.numel()} (shape {tuple(t.shape)})")


def _validate_mla(a: "MlaPrologV2Args", t: dict):
    """Element types and counts of the MlaPrologV2 tensors for the
    dimensions and quant mode in `a` (the dtype/shape table of
    include/qkvnr.h; packed weights hold whole 32-column blocks)."""
    m = a.quant_mode
    full, quant = m in (3, 4), m != 0
    kv8, kr8, q8 = m in (2, 4), m == 2, m == 4
    T = a.B * a.S
    bf, i8, f32 = torch.bfloat16, torch.int8, torch.float32
    cols = _pad32 if a.weight_layout == MLA_WEIGHT_PACKED_K16 else int
    down = i8 if full else bf
    slots = a.block_num * a.block_size * a.Nkv
    _expect(t.get("token_x"), down, T * a.He, "token_x")
    _expect(t.get("weight_dq"), down, a.He * cols(a.Hcq), "weight_dq")
    _expect(t.get("weight_dkv_kr"), down, a.He * cols(a.Hckv + a.Dr),
            "weight_dkv_kr")
    _expect(t.get("weight_uq_qr"), i8 if quant else bf,
            a.Hcq * cols(a.N * (a.D + a.Dr)), "weight_uq_qr")
    _expect(t.get("weight_uk"), bf, a.N * a.D * cols(a.Hckv), "weight_uk")
    _expect(t.get("rmsnorm_gamma_cq"), bf, a.Hcq, "rmsnorm_gamma_cq")
    _expect(t.get("rmsnorm_gamma_ckv"), bf, a.Hckv, "rmsnorm_gamma_ckv")
    _expect(t.get("rope_sin"), bf, T * a.Dr, "rope_sin")
    _expect(t.get("rope_cos"), bf, T * a.Dr, "rope_cos")
    _expect(t.get("cache_index"), torch.int64, T, "cache_index")
    _expect(t.get("kv_cache"), i8 if kv8 else bf, slots * a.Hckv, "kv_cache")
    _expect(t.get("kr_cache"), i8 if kr8 else bf, slots * a.Dr, "kr_cache")
    _expect(t.get("query"), i8 if q8 else bf, T * a.N * a.Hckv, "query")
    _expect(t.get("query_rope"), bf, T * a.N * a.Dr, "query_rope")
    if quant:
        _expect(t.get("dequant_scale_w_uq_qr"), f32, a.N * (a.D + a.Dr),
                "dequant_scale_w_uq_qr")
        _expect(t.get("smooth_scales_cq"), f32, a.Hcq, "smooth_scales_cq")
        _expect(t.get("dbg_cq_int8"), i8, T * a.Hcq, "cq_int8")
        _expect(t.get("dbg_cq_scale"), f32, T, "cq_scale")
    if kv8:
        _expect(t.get("quant_scale_ckv"), f32, a.Hckv, "quant_scale_ckv")
    if kr8:
        _expect(t.get("quant_scale_ckr"), f32, a.Dr, "quant_scale_ckr")
    if full:
        _expect(t.get("dequant_scale_x"), f32, T, "dequant_scale_x")
        _expect(t.get("dequant_scale_w_dq"), f32, a.Hcq, "dequant_scale_w_dq")
        _expect(t.get("dequant_scale_w_dkv_kr"), f32, a.Hckv + a.Dr,
                "dequant_scale_w_dkv_kr")
    if q8:
        _expect(t.get("dequant_scale_q_nope"), f32, T * a.N,
                "dequant_scale_q_nope")


def _validate_qkv(a: "QkvRmsNormRopeCacheArgs", t: dict):
    """Element types and counts of the QkvRmsNormRopeCache tensors for the
    dimensions and quant mode in `a`."""
    dt = {0: torch.float16, 1: torch.bfloat16}.get(a.dtype)
    if dt is None:
        raise TypeError("qkv must be float16 or bfloat16")
    T, D = a.B * a.S, a.D
    cache = dt if a.quant_mode == QKV_QUANT["none"] else torch.int8
    slots = a.block_num * a.block_size
    _expect(t.get("qkv"), dt, T * (a.Nq + a.Nk + a.Nv) * D, "qkv")
    _expect(t.get("gamma_q"), dt, D, "gamma_q")
    _expect(t.get("gamma_k"), dt, D, "gamma_k")
    _expect(t.get("cos"), dt, T * D, "cos")
    _expect(t.get("sin"), dt, T * D, "sin")
    _expect(t.get("index"), torch.int64, T, "index")
    _expect(t.get("k_cache"), cache, slots * a.Nk * D, "k_cache")
    _expect(t.get("v_cache"), cache, slots * a.Nv * D, "v_cache")
    _expect(t.get("q_out"), dt, T * a.Nq * D, "q_out")
    _expect(t.get("q_before_quant"), dt, T * a.Nq * D, "q_before_quant")
    _expect(t.get("k_before_quant"), dt, T * a.Nk * D, "k_before_quant")
    _expect(t.get("v_before_quant"), dt, T * a.Nv * D, "v_before_quant")
    if a.quant_mode != QKV_QUANT["none"]:
        _expect(t.get("k_scale"), torch.float32, a.Nk * D, "k_scale")
        _expect(t.get("v_scale"), torch.float32, a.Nv * D, "v_scale")
    if a.quant_mode == QKV_QUANT["asymmetric"]:
        _expect(t.get("k_offset"), torch.float32, a.Nk * D, "k_offset")
        _expect(t.get("v_offset"), torch.float32, a.Nv * D, "v_offset")


# ---------------------------------------------------------------------------
# measurement probes
# ---------------------------------------------------------------------------

def mla_probe_read(src: torch.Tensor, sink: torch.Tensor, stream=None):
    """Enqueue one streaming read of src (device, contiguous, a multiple of
    16 bytes); sink is a device tensor of at least 4 bytes."""
    _check(load_library().mla_probe_read(
        _ptr(src), src.numel() * src.element_size(), _ptr(sink),
        _stream(stream)), "mla_probe_read")


def mla_probe_mfma_bf16(iters: int, sink: torch.Tensor, stream=None) -> int:
    """Enqueue the dense bf16 MFMA loop; returns its flop count."""
    _check(load_library().mla_probe_mfma_bf16(int(iters), _ptr(sink),
                                              _stream(stream)),
           "mla_probe_mfma_bf16")
    return (1 << 28) * int(iters)


# ---------------------------------------------------------------------------
# weight packing
# ---------------------------------------------------------------------------

def mla_pack_weight(w: torch.Tensor, stream=None) -> torch.Tensor:
    """Pack a (K, N) or (batch, K, N) weight into the K16 blocked layout.

    Returns a tensor of shape (K, Np) or (batch, K, Np) with Np = N rounded
    up to a multiple of 32 and w's dtype; only the element order (and the
    zero padding) differ (see MLA_WEIGHT_PACKED_K16 in include/qkvnr.h).
    """
    lib = load_library()
    if w.dim() not in (2, 3):
        raise ValueError("weight must be (K, N) or (batch, K, N)")
    batch = 1 if w.dim() == 2 else w.shape[0]
    K, N = w.shape[-2], w.shape[-1]
    eb = w.element_size()
    out = torch.empty(tuple(w.shape[:-1]) + ((N + 31) // 32 * 32,),
                      dtype=w.dtype, device=w.device)
    _check(lib.mla_pack_weight(_ptr(w), _ptr(out), batch, K, N, eb,
                               _stream(stream)), "mla_pack_weight")
    return out


def mla_pack_weight_uk(w: torch.Tensor, stream=None) -> torch.Tensor:
    """Pack weight_uk (N, D, Hckv) bf16 into the K16 blocked layout with the
    k order of include/qkvnr.h (MLA_WEIGHT_PACKED_K16).  Returns (N, D, Hp),
    Hp = Hckv rounded up to a multiple of 32."""
    lib = load_library()
    if w.dim() != 3 or w.dtype != torch.bfloat16:
        raise ValueError("weight_uk must be a bf16 (N, D, Hckv) tensor")
    N, D, H = w.shape
    out = torch.empty((N, D, (H + 31) // 32 * 32), dtype=w.dtype,
                      device=w.device)
    _check(lib.mla_pack_weight_uk(_ptr(w), _ptr(out), N, D, H,
                                  _stream(stream)), "mla_pack_weight_uk")
    return out


def mla_pack_weight_uq_qr(w: torch.Tensor, N: int, D: int, Dr: int,
                          stream=None) -> torch.Tensor:
    """Pack weight_uq_qr (Hcq, N*(D+Dr)) into the K16 blocked layout with
    the RoPE-partner column order of its W^QR part (include/qkvnr.h,
    MLA_WEIGHT_PACKED_K16).  Returns (Hcq, Np), Np = N*(D+Dr) rounded up to
    a multiple of 32, with w's dtype."""
    lib = load_library()
    if w.dim() != 2 or w.shape[1] != N * (D + Dr):
        raise ValueError("weight_uq_qr must be (Hcq, N*(D+Dr))")
    Hcq, NDR = w.shape
    out = torch.empty((Hcq, (NDR + 31) // 32 * 32), dtype=w.dtype,
                      device=w.device)
    _check(lib.mla_pack_weight_uq_qr(_ptr(w), _ptr(out), Hcq, N, D, Dr,
                                     w.element_size(), _stream(stream)),
           "mla_pack_weight_uq_qr")
    return out


# ---------------------------------------------------------------------------
# MlaPrologV2
# ---------------------------------------------------------------------------

def mla_prolog_v2_args(token_x, weight_dq, weight_uq_qr, weight_uk,
                       weight_dkv_kr, rmsnorm_gamma_cq, rmsnorm_gamma_ckv,
                       rope_sin, rope_cos, cache_index, kv_cache, kr_cache,
                       query, query_rope, *, quant_mode="none",
                       weight_layout=MLA_WEIGHT_PACKED_K16,
                       rmsnorm_epsilon_cq=1e-5, rmsnorm_epsilon_ckv=1e-5,
                       dequant_scale_w_uq_qr=None, quant_scale_ckv=None,
                       quant_scale_ckr=None, smooth_scales_cq=None,
                       dequant_scale_x=None, dequant_scale_w_dq=None,
                       dequant_scale_w_dkv_kr=None, dequant_scale_q_nope=None,
                       dbg_cq_int8=None, dbg_cq_scale=None, cache_mode=None,
                       B=None, S=None, flags=0) -> MlaPrologV2Args:
    """Fill the C struct from tensors.  Dims come from the tensor shapes:
    token_x (T, He) or (B, S, He); weight_dq (He, Hcq); weight_uk
    (N, D, Hckv); rope tables (T, Dr); caches (BlockNum, BlockSize, Nkv, H).
    """
    a = MlaPrologV2Args()
    a.struct_size = ctypes.sizeof(MlaPrologV2Args)
    a.quant_mode = MLA_QUANT[quant_mode] if isinstance(quant_mode, str) \
        else int(quant_mode)
    a.weight_layout = int(weight_layout)
    a.flags = int(flags)
    He = token_x.shape[-1]
    T = token_x.numel() // He if He else 0
    if B is None:
        B, S = (token_x.shape[0], token_x.shape[1]) if token_x.dim() == 3 \
            else (T, 1)
    a.B, a.S = int(B), int(S)
    a.He = int(He)
    # Hcq and Hckv come from the gammas: packed weights pad their columns.
    a.Hcq = int(rmsnorm_gamma_cq.shape[-1])
    a.N, a.D = int(weight_uk.shape[0]), int(weight_uk.shape[1])
    a.Hckv = int(rmsnorm_gamma_ckv.shape[-1])
    a.Dr = int(rope_sin.shape[-1])
    a.Nkv = int(kv_cache.shape[2])
    a.block_num, a.block_size = int(kv_cache.shape[0]), int(kv_cache.shape[1])
    a.rmsnorm_epsilon_cq = float(rmsnorm_epsilon_cq)
    a.rmsnorm_epsilon_ckv = float(rmsnorm_epsilon_ckv)
    a.cache_mode = cache_mode.encode() if cache_mode else None
    if T > 0:
        a.token_x = _ptr(token_x)
        a.rope_sin = _ptr(rope_sin)
        a.rope_cos = _ptr(rope_cos)
        a.cache_index = _ptr(cache_index)
        a.query = _ptr(query)
        a.query_rope = _ptr(query_rope)
        a.dbg_cq_int8 = _ptr(dbg_cq_int8)
        a.dbg_cq_scale = _ptr(dbg_cq_scale)
        a.dequant_scale_x = _ptr(dequant_scale_x)
        a.dequant_scale_q_nope = _ptr(dequant_scale_q_nope)
    a.weight_dq = _ptr(weight_dq)
    a.weight_uq_qr = _ptr(weight_uq_qr)
    a.weight_uk = _ptr(weight_uk)
    a.weight_dkv_kr = _ptr(weight_dkv_kr)
    a.rmsnorm_gamma_cq = _ptr(rmsnorm_gamma_cq)
    a.rmsnorm_gamma_ckv = _ptr(rmsnorm_gamma_ckv)
    if kv_cache.numel():
        a.kv_cache = _ptr(kv_cache)
    if kr_cache.numel():
        a.kr_cache = _ptr(kr_cache)
    a.dequant_scale_w_uq_qr = _ptr(dequant_scale_w_uq_qr)
    a.quant_scale_ckv = _ptr(quant_scale_ckv)
    a.quant_scale_ckr = _ptr(quant_scale_ckr)
    a.smooth_scales_cq = _ptr(smooth_scales_cq)
    a.dequant_scale_w_dq = _ptr(dequant_scale_w_dq)
    a.dequant_scale_w_dkv_kr = _ptr(dequant_scale_w_dkv_kr)
    return a


def mla_prolog_v2_workspace_size(args: MlaPrologV2Args) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().mla_prolog_v2_workspace_size(ctypes.byref(args),
                                                       ctypes.byref(n)),
           "mla_prolog_v2_workspace_size")
    return n.value


def mla_prolog_v2_kernels(args: MlaPrologV2Args) -> tuple:
    """Names (from MLA_KERNELS) of the main kernels a call with these args
    launches, i.e. whose kernel_events it records."""
    m = ctypes.c_uint32(0)
    _check(load_library().mla_prolog_v2_kernels(ctypes.byref(args),
                                                ctypes.byref(m)),
           "mla_prolog_v2_kernels")
    return tuple(k for i, k in enumerate(MLA_KERNELS) if m.value >> i & 1)


def mla_prolog_v2(token_x, weight_dq, weight_uq_qr, weight_uk, weight_dkv_kr,
                  rmsnorm_gamma_cq, rmsnorm_gamma_ckv, rope_sin, rope_cos,
                  cache_index, kv_cache, kr_cache, *, quant_mode="none",
                  weight_layout=MLA_WEIGHT_PACKED_K16,
                  rmsnorm_epsilon_cq=1e-5, rmsnorm_epsilon_ckv=1e-5,
                  dequant_scale_w_uq_qr=None, quant_scale_ckv=None,
                  quant_scale_ckr=None, smooth_scales_cq=None,
                  dequant_scale_x=None, dequant_scale_w_dq=None,
                  dequant_scale_w_dkv_kr=None, dequant_scale_q_nope=None,
                  query=None, query_rope=None, workspace=None,
                  return_cq_quant=False, cache_mode=None, stream=None,
                  phase_events=None, kernel_events=None,
                  debug_check_index=False, no_alloc=False):
    """Run MlaPrologV2; kv_cache and kr_cache are updated in place.

    no_alloc: run mla_prolog_v2_no_alloc (the library's fixed per-device
    scratch instead of a workspace; `workspace` is ignored).

    debug_check_index: the library copies cache_index to the host first
    (synchronising the stream) and refuses an out-of-range or repeated index
    with QKVNR_ERR_BAD_INDEX before launching anything.

    Returns (query, query_rope), with dequant_scale_q_nope (T, N, 1) after
    them in "full_kv_int8" (int8 query), plus (cq_int8, cq_scale) when
    return_cq_quant is set in a partial- or full-quant mode.  phase_events: optional
    list of recorded torch.cuda.Event(enable_timing=True) objects, recorded
    again by the library at the MLA_PHASES boundaries.
    """
    lib = load_library()
    He = token_x.shape[-1]
    lead = tuple(token_x.shape[:-1])
    T = token_x.numel() // He if He else 0
    N = weight_uk.shape[0]
    Hckv = rmsnorm_gamma_ckv.shape[-1]
    Dr = rope_sin.shape[-1]
    dev = token_x.device
    q8 = quant_mode in ("full_kv_int8", MLA_QUANT["full_kv_int8"])
    if query is None:
        query = torch.empty(lead + (N, Hckv),
                            dtype=torch.int8 if q8 else torch.bfloat16,
                            device=dev)
    if q8 and dequant_scale_q_nope is None:
        dequant_scale_q_nope = torch.empty(lead + (N, 1), dtype=torch.float32,
                                           device=dev)
    if query_rope is None:
        query_rope = torch.empty(lead + (N, Dr), dtype=torch.bfloat16,
                                 device=dev)
    dbg8 = dbgs = None
    if return_cq_quant:
        dbg8 = torch.empty((T, rmsnorm_gamma_cq.shape[-1]), dtype=torch.int8,
                           device=dev)
        dbgs = torch.empty((T,), dtype=torch.float32, device=dev)
    a = mla_prolog_v2_args(
        token_x, weight_dq, weight_uq_qr, weight_uk, weight_dkv_kr,
        rmsnorm_gamma_cq, rmsnorm_gamma_ckv, rope_sin, rope_cos, cache_index,
        kv_cache, kr_cache, query, query_rope, quant_mode=quant_mode,
        weight_layout=weight_layout, rmsnorm_epsilon_cq=rmsnorm_epsilon_cq,
        rmsnorm_epsilon_ckv=rmsnorm_epsilon_ckv,
        dequant_scale_w_uq_qr=dequant_scale_w_uq_qr,
        quant_scale_ckv=quant_scale_ckv, quant_scale_ckr=quant_scale_ckr,
        smooth_scales_cq=smooth_scales_cq, dequant_scale_x=dequant_scale_x,
        dequant_scale_w_dq=dequant_scale_w_dq,
        dequant_scale_w_dkv_kr=dequant_scale_w_dkv_kr,
        dequant_scale_q_nope=dequant_scale_q_nope if q8 else None,
        dbg_cq_int8=dbg8, dbg_cq_scale=dbgs,
        cache_mode=cache_mode,
        B=lead[0] if len(lead) == 2 else None,
        S=lead[1] if len(lead) == 2 else None,
        flags=MLA_FLAG_CHECK_INDEX if debug_check_index else 0)
    _validate_mla(a, dict(
        token_x=token_x, weight_dq=weight_dq, weight_uq_qr=weight_uq_qr,
        weight_uk=weight_uk, weight_dkv_kr=weight_dkv_kr,
        rmsnorm_gamma_cq=rmsnorm_gamma_cq, rmsnorm_gamma_ckv=rmsnorm_gamma_ckv,
        rope_sin=rope_sin, rope_cos=rope_cos, cache_index=cache_index,
        kv_cache=kv_cache, kr_cache=kr_cache, query=query,
        query_rope=query_rope, dequant_scale_w_uq_qr=dequant_scale_w_uq_qr,
        quant_scale_ckv=quant_scale_ckv, quant_scale_ckr=quant_scale_ckr,
        smooth_scales_cq=smooth_scales_cq, dequant_scale_x=dequant_scale_x,
        dequant_scale_w_dq=dequant_scale_w_dq,
        dequant_scale_w_dkv_kr=dequant_scale_w_dkv_kr,
        dequant_scale_q_nope=dequant_scale_q_nope, dbg_cq_int8=dbg8,
        dbg_cq_scale=dbgs))
    if phase_events:
        handles = (_vp * len(phase_events))(*[e.cuda_event for e in phase_events])
        a.phase_events = ctypes.cast(handles, ctypes.POINTER(_vp))
        a.n_phase_events = len(phase_events)
    if kernel_events:
        khandles = (_vp * len(kernel_events))(
            *[e.cuda_event for e in kernel_events])
        a.kernel_events = ctypes.cast(khandles, ctypes.POINTER(_vp))
        a.n_kernel_events = len(kernel_events)
    if no_alloc:
        _check(lib.mla_prolog_v2_no_alloc(ctypes.byref(a), _stream(stream)),
               "mla_prolog_v2_no_alloc")
    else:
        nbytes = mla_prolog_v2_workspace_size(a)
        if workspace is None or \
                workspace.numel() * workspace.element_size() < nbytes:
            workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8,
                                    device=dev)
        _check(lib.mla_prolog_v2(ctypes.byref(a), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(),
                                 _stream(stream)), "mla_prolog_v2")
    out = (query, query_rope) + ((dequant_scale_q_nope,) if q8 else ())
    if return_cq_quant:
        return out + (dbg8, dbgs)
    return out


def mla_prolog_v2_no_alloc(*args, **kw):
    """mla_prolog_v2 through the no-allocation entry point: the workspace is
    the library's fixed per-device scratch (MLA_NO_ALLOC_SCRATCH_BYTES); the
    outputs are allocated here unless passed in (query=, query_rope=)."""
    kw.pop("workspace", None)
    return mla_prolog_v2(*args, no_alloc=True, **kw)


class PreparedMlaPrologV2:
    """One mla_prolog_v2 call with its argument struct and workspace built
    once, for callers that issue the same call repeatedly (serving loops,
    graph capture).  Calling it runs the library on the current stream;
    the tensors passed at construction must stay alive and in place.
    """

    def __init__(self, token_x, weight_dq, weight_uq_qr, weight_uk,
                 weight_dkv_kr, rmsnorm_gamma_cq, rmsnorm_gamma_ckv, rope_sin,
                 rope_cos, cache_index, kv_cache, kr_cache, query, query_rope,
                 workspace=None, **kw):
        self._lib = load_library()
        lead = tuple(token_x.shape[:-1])
        self._keep = (token_x, weight_dq, weight_uq_qr, weight_uk,
                      weight_dkv_kr, rmsnorm_gamma_cq, rmsnorm_gamma_ckv,
                      rope_sin, rope_cos, cache_index, kv_cache, kr_cache,
                      query, query_rope, kw)
        self.args = mla_prolog_v2_args(
            token_x, weight_dq, weight_uq_qr, weight_uk, weight_dkv_kr,
            rmsnorm_gamma_cq, rmsnorm_gamma_ckv, rope_sin, rope_cos,
            cache_index, kv_cache, kr_cache, query, query_rope,
            B=lead[0] if len(lead) == 2 else None,
            S=lead[1] if len(lead) == 2 else None, **kw)
        _validate_mla(self.args, dict(
            kw, token_x=token_x, weight_dq=weight_dq,
            weight_uq_qr=weight_uq_qr, weight_uk=weight_uk,
            weight_dkv_kr=weight_dkv_kr, rmsnorm_gamma_cq=rmsnorm_gamma_cq,
            rmsnorm_gamma_ckv=rmsnorm_gamma_ckv, rope_sin=rope_sin,
            rope_cos=rope_cos, cache_index=cache_index, kv_cache=kv_cache,
            kr_cache=kr_cache, query=query, query_rope=query_rope))
        nbytes = mla_prolog_v2_workspace_size(self.args)
        if workspace is None or \
                workspace.numel() * workspace.element_size() < nbytes:
            workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8,
                                    device=token_x.device)
        self.workspace = workspace
        self._ws = ctypes.c_void_p(_ptr(workspace))
        self._nbytes = workspace.numel() * workspace.element_size()
        self._ref = ctypes.byref(self.args)
        self.query, self.query_rope = query, query_rope

    def __call__(self, stream=None, phase_events=None, kernel_events=None):
        """phase_events: MLA_PHASES events recorded between the launches;
        kernel_events: 2 * len(MLA_KERNELS) events, (start, stop) of each
        main kernel taken at its dispatch.  Either may be a list of
        torch.cuda.Event or of raw hipEvent_t handles (ints)."""
        a = self.args

        def handles_of(evs):
            return (_vp * len(evs))(*[getattr(e, "cuda_event", e) for e in evs])
        if phase_events:
            handles = handles_of(phase_events)
            a.phase_events = ctypes.cast(handles, ctypes.POINTER(_vp))
            a.n_phase_events = len(phase_events)
        else:
            handles = None
            a.n_phase_events = 0
            a.phase_events = None
        if kernel_events:
            khandles = handles_of(kernel_events)
            a.kernel_events = ctypes.cast(khandles, ctypes.POINTER(_vp))
            a.n_kernel_events = len(kernel_events)
        else:
            khandles = None
            a.n_kernel_events = 0
            a.kernel_events = None
        rc = self._lib.mla_prolog_v2(self._ref, self._ws, self._nbytes,
                                     _stream(stream))
        _check(rc, "mla_prolog_v2")
        return self.query, self.query_rope


# ---------------------------------------------------------------------------
# MlaPreprocessV2
# ---------------------------------------------------------------------------

def _validate_pre(a: "MlaPreprocessV2Args", t: dict):
    """Element types and counts of the MlaPreprocessV2 tensors for the
    dimensions in `a` (include/qkvnr.h; packed weights hold whole
    32-column blocks)."""
    T = a.B * a.S
    bf, i8, f32 = torch.bfloat16, torch.int8, torch.float32
    cols = _pad32 if a.weight_layout == MLA_WEIGHT_PACKED_K16 else int
    ntot = a.Hcq + a.Hckv + a.Dr
    slots = a.block_num * a.block_size
    _expect(t.get("token_x"), bf, T * a.He, "token_x")
    _expect(t.get("gamma_x"), bf, a.He, "gamma_x")
    _expect(t.get("bias_x"), f32, a.He, "bias_x")
    _expect(t.get("weight_dqkv"), i8, a.He * cols(ntot), "weight_dqkv")
    _expect(t.get("dequant_scale_dqkv"), f32, ntot, "dequant_scale_dqkv")
    _expect(t.get("gamma_cq"), bf, a.Hcq, "gamma_cq")
    _expect(t.get("bias_cq"), f32, a.Hcq, "bias_cq")
    _expect(t.get("weight_uq_qr"), i8, a.Hcq * cols(a.N * (a.D + a.Dr)),
            "weight_uq_qr")
    _expect(t.get("dequant_scale_uq_qr"), f32, a.N * (a.D + a.Dr),
            "dequant_scale_uq_qr")
    _expect(t.get("weight_uk"), bf, a.N * a.D * cols(a.Hckv), "weight_uk")
    _expect(t.get("gamma_ckv"), bf, a.Hckv, "gamma_ckv")
    _expect(t.get("rope_sin"), bf, T * a.Dr, "rope_sin")
    _expect(t.get("rope_cos"), bf, T * a.Dr, "rope_cos")
    _expect(t.get("cache_index"), torch.int64, T, "cache_index")
    _expect(t.get("kv_cache"), bf, slots * a.Hckv, "kv_cache")
    _expect(t.get("kr_cache"), bf, slots * a.Dr, "kr_cache")
    _expect(t.get("query"), bf, T * a.N * a.Hckv, "query")
    _expect(t.get("query_rope"), bf, T * a.N * a.Dr, "query_rope")
    _expect(t.get("dbg_x_int8"), i8, T * a.He, "x_int8")
    _expect(t.get("dbg_cq_int8"), i8, T * a.Hcq, "cq_int8")


def mla_preprocess_v2(token_x, gamma_x, bias_x, quant_scale_x, weight_dqkv,
                      dequant_scale_dqkv, gamma_cq, bias_cq, quant_scale_cq,
                      weight_uq_qr, dequant_scale_uq_qr, weight_uk, gamma_ckv,
                      rope_sin, rope_cos, cache_index, kv_cache, kr_cache, *,
                      epsilon=1e-6, weight_layout=MLA_WEIGHT_PACKED_K16,
                      query=None, query_rope=None, workspace=None,
                      return_codes=False, debug_check_index=False,
                      cache_mode=None, stream=None):
    """Run MlaPreprocessV2; kv_cache and kr_cache are updated in place.

    token_x (T, He) or (B, S, He) bf16; weight_dqkv (He, Hcq+Hckv+Dr) int8
    (packed with mla_pack_weight unless weight_layout is MLA_WEIGHT_ND);
    weight_uq_qr (Hcq, N*(D+Dr)) int8 (mla_pack_weight_uq_qr); weight_uk
    (N, D, Hckv) bf16 (mla_pack_weight_uk); quant_scale_x / quant_scale_cq
    Python floats.  Returns (query, query_rope), plus the int8 codes of the
    two RmsNormQuant steps, (T, He) and (T, Hcq), when return_codes is set.
    """
    lib = load_library()
    He = token_x.shape[-1]
    lead = tuple(token_x.shape[:-1])
    T = token_x.numel() // He if He else 0
    N, D = weight_uk.shape[0], weight_uk.shape[1]
    Hcq, Hckv = gamma_cq.shape[-1], gamma_ckv.shape[-1]
    Dr = rope_sin.shape[-1]
    dev = token_x.device
    if query is None:
        query = torch.empty(lead + (N, Hckv), dtype=torch.bfloat16, device=dev)
    if query_rope is None:
        query_rope = torch.empty(lead + (N, Dr), dtype=torch.bfloat16,
                                 device=dev)
    dx = dc = None
    if return_codes:
        dx = torch.empty((T, He), dtype=torch.int8, device=dev)
        dc = torch.empty((T, Hcq), dtype=torch.int8, device=dev)
    a = MlaPreprocessV2Args()
    a.struct_size = ctypes.sizeof(MlaPreprocessV2Args)
    a.weight_layout = int(weight_layout)
    a.flags = MLA_FLAG_CHECK_INDEX if debug_check_index else 0
    B, S = (lead[0], lead[1]) if len(lead) == 2 else (T, 1)
    a.B, a.S, a.He, a.Hcq, a.N, a.D = int(B), int(S), int(He), int(Hcq), \
        int(N), int(D)
    a.Hckv, a.Dr = int(Hckv), int(Dr)
    a.block_num, a.block_size = int(kv_cache.shape[0]), int(kv_cache.shape[1])
    a.epsilon = float(epsilon)
    a.quant_scale_x, a.quant_scale_cq = float(quant_scale_x), \
        float(quant_scale_cq)
    a.cache_mode = cache_mode.encode() if cache_mode else None
    if T > 0:
        a.token_x, a.rope_sin, a.rope_cos = _ptr(token_x), _ptr(rope_sin), \
            _ptr(rope_cos)
        a.cache_index, a.query = _ptr(cache_index), _ptr(query)
        a.query_rope = _ptr(query_rope)
        a.dbg_x_int8, a.dbg_cq_int8 = _ptr(dx), _ptr(dc)
    a.gamma_x, a.bias_x = _ptr(gamma_x), _ptr(bias_x)
    a.weight_dqkv, a.dequant_scale_dqkv = _ptr(weight_dqkv), \
        _ptr(dequant_scale_dqkv)
    a.gamma_cq, a.bias_cq = _ptr(gamma_cq), _ptr(bias_cq)
    a.weight_uq_qr, a.dequant_scale_uq_qr = _ptr(weight_uq_qr), \
        _ptr(dequant_scale_uq_qr)
    a.weight_uk, a.gamma_ckv = _ptr(weight_uk), _ptr(gamma_ckv)
    if kv_cache.numel():
        a.kv_cache = _ptr(kv_cache)
    if kr_cache.numel():
        a.kr_cache = _ptr(kr_cache)
    _validate_pre(a, dict(
        token_x=token_x, gamma_x=gamma_x, bias_x=bias_x,
        weight_dqkv=weight_dqkv, dequant_scale_dqkv=dequant_scale_dqkv,
        gamma_cq=gamma_cq, bias_cq=bias_cq, weight_uq_qr=weight_uq_qr,
        dequant_scale_uq_qr=dequant_scale_uq_qr, weight_uk=weight_uk,
        gamma_ckv=gamma_ckv, rope_sin=rope_sin, rope_cos=rope_cos,
        cache_index=cache_index, kv_cache=kv_cache, kr_cache=kr_cache,
        query=query, query_rope=query_rope, dbg_x_int8=dx, dbg_cq_int8=dc))
    n = ctypes.c_size_t(0)
    _check(lib.mla_preprocess_v2_workspace_size(ctypes.byref(a),
                                                 ctypes.byref(n)),
           "mla_preprocess_v2_workspace_size")
    if workspace is None or \
            workspace.numel() * workspace.element_size() < n.value:
        workspace = torch.empty(max(n.value, 1), dtype=torch.uint8, device=dev)
    _check(lib.mla_preprocess_v2(ctypes.byref(a), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(),
                                 _stream(stream)), "mla_preprocess_v2")
    if return_codes:
        return query, query_rope, dx, dc
    return query, query_rope


# ---------------------------------------------------------------------------
# QkvRmsNormRopeCache
# ---------------------------------------------------------------------------

def qkv_rmsnorm_rope_cache_args(qkv, gamma_q, gamma_k, cos, sin, index,
                                k_cache, v_cache, q_out, *, Nq, Nk, Nv,
                                quant_mode="symmetric", epsilon=1e-6,
                                k_scale=None, v_scale=None, k_offset=None,
                                v_offset=None, q_before_quant=None,
                                k_before_quant=None, v_before_quant=None,
                                B=None, S=None, cache_mode=None, flags=0):
    a = QkvRmsNormRopeCacheArgs()
    a.struct_size = ctypes.sizeof(QkvRmsNormRopeCacheArgs)
    a.flags = int(flags)
    a.quant_mode = QKV_QUANT[quant_mode] if isinstance(quant_mode, str) \
        else int(quant_mode)
    a.dtype = QKV_DTYPE.get(qkv.dtype, -1)
    D = qkv.shape[-1] if qkv.dim() >= 1 else 0
    T = index.numel()
    if B is None:
        B, S = T, 1
    a.B, a.S = int(B), int(S)
    a.Nq, a.Nk, a.Nv, a.D = int(Nq), int(Nk), int(Nv), int(D)
    a.block_num, a.block_size = int(k_cache.shape[0]), int(k_cache.shape[1])
    a.epsilon = float(epsilon)
    a.cache_mode = cache_mode.encode() if cache_mode else None
    if T > 0:
        a.qkv, a.cos, a.sin, a.index = _ptr(qkv), _ptr(cos), _ptr(sin), \
            _ptr(index)
        a.q_out = _ptr(q_out)
        a.q_before_quant = _ptr(q_before_quant)
        a.k_before_quant = _ptr(k_before_quant)
        a.v_before_quant = _ptr(v_before_quant)
    a.gamma_q, a.gamma_k = _ptr(gamma_q), _ptr(gamma_k)
    a.k_cache, a.v_cache = _ptr(k_cache), _ptr(v_cache)
    a.k_scale, a.v_scale = _ptr(k_scale), _ptr(v_scale)
    a.k_offset, a.v_offset = _ptr(k_offset), _ptr(v_offset)
    return a


def qkv_rmsnorm_rope_cache(qkv, gamma_q, gamma_k, cos, sin, index, k_cache,
                           v_cache, *, Nq, Nk, Nv, quant_mode="symmetric",
                           epsilon=1e-6, k_scale=None, v_scale=None,
                           k_offset=None, v_offset=None, q_out=None,
                           before_quant=False, B=None, S=None,
                           cache_mode=None, stream=None,
                           debug_check_inputs=False):
    """Run QkvRmsNormRopeCache; k_cache and v_cache are updated in place.

    debug_check_inputs: the library copies the index (and the quant scales)
    to the host first, synchronising the stream, and refuses an
    out-of-range or repeated index (QKVNR_ERR_BAD_INDEX) or a zero scale
    (QKVNR_ERR_BAD_SCALE) before launching anything.

    qkv: (T, Nq+Nk+Nv, D) or (B, S, (Nq+Nk+Nv)*D).  Returns q_out (T, Nq, D),
    plus (q_before_quant, k_before_quant, v_before_quant) when
    before_quant is set.
    """
    lib = load_library()
    T = index.numel()
    D = qkv.shape[-1] if qkv.dim() == 3 and qkv.shape[1] == Nq + Nk + Nv \
        else qkv.shape[-1] // (Nq + Nk + Nv)
    dev = qkv.device
    if q_out is None:
        q_out = torch.empty((T, Nq, D), dtype=qkv.dtype, device=dev)
    qb = kb = vb = None
    if before_quant:
        qb = torch.empty((T, Nq, D), dtype=qkv.dtype, device=dev)
        kb = torch.empty((T, Nk, D), dtype=qkv.dtype, device=dev)
        vb = torch.empty((T, Nv, D), dtype=qkv.dtype, device=dev)
    qkv3 = qkv.reshape(T, Nq + Nk + Nv, D) if T else qkv
    a = qkv_rmsnorm_rope_cache_args(
        qkv3, gamma_q, gamma_k, cos, sin, index, k_cache, v_cache, q_out,
        Nq=Nq, Nk=Nk, Nv=Nv, quant_mode=quant_mode, epsilon=epsilon,
        k_scale=k_scale, v_scale=v_scale, k_offset=k_offset,
        v_offset=v_offset, q_before_quant=qb, k_before_quant=kb,
        v_before_quant=vb, B=B, S=S, cache_mode=cache_mode,
        flags=QKV_FLAG_CHECK_INPUTS if debug_check_inputs else 0)
    a.D = int(D)
    _validate_qkv(a, dict(
        qkv=qkv3, gamma_q=gamma_q, gamma_k=gamma_k, cos=cos, sin=sin,
        index=index, k_cache=k_cache, v_cache=v_cache, q_out=q_out,
        q_before_quant=qb, k_before_quant=kb, v_before_quant=vb,
        k_scale=k_scale, v_scale=v_scale, k_offset=k_offset,
        v_offset=v_offset))
    _check(lib.qkv_rmsnorm_rope_cache(ctypes.byref(a), _stream(stream)),
           "qkv_rmsnorm_rope_cache")
    if before_quant:
        return q_out, qb, kb, vb
    return q_out
