// C ABI of the library: argument validation (host only, no HIP calls),
// workspace sizing and dispatch to the kernel launchers.
#include <math.h>
#include <string.h>

#include "launch.h"

namespace {

using namespace qkvnr;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned8(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 7u) == 0; }

bool good_eps(double e) { return isfinite(e) && e >= 0.0; }

// NULL, "" and "PA_ND" name the row-major paged cache the kernels write.
// "PA_NZ" (the pages' blocked cache layout) is valid on the pages but not
// built here; anything else is an unknown mode.
int check_cache_mode(const char* m) {
  if (m == nullptr || m[0] == '\0' || strcmp(m, "PA_ND") == 0) return QKVNR_OK;
  if (strcmp(m, "PA_NZ") == 0) return QKVNR_ERR_UNSUPPORTED;
  return QKVNR_ERR_BAD_MODE;
}

constexpr int64_t kDimCap = int64_t(1) << 30;
constexpr int64_t kKCap = int64_t(1) << 22;

// The packers' bounds: batch (or heads) <= 65535, each dim <= 2^30 and at
// most 2^46 packed elements, so no size product below overflows int64.
bool pack_dims_ok(int64_t batch, int64_t K, int64_t N) {
  if (batch < 0 || K < 0 || N < 0 || batch > 65535 || K > kDimCap || N > kDimCap) return false;
  const int64_t per = K * ((N + 31) / 32) * 32;  // < 2^61
  return batch == 0 || per <= (int64_t(1) << 46) / batch;
}

int validate_mla(const MlaPrologV2Args* a) {
  if (a == nullptr) return QKVNR_ERR_NULL_ARG;
  if (a->struct_size != sizeof(MlaPrologV2Args) || a->reserved0 != 0) return QKVNR_ERR_BAD_STRUCT;
  if (a->n_phase_events < 0 || (a->n_phase_events > 0 && a->phase_events == nullptr))
    return QKVNR_ERR_NULL_ARG;
  if (a->n_kernel_events < 0 || (a->n_kernel_events > 0 && a->kernel_events == nullptr))
    return QKVNR_ERR_NULL_ARG;
  if (a->quant_mode < MLA_QUANT_NONE || a->quant_mode > MLA_QUANT_FULL_KV_INT8)
    return QKVNR_ERR_BAD_MODE;
  if (a->weight_layout != MLA_WEIGHT_ND && a->weight_layout != MLA_WEIGHT_PACKED_K16)
    return QKVNR_ERR_BAD_MODE;
  int rc = check_cache_mode(a->cache_mode);
  if (rc != QKVNR_OK) return rc;

  // Shapes (MlaPrologV2 README, constraints: B, S, T may be 0; the other
  // dims are positive).
  if (a->B < 0 || a->S < 0 || a->block_num < 0 || a->block_size < 0) return QKVNR_ERR_BAD_SHAPE;
  if (a->He <= 0 || a->Hcq <= 0 || a->N <= 0 || a->D <= 0 || a->Hckv <= 0 || a->Dr <= 0 ||
      a->Nkv <= 0)
    return QKVNR_ERR_BAD_SHAPE;
  if (a->He > kDimCap || a->Hcq > kDimCap || a->N > 65535 || a->D > kDimCap ||
      a->Hckv > kDimCap || a->Dr > kDimCap || a->B > kDimCap || a->S > kDimCap ||
      a->block_num > kDimCap || a->block_size > kDimCap)
    return QKVNR_ERR_BAD_SHAPE;
  if (a->Dr % 2 != 0) return QKVNR_ERR_BAD_SHAPE;  // RoPE pairs halves
  const int64_t T = a->B * a->S;
  if (T > (int64_t(1) << 23)) return QKVNR_ERR_BAD_SHAPE;
  // Limits of the kernels built here.
  if (a->Nkv != 1) return QKVNR_ERR_UNSUPPORTED;
  const bool quant = a->quant_mode != MLA_QUANT_NONE;
  const bool full =
      a->quant_mode == MLA_QUANT_FULL_KV_BF16 || a->quant_mode == MLA_QUANT_FULL_KV_INT8;
  const bool kv8 =
      a->quant_mode == MLA_QUANT_PARTIAL_KV_INT8 || a->quant_mode == MLA_QUANT_FULL_KV_INT8;
  if (a->He % (full ? 64 : 32) || a->Hcq % (quant ? 64 : 32) || a->D % 32 || a->Hckv % 16)
    return QKVNR_ERR_UNSUPPORTED;
  if (!(a->Dr == 16 || a->Dr == 32 || a->Dr == 64) || (a->N * a->D) % a->Dr != 0)
    return QKVNR_ERR_UNSUPPORTED;
  if ((a->Hcq + a->Hckv + a->Dr) * 4 > 64 * 1024) return QKVNR_ERR_UNSUPPORTED;
  // GEMM K dims: the weight-streaming kernels address one column block's
  // run and one A operand with 32-bit buffer offsets.
  if (a->He > kKCap || a->Hcq > kKCap || a->D > kKCap) return QKVNR_ERR_UNSUPPORTED;
  // Output column indexes are 32-bit in the epilogues.
  if (a->N * (a->D + a->Dr) >= (int64_t(1) << 31)) return QKVNR_ERR_UNSUPPORTED;
  if (!good_eps(a->rmsnorm_epsilon_cq) || !good_eps(a->rmsnorm_epsilon_ckv))
    return QKVNR_ERR_BAD_EPS;

  // Parameters a scenario does not use (README dtype/shape table: "no
  // value needed") must be NULL: the x and down-projection dequant scales
  // outside full quantisation, the query's dequant scale outside
  // FULL_KV_INT8, the cache quant scales where the caches are bf16, and
  // the kr_cache scale in full quantisation (its kr_cache stays bf16).
  if (!full && (a->dequant_scale_x || a->dequant_scale_w_dq || a->dequant_scale_w_dkv_kr))
    return QKVNR_ERR_RESERVED_NONNULL;
  if (a->quant_mode != MLA_QUANT_FULL_KV_INT8 && a->dequant_scale_q_nope)
    return QKVNR_ERR_RESERVED_NONNULL;
  if ((!kv8 && a->quant_scale_ckv) || (full && a->quant_scale_ckr))
    return QKVNR_ERR_RESERVED_NONNULL;

  if (T == 0) return QKVNR_OK;  // empty tensors are allowed; nothing runs
  const void* need[] = {a->token_x,   a->weight_dq,       a->weight_uq_qr,      a->weight_uk,
                        a->weight_dkv_kr, a->rmsnorm_gamma_cq, a->rmsnorm_gamma_ckv, a->rope_sin,
                        a->rope_cos,  a->cache_index,     a->query,             a->query_rope};
  for (const void* p : need)
    if (p == nullptr) return QKVNR_ERR_NULL_ARG;
  const bool slots = a->block_num * a->block_size > 0;
  if (slots && (a->kv_cache == nullptr || a->kr_cache == nullptr)) return QKVNR_ERR_NULL_ARG;
  if (quant && (a->dequant_scale_w_uq_qr == nullptr || a->smooth_scales_cq == nullptr))
    return QKVNR_ERR_NULL_ARG;
  if (a->quant_mode == MLA_QUANT_PARTIAL_KV_INT8 &&
      (a->quant_scale_ckv == nullptr || a->quant_scale_ckr == nullptr))
    return QKVNR_ERR_NULL_ARG;
  if (full && (a->dequant_scale_x == nullptr || a->dequant_scale_w_dq == nullptr ||
               a->dequant_scale_w_dkv_kr == nullptr))
    return QKVNR_ERR_NULL_ARG;
  if (a->quant_mode == MLA_QUANT_FULL_KV_INT8 &&
      (a->quant_scale_ckv == nullptr || a->dequant_scale_q_nope == nullptr))
    return QKVNR_ERR_NULL_ARG;

  const void* al16[] = {a->token_x,   a->weight_dq,       a->weight_uq_qr,      a->weight_uk,
                        a->weight_dkv_kr, a->rmsnorm_gamma_cq, a->rmsnorm_gamma_ckv, a->rope_sin,
                        a->rope_cos,  a->query,           a->query_rope};
  for (const void* p : al16)
    if (!aligned16(p)) return QKVNR_ERR_BAD_ALIGNMENT;
  if (!aligned8(a->cache_index)) return QKVNR_ERR_BAD_ALIGNMENT;
  if (quant && (!aligned16(a->dequant_scale_w_uq_qr) || !aligned16(a->smooth_scales_cq)))
    return QKVNR_ERR_BAD_ALIGNMENT;
  if (slots && (!aligned16(a->kv_cache) || !aligned16(a->kr_cache))) return QKVNR_ERR_BAD_ALIGNMENT;
  if (a->quant_mode == MLA_QUANT_PARTIAL_KV_INT8 &&
      (!aligned16(a->quant_scale_ckv) || !aligned16(a->quant_scale_ckr)))
    return QKVNR_ERR_BAD_ALIGNMENT;
  if (full && ((reinterpret_cast<uintptr_t>(a->dequant_scale_x) & 3u) ||
               !aligned16(a->dequant_scale_w_dq) ||
               !aligned16(a->dequant_scale_w_dkv_kr)))
    return QKVNR_ERR_BAD_ALIGNMENT;
  if (a->quant_mode == MLA_QUANT_FULL_KV_INT8 &&
      (!aligned16(a->quant_scale_ckv) || (reinterpret_cast<uintptr_t>(a->dequant_scale_q_nope) & 3u)))
    return QKVNR_ERR_BAD_ALIGNMENT;
  if ((a->dbg_cq_int8 && !aligned8(a->dbg_cq_int8)) ||
      (a->dbg_cq_scale && (reinterpret_cast<uintptr_t>(a->dbg_cq_scale) & 3u)))
    return QKVNR_ERR_BAD_ALIGNMENT;
  return QKVNR_OK;
}

int validate_qkv(const QkvRmsNormRopeCacheArgs* a) {
  if (a == nullptr) return QKVNR_ERR_NULL_ARG;
  if (a->struct_size != sizeof(QkvRmsNormRopeCacheArgs) || a->reserved0 != 0)
    return QKVNR_ERR_BAD_STRUCT;
  if (a->quant_mode < QKV_QUANT_NONE || a->quant_mode > QKV_QUANT_ASYMMETRIC)
    return QKVNR_ERR_BAD_MODE;
  if (a->dtype != QKV_DTYPE_FP16 && a->dtype != QKV_DTYPE_BF16) return QKVNR_ERR_BAD_MODE;
  int rc = check_cache_mode(a->cache_mode);
  if (rc != QKVNR_OK) return rc;
  // aclnnQkvRmsNormRopeCache, input shape restrictions: Nk == Nv, D even and
  // (only 128 supported) D == 128.
  if (a->B < 0 || a->S < 0 || a->Nq < 1 || a->Nk < 1 || a->Nv < 1 || a->D < 1 ||
      a->block_num < 0 || a->block_size < 0)
    return QKVNR_ERR_BAD_SHAPE;
  if (a->B > kDimCap || a->S > kDimCap || a->Nq > 4096 || a->Nk > 4096 || a->Nv > 4096 ||
      a->block_num > kDimCap || a->block_size > kDimCap)
    return QKVNR_ERR_BAD_SHAPE;
  if (a->Nk != a->Nv || a->D % 2 != 0) return QKVNR_ERR_BAD_SHAPE;
  if (a->D != 128) return QKVNR_ERR_UNSUPPORTED;
  if (!good_eps(a->epsilon)) return QKVNR_ERR_BAD_EPS;
  const int64_t T = a->B * a->S;
  if (T > (int64_t(1) << 31)) return QKVNR_ERR_BAD_SHAPE;
  if (T == 0) return QKVNR_OK;
  // BlockNum >= ceil(S / BlockSize) * B
  if (a->block_size == 0) return QKVNR_ERR_BAD_SHAPE;
  if (a->block_num < ((a->S + a->block_size - 1) / a->block_size) * a->B)
    return QKVNR_ERR_BAD_SHAPE;
  const void* need[] = {a->qkv,     a->gamma_q, a->gamma_k, a->cos,  a->sin,
                        a->index,   a->k_cache, a->v_cache, a->q_out};
  for (const void* p : need)
    if (p == nullptr) return QKVNR_ERR_NULL_ARG;
  const bool q = a->quant_mode != QKV_QUANT_NONE;
  if (q && (a->k_scale == nullptr || a->v_scale == nullptr)) return QKVNR_ERR_NULL_ARG;
  if (a->quant_mode == QKV_QUANT_ASYMMETRIC && (a->k_offset == nullptr || a->v_offset == nullptr))
    return QKVNR_ERR_NULL_ARG;
  const void* al16[] = {a->qkv, a->gamma_q, a->gamma_k, a->cos,
                        a->sin, a->k_cache, a->v_cache, a->q_out};
  for (const void* p : al16)
    if (!aligned16(p)) return QKVNR_ERR_BAD_ALIGNMENT;
  const void* opt16[] = {a->q_before_quant, a->k_before_quant, a->v_before_quant,
                         q ? a->k_scale : nullptr, q ? a->v_scale : nullptr,
                         a->quant_mode == QKV_QUANT_ASYMMETRIC ? a->k_offset : nullptr,
                         a->quant_mode == QKV_QUANT_ASYMMETRIC ? a->v_offset : nullptr};
  for (const void* p : opt16)
    if (p && !aligned16(p)) return QKVNR_ERR_BAD_ALIGNMENT;
  if (!aligned8(a->index)) return QKVNR_ERR_BAD_ALIGNMENT;
  return QKVNR_OK;
}

}  // namespace

extern "C" {

const char* qkvnr_status_string(int s) {
  switch (s) {
    case QKVNR_OK: return "ok";
    case QKVNR_ERR_NULL_ARG: return "a required pointer is NULL";
    case QKVNR_ERR_BAD_SHAPE: return "bad shape";
    case QKVNR_ERR_BAD_MODE: return "unknown quant mode, dtype, layout or cache mode";
    case QKVNR_ERR_UNSUPPORTED: return "unsupported configuration";
    case QKVNR_ERR_RESERVED_NONNULL: return "a reserved pointer is not NULL";
    case QKVNR_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case QKVNR_ERR_BAD_EPS: return "epsilon must be finite and >= 0";
    case QKVNR_ERR_BAD_STRUCT: return "argument struct size mismatch";
    case QKVNR_ERR_BAD_ALIGNMENT: return "pointer not 16-byte aligned";
    case QKVNR_ERR_LAUNCH_FAILED: return "kernel launch failed";
    case QKVNR_ERR_BAD_INDEX: return "cache index out of range or repeated";
    default: return "unknown status";
  }
}

const char* qkvnr_version(void) { return QKVNR_VERSION_STRING; }

int mla_prolog_v2_validate(const MlaPrologV2Args* args) { return validate_mla(args); }

int mla_prolog_v2_workspace_size(const MlaPrologV2Args* args, size_t* bytes) {
  if (bytes == nullptr) return QKVNR_ERR_NULL_ARG;
  *bytes = 0;
  const int rc = validate_mla(args);
  if (rc != QKVNR_OK) return rc;
  *bytes = make_mla_plan(args).total;
  return QKVNR_OK;
}

int mla_prolog_v2(const MlaPrologV2Args* args, void* workspace, size_t workspace_bytes,
                  void* stream) {
  const int rc = validate_mla(args);
  if (rc != QKVNR_OK) return rc;
  if (args->B * args->S == 0) return QKVNR_OK;
  const MlaPlan plan = make_mla_plan(args);
  if (workspace_bytes < plan.total) return QKVNR_ERR_WORKSPACE_TOO_SMALL;
  if (plan.total > 0 && workspace == nullptr) return QKVNR_ERR_NULL_ARG;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return QKVNR_ERR_BAD_ALIGNMENT;
  return launch_mla_prolog_v2(args, plan, workspace, static_cast<hipStream_t>(stream));
}

int mla_pack_weight(const void* src, void* dst, int64_t batch, int64_t K, int64_t N,
                    int32_t elem_bytes, void* stream) {
  if (elem_bytes != 1 && elem_bytes != 2) return QKVNR_ERR_BAD_MODE;
  if (!pack_dims_ok(batch, K, N) || K % (16 / elem_bytes) != 0) return QKVNR_ERR_BAD_SHAPE;
  if (batch * K * N == 0) return QKVNR_OK;
  if (src == nullptr || dst == nullptr) return QKVNR_ERR_NULL_ARG;
  if (!aligned16(dst) || (elem_bytes == 2 && (reinterpret_cast<uintptr_t>(src) & 1u)))
    return QKVNR_ERR_BAD_ALIGNMENT;
  return launch_pack_weight(src, dst, batch, K, N, elem_bytes, N, 0,
                            static_cast<hipStream_t>(stream));
}

int mla_pack_weight_uk(const void* src, void* dst, int64_t N, int64_t D, int64_t Hckv,
                       void* stream) {
  if (!pack_dims_ok(N, D, Hckv) || D % 16 != 0) return QKVNR_ERR_BAD_SHAPE;
  if (N * D * Hckv == 0) return QKVNR_OK;
  if (src == nullptr || dst == nullptr) return QKVNR_ERR_NULL_ARG;
  if (!aligned16(dst) || (reinterpret_cast<uintptr_t>(src) & 1u)) return QKVNR_ERR_BAD_ALIGNMENT;
  return launch_pack_weight(src, dst, N, D, Hckv, 2, Hckv, 0, static_cast<hipStream_t>(stream),
                            /*kperm=*/true);
}

int mla_pack_weight_uq_qr(const void* src, void* dst, int64_t Hcq, int64_t N, int64_t D,
                          int64_t Dr, int32_t elem_bytes, void* stream) {
  if (elem_bytes != 1 && elem_bytes != 2) return QKVNR_ERR_BAD_MODE;
  if (Hcq < 0 || N < 0 || D < 0 || Dr < 0 || Hcq > kDimCap || N > 65535 || D > kDimCap ||
      Dr > kDimCap || !pack_dims_ok(1, Hcq, N * (D + Dr)) || Hcq % (16 / elem_bytes) != 0)
    return QKVNR_ERR_BAD_SHAPE;
  if (Hcq * N == 0) return QKVNR_OK;
  if (D % 32 != 0 || !(Dr == 16 || Dr == 32 || Dr == 64)) return QKVNR_ERR_UNSUPPORTED;
  if (src == nullptr || dst == nullptr) return QKVNR_ERR_NULL_ARG;
  if (!aligned16(dst) || (elem_bytes == 2 && (reinterpret_cast<uintptr_t>(src) & 1u)))
    return QKVNR_ERR_BAD_ALIGNMENT;
  return launch_pack_weight(src, dst, 1, Hcq, N * (D + Dr), elem_bytes, N * D, Dr,
                            static_cast<hipStream_t>(stream));
}

int qkv_rmsnorm_rope_cache_validate(const QkvRmsNormRopeCacheArgs* args) {
  return validate_qkv(args);
}

int qkv_rmsnorm_rope_cache(const QkvRmsNormRopeCacheArgs* args, void* stream) {
  const int rc = validate_qkv(args);
  if (rc != QKVNR_OK) return rc;
  return launch_qkv_rmsnorm_rope_cache(args, static_cast<hipStream_t>(stream));
}

}  // extern "C"
