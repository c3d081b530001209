// C ABI of the library (include/qkvnr.h): argument validation, the
// execution plan and workspace sizing, the host debug checks, and dispatch
// to the HIP launchers.  Plain C++ with no HIP dependency, so the whole
// host side can also be built and tested under the address and
// undefined-behaviour sanitizers without a GPU.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "launch.h"

namespace qkvnr {

namespace {
size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }
}  // namespace

MlaPlan make_mla_plan(const MlaPrologV2Args* a) {
  MlaPlan pl{};
  const int64_t T = a->B * a->S;
  const bool quant = a->quant_mode != MLA_QUANT_NONE;
  const bool xq = a->quant_mode == MLA_QUANT_FULL_KV_BF16 || a->quant_mode == MLA_QUANT_FULL_KV_INT8;
  const int64_t ntot = a->Hcq + a->Hckv + a->Dr;
  pl.skinny = T <= 128;
  pl.gemm256 = !pl.skinny;
  pl.mb = T <= 32 ? 1 : (T <= 64 ? 2 : 4);
  // k-steps of the down projection: 16 k (bf16) or 32 k (int8 x)
  const int64_t steps = a->He / (xq ? 32 : 16);
  if (pl.gemm256) {
    // Split the down projection over K so that its 256x256 tiles (one
    // workgroup per CU) times the splits fill whole rounds of the 256 CUs
    // best: minimise ceil(tiles * ks / 256) / ks over ks <= 4 (more splits
    // cost partial-sum traffic), with steps per split even (32-k pipeline
    // stages).
    const int64_t tiles = (T + 255) / 256 *
                          ((a->Hcq + G_TN - 1) / G_TN + (a->Hckv + a->Dr + G_TN - 1) / G_TN);
    int64_t best = 1;
    double best_cost = 1e30;
    for (int64_t ks = 1; ks <= 4; ++ks) {
      const double cost = static_cast<double>((tiles * ks + 255) / 256) / static_cast<double>(ks);
      if (cost < best_cost - 1e-9) {
        best_cost = cost;
        best = ks;
      }
    }
    int64_t sps = (steps + best - 1) / best;
    sps += sps & 1;
    pl.steps_per_split = sps;
    pl.ksplit = static_cast<int>((steps + sps - 1) / sps);
  } else if (pl.skinny) {
    // Split the down projection over K so that (64-column tiles x splits)
    // stays within one wave of workgroups over the 256 CUs (no tail round),
    // at most FIN_MAXSPLIT splits (the finish kernel sums them) and at least
    // one k-step per wave.
    const int kw = pl.mb >= 4 ? 2 : (pl.mb == 2 ? 4 : 8);
    const int64_t ntiles = (a->Hcq + kA1Cols - 1) / kA1Cols + (a->Hckv + a->Dr + kA1Cols - 1) / kA1Cols;
    int64_t ks = 256 / (ntiles > 0 ? ntiles : 1);
    if (ks > FIN_MAXSPLIT) ks = FIN_MAXSPLIT;
    if (ks > steps / kw) ks = steps / kw;
    if (ks < 1) ks = 1;
    pl.steps_per_split = (steps + ks - 1) / ks;
    pl.ksplit = static_cast<int>((steps + pl.steps_per_split - 1) / pl.steps_per_split);
  } else {
    pl.steps_per_split = steps;
    pl.ksplit = 1;
  }
  pl.rows = pl.skinny ? 32 * pl.mb : (pl.gemm256 ? (T + 31) / 32 * 32 : T);
  // Prefill fuses the W^UK product into the q^C tiles of A6 when a wave's
  // 128 q^C columns are exactly one head (D = 128) and the q^C columns end
  // on a tile boundary.
  // (FULL_KV_INT8 keeps the unfused path: its query quant needs q^N in fp32)
  pl.fuse_uk = pl.gemm256 && a->quant_mode != MLA_QUANT_FULL_KV_INT8 && a->D == 128 &&
               (a->N * a->D) % G_TN == 0;
  // Decode with one row block in bf16 runs the up projection and the W^UK
  // product as one launch when a head's q^C and W^UK slices fit a wave's
  // registers (D <= 128).
  pl.merge_uk = pl.skinny && pl.mb == 1 && !quant && a->D <= 128;
  // The quantised scenarios with a bf16 query (T <= 64) when their up
  // projection runs on 32-column tiles (fewer than 128 of the 96-column
  // ones: few heads) and a head's q^C is whole 32-column k-steps (D a
  // multiple of 32 up to 128).
  pl.merge_uk_q = pl.skinny && pl.mb <= 2 && quant &&
                  a->quant_mode != MLA_QUANT_FULL_KV_INT8 && a->D % 32 == 0 && a->D <= 128 &&
                  (a->N * (a->D + a->Dr) + 95) / 96 < 128;
  // FULL_KV_INT8 decode with one row block quantises the query in the W^UK
  // product's epilogue when a head's Hckv fits one tile of at most 16 waves;
  // otherwise q^N goes out in fp32 for a separate quant kernel.
  pl.qh = pl.skinny && pl.mb == 1 && a->quant_mode == MLA_QUANT_FULL_KV_INT8 && a->Hckv <= 512;
  size_t off = 0;
  if (a->weight_layout == MLA_WEIGHT_ND) {
    // packed copies: columns padded to whole 32-column blocks
    const size_t eb_uq = quant ? 1 : 2;
    auto pad32 = [](int64_t n) { return static_cast<size_t>((n + 31) / 32 * 32); };
    pl.off_wdq = off;
    off += align256(static_cast<size_t>(a->He) * pad32(a->Hcq) * (xq ? 1 : 2));
    pl.off_wdkvkr = off;
    off += align256(static_cast<size_t>(a->He) * pad32(a->Hckv + a->Dr) * (xq ? 1 : 2));
    pl.off_wuqqr = off;
    off += align256(static_cast<size_t>(a->Hcq) * pad32(a->N * (a->D + a->Dr)) * eb_uq);
    pl.off_wuk = off;
    off += align256(static_cast<size_t>(a->N * a->D) * pad32(a->Hckv) * 2);
  }
  pl.off_part = off;
  off += align256(static_cast<size_t>(pl.ksplit) * T * ntot * 4);
  pl.off_cq = off;
  off += align256(static_cast<size_t>(pl.rows * a->Hcq) * (quant ? 1 : 2));
  pl.off_cq_scale = off;
  off += align256(static_cast<size_t>(T) * 4);
  pl.off_qc = off;
  off += align256(static_cast<size_t>(pl.rows * a->N * a->D) * (quant ? 4 : 2));
  pl.off_qn = off;
  if (a->quant_mode == MLA_QUANT_FULL_KV_INT8 && !pl.qh)
    off += align256(static_cast<size_t>(T * a->N * a->Hckv) * sizeof(float));
  pl.off_xfrag = off;
  if (pl.gemm256) off += align256(static_cast<size_t>(pl.rows * a->He) * 2);
  pl.off_sync = off;
  if (pl.merge_uk || pl.merge_uk_q) off += static_cast<size_t>(a->N) * SYNC_STRIDE * 4;
  pl.total = T > 0 ? off : 0;
  return pl;
}

MlaPlan make_preprocess_plan(const MlaPrologV2Args* m) {
  MlaPlan pl = make_mla_plan(m);
  const int64_t T = m->B * m->S;
  if (T == 0) return pl;
  size_t off = pl.total;
  pl.off_prex8 = off;
  off += align256(static_cast<size_t>(T) * static_cast<size_t>(m->He));
  pl.off_presx = off;
  off += align256(static_cast<size_t>(T) * sizeof(float));
  pl.total = off;
  return pl;
}

}  // namespace qkvnr

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
  if (a->struct_size != sizeof(MlaPrologV2Args)) return QKVNR_ERR_BAD_STRUCT;
  if (a->flags & ~MLA_FLAG_CHECK_INDEX) return QKVNR_ERR_BAD_MODE;
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
  if (a->struct_size != sizeof(QkvRmsNormRopeCacheArgs)) return QKVNR_ERR_BAD_STRUCT;
  if (a->flags & ~QKV_FLAG_CHECK_INPUTS) return QKVNR_ERR_BAD_MODE;
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


// MlaPreprocessV2 as the equivalent prolog arguments: full quantisation
// with bf16 caches, W^DQKV as weight_dq (the launcher splits it), the c^Q
// bias in smooth_scales_cq, and placeholders (never read) where the
// launcher substitutes workspace regions (x's codes and their unit token
// scales).
MlaPrologV2Args preprocess_as_prolog(const MlaPreprocessV2Args* a) {
  MlaPrologV2Args m{};
  m.struct_size = sizeof(MlaPrologV2Args);
  m.quant_mode = MLA_QUANT_FULL_KV_BF16;
  m.weight_layout = a->weight_layout;
  m.flags = a->flags;
  m.B = a->B;
  m.S = a->S;
  m.He = a->He;
  m.Hcq = a->Hcq;
  m.N = a->N;
  m.D = a->D;
  m.Hckv = a->Hckv;
  m.Dr = a->Dr;
  m.Nkv = 1;
  m.block_num = a->block_num;
  m.block_size = a->block_size;
  m.rmsnorm_epsilon_cq = a->epsilon;
  m.rmsnorm_epsilon_ckv = a->epsilon;
  m.cache_mode = a->cache_mode;
  m.token_x = a->token_x;
  m.weight_dq = a->weight_dqkv;
  m.weight_dkv_kr = a->weight_dqkv;
  m.weight_uq_qr = a->weight_uq_qr;
  m.weight_uk = a->weight_uk;
  m.rmsnorm_gamma_cq = a->gamma_cq;
  m.rmsnorm_gamma_ckv = a->gamma_ckv;
  m.rope_sin = a->rope_sin;
  m.rope_cos = a->rope_cos;
  m.cache_index = a->cache_index;
  m.dequant_scale_x = a->dequant_scale_dqkv;  // placeholder: unit scales
  m.dequant_scale_w_dq = a->dequant_scale_dqkv;
  // the W^DKV | W^KR part of the scales (an out-of-range Hcq is refused by
  // the validation; the pointer is then not formed)
  m.dequant_scale_w_dkv_kr = a->dequant_scale_dqkv != nullptr && a->Hcq > 0 && a->Hcq <= kDimCap
                                 ? a->dequant_scale_dqkv + a->Hcq
                                 : a->dequant_scale_dqkv;
  m.dequant_scale_w_uq_qr = a->dequant_scale_uq_qr;
  m.smooth_scales_cq = a->bias_cq;
  m.kv_cache = a->kv_cache;
  m.kr_cache = a->kr_cache;
  m.query = a->query;
  m.query_rope = a->query_rope;
  m.dbg_cq_int8 = a->dbg_cq_int8;
  return m;
}

int validate_pre(const MlaPreprocessV2Args* a) {
  if (a == nullptr) return QKVNR_ERR_NULL_ARG;
  if (a->struct_size != sizeof(MlaPreprocessV2Args) || a->reserved0 != 0)
    return QKVNR_ERR_BAD_STRUCT;
  if (a->flags & ~MLA_FLAG_CHECK_INDEX) return QKVNR_ERR_BAD_MODE;
  if (!isfinite(a->quant_scale_x) || !isfinite(a->quant_scale_cq)) return QKVNR_ERR_BAD_SCALE;
  const MlaPrologV2Args m = preprocess_as_prolog(a);
  const int rc = validate_mla(&m);
  if (rc != QKVNR_OK || a->B * a->S == 0) return rc;
  if (a->gamma_x == nullptr || a->bias_x == nullptr || a->bias_cq == nullptr ||
      a->dequant_scale_dqkv == nullptr)
    return QKVNR_ERR_NULL_ARG;
  if (!aligned16(a->gamma_x) || !aligned16(a->bias_x) || !aligned16(a->bias_cq) ||
      (a->dbg_x_int8 && !aligned8(a->dbg_x_int8)))
    return QKVNR_ERR_BAD_ALIGNMENT;
  return QKVNR_OK;
}

// Host copy of a device array of n elements (debug checks only).
template <typename V>
int fetch(std::vector<V>& out, const V* dev, int64_t n, void* stream) {
  out.resize(static_cast<size_t>(n));
  if (n == 0) return QKVNR_OK;
  return copy_to_host_sync(out.data(), dev, static_cast<size_t>(n) * sizeof(V), stream);
}

// Both operators' index restriction: every index in [-1, slots), no
// repeats among the non-negative ones.
int check_index_host(const int64_t* idx, int64_t n, int64_t slots) {
  std::vector<int64_t> v;
  v.reserve(static_cast<size_t>(n));
  for (int64_t i = 0; i < n; ++i) {
    if (idx[i] < -1 || idx[i] >= slots) return QKVNR_ERR_BAD_INDEX;
    if (idx[i] >= 0) v.push_back(idx[i]);
  }
  std::sort(v.begin(), v.end());
  return std::adjacent_find(v.begin(), v.end()) == v.end() ? QKVNR_OK : QKVNR_ERR_BAD_INDEX;
}

// MLA_FLAG_CHECK_INDEX: the call's cache_index, copied to the host.
int debug_check_mla(const MlaPrologV2Args* a, void* stream) {
  const int64_t T = a->B * a->S;
  std::vector<int64_t> idx;
  int rc = fetch(idx, a->cache_index, T, stream);
  if (rc != QKVNR_OK) return rc;
  return check_index_host(idx.data(), T, a->block_num * a->block_size);
}

// QKV_FLAG_CHECK_INPUTS: the index restriction, and the quant scales must
// be non-zero (aclnnQkvRmsNormRopeCache, other restrictions).
int debug_check_qkv(const QkvRmsNormRopeCacheArgs* a, void* stream) {
  const int64_t T = a->B * a->S;
  std::vector<int64_t> idx;
  int rc = fetch(idx, a->index, T, stream);
  if (rc != QKVNR_OK) return rc;
  rc = check_index_host(idx.data(), T, a->block_num * a->block_size);
  if (rc != QKVNR_OK || a->quant_mode == QKV_QUANT_NONE) return rc;
  std::vector<float> ks, vs;
  rc = fetch(ks, a->k_scale, a->Nk * a->D, stream);
  if (rc == QKVNR_OK) rc = fetch(vs, a->v_scale, a->Nv * a->D, stream);
  if (rc != QKVNR_OK) return rc;
  for (float s : ks)
    if (s == 0.0f) return QKVNR_ERR_BAD_SCALE;
  for (float s : vs)
    if (s == 0.0f) return QKVNR_ERR_BAD_SCALE;
  return QKVNR_OK;
}

}  // namespace

extern "C" {

const char* mla_status_string(int s) {
  switch (s) {
    case QKVNR_OK: return "ok";
    case QKVNR_ERR_NULL_ARG: return "a required pointer is NULL";
    case QKVNR_ERR_BAD_SHAPE: return "bad shape";
    case QKVNR_ERR_BAD_MODE: return "unknown quant mode, dtype, layout, cache mode or flag";
    case QKVNR_ERR_UNSUPPORTED: return "unsupported configuration";
    case QKVNR_ERR_RESERVED_NONNULL: return "a reserved pointer is not NULL";
    case QKVNR_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case QKVNR_ERR_BAD_EPS: return "epsilon must be finite and >= 0";
    case QKVNR_ERR_BAD_STRUCT: return "argument struct size mismatch";
    case QKVNR_ERR_BAD_ALIGNMENT: return "pointer not 16-byte aligned";
    case QKVNR_ERR_LAUNCH_FAILED: return "kernel launch failed";
    case QKVNR_ERR_BAD_INDEX: return "cache index out of range or repeated";
    case QKVNR_ERR_BAD_SCALE: return "a quant scale is zero";
    case QKVNR_ERR_SCRATCH_TOO_SMALL:
      return "the call needs more than the no-allocation entry point's fixed scratch";
    default: return "unknown status";
  }
}

const char* mla_lib_version(void) { return QKVNR_VERSION_STRING; }

int mla_check_cache_index(const int64_t* index, int64_t n, int64_t slots) {
  if (n < 0 || slots < 0) return QKVNR_ERR_BAD_SHAPE;
  if (n > 0 && index == nullptr) return QKVNR_ERR_NULL_ARG;
  return check_index_host(index, n, slots);
}

int mla_prolog_v2_validate(const MlaPrologV2Args* args) { return validate_mla(args); }

int mla_prolog_v2_workspace_size(const MlaPrologV2Args* args, size_t* bytes) {
  if (bytes == nullptr) return QKVNR_ERR_NULL_ARG;
  *bytes = 0;
  const int rc = validate_mla(args);
  if (rc != QKVNR_OK) return rc;
  *bytes = make_mla_plan(args).total;
  return QKVNR_OK;
}

int mla_prolog_v2_kernels(const MlaPrologV2Args* args, uint32_t* mask) {
  if (mask == nullptr) return QKVNR_ERR_NULL_ARG;
  *mask = 0;
  const int rc = validate_mla(args);
  if (rc != QKVNR_OK) return rc;
  // Every plan launches each of the main kernels once when there are
  // tokens, except that the merged decode launch runs the W^UK product
  // inside the up projection's kernel, and the fused large-T launch runs
  // the q^R columns inside the W^UK one.
  if (args->B * args->S > 0) {
    *mask = (1u << MLA_KERNEL_COUNT) - 1u;
    const MlaPlan pl = make_mla_plan(args);
    if (pl.merge_uk || pl.merge_uk_q) *mask &= ~(1u << MLA_KERNEL_UK);
    if (pl.fuse_uk) *mask &= ~(1u << MLA_KERNEL_UQQR);

  }
  return QKVNR_OK;
}

int mla_prolog_v2(const MlaPrologV2Args* args, void* workspace, size_t workspace_bytes,
                  void* stream) {
  int rc = validate_mla(args);
  if (rc != QKVNR_OK) return rc;
  if (args->B * args->S == 0) return QKVNR_OK;
  const MlaPlan plan = make_mla_plan(args);
  if (workspace_bytes < plan.total) return QKVNR_ERR_WORKSPACE_TOO_SMALL;
  if (plan.total > 0 && workspace == nullptr) return QKVNR_ERR_NULL_ARG;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return QKVNR_ERR_BAD_ALIGNMENT;
  if (args->flags & MLA_FLAG_CHECK_INDEX) {
    rc = debug_check_mla(args, stream);
    if (rc != QKVNR_OK) return rc;
  }
  return launch_mla_prolog_v2(args, plan, workspace, stream);
}

int mla_preprocess_v2_validate(const MlaPreprocessV2Args* args) { return validate_pre(args); }

int mla_preprocess_v2_workspace_size(const MlaPreprocessV2Args* args, size_t* bytes) {
  if (bytes == nullptr) return QKVNR_ERR_NULL_ARG;
  *bytes = 0;
  const int rc = validate_pre(args);
  if (rc != QKVNR_OK) return rc;
  const MlaPrologV2Args m = preprocess_as_prolog(args);
  *bytes = make_preprocess_plan(&m).total;
  return QKVNR_OK;
}

int mla_preprocess_v2(const MlaPreprocessV2Args* args, void* workspace, size_t workspace_bytes,
                      void* stream) {
  int rc = validate_pre(args);
  if (rc != QKVNR_OK) return rc;
  if (args->B * args->S == 0) return QKVNR_OK;
  const MlaPrologV2Args m = preprocess_as_prolog(args);
  const MlaPlan plan = make_preprocess_plan(&m);
  if (workspace_bytes < plan.total) return QKVNR_ERR_WORKSPACE_TOO_SMALL;
  if (workspace == nullptr) return QKVNR_ERR_NULL_ARG;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return QKVNR_ERR_BAD_ALIGNMENT;
  if (args->flags & MLA_FLAG_CHECK_INDEX) {
    rc = debug_check_mla(&m, stream);
    if (rc != QKVNR_OK) return rc;
  }
  const PreprocessExtra pre{args->gamma_x, args->bias_x, args->quant_scale_x,
                            args->quant_scale_cq, args->dbg_x_int8};
  return launch_mla_prolog_v2(&m, plan, workspace, stream, &pre);
}

int mla_prolog_v2_no_alloc(const MlaPrologV2Args* args, void* stream) {
  const int rc = validate_mla(args);
  if (rc != QKVNR_OK) return rc;
  // the debug copy would allocate host memory and synchronise
  if (args->flags & MLA_FLAG_CHECK_INDEX) return QKVNR_ERR_BAD_MODE;
  if (args->B * args->S == 0) return QKVNR_OK;
  const MlaPlan plan = make_mla_plan(args);
  if (plan.total > MLA_NO_ALLOC_SCRATCH_BYTES) return QKVNR_ERR_SCRATCH_TOO_SMALL;
  return launch_mla_prolog_v2_no_alloc(args, plan, stream);
}

int mla_pack_weight(const void* src, void* dst, int64_t batch, int64_t K, int64_t N,
                    int32_t elem_bytes, void* stream) {
  if (elem_bytes != 1 && elem_bytes != 2) return QKVNR_ERR_BAD_MODE;
  if (!pack_dims_ok(batch, K, N) || K % (16 / elem_bytes) != 0) return QKVNR_ERR_BAD_SHAPE;
  if (batch * K * N == 0) return QKVNR_OK;
  if (src == nullptr || dst == nullptr) return QKVNR_ERR_NULL_ARG;
  if (!aligned16(dst) || (elem_bytes == 2 && (reinterpret_cast<uintptr_t>(src) & 1u)))
    return QKVNR_ERR_BAD_ALIGNMENT;
  return launch_pack_weight(src, dst, batch, K, N, elem_bytes, N, 0, stream);
}

int mla_pack_weight_uk(const void* src, void* dst, int64_t N, int64_t D, int64_t Hckv,
                       void* stream) {
  if (!pack_dims_ok(N, D, Hckv) || D % 16 != 0) return QKVNR_ERR_BAD_SHAPE;
  if (N * D * Hckv == 0) return QKVNR_OK;
  if (src == nullptr || dst == nullptr) return QKVNR_ERR_NULL_ARG;
  if (!aligned16(dst) || (reinterpret_cast<uintptr_t>(src) & 1u)) return QKVNR_ERR_BAD_ALIGNMENT;
  return launch_pack_weight(src, dst, N, D, Hckv, 2, Hckv, 0, stream, /*kperm=*/true);
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
  return launch_pack_weight(src, dst, 1, Hcq, N * (D + Dr), elem_bytes, N * D, Dr, stream);
}

int qkv_rmsnorm_rope_cache_validate(const QkvRmsNormRopeCacheArgs* args) {
  return validate_qkv(args);
}

int qkv_rmsnorm_rope_cache(const QkvRmsNormRopeCacheArgs* args, void* stream) {
  int rc = validate_qkv(args);
  if (rc != QKVNR_OK) return rc;
  if (args->B * args->S == 0) return QKVNR_OK;  // empty tensors: nothing runs
  if (args->flags & QKV_FLAG_CHECK_INPUTS) {
    rc = debug_check_qkv(args, stream);
    if (rc != QKVNR_OK) return rc;
  }
  return launch_qkv_rmsnorm_rope_cache(args, stream);
}

int mla_probe_read(const void* src, size_t bytes, void* sink, void* stream) {
  if (bytes == 0) return QKVNR_OK;
  if (src == nullptr || sink == nullptr) return QKVNR_ERR_NULL_ARG;
  if (bytes % 16 != 0) return QKVNR_ERR_BAD_SHAPE;
  if (!aligned16(src) || (reinterpret_cast<uintptr_t>(sink) & 3u)) return QKVNR_ERR_BAD_ALIGNMENT;
  return probe_read(src, bytes, sink, stream);
}

int mla_probe_mfma_bf16(int64_t iters, void* sink, void* stream) {
  if (iters <= 0 || iters > (int64_t(1) << 31)) return QKVNR_ERR_BAD_SHAPE;
  if (sink == nullptr) return QKVNR_ERR_NULL_ARG;
  if (reinterpret_cast<uintptr_t>(sink) & 3u) return QKVNR_ERR_BAD_ALIGNMENT;
  return probe_mfma(iters, sink, stream);
}

}  // extern "C"
