/*
 * qkvnr.h - C ABI of the MI355X (gfx950) MLA-prolog / qkv RmsNorm-RoPE-cache
 * library.
 *
 * Two operations, both from public operator documentation:
 *
 *  - MlaPrologV2 ("MlaPrologV2" README, ops-transformer, attention/
 *    mla_prolog_v2: function description and formulas, parameter table,
 *    constraints).  It computes, per token t:
 *        c^Q  = RmsNorm(x . W^DQ)
 *        q^N  = (c^Q . W^UQ) . W^UK           per head   -> query
 *        q^R  = RoPE(c^Q . W^QR)                         -> query_rope
 *        c^KV = RmsNorm(x . W^DKV)     written to kv_cache at cache_index[t]
 *        k^R  = RoPE(x . W^KR)         written to kr_cache at cache_index[t]
 *
 *  - QkvRmsNormRopeCache ("aclnnQkvRmsNormRopeCache", CANN API reference:
 *    function description and formulas (1)-(4)).  It splits a fused qkv
 *    tensor into q, k and v (SplitVD), RmsNorms q and k, applies
 *    half-and-half RoPE to both, quantises k and v, writes q to q_out and
 *    scatters k and v into paged caches.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every pointer named in an argument struct is a DEVICE pointer into
 *    memory the caller owns (the struct itself lives in host memory).  The
 *    library never allocates, frees or synchronises, keeps no state between
 *    calls, and launches all work on the caller's stream (`stream` is a
 *    hipStream_t passed as void*; NULL is the default stream).  Calls on one
 *    stream are ordered by that stream; calls that share output buffers on
 *    different streams race.
 *  - Tensors are dense and row-major (C order) with the shapes given below.
 *    bf16 and fp16 are IEEE-style 16-bit floats; int8 is two's complement.
 *  - Every entry point validates its arguments on the host first and
 *    returns a negative QKVNR_ERR_* code without launching anything when a
 *    check fails.  QKVNR_OK (0) means all work was enqueued; kernel faults
 *    surface on the stream like any other HIP error.
 *  - Results are deterministic: the same inputs give bit-identical outputs
 *    and caches (no floating-point atomics; fixed-order reductions).
 *  - Cache updates: a token whose index is -1 writes nothing.  Indexes must
 *    lie in [-1, BlockNum*BlockSize) and must not repeat (both operators'
 *    index restrictions).  The kernels skip any index outside that range
 *    (memory safety); a repeated slot gets an unspecified winner.  The
 *    opt-in debug flags (MLA_FLAG_CHECK_INDEX, QKV_FLAG_CHECK_INPUTS) copy
 *    the index to the host first, synchronising the stream, and refuse a
 *    violation with QKVNR_ERR_BAD_INDEX before anything is launched; a
 *    call with a debug flag must not be captured into a HIP graph.
 */
#ifndef QKVNR_H
#define QKVNR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QKVNR_VERSION_STRING "0.1.0"

/* ---- status codes ------------------------------------------------------ */
enum {
  QKVNR_OK = 0,
  QKVNR_ERR_NULL_ARG = -1,          /* a required pointer is NULL */
  QKVNR_ERR_BAD_SHAPE = -2,         /* a dimension is negative or breaks a
                                       shape rule */
  QKVNR_ERR_BAD_MODE = -3,          /* unknown quant mode, dtype, layout,
                                       cache mode or flag bit */
  QKVNR_ERR_UNSUPPORTED = -4,       /* valid on the pages, not built here
                                       (PA_NZ caches, Nkv != 1, dims off
                                       the kernels' multiples, ...) */
  QKVNR_ERR_RESERVED_NONNULL = -5,  /* a reserved pointer is not NULL */
  QKVNR_ERR_WORKSPACE_TOO_SMALL = -6,
  QKVNR_ERR_BAD_EPS = -7,           /* epsilon negative or not finite */
  QKVNR_ERR_BAD_STRUCT = -8,        /* struct_size does not match */
  QKVNR_ERR_BAD_ALIGNMENT = -9,     /* a pointer is not 16-byte aligned
                                       (cache_index and dbg_cq_int8: 8,
                                       dbg_cq_scale: 4) */
  QKVNR_ERR_LAUNCH_FAILED = -10,    /* a HIP call failed (hipGetLastError
                                       after a launch, or the debug checks'
                                       copy) */
  QKVNR_ERR_BAD_INDEX = -11,        /* an index outside [-1, BlockNum *
                                       BlockSize) or a repeated one: only
                                       from mla_check_cache_index and the
                                       opt-in debug checks (MLA_FLAG_CHECK_
                                       INDEX, QKV_FLAG_CHECK_INPUTS) */
  QKVNR_ERR_BAD_SCALE = -12,        /* a zero quant scale: only from the
                                       opt-in QKV_FLAG_CHECK_INPUTS check */
  QKVNR_ERR_SCRATCH_TOO_SMALL = -13  /* mla_prolog_v2_no_alloc: the call
                                        needs more workspace than
                                        MLA_NO_ALLOC_SCRATCH_BYTES */
};

/* Human-readable name of a status code (static storage, never NULL; an
 * unknown code gives "unknown status").  Errors: none. */
const char* mla_status_string(int status);

/* Library version, QKVNR_VERSION_STRING (static storage).  Errors: none. */
const char* mla_lib_version(void);

/* Both operators' index restriction (aclnnQkvRmsNormRopeCache, other
 * restrictions; the MlaPrologV2 cache_index follows the same rule): every
 * index[i], i < n, lies in [-1, slots) and no non-negative value repeats.
 * `index` is HOST memory (may be NULL when n == 0); nothing is launched.
 * Returns QKVNR_OK, QKVNR_ERR_BAD_INDEX, QKVNR_ERR_BAD_SHAPE (n < 0 or
 * slots < 0) or QKVNR_ERR_NULL_ARG. */
int mla_check_cache_index(const int64_t* index, int64_t n, int64_t slots);

/* ======================================================================= */
/* MlaPrologV2                                                              */
/* ======================================================================= */

/* Quantisation scenarios of the MlaPrologV2 README's scenario table.
 * NONE: every input and output is bf16.
 * PARTIAL_KV_BF16: weight_uq_qr is int8 with a per-channel fp32 dequant
 *   scale (dequant_scale_w_uq_qr); c^Q is quantised per token to int8 after
 *   multiplying by smooth_scales_cq; caches stay bf16.
 * PARTIAL_KV_INT8: as PARTIAL_KV_BF16, plus int8 kv_cache / kr_cache
 *   quantised per channel by quant_scale_ckv / quant_scale_ckr
 *   (code = saturate(round_half_even(value / scale))).
 * FULL_KV_BF16: as PARTIAL_KV_BF16, plus int8 token_x with a per-token
 *   fp32 dequant scale (dequant_scale_x) and int8 weight_dq / weight_dkv_kr
 *   with per-channel fp32 dequant scales (dequant_scale_w_dq,
 *   dequant_scale_w_dkv_kr): h = (sum_k x8 * w8) * dequant_scale_x[t] *
 *   dequant_scale_w[j].  Caches and outputs bf16.
 * FULL_KV_INT8: as FULL_KV_BF16 with an int8 kv_cache quantised per channel
 *   by quant_scale_ckv (the README's dtype/shape table gives it shape
 *   (1, Hckv); its scenario table's "per-tensor" is the case of equal
 *   entries), a bf16 kr_cache, and an int8 query quantised per (token,
 *   head): dequant_scale_q_nope[t, n] = max_j |q^N[t, n, j]| / 127 and
 *   query = round_half_even(q^N / that scale) in [-127, 127] (0 for an
 *   all-zero head). */
enum {
  MLA_QUANT_NONE = 0,
  MLA_QUANT_PARTIAL_KV_BF16 = 1,
  MLA_QUANT_PARTIAL_KV_INT8 = 2,
  MLA_QUANT_FULL_KV_BF16 = 3,
  MLA_QUANT_FULL_KV_INT8 = 4
};

/* Weight layouts for weight_dq, weight_dkv_kr, weight_uq_qr, weight_uk.
 * ND: the page's unblocked (k, n) row-major layout ((N, D, Hckv) for
 *   weight_uk).  The library packs ND weights into the workspace on every
 *   call (convenient, slower).
 * PACKED_K16: the MFMA-native blocked layout produced once by
 *   mla_pack_weight().  For a (K, N) matrix with G = 16 / element_bytes
 *   (8 for bf16, 16 for int8), KC = K / G chunk rows and NB = ceil(N / 32)
 *   column blocks (the last one zero-padded), element (k, n) is stored at
 *       ((((n / 32) * KC + k / G) * 32) + n % 32) * G + k % G.
 *   The G consecutive-k values of one column form one 16-byte chunk (one
 *   lane's MFMA operand), and each 32-column block's whole K range is one
 *   contiguous run, so a weight-streaming wave reads one contiguous stream.
 *   A packed matrix holds K * NB * 32 elements.
 *   weight_uk is packed by mla_pack_weight_uk(): each head's (D, Hckv)
 *   matrix this way, heads in order, except that within every 16-k step
 *   the two 8-k chunks hold k offsets {0-3, 8-11} and {4-7, 12-15} (the
 *   order in which an MFMA result holds the rows it feeds into the W^UK
 *   product).  This plays the role that the
 *   pages' FRACTAL_NZ weight format plays for their hardware.
 *   weight_uq_qr is packed by mla_pack_weight_uq_qr(), which also reorders
 *   the W^QR columns when Dr = 64: within each head, packed 32-column block
 *   b (b = 0, 1) holds rope columns [16b, 16b + 16) followed by
 *   [32 + 16b, 32 + 16b + 16), so every column and its RoPE partner (the
 *   column Dr/2 away) sit in one 32-column block.  For Dr = 16 and 32 the
 *   natural order already has that property and is kept. */
enum { MLA_WEIGHT_ND = 0, MLA_WEIGHT_PACKED_K16 = 1 };

/* Debug flags of MlaPrologV2Args.flags.  MLA_FLAG_CHECK_INDEX: before
 * launching, copy cache_index to the host (synchronises `stream`) and
 * return QKVNR_ERR_BAD_INDEX if an index lies outside [-1, BlockNum *
 * BlockSize) or repeats.  Unknown bits: QKVNR_ERR_BAD_MODE. */
enum { MLA_FLAG_CHECK_INDEX = 1 };

/* Arguments of one MlaPrologV2 call: the tensors of the MlaPrologV2 README
 * parameter table, with the shapes and dtypes of its constraints section
 * (shape rules and dtype/shape table). */
typedef struct MlaPrologV2Args {
  uint32_t struct_size;      /* = sizeof(MlaPrologV2Args) */
  int32_t quant_mode;        /* MLA_QUANT_* */
  int32_t weight_layout;     /* MLA_WEIGHT_* */
  int32_t flags;             /* MLA_FLAG_* (0 in production) */

  /* Dimensions (MlaPrologV2 README, constraints).  T = B*S tokens; for the
   * (T, He) layout pass B = T, S = 1.  Requirements checked here:
   * He, Hcq, D multiples of 32 (K dims of the MFMA tiles; He of 64 in
   * FULL_*, Hcq of 64 in PARTIAL_* and FULL_*), Hckv a multiple
   * of 16, Dr in {16, 32, 64} with (N*D) % Dr == 0, Nkv == 1, all > 0
   * except B, S (either may be 0: nothing is done) and block_num /
   * block_size (either 0: the caches are left untouched, queries are still
   * computed). */
  int64_t B, S, He, Hcq, N, D, Hckv, Dr, Nkv, block_num, block_size;

  double rmsnorm_epsilon_cq;   /* epsilon of c^Q's RmsNorm, >= 0 */
  double rmsnorm_epsilon_ckv;  /* epsilon of c^KV's RmsNorm, >= 0 */
  const char* cache_mode;      /* NULL, "" or "PA_ND" (paged, row-major);
                                  "PA_NZ" -> QKVNR_ERR_UNSUPPORTED */

  /* ---- inputs (device) ---- */
  const void* token_x;         /* (T, He) bf16, int8 in FULL_* */
  const void* weight_dq;       /* (He, Hcq) bf16, int8 in FULL_* */
  const void* weight_uq_qr;    /* (Hcq, N*(D+Dr)): bf16 (NONE) or int8
                                  (PARTIAL_*, FULL_*).  Columns [0, N*D) are W^UQ,
                                  head n at n*D; columns [N*D, N*(D+Dr)) are
                                  W^QR, head n at N*D + n*Dr. */
  const void* weight_uk;       /* (N, D, Hckv) bf16 */
  const void* weight_dkv_kr;   /* (He, Hckv+Dr): [W^DKV | W^KR], bf16,
                                  int8 in FULL_* */
  const void* rmsnorm_gamma_cq;   /* (Hcq) bf16 */
  const void* rmsnorm_gamma_ckv;  /* (Hckv) bf16 */
  const void* rope_sin;        /* (T, Dr) bf16 */
  const void* rope_cos;        /* (T, Dr) bf16 */
  const int64_t* cache_index;  /* (T) flat slot ids, -1 = skip */
  /* Scales a scenario does not use must be NULL (else
   * QKVNR_ERR_RESERVED_NONNULL). */
  const float* dequant_scale_x;        /* (T) fp32, FULL_* only */
  const float* dequant_scale_w_dq;     /* (Hcq) fp32, FULL_* only */
  const float* dequant_scale_w_uq_qr;  /* (N*(D+Dr)) fp32, PARTIAL_*, FULL_* */
  const float* dequant_scale_w_dkv_kr; /* (Hckv+Dr) fp32, FULL_* only */
  const float* quant_scale_ckv;        /* (Hckv) fp32, PARTIAL_KV_INT8 and
                                          FULL_KV_INT8 only */
  const float* quant_scale_ckr;        /* (Dr) fp32, PARTIAL_KV_INT8 only */
  const float* smooth_scales_cq;       /* (Hcq) fp32, PARTIAL_*, FULL_* */

  /* ---- in/out (device), updated in place at indexed slots only ---- */
  void* kv_cache;              /* (BlockNum, BlockSize, Nkv, Hckv): bf16, or
                                  int8 in PARTIAL_KV_INT8 and FULL_KV_INT8 */
  void* kr_cache;              /* (BlockNum, BlockSize, Nkv, Dr): bf16, or
                                  int8 in PARTIAL_KV_INT8 */

  /* ---- outputs (device), fully overwritten ---- */
  void* query;                 /* (T, N, Hckv) bf16, int8 in FULL_KV_INT8 */
  void* query_rope;            /* (T, N, Dr) bf16 */
  float* dequant_scale_q_nope; /* (T, N) fp32, FULL_KV_INT8 only */

  /* ---- optional diagnostics (device), NULL when not wanted ----
   * PARTIAL_* and FULL_*: the int8 codes of c^Q (T, Hcq) and their per-token
   * scales (T) exactly as the up-projection consumed them. */
  int8_t* dbg_cq_int8;
  float* dbg_cq_scale;

  /* ---- optional instrumentation (host array of hipEvent_t handles) ----
   * When n_phase_events > 0 the library records phase_events[i] on `stream`
   * at the phase boundaries MLA_PHASE_* below (only the first
   * n_phase_events of them).  The work is exactly that of a normal call;
   * ND-layout weight packing happens before MLA_PHASE_START. */
  void* const* phase_events;
  int32_t n_phase_events;

  /* ---- optional per-kernel timing (host array of hipEvent_t handles) ----
   * When n_kernel_events > 2*i+1, the main kernel MLA_KERNEL_i below is
   * launched with kernel_events[2*i] and kernel_events[2*i+1] as its start
   * and stop events (hipExtLaunchKernel: taken by the kernel's own dispatch,
   * so their interval is the kernel's execution time).  The work is exactly
   * that of a normal call. */
  void* const* kernel_events;
  int32_t n_kernel_events;
} MlaPrologV2Args;

/* The main kernels of one call, for kernel_events.  With the large-T plan
 * that fuses the W^UK product (D = 128), MLA_KERNEL_UK is one launch that
 * runs the q^C columns with the fused W^UK product and the q^R columns, and
 * MLA_KERNEL_UQQR is not launched.  With
 * the bf16 decode plan for T <= 32 and D <= 128, and with the quantised
 * decode plans that write a bf16 query for T <= 64 when the up projection
 * has fewer than 128 x 96 columns (D a multiple of 32 up to 128),
 * MLA_KERNEL_UQQR is one launch that runs the up projection and the W^UK
 * product, and MLA_KERNEL_UK is not launched (mla_prolog_v2_kernels
 * reports which). */
enum {
  MLA_KERNEL_DOWN = 0,  /* x . [W^DQ | W^DKV_KR] */
  MLA_KERNEL_NORM = 1,  /* RmsNorms, c^Q quant, RoPE k^R, cache scatter */
  MLA_KERNEL_UQQR = 2,  /* c^Q . [W^UQ | W^QR], RoPE q^R */
  MLA_KERNEL_UK = 3,    /* q^C . W^UK per head */
  MLA_KERNEL_COUNT = 4
};

/* Phase boundaries of one mla_prolog_v2 call, in launch order; each one
 * follows one kernel. */
enum {
  MLA_PHASE_START = 0,        /* before the first kernel */
  MLA_PHASE_AFTER_DOWN = 1,   /* after x . [W^DQ | W^DKV_KR] */
  MLA_PHASE_AFTER_NORM = 2,   /* after RmsNorms, c^Q quant, RoPE k^R, scatter */
  MLA_PHASE_AFTER_UQQR = 3,   /* after c^Q . [W^UQ | W^QR] and RoPE q^R */
  MLA_PHASE_AFTER_UK = 4,     /* after q^C . W^UK per head (end of call) */
  MLA_PHASE_COUNT = 5
};

/* Bytes of device workspace mla_prolog_v2() needs for these arguments
 * (depends on the dims, T, quant mode and weight layout; the pages' first
 * phase, which sizes the workspace, as one call).  Writes *bytes and
 * returns QKVNR_OK, or a validation error (then *bytes is 0).  The size
 * comes back through a pointer so that an error is never mistaken for a
 * zero-byte workspace.  Host only, no HIP call. */
int mla_prolog_v2_workspace_size(const MlaPrologV2Args* args, size_t* bytes);

/* Host-only validation of args against the MlaPrologV2 README constraints
 * (shape rules, scenario and dtype/shape tables) and this library's kernel
 * limits: the checks mla_prolog_v2 runs first.  Makes no HIP call.
 * Returns QKVNR_OK or the first failing check's QKVNR_ERR_* code. */
int mla_prolog_v2_validate(const MlaPrologV2Args* args);

/* Which main kernels (bit i = MLA_KERNEL_i) a call with these args
 * launches, and so which kernel_events pairs it records.  Writes *mask and
 * returns QKVNR_OK, or a validation error (then *mask is 0).  Host only. */
int mla_prolog_v2_kernels(const MlaPrologV2Args* args, uint32_t* mask);

/* Run the prolog: the five formulas of the MlaPrologV2 README function
 * description (c^Q, q^N, q^R, c^KV -> kv_cache, k^R -> kr_cache) in the
 * quantisation scenario args->quant_mode.  workspace: device scratch of at
 * least mla_prolog_v2_workspace_size() bytes, 256-byte aligned, owned by
 * the caller, contents undefined on entry and exit (may be NULL when the
 * size is 0).  Enqueues on `stream` and returns without synchronising
 * (except under MLA_FLAG_CHECK_INDEX).  Errors: any validation code,
 * QKVNR_ERR_WORKSPACE_TOO_SMALL, QKVNR_ERR_BAD_INDEX (debug flag),
 * QKVNR_ERR_LAUNCH_FAILED; nothing is launched on a validation error. */
int mla_prolog_v2(const MlaPrologV2Args* args, void* workspace,
                  size_t workspace_bytes, void* stream);

/* Size of the fixed per-device scratch array of mla_prolog_v2_no_alloc. */
#define MLA_NO_ALLOC_SCRATCH_BYTES ((size_t)16 << 20)

/* mla_prolog_v2 for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same kernels and results, with the workspace taken from a
 * 16 MiB array the library holds on each GPU it runs on (allocated with
 * the code object, kept until the process ends) instead of a caller buffer.
 * The call itself allocates nothing.  It needs nothing cleared.  Calls that
 * overlap in time on one GPU share that array and race: order them on one
 * stream.  Limit: calls whose mla_prolog_v2_workspace_size exceeds
 * MLA_NO_ALLOC_SCRATCH_BYTES are refused with QKVNR_ERR_SCRATCH_TOO_SMALL
 * (at the DeepSeek-V3 dims every decode-sized call with T <= 128 fits,
 * except FULL_KV_INT8 above T = 32; ND-layout weights, packed into the
 * workspace, need far more).  MLA_FLAG_CHECK_INDEX is refused
 * (QKVNR_ERR_BAD_MODE).  Other errors as mla_prolog_v2. */
int mla_prolog_v2_no_alloc(const MlaPrologV2Args* args, void* stream);

/* Weight packing: the MFMA-native counterpart of the MlaPrologV2 pages'
 * FRACTAL_NZ weight format (MLA_WEIGHT_PACKED_K16 above); done once per
 * weight, outside the per-token path.
 *
 * Pack `batch` row-major (K, N) matrices (each K*N elements of
 * `elem_bytes` = 2 (bf16/fp16) or 1 (int8), batches contiguous) into the
 * MLA_WEIGHT_PACKED_K16 layout at dst, a distinct buffer of
 * batch * K * ceil(N/32)*32 elements.  K must be a multiple of
 * 16 / elem_bytes.  batch <= 65535, K and N <= 2^30 and the packed
 * element count <= 2^46, else QKVNR_ERR_BAD_SHAPE (the same bounds hold for
 * the two packers below).  Device pointers; enqueued on `stream`. */
int mla_pack_weight(const void* src, void* dst, int64_t batch, int64_t K,
                    int64_t N, int32_t elem_bytes, void* stream);

/* Pack weight_uk, N row-major (D, Hckv) bf16 matrices, into the
 * MLA_WEIGHT_PACKED_K16 layout with the k order described above, at dst (a
 * distinct buffer of N * D * ceil(Hckv/32)*32 elements).  D must be a
 * multiple of 16, else QKVNR_ERR_BAD_SHAPE.  Device pointers; enqueued on
 * `stream`. */
int mla_pack_weight_uk(const void* src, void* dst, int64_t N, int64_t D,
                       int64_t Hckv, void* stream);

/* Pack weight_uq_qr, a row-major (Hcq, N*(D+Dr)) matrix of `elem_bytes` = 2
 * (bf16) or 1 (int8) elements, into the MLA_WEIGHT_PACKED_K16 layout with
 * the W^QR column order described above, at dst (a distinct buffer of
 * Hcq * ceil(N*(D+Dr)/32)*32 elements).  Dims must pass the same checks as
 * mla_prolog_v2 (D a multiple of 32, Dr in {16, 32, 64}, Hcq a multiple of
 * 16 / elem_bytes), else QKVNR_ERR_BAD_SHAPE or QKVNR_ERR_UNSUPPORTED.
 * Device pointers; enqueued on `stream`. */
int mla_pack_weight_uq_qr(const void* src, void* dst, int64_t Hcq, int64_t N,
                          int64_t D, int64_t Dr, int32_t elem_bytes,
                          void* stream);

/* ======================================================================= */
/* MlaPreprocessV2                                                          */
/* ======================================================================= */

/* aclnnMlaPreprocessV2 (CANN API reference: interface function bullets,
 * formula block).  Per token t, in the bullets' order:
 *     x8 = RmsNormQuant(x)               (He: gamma_x, bias_x, quant_scale_x)
 *     [h | g_kv | g_r] = x8 . W^DQKV     (int8 product, dequant per channel)
 *     path 1: c8 = RmsNormQuant(h)       (Hcq: gamma_cq, bias_cq, quant_scale_cq)
 *             y  = c8 . [W^UQ | W^QR]    (int8 product, dequant per channel)
 *             path 3: query = y's q^C . W^UK per head
 *             path 4: query_rope = RoPE(y's rope block)
 *     path 2: path 5: RmsNorm(g_kv) (gamma_ckv) -> kv_cache[cache_index[t]]
 *             path 6: RoPE(g_r)                   -> kr_cache[cache_index[t]]
 * RmsNormQuant(v) = (gamma * v / RMS(v) + bias) * quant_scale as the
 * formula block prints it, then rounded half to even and saturated to
 * [-128, 127]; RMS(v) = sqrt(mean(v^2) + epsilon), one epsilon for all
 * three norms.  The int8 products are exact integer sums times a
 * per-output-channel fp32 dequant scale.  The page's parameter tables did
 * not survive extraction: the names below are this library's.  Shapes as
 * MlaPrologV2 (T = B*S tokens, Nkv = 1); He and Hcq multiples of 64, D of
 * 32, Hckv of 16, Dr in {16, 32, 64}.  The page's ranges (B <= 256, He in
 * [2048, 10240], N in {16, 32, 64, 128}, BlockNum 192, BlockSize 128)
 * describe its own kernels; any shape above is accepted. */
typedef struct MlaPreprocessV2Args {
  uint32_t struct_size;      /* = sizeof(MlaPreprocessV2Args) */
  int32_t weight_layout;     /* MLA_WEIGHT_* for weight_dqkv, weight_uq_qr,
                                weight_uk (packed: mla_pack_weight for
                                weight_dqkv, mla_pack_weight_uq_qr,
                                mla_pack_weight_uk) */
  int32_t flags;             /* MLA_FLAG_CHECK_INDEX, else 0 */
  int32_t reserved0;         /* must be 0 */
  int64_t B, S, He, Hcq, N, D, Hckv, Dr, block_num, block_size;
  double epsilon;            /* RmsNorm epsilon, >= 0 */
  float quant_scale_x;       /* RmsNormQuant scale of x (finite) */
  float quant_scale_cq;      /* RmsNormQuant scale of the query latent */
  const char* cache_mode;    /* NULL, "" or "PA_ND" */

  /* ---- inputs (device) ---- */
  const void* token_x;       /* (T, He) bf16 */
  const void* gamma_x;       /* (He) bf16 */
  const float* bias_x;       /* (He) fp32 */
  const void* weight_dqkv;   /* (He, Hcq+Hckv+Dr) int8: [W^DQ | W^DKV | W^KR] */
  const float* dequant_scale_dqkv;   /* (Hcq+Hckv+Dr) fp32 */
  const void* gamma_cq;      /* (Hcq) bf16 */
  const float* bias_cq;      /* (Hcq) fp32 */
  const void* weight_uq_qr;  /* (Hcq, N*(D+Dr)) int8, column order as
                                MlaPrologV2's weight_uq_qr */
  const float* dequant_scale_uq_qr;  /* (N*(D+Dr)) fp32 */
  const void* weight_uk;     /* (N, D, Hckv) bf16 */
  const void* gamma_ckv;     /* (Hckv) bf16 */
  const void* rope_sin;      /* (T, Dr) bf16 */
  const void* rope_cos;      /* (T, Dr) bf16 */
  const int64_t* cache_index;  /* (T) flat slot ids, -1 = skip */

  /* ---- in/out (device) ---- */
  void* kv_cache;            /* (BlockNum, BlockSize, 1, Hckv) bf16 */
  void* kr_cache;            /* (BlockNum, BlockSize, 1, Dr) bf16 */
  /* ---- outputs (device) ---- */
  void* query;               /* (T, N, Hckv) bf16: q^N */
  void* query_rope;          /* (T, N, Dr) bf16: q^R */
  /* ---- optional diagnostics (device), NULL when not wanted: the int8
   * codes of the two RmsNormQuant steps, (T, He) and (T, Hcq) ---- */
  int8_t* dbg_x_int8;
  int8_t* dbg_cq_int8;
} MlaPreprocessV2Args;

/* Host-only validation (no HIP call): QKVNR_OK or the first failing
 * check's code (a non-finite quant scale: QKVNR_ERR_BAD_SCALE). */
int mla_preprocess_v2_validate(const MlaPreprocessV2Args* args);

/* Bytes of device workspace mla_preprocess_v2() needs; as
 * mla_prolog_v2_workspace_size.  Host only. */
int mla_preprocess_v2_workspace_size(const MlaPreprocessV2Args* args,
                                     size_t* bytes);

/* Run MlaPreprocessV2 on `stream` (workspace as mla_prolog_v2).  Errors:
 * any validation code, QKVNR_ERR_WORKSPACE_TOO_SMALL, QKVNR_ERR_BAD_INDEX
 * (MLA_FLAG_CHECK_INDEX), QKVNR_ERR_LAUNCH_FAILED; nothing is launched on
 * a validation error. */
int mla_preprocess_v2(const MlaPreprocessV2Args* args, void* workspace,
                      size_t workspace_bytes, void* stream);

/* ======================================================================= */
/* QkvRmsNormRopeCache                                                      */
/* ======================================================================= */

/* Quant step of formula (4): NONE (caches have the input dtype), SYMMETRIC
 * (int8 = sat(rne(x / scale))), ASYMMETRIC (int8 = sat(rne(x / scale +
 * offset))).  Scales and offsets are per channel over (head, dim). */
enum { QKV_QUANT_NONE = 0, QKV_QUANT_SYMMETRIC = 1, QKV_QUANT_ASYMMETRIC = 2 };

/* Element type of qkv, gamma, cos, sin, q_out and the BeforeQuant outputs
 * (and of the caches in QKV_QUANT_NONE). */
enum { QKV_DTYPE_FP16 = 0, QKV_DTYPE_BF16 = 1 };

/* Debug flags of QkvRmsNormRopeCacheArgs.flags.  QKV_FLAG_CHECK_INPUTS:
 * before launching, copy the index (and, quantised, k_scale / v_scale) to
 * the host (synchronises `stream`) and return QKVNR_ERR_BAD_INDEX for an
 * index outside [-1, BlockNum * BlockSize) or a repeated one, or
 * QKVNR_ERR_BAD_SCALE for a zero scale (the page's other restrictions).
 * Unknown bits: QKVNR_ERR_BAD_MODE. */
enum { QKV_FLAG_CHECK_INPUTS = 1 };

/* Arguments of one QkvRmsNormRopeCache call.  The page's parameter tables
 * did not survive extraction; the tensors below are rebuilt from its
 * function description, formulas (1)-(4) and the requireMemory sum of its
 * other restrictions. */
typedef struct QkvRmsNormRopeCacheArgs {
  uint32_t struct_size;      /* = sizeof(QkvRmsNormRopeCacheArgs) */
  int32_t quant_mode;        /* QKV_QUANT_* */
  int32_t dtype;             /* QKV_DTYPE_* */
  int32_t flags;             /* QKV_FLAG_* (0 in production) */

  /* Dimensions (aclnnQkvRmsNormRopeCache, input shape restrictions):
   * D == 128; Nk == Nv; Nq, Nk >= 1; block_num >= ceil(S / block_size) * B
   * when B*S > 0. */
  int64_t B, S, Nq, Nk, Nv, D, block_num, block_size;
  double epsilon;            /* RmsNorm epsilon, >= 0 */
  const char* cache_mode;    /* NULL, "" or "PA_ND"; "PA_NZ" unsupported */

  /* ---- inputs (device) ---- */
  const void* qkv;           /* (B*S, Nq+Nk+Nv, D): q heads, then k, then v */
  const void* gamma_q;       /* (D) */
  const void* gamma_k;       /* (D) */
  const void* cos;           /* (B*S, D) */
  const void* sin;           /* (B*S, D) */
  const int64_t* index;      /* (B*S) flat slot ids, -1 = skip */
  const float* k_scale;      /* (Nk*D), nonzero; quantised modes only */
  const float* v_scale;      /* (Nv*D), nonzero; quantised modes only */
  const float* k_offset;     /* (Nk*D); ASYMMETRIC only, else NULL */
  const float* v_offset;     /* (Nv*D); ASYMMETRIC only, else NULL */

  /* ---- in/out (device) ---- */
  void* k_cache;             /* (block_num, block_size, Nk, D) */
  void* v_cache;             /* (block_num, block_size, Nv, D) */

  /* ---- outputs (device) ---- */
  void* q_out;               /* (B*S, Nq, D), the rotated q */
  void* q_before_quant;      /* optional (B*S, Nq, D): same as q_out */
  void* k_before_quant;      /* optional (B*S, Nk, D): k after RoPE */
  void* v_before_quant;      /* optional (B*S, Nv, D): v as split */
} QkvRmsNormRopeCacheArgs;

/* Host-only validation against the aclnnQkvRmsNormRopeCache input shape
 * restrictions and this library's kernel limits (makes no HIP call).
 * Returns QKVNR_OK or the first failing check's QKVNR_ERR_* code. */
int qkv_rmsnorm_rope_cache_validate(const QkvRmsNormRopeCacheArgs* args);

/* Run the fused op, aclnnQkvRmsNormRopeCache formulas (1) SplitVD, (2)
 * RmsNorm of q and k, (3) half-and-half RoPE of q and k, (4) quant of k
 * and v, then q_out and the paged scatter: one pass over qkv, no
 * workspace.  Enqueues on `stream` and returns without synchronising
 * (except under QKV_FLAG_CHECK_INPUTS).  Errors: any validation code,
 * QKVNR_ERR_BAD_INDEX / QKVNR_ERR_BAD_SCALE (debug flag),
 * QKVNR_ERR_LAUNCH_FAILED; nothing is launched on a validation error. */
int qkv_rmsnorm_rope_cache(const QkvRmsNormRopeCacheArgs* args, void* stream);

/* ======================================================================= */
/* Measurement probes                                                       */
/* ======================================================================= */

/* Not part of either operator: reference points for the roofline figures a
 * benchmark reports beside the published peaks (HBM bandwidth, dense bf16
 * MFMA rate).  Both enqueue one kernel on `stream` and return without
 * synchronising; time them with events.
 *
 * mla_probe_read: stream `bytes` (a multiple of 16, src 16-byte aligned)
 * of device memory once with nontemporal loads.  `sink`: a device word,
 * written only in a case that does not happen in practice (it keeps the
 * loads from being optimised away).  Errors: QKVNR_ERR_NULL_ARG,
 * QKVNR_ERR_BAD_SHAPE, QKVNR_ERR_BAD_ALIGNMENT, QKVNR_ERR_LAUNCH_FAILED.
 *
 * mla_probe_mfma_bf16: 512 workgroups x 4 waves, each wave `iters` steps
 * of four independent v_mfma_f32_32x32x16_bf16 chains: 2^28 * iters flop,
 * no memory traffic in the loop.  `sink` as above.  iters in [1, 2^31],
 * else QKVNR_ERR_BAD_SHAPE. */
int mla_probe_read(const void* src, size_t bytes, void* sink, void* stream);
int mla_probe_mfma_bf16(int64_t iters, void* sink, void* stream);

#ifdef __cplusplus
} /* extern "C" */
#endif

#endif /* QKVNR_H */
