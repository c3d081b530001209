// Internal interface between the C-ABI layer (host.cpp, plain C++) and the
// HIP launchers.  Not installed; the public header is include/qkvnr.h.
// Streams are hipStream_t passed as void*, so this header needs no HIP.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "plan.h"
#include "qkvnr.h"

namespace qkvnr {

// Launch the fused qkv kernel; arguments already validated.
int launch_qkv_rmsnorm_rope_cache(const QkvRmsNormRopeCacheArgs* a, void* stream);

// Pack (batch, K, N) row-major weights into the K16 blocked layout; columns
// from rope_col0 on are rope heads of rope_dim columns, reordered into the
// partner-in-block order when rope_dim > 32 (rope_col0 = N: no rope columns).
// kperm (bf16, K % 16 == 0): within each 16-k step the two 8-k chunks hold
// k offsets {0-3, 8-11} and {4-7, 12-15}.
int launch_pack_weight(const void* src, void* dst, int64_t batch, int64_t K, int64_t N,
                       int elem_bytes, int64_t rope_col0, int64_t rope_dim, void* stream,
                       bool kperm = false);

// MlaPreprocessV2 on the prolog's full-quantisation kernels: RmsNormQuant of
// x first (into the workspace), then the int8 path with the static c^Q
// quant finish.  `a` then holds the equivalent prolog arguments: token_x
// the bf16 x, weight_dq the whole packed (or ND) W^DQKV, smooth_scales_cq
// the c^Q bias.
struct PreprocessExtra {
  const void* gamma_x;  // (He) bf16
  const float* bias_x;  // (He) fp32
  float qs_x, qs_cq;    // the two RmsNormQuant scales
  int8_t* dbg_x_int8;   // optional (T, He) copy of x's codes
};

// Launch the prolog (pre == nullptr) or MlaPreprocessV2; arguments
// validated, workspace large enough.
int launch_mla_prolog_v2(const MlaPrologV2Args* a, const MlaPlan& plan, void* workspace,
                         void* stream, const PreprocessExtra* pre = nullptr);

// The same on this library's fixed per-device scratch array (no_alloc.hip);
// plan.total <= MLA_NO_ALLOC_SCRATCH_BYTES already checked.
int launch_mla_prolog_v2_no_alloc(const MlaPrologV2Args* a, const MlaPlan& plan, void* stream);

// Copy `bytes` of device memory to host memory in stream order and wait for
// the copy (the debug checks only).  QKVNR_OK or QKVNR_ERR_LAUNCH_FAILED.
int copy_to_host_sync(void* host_dst, const void* dev_src, size_t bytes, void* stream);

// Measurement probes (runtime.hip): a streaming read of `bytes` (a multiple
// of 16) from device memory, and a dense bf16 MFMA loop of `iters` steps per
// chain over 512 workgroups x 4 waves x 4 chains.  `sink` is a device word
// that is written only in a case that does not happen.
int probe_read(const void* src, size_t bytes, void* sink, void* stream);
int probe_mfma(int64_t iters, void* sink, void* stream);

}  // namespace qkvnr
