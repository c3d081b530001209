// Internal interface between the C-ABI layer (capi.hip) and the kernel
// launchers.  Not installed; the public header is include/qkvnr.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "qkvnr.h"

namespace qkvnr {

// Launch the fused qkv kernel; arguments already validated.
int launch_qkv_rmsnorm_rope_cache(const QkvRmsNormRopeCacheArgs* a, hipStream_t stream);

// Pack (batch, K, N) row-major weights into the K16 blocked layout; columns
// from rope_col0 on are rope heads of rope_dim columns, reordered into the
// partner-in-block order when rope_dim > 32 (rope_col0 = N: no rope columns).
// kperm (bf16, K % 16 == 0): within each 16-k step the two 8-k chunks hold
// k offsets {0-3, 8-11} and {4-7, 12-15}.
int launch_pack_weight(const void* src, void* dst, int64_t batch, int64_t K, int64_t N,
                       int elem_bytes, int64_t rope_col0, int64_t rope_dim, hipStream_t stream,
                       bool kperm = false);

// Execution plan of one MlaPrologV2 call: which kernel family runs, the
// split-K factor of the down projection and the workspace carve-up.  A pure
// function of the arguments, so workspace sizing and execution agree.
struct MlaPlan {
  bool skinny;        // decode-sized T: weight-streaming kernels
  bool gemm256;       // large T, bf16: 256x256-tile MFMA GEMMs
  bool fuse_uk;       // gemm256 with the W^UK product fused into A6's q^C tiles
  int mb;             // 32-row blocks held per wave (skinny only)
  int ksplit;         // down-projection split-K factor
  int64_t steps_per_split;
  // workspace offsets (bytes) and total size
  size_t off_wdq, off_wdkvkr, off_wuqqr, off_wuk;  // packed weights (ND layout only)
  size_t off_part, off_cq, off_cq_scale, off_qc;
  size_t off_qn;      // FULL_KV_INT8: q^N in fp32 before its per-head quant
  size_t off_xfrag;   // token_x in fragment layout (256-tile plan)
  int64_t rows;       // token rows padded to the plan's 32-row blocks
  size_t total;
};

MlaPlan make_mla_plan(const MlaPrologV2Args* a);

// Launch the prolog; arguments validated, workspace large enough.
int launch_mla_prolog_v2(const MlaPrologV2Args* a, const MlaPlan& plan, void* workspace,
                         hipStream_t stream);

}  // namespace qkvnr
