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

// Pack (batch, K, N) row-major weights into the K16 blocked layout.
int launch_pack_weight(const void* src, void* dst, int64_t batch, int64_t K, int64_t N,
                       int elem_bytes, hipStream_t stream);

// Execution plan of one MlaPrologV2 call: which kernel family runs, the
// split-K factor of the down projection and the workspace carve-up.  A pure
// function of the arguments, so workspace sizing and execution agree.
struct MlaPlan {
  bool fused;         // persistent fused decode kernel (T <= 32, bf16)
  bool skinny;        // decode-sized T: weight-streaming kernels
  int mb;             // 32-row blocks held per wave (skinny only)
  int ksplit;         // down-projection split-K factor
  int64_t steps_per_split;
  // workspace offsets (bytes) and total size
  size_t off_wdq, off_wdkvkr, off_wuqqr, off_wuk;  // packed weights (ND layout only)
  size_t off_part, off_cq, off_cq_scale, off_qc;
  size_t off_xfrag;   // token_x in fragment layout (skinny plan)
  size_t off_fused;   // start of the fused path's region (fused plan)
  int64_t rows;       // token rows padded to the plan's 32-row blocks
  size_t total;
};

MlaPlan make_mla_plan(const MlaPrologV2Args* a);

// Fused decode path (mla_decode_fused.hip).
struct FusedLayout {
  size_t off_bar, off_part, off_cq, off_qc, off_yrope, off_xfrag, total;
};
bool mla_fused_supported(const MlaPrologV2Args* a);
void mla_fused_layout(const MlaPrologV2Args* a, int64_t ksplit, FusedLayout* layout);
int launch_mla_decode_fused(const MlaPrologV2Args* a, const MlaPlan& plan, void* workspace,
                            const void* wdq, const void* wdkvkr, const void* wuqqr,
                            const void* wuk, hipStream_t stream);

// Launch the prolog; arguments validated, workspace large enough.
int launch_mla_prolog_v2(const MlaPrologV2Args* a, const MlaPlan& plan, void* workspace,
                         hipStream_t stream);

}  // namespace qkvnr
