// Execution plan of one MlaPrologV2 call and the launch-shape constants it
// is computed from.  Host-only C++ (no HIP): the entry points in host.cpp
// size the workspace from it and the launchers in mla_prolog_v2.hip execute
// it, so sizing and execution always agree.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "qkvnr.h"

namespace qkvnr {

// Prefill GEMM tile width (columns) and the height of its two-per-CU tiles.
constexpr int G_TN = 256;
constexpr int G_TM_HALF = 128;
// Most split-K partials the down-projection finish sums, and the bound of
// the large-T plan's split factor (its finish is instantiated for it).
constexpr int FIN_MAXSPLIT = 8;
constexpr int FIN_SPLIT_SMALL = 4;
// Decode down-projection tile width: two 32-column blocks.
constexpr int kA1Cols = 64;
// Handoff counters of the merged decode launch: one per 256-byte line
// (SYNC_STRIDE uint32 apart).
constexpr int SYNC_STRIDE = 64;

// Which kernel family runs, the split-K factor of the down projection and
// the workspace carve-up.  A pure function of the arguments.
struct MlaPlan {
  bool skinny;        // decode-sized T: weight-streaming kernels
  bool gemm256;       // large T (every mode): LDS-pipelined MFMA GEMMs
  bool fuse_uk;       // gemm256 with the W^UK product fused into A6's q^C tiles
                      // (bf16, or int8 with q^C as bf16 hi + lo)
  bool merge_uk;      // skinny bf16, one row block: A6 and the W^UK product in
                      // one launch (k_decode_tail), handing q^C over per head
  bool merge_uk_q;    // skinny quantised with a bf16 query, at most two row
                      // blocks, few up-projection columns: the same in one
                      // launch with fp32 q^C (k_decode_tail_q)
  bool qh;            // FULL_KV_INT8 decode, one row block, Hckv <= 512: the
                      // query quant runs in the W^UK product's epilogue
  int mb;             // 32-row blocks held per wave (skinny only)
  int ksplit;         // down-projection split-K factor
  int64_t steps_per_split;
  // workspace offsets (bytes) and total size
  size_t off_wdq, off_wdkvkr, off_wuqqr, off_wuk;  // packed weights (ND layout only)
  size_t off_part, off_cq, off_cq_scale, off_qc;
  size_t off_qn;      // FULL_KV_INT8 without qh: q^N in fp32 before its
                      // per-head quant
  size_t off_xfrag;   // token_x in fragment layout (256-tile plan)
  size_t off_sync;    // merge_uk(_q): N per-head handoff counters, one per
                      // 256-byte line
  size_t off_prex8, off_presx;  // MlaPreprocessV2: RmsNormQuant codes of x
                                // (T, He) int8 and their unit token scales
  int64_t rows;       // token rows padded to the plan's 32-row blocks
  size_t total;
};

// Arguments must have passed validation.
MlaPlan make_mla_plan(const MlaPrologV2Args* a);

// MlaPreprocessV2 runs on the full-quantisation plan of the equivalent
// prolog arguments `m`, plus room for the RmsNormQuant codes of x.
MlaPlan make_preprocess_plan(const MlaPrologV2Args* m);

}  // namespace qkvnr
