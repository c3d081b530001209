// MlaPrologV2 on gfx950 ("MlaPrologV2" README, ops-transformer: function
// description and formulas; parameter table; constraints incl. the
// quantisation-scenario and dtype/shape tables).
//
//   A1  h = x . W^DQ, g = x . [W^DKV | W^KR]   one logical GEMM, N = Hcq+Hckv+Dr
//   A2  c^Q = RmsNorm(h)                       (+ smooth, per-token int8 in the
//                                               partial-quant scenarios)
//   A3  c^KV = RmsNorm(g[:, :Hckv])  -> kv_cache[cache_index[t]]
//   A4  k^R = RoPE(g[:, Hckv:])      -> kr_cache[cache_index[t]]
//   A6  y = c^Q . [W^UQ | W^QR]                (int8 x int8 -> int32, dequant
//                                               per token x per channel)
//   A7  q^R = RoPE(y[:, N*D:])       -> query_rope; q^C = y[:, :N*D]
//   A8  q^N[:, n] = q^C[:, n] . W^UK[n] -> query
//
// Two plans.  Decode-sized T (<= 128) streams every weight byte exactly once
// through "skinny" kernels: each wave owns a 32-column slice of the packed
// weight and a range of K, holds all T rows (up to four 32-row MFMA blocks)
// in registers, and the down projection is split over K across workgroups
// with fp32 partials reduced in a fixed order (deterministic, no atomics).
// Larger T uses 128x128 LDS-tiled MFMA GEMMs.  Both share the epilogues.
//
// Weights arrive in the K16 blocked layout (see mla_pack_weight in the
// public header): the 8 (bf16) or 16 (int8) consecutive-k values of one
// column are one 16-byte chunk, which is exactly one lane's MFMA operand.
#include <hip/hip_ext.h>

#include <algorithm>
#include <type_traits>

#include "device_common.h"
#include "launch.h"
#include "mla_device.h"

namespace qkvnr {

namespace {

enum EpiKind { EPI_PARTIAL = 0, EPI_UQQR = 1, EPI_UK = 2, EPI_QN = 3 };

struct GemmParams {
  // A: activations.  Row-major (a_frag == 0): row m of batch z starts at
  // A + z*a_bstride + m*lda (element units of the A type).  Fragment layout
  // (a_frag == 1, skinny kernels only): the 32-row block mb, k-step s of
  // batch z is 64 lanes x CB contiguous bytes at
  // A + z*a_zs + mb*a_mbs + s*64*CB, lane (g, i) holding row 32*mb + i and
  // the k-step's g-th half (CB = 16, or 32 for fp32 A).
  const void* A;
  int64_t lda;
  int64_t a_bstride;
  int a_frag;
  int64_t a_mbs, a_zs;
  // B: packed weights as 16-byte chunks; chunk (kc, n) at kc*N + n.  Tiles
  // [0, ntiles0) read B0 (N0 columns), the rest read B1 (N1 columns, output
  // columns offset by N0).  Batch z adds z*b_bstride chunks.
  const uint4* B0;
  int64_t N0;
  const uint4* B1;
  int64_t N1;
  int64_t b_bstride;
  int64_t M, K;
  int64_t KB;  // k_gemm: B's K when it is shorter than A's (EPI_UK over q^C
               // hi | lo: A's k-step s pairs with B's k-step s mod KB-steps);
               // 0: KB = K
  int ntiles0;
  int64_t steps_per_split;  // k-steps handled per blockIdx.y
  // EPI_PARTIAL: part[m][part_ld] of this launch's split (the skinny kernel
  // offsets it by its split index)
  float* part;
  int64_t part_ld;
  // EPI_UQQR
  int64_t ND;  // N*D: first rope column
  int Dr;
  const uint16_t* cosb;  // (T, Dr)
  const uint16_t* sinb;
  const float* cq_scale;  // (T) per-token scale (int8 A)
  const float* dq;        // per-column dequant (int8 A)
  void* qc_out;           // (T, N*D): bf16, or fp32 when qc_f32
  int qc_f32;
  int qc_frag;            // write q^C in per-head fragment layout
  int64_t qc_D;           // head dim D (fragment layout)
  int64_t qc_mblocks;     // 32-row blocks per head (fragment layout)
  int qc_coherent;        // fragment q^C (bf16 or fp32) with device-scope
                          // stores, for a consumer in the same launch
                          // (k_decode_tail, k_decode_tail_q)
  int qc_split;           // fragment q^C as bf16 hi and lo = bf16(v - hi):
                          // per head 2*D k, hi in k-steps [0, D/16), lo after
  // Handoff words of the merged decode launch that this launch zeroes
  // first (workgroup 0), SYNC_STRIDE words apart; NULL: none.
  unsigned* zero_words;
  int zero_count;
  uint16_t* qr_out;  // (T, N, Dr)
  int64_t qr_ld;     // N*Dr
  // EPI_UK (and EPI_QN's output)
  uint16_t* q_out;  // (T, N, Hckv)
  float* q_f32;     // when set, q^N goes here in fp32 instead (same indexing)
  // EPI_UK with the per-(token, head) int8 quantisation fused (QH): codes
  // (T, N, Hckv) and scales (T, N), one workgroup covering a head's Hckv
  int8_t* q8_out;
  float* q8_scale;
  int64_t q_ld;     // N*Hckv
  int64_t q_bstride;  // Hckv (per head)
  // EPI_QN: q^C never leaves registers; the W^UK product runs in the
  // epilogue.  Buk: packed W^UK (heads uk_bstride chunks apart), uk_N = Hckv;
  // qc_D is the head dim D.
  const uint4* Buk;
  int64_t uk_bstride;
  int64_t uk_N;
};

// ---------------------------------------------------------------------------
// Epilogue over 8 consecutive output columns of one row.  `v` are the raw
// accumulator sums (int32 bit patterns for int8 A), `vp` the same for the
// RoPE partner columns (col +/- Dr/2) when the columns are rope columns.
// ---------------------------------------------------------------------------
template <int AK, int EPI>
struct Epilogue {
  static __device__ __forceinline__ void to_float(const uint32_t* raw, float* v) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      v[e] = (AK == A_I8) ? static_cast<float>(static_cast<int>(raw[e])) : __uint_as_float(raw[e]);
  }

  // Does this 8-column group need its RoPE partner, and where is it (offset
  // in packed columns relative to the group)?  The rope region starts on a
  // 32-column block and its packed order keeps every partner in the same
  // block: Dr = 16 pairs columns 8 apart, Dr = 32 and the reordered Dr = 64
  // pair columns 16 apart.
  // (Column and row indexes fit 32 bits: N*(D+Dr) < 2^31 and T <= 2^23
  // are validated, so the index arithmetic below is 32-bit.)
  static __device__ __forceinline__ int partner_offset(const GemmParams& p, int64_t gcol) {
    if (EPI != EPI_UQQR || gcol < p.ND) return 0;
    const int w = static_cast<int>((gcol - p.ND) & 31);
    const int hp = p.Dr >= 32 ? 16 : (p.Dr >> 1);
    return (w & (2 * hp - 1)) < hp ? hp : -hp;
  }

  // Natural rope index (position within the head's Dr columns) of packed
  // rope column r = gcol - ND.  For Dr = 64, packed block b of a head holds
  // natural columns [16b, 16b + 16) then [32 + 16b, 32 + 16b + 16).
  static __device__ __forceinline__ int rope_index(const GemmParams& p, int64_t r) {
    const int pj = static_cast<int>(static_cast<uint32_t>(r) % static_cast<uint32_t>(p.Dr));
    if (p.Dr <= 32) return pj;
    const int b = pj >> 5, w = pj & 31;
    return w < 16 ? 16 * b + w : (p.Dr >> 1) + 16 * b + (w - 16);
  }

  // Everything the epilogue of one 8-column group reads from global memory
  // besides the accumulators: the token's RoPE cos/sin for rope columns and,
  // for int8 A, the token's scale and the columns' (and partners')
  // dequant scales.  Loaded by prefetch() before the main loop so the
  // epilogue does not wait on memory.
  struct Pre {
    uint4 c4, s4;
    float cs;
    float d[8], dp[8];
  };

  // Branch-free: every address is valid for any in-range (m, gcol), so the
  // loads can stay in flight across the main loop (a load under a divergent
  // branch would be waited for at the branch's join).
  static __device__ __forceinline__ Pre prefetch(const GemmParams& p, int64_t m, int64_t gcol) {
    Pre r{};
    if constexpr (EPI == EPI_UQQR) {
      const bool rope = gcol >= p.ND;
      const int64_t rr = rope ? gcol - p.ND : 0;
      const int i0 = rope_index(p, rr);
      const int half = p.Dr >> 1;
      const uint32_t hd = static_cast<uint32_t>(rr) / static_cast<uint32_t>(p.Dr);
      const int64_t ncol = rope ? p.ND + static_cast<int64_t>(hd) * p.Dr + i0 : gcol;
      const int64_t pcol = rope ? (i0 < half ? ncol + half : ncol - half) : gcol;
      r.c4 = ld16(p.cosb + m * p.Dr + i0);
      r.s4 = ld16(p.sinb + m * p.Dr + i0);
      if constexpr (AK == A_I8) {
        r.cs = gld(p.cq_scale + m);
        ld8f(p.dq + ncol, r.d);
        ld8f(p.dq + pcol, r.dp);
      }
    }
    return r;
  }

  static __device__ __forceinline__ void dequant(float s, const float* d, float* v) {
    if constexpr (AK == A_I8) {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = v[e] * s * d[e];
    }
  }

  // m: token row; gcol: column within this weight; ocol: output column in
  // the partial buffer (gcol + offset of B1); z: batch (head) index; pre:
  // prefetch(p, m, gcol).
  static __device__ __forceinline__ void apply(const GemmParams& p, int64_t m, int64_t gcol,
                                               int64_t ocol, int z, const uint32_t* raw,
                                               const uint32_t* raw_partner, const Pre& pre) {
    float v[8];
    to_float(raw, v);
    if constexpr (EPI == EPI_PARTIAL) {
      st8f(p.part + m * p.part_ld + ocol, v);
    } else if constexpr (EPI == EPI_UK) {
      const int64_t o = m * p.q_ld + static_cast<int64_t>(z) * p.q_bstride + gcol;
      if (p.q_f32 != nullptr) {
        st8f(p.q_f32 + o, v);  // full quantisation: quantised per (token, head) next
      } else {
        st16_nt(p.q_out + o, make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                        pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])));
      }
    } else {  // EPI_UQQR
      if (gcol < p.ND) {
        dequant(pre.cs, pre.d, v);
        // 8 columns of q^C = 8 consecutive k of one head: one A chunk of the
        // per-head product in fragment layout, or 8 row-major elements.
        if (p.qc_frag) {
          // The W^UK product's A operand, in the k order of the packed W^UK:
          // within a 16-k step, lane half h holds d offsets {4h..4h+3} in
          // slots 0-3 and {8+4h..8+4h+3} in slots 4-7.  These 8 columns
          // (d0 = 8*(d/8)) split into two 4-element halves.
          const uint32_t gc = static_cast<uint32_t>(gcol), D = static_cast<uint32_t>(p.qc_D);
          const uint32_t head = gc / D, d = gc - head * D;
          const uint32_t mm = static_cast<uint32_t>(m);
          const uint32_t hsteps = (D >> 4) * (p.qc_split ? 2u : 1u);  // k-steps per head
          const int64_t base =
              ((static_cast<int64_t>(head) * p.qc_mblocks + (mm >> 5)) * hsteps + (d >> 4)) * 512 +
              (mm & 31) * 8 + ((d >> 3) & 1) * 4;  // slots 0-3 or 4-7
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const int64_t off = base + hh * 32 * 8;  // lane half hh
            if (p.qc_split) {
              uint32_t hw[2], lw[2];
#pragma unroll
              for (int e = 0; e < 2; ++e) {
                const float a = v[4 * hh + 2 * e], b = v[4 * hh + 2 * e + 1];
                const uint16_t ha = f32_to_bf16(a), hb = f32_to_bf16(b);
                hw[e] = static_cast<uint32_t>(ha) | (static_cast<uint32_t>(hb) << 16);
                lw[e] = pack_bf16x2(a - bf16_to_f32(ha), b - bf16_to_f32(hb));
              }
              uint16_t* q = static_cast<uint16_t*>(p.qc_out);
              st8(q + off, make_uint2(hw[0], hw[1]));
              st8(q + off + static_cast<int64_t>(D >> 4) * 512, make_uint2(lw[0], lw[1]));
            } else if (p.qc_f32) {
              const uint4 f = make_uint4(__float_as_uint(v[4 * hh]), __float_as_uint(v[4 * hh + 1]),
                                         __float_as_uint(v[4 * hh + 2]), __float_as_uint(v[4 * hh + 3]));
              if (p.qc_coherent)  // (decode q^C, < 2^31 bytes: one resource)
                bst16_dev(make_rsrc(p.qc_out, 0x7fffffffu), static_cast<uint32_t>(off) * 4u, f);
              else
                st16(static_cast<float*>(p.qc_out) + off, f);
            } else if (p.qc_coherent) {
              // decode q^C (< 2^31 bytes): one resource over the buffer
              bst8_dev(make_rsrc(p.qc_out, 0x7fffffffu), static_cast<uint32_t>(off) * 2u,
                       make_uint2(pack_bf16x2(v[4 * hh], v[4 * hh + 1]),
                                  pack_bf16x2(v[4 * hh + 2], v[4 * hh + 3])));
            } else {
              st8(static_cast<uint16_t*>(p.qc_out) + off,
                  make_uint2(pack_bf16x2(v[4 * hh], v[4 * hh + 1]),
                             pack_bf16x2(v[4 * hh + 2], v[4 * hh + 3])));
            }
          }
        } else {
          const int64_t off = m * p.ND + gcol;
          if (p.qc_f32) {
            st8f(static_cast<float*>(p.qc_out) + off, v);
          } else {
            st16(static_cast<uint16_t*>(p.qc_out) + off,
                 make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                            pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])));
          }
        }
      } else {
        const int64_t r = gcol - p.ND;
        const int64_t head = static_cast<uint32_t>(r) / static_cast<uint32_t>(p.Dr);
        const int i0 = rope_index(p, r);
        const int half = p.Dr >> 1;
        dequant(pre.cs, pre.d, v);
        float w[8];
        to_float(raw_partner, w);
        dequant(pre.cs, pre.dp, w);
        const uint32_t cw[4] = {pre.c4.x, pre.c4.y, pre.c4.z, pre.c4.w};
        const uint32_t sw[4] = {pre.s4.x, pre.s4.y, pre.s4.z, pre.s4.w};
        float o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float c = (e & 1) ? bf16hi(cw[e >> 1]) : bf16lo(cw[e >> 1]);
          const float s = (e & 1) ? bf16hi(sw[e >> 1]) : bf16lo(sw[e >> 1]);
          // cat(-y2, y1) * sin: first half subtracts the partner
          o[e] = i0 < half ? v[e] * c - w[e] * s : v[e] * c + w[e] * s;
        }
        uint16_t* out = p.qr_out + m * p.qr_ld + head * p.Dr + i0;
        st16_nt(out, make_uint4(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]),
                             pack_bf16x2(o[4], o[5]), pack_bf16x2(o[6], o[7])));
      }
    }
  }
};

// ---------------------------------------------------------------------------
// Skinny GEMM (decode): all M (<= 32*MB) rows stay in registers while the
// weight streams past.  A workgroup owns a tile of NW*NB 32-column blocks and
// a K range split over KW waves; each wave streams NB column blocks over its
// K sub-range.  In the N32-blocked packed layout one k-step of one column
// block is 1 KB contiguous (64 lanes x 16 B), and a wave's whole K sub-range
// is one contiguous run, read exactly once.  Loads are software-pipelined in
// register batches of P k-steps (the next batch is in flight while the
// current one feeds the MFMAs).  The KW partial tiles are summed in LDS in
// wave order (deterministic), then the epilogue runs on 8-column groups.
// ---------------------------------------------------------------------------
template <int AK, int MB, int NB>
struct SkinnyDepth {
  // k-steps per register batch: about 32 VGPRs of loads per batch (two
  // batches live), the rest of the in-flight bytes coming from many waves.
  static constexpr int per_step = NB + MB * ((AK == A_F32SPLIT) ? 2 : 1);
  static constexpr int value = (8 / per_step) > 0 ? (8 / per_step) : 1;
};

// ---------------------------------------------------------------------------
// Handoff counters between the workgroups of the merged decode launch
// (k_decode_tail) sit in the workspace one per 256-byte line (SYNC_STRIDE
// words apart, plan.h): hundreds of workgroups polling a few shared lines
// measured 4 us slower than the same polls spread over lines.  The down
// projection, the launch before, zeroes them.
// ---------------------------------------------------------------------------
constexpr uint32_t SYNC_SPIN_LIMIT = 1u << 18;  // polls before a wait gives up

// A_LDS_STEPS: most k-steps of one split whose A operand (32 rows, bf16) a
// workgroup stages in LDS by default (64 KB).
constexpr int A_LDS_STEPS = 64;

// Where the skinny kernel's A operand comes from: global memory on every
// k-step, or staged once per workgroup in LDS (in fragment order) from a
// row-major or a fragment-layout A.  Staging reads A once per workgroup
// instead of once per wave, and leaves the vector-memory queue to the weight
// stream.
enum { ALDS_NONE = 0, ALDS_ROWMAJOR = 1, ALDS_FRAG = 2 };

// One tile of the skinny GEMM: tile bx (column tiles of B0 then of B1),
// split by, batch bz; run by a 64*NW*KW-thread workgroup, plus XW extra
// waves that skip the main loop and share the epilogue.
template <int AK, int MB, int NB, int NW, int KW, int EPI,
          int P = SkinnyDepth<AK, MB, NB>::value, int ALDS = ALDS_NONE, int ACAP = A_LDS_STEPS,
          bool QH = false, int XW = 0>
__device__ __forceinline__ void skinny_tile(const GemmParams& p, const int bx, const int by,
                                            const int bz) {
  static_assert(XW == 0 || (ALDS == ALDS_NONE && !QH), "extra waves: plain tiles only");
  constexpr int NALL = 64 * (NW * KW + XW);  // threads of the workgroup
  typedef typename AccT<AK>::type Acc;
  constexpr int KSTEP = (AK == A_I8) ? 32 : 16;  // k per MFMA
  constexpr int G = (AK == A_I8) ? 16 : 8;       // k per 16-byte chunk
  constexpr int TN = 32 * NB * NW;
  constexpr int PITCH = TN + 4;  // words per LDS row
  constexpr int NA = (AK == A_F32SPLIT) ? 2 : 1;  // 16-byte A loads per fragment
  // LDS-staged A, up to ACAP k-steps of this workgroup's split: row-major
  // bf16 A, or fragment-layout bf16 or fp32-split A (MB row blocks).  Chunk
  // n (of NA) of lane `lane`, k-step s, row block mb sits at
  // ((mb*NA + n)*ACAP + s - s_lo)*64 + lane, so each wave's read of one
  // operand chunk is 64 consecutive 16-byte words.
  static_assert(ALDS == ALDS_NONE || (ALDS == ALDS_ROWMAJOR && MB <= 2 && AK != A_F32SPLIT) ||
                    (ALDS == ALDS_FRAG && AK != A_I8),
                "LDS-staged A: row-major bf16 or int8 (one or two row blocks), or bf16 / fp32 "
                "fragments");
  // The waves' partial tiles (summed over KW in the epilogue).  With two
  // row-major row blocks staged, they share the staged A's memory (both
  // together would exceed the CU's 160 KB): a barrier separates the main
  // loop's last A read from the first partial-tile write.
  constexpr bool ALIAS = ALDS == ALDS_ROWMAJOR && MB > 1;
  constexpr int ALDS_CH = ALDS != ALDS_NONE ? ACAP * 64 * NA * MB : 1;
  constexpr int TILE_CH = (KW * MB * 32 * PITCH + 3) / 4;
  __shared__ uint4 alds[ALIAS && TILE_CH > ALDS_CH ? TILE_CH : ALDS_CH];
  __shared__ uint32_t lds_own[ALIAS ? 1 : KW][ALIAS ? 1 : MB * 32][ALIAS ? 1 : PITCH];
  typedef uint32_t TileLds[KW][MB * 32][PITCH];
  TileLds& lds = *reinterpret_cast<TileLds*>(ALIAS ? static_cast<void*>(alds)
                                                   : static_cast<void*>(lds_own));

  const int lane = threadIdx.x & 63;
  // Wave-level quantities live in SGPRs: the per-step load offsets below are
  // scalar, so the loop's address arithmetic costs no VGPRs.
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const bool active = wave < NW * KW;  // a streaming wave (wave-uniform)
  const int nw = wave % NW;
  const int kw = active ? wave / NW : 0;
  const int g = lane >> 5;
  const int li = lane & 31;
  const int z = bz;

  // (the weight pointer is chosen arithmetically: a branch over the two
  // kernel-argument pointers has been lowered to a private-memory table)
  const bool second = bx >= p.ntiles0;
  const uint4* B = reinterpret_cast<const uint4*>(
      second ? reinterpret_cast<uintptr_t>(p.B1) : reinterpret_cast<uintptr_t>(p.B0));
  const int64_t N = second ? p.N1 : p.N0;
  const int64_t n0 = static_cast<int64_t>(second ? bx - p.ntiles0 : bx) * TN;
  const int64_t ocol0 = second ? p.N0 : 0;
  B += static_cast<int64_t>(z) * p.b_bstride;
  const int KC = static_cast<int>(p.K / G);  // 16-byte chunk rows per column

  const int nsteps = static_cast<int>(p.K / KSTEP);
  const int s_lo = static_cast<int>(by * p.steps_per_split);
  const int s_hi = min(s_lo + static_cast<int>(p.steps_per_split), nsteps);
  const int cnt = s_hi > s_lo ? s_hi - s_lo : 0;
  const int w_lo = s_lo + cnt * kw / KW;
  const int w_hi = s_lo + cnt * (kw + 1) / KW;

  // Column blocks of this wave: chunk (block nb, row kc, column j) sits at
  // (nb*KC + kc)*32 + j, and lane (g, j) of k-step s reads row 2s+g, so the
  // lane's chunk for step s is 16*lane + 1024*s bytes into the block's run.
  //
  // Every load below is unconditional: a column block past N, a row past M
  // and a step past the wave's range are clamped to valid memory and their
  // products are never stored (rows and columns of a product are
  // independent).  Branch-free loads let the compiler wait only for the
  // batch being consumed instead of draining every load in flight.
  const int64_t nblk = (N + 31) / 32;
  rsrc_t rb[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    int64_t nb = n0 / 32 + nw * NB + b;
    nb = nb < nblk ? nb : nblk - 1;
    rb[b] = make_rsrc(B + nb * KC * 32, static_cast<uint32_t>(KC) * 512u);
  }
  const uint32_t vb = static_cast<uint32_t>(lane) * 16u;

  constexpr int AEB = (AK == A_I8) ? 1 : (AK == A_F32SPLIT ? 4 : 2);  // A element bytes
  constexpr int CB = (AK == A_F32SPLIT) ? 32 : 16;  // A bytes per lane per k-step
  rsrc_t ra[MB];
  uint32_t va[MB];     // lane's byte offset into its A resource
  uint32_t astep;      // A bytes between consecutive k-steps (scalar)
  if (p.a_frag) {
    const char* base = static_cast<const char*>(p.A) + static_cast<int64_t>(z) * p.a_zs;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      ra[mb] = make_rsrc(base + mb * p.a_mbs, static_cast<uint32_t>(nsteps) * 64u * CB);
      va[mb] = static_cast<uint32_t>(lane) * CB;
    }
    astep = 64 * CB;
  } else {
    const char* base =
        static_cast<const char*>(p.A) + (static_cast<int64_t>(z) * p.a_bstride) * AEB;
    const uint32_t a_row_bytes = static_cast<uint32_t>(p.lda) * AEB;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      int m = mb * 32 + li;
      m = m < p.M ? m : static_cast<int>(p.M) - 1;
      // bf16: 16 k = 32 bytes per step, lane group g takes bytes [16g, 16g+16);
      // int8: 32 k = 32 bytes, same offsets; fp32: 16 k = 64 bytes, group g
      // takes [32g, 32g+32).
      ra[mb] = make_rsrc(base, static_cast<uint32_t>(p.M) * a_row_bytes);
      va[mb] = static_cast<uint32_t>(m) * a_row_bytes + g * CB;
    }
    astep = 2 * CB;
  }

  // Epilogue operands of this thread's first 8-column group, loaded now so
  // they arrive during the main loop.
  constexpr int GROUPS = MB * 32 * (TN / 8);
  typedef Epilogue<AK, EPI> Epi;
  typename Epi::Pre pre0;
  {
    // clamped into range; the values of clamped groups are never used
    int64_t m = static_cast<int>(threadIdx.x % GROUPS) / (TN / 8);
    int64_t gcol = n0 + (threadIdx.x % (TN / 8)) * 8;
    m = m < p.M ? m : p.M - 1;
    gcol = gcol < N ? gcol : N - 8;
    pre0 = Epi::prefetch(p, m, gcol);
  }

  Acc acc[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[mb][b] = Acc{};

  // One register batch: B chunks and raw A chunks of P k-steps.
  struct Batch {
    uint4 b[P][NB];
    uint4 a[P][MB][NA];
  };
  const int s_last = w_hi - 1;
  auto load_b = [&](Batch& x, int s0) {
#pragma unroll
    for (int u = 0; u < P; ++u) {
      int s = (s0 + u) < s_last ? (s0 + u) : s_last;
      s = s > 0 ? s : 0;  // a wave with an empty range still loads in bounds
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        // streaming loads for the up projections' weights (A6 15.3 vs 16.0
        // us); the down projection measured faster with cached loads
        if constexpr (EPI == EPI_PARTIAL)
          x.b[u][b] = bld16(rb[b], vb, static_cast<uint32_t>(s) * 1024u);
        else
          x.b[u][b] = bld16_nt(rb[b], vb, static_cast<uint32_t>(s) * 1024u);
      }
    }
  };
  // Row-major staged A is read from LDS where each MFMA uses it (so a batch
  // holds only weight chunks and can cover a wave's whole k range); the
  // other staged forms are read a batch ahead like the global ones.
  constexpr bool A_AT_USE = ALDS == ALDS_ROWMAJOR;
  auto load_a = [&](Batch& x, int s0) {
    if constexpr (A_AT_USE) return;
#pragma unroll
    for (int u = 0; u < P; ++u) {
      const int s = (s0 + u) < s_last ? (s0 + u) : s_last;
      if constexpr (ALDS != ALDS_NONE) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int n = 0; n < NA; ++n)
            x.a[u][mb][n] = alds[((mb * NA + n) * ACAP + (s - s_lo)) * 64 + lane];
      } else {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          x.a[u][mb][0] = bld16(ra[mb], va[mb], static_cast<uint32_t>(s) * astep);
          if constexpr (AK == A_F32SPLIT)
            x.a[u][mb][1] = bld16(ra[mb], va[mb] + 16u, static_cast<uint32_t>(s) * astep);
        }
      }
    }
  };
  auto load = [&](Batch& x, int s0) {
    load_b(x, s0);
    load_a(x, s0);
  };
  auto compute = [&](const Batch& x, int s0, int count) {
#pragma unroll
    for (int u = 0; u < P; ++u) {
      if (u >= count) break;  // wave-uniform; only MFMAs are skipped
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        if constexpr (A_AT_USE) {
          const uint4 av = alds[(mb * ACAP + (s0 + u - s_lo)) * 64 + lane];
#pragma unroll
          for (int b = 0; b < NB; ++b) mfma_step<AK>(acc[mb][b], av, x.b[u][b]);
          continue;
        }
        if constexpr (AK == A_F32SPLIT) {
          uint4 hi, lo;
          const uint4 r0 = x.a[u][mb][0], r1 = x.a[u][mb][1];
          split8(make_float4(__uint_as_float(r0.x), __uint_as_float(r0.y), __uint_as_float(r0.z),
                             __uint_as_float(r0.w)),
                 make_float4(__uint_as_float(r1.x), __uint_as_float(r1.y), __uint_as_float(r1.z),
                             __uint_as_float(r1.w)),
                 hi, lo);
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            mfma_step<AK>(acc[mb][b], hi, x.b[u][b]);
            mfma_step<AK>(acc[mb][b], lo, x.b[u][b]);
          }
        } else {
#pragma unroll
          for (int b = 0; b < NB; ++b) mfma_step<AK>(acc[mb][b], x.a[u][mb][0], x.b[u][b]);
        }
      }
    }
  };

  // Ping-pong over batches: the next batch's loads are issued before the
  // current batch's MFMAs.  The last prefetch re-reads the final batch (cache
  // hits) so the load sequence never depends on a branch.
  Batch X, Y;
  if constexpr (ALDS == ALDS_FRAG) if (cnt > 0) {  // cnt is uniform over the workgroup
    // Fragment-layout A: per row block the split's chunks are one
    // contiguous run of 64*NA*cnt 16-byte chunks (cnt <= ACAP); chunk r of
    // row block mb is lane (r / NA) % 64, part r % NA, k-step s_lo + r /
    // (64*NA), and lands at its LDS slot.
    constexpr int NT = 64 * NW * KW;
    constexpr int PER = (ACAP * 64 * NA * MB + NT - 1) / NT;
    const int run = 64 * NA * cnt;  // chunks per row block
    const int total = MB * run;
    const rsrc_t rx = make_rsrc(static_cast<const char*>(p.A) + static_cast<int64_t>(z) * p.a_zs,
                                static_cast<uint32_t>(MB * p.a_mbs));
    uint4 st[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      int c = static_cast<int>(threadIdx.x) + i * NT;
      c = c < total ? c : total - 1;
      const int mb = c / run, r = c - mb * run;
      st[i] = bld16(rx,
                    static_cast<uint32_t>(mb * p.a_mbs) +
                        (static_cast<uint32_t>(s_lo) * 64u * NA + static_cast<uint32_t>(r)) * 16u,
                    0u);
    }
    load_b(X, w_lo);  // unconditional: a branch here would drain the staging loads
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = static_cast<int>(threadIdx.x) + i * NT;
      if (c < total) {
        const int mb = c / run, r = c - mb * run;
        const int ls = r / (64 * NA), rem = r - ls * 64 * NA;
        alds[((mb * NA + rem % NA) * ACAP + ls) * 64 + rem / NA] = st[i];
      }
    }
    lds_barrier();  // keeps the first weight batch in flight
    if (w_lo < w_hi) load_a(X, w_lo);
  }
  if constexpr (ALDS == ALDS_ROWMAJOR) if (cnt > 0) {
    // Stage rows 0..32*MB-1 of A over this split's k range [16*s_lo,
    // 16*s_hi): thread c of the 64*cnt*MB 16-byte chunks takes row
    // c / (2*cnt), chunk c % (2*cnt), so each wave reads 1 KB of consecutive
    // row bytes.  Rows past M repeat row M-1 (their products are never
    // stored); surplus threads repeat the last chunk.  The loads are issued
    // before the first weight batch, so both are in flight together.
    constexpr int NT = 64 * NW * KW;
    constexpr int PER = (ACAP * 64 * MB + NT - 1) / NT;
    const int total = 64 * cnt * MB;
    const int per_row = 2 * cnt;
    // Buffer loads like the weight stream (loads of one kind complete in
    // order, so waiting for these does not drain the weight batch).
    // (a k-step is 32 bytes of a row: 16 bf16 or 32 int8 k)
    const rsrc_t rx = make_rsrc(static_cast<const char*>(p.A) + static_cast<int64_t>(s_lo) * 32,
                                static_cast<uint32_t>(p.M * p.lda * AEB - s_lo * 32));
    uint4 st[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      int c = static_cast<int>(threadIdx.x) + i * NT;
      c = c < total ? c : total - 1;
      int m = c / per_row;
      m = m < p.M ? m : static_cast<int>(p.M) - 1;
      st[i] = bld16(rx, static_cast<uint32_t>(m * p.lda * AEB + (c % per_row) * 16), 0u);
    }
    load_b(X, w_lo);  // unconditional: a branch here would drain the staging loads
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      int c = static_cast<int>(threadIdx.x) + i * NT;
      c = c < total ? c : total - 1;
      const int row = c / per_row, q = c % per_row;
      alds[((row >> 5) * ACAP + (q >> 1)) * 64 + (q & 1) * 32 + (row & 31)] = st[i];
    }
    lds_barrier();  // keeps the first weight batch in flight
    if (w_lo < w_hi) load_a(X, w_lo);
  }
  // A batch as deep as a wave's whole k range (row-major staged A, at most
  // ACAP steps over KW waves) is loaded once, with no re-read prefetch.
  constexpr bool ONE_BATCH = A_AT_USE && P * KW >= ACAP;
  if (active && w_lo < w_hi) {
    int s = w_lo;
    if constexpr (ALDS == ALDS_NONE) load(X, s);
    if constexpr (ONE_BATCH) compute(X, s, w_hi - s);
    else for (;;) {
      load(Y, s + P < w_hi ? s + P : s);
      compute(X, s, w_hi - s);
      s += P;
      if (s >= w_hi) break;
      load(X, s + P < w_hi ? s + P : s);
      compute(Y, s, w_hi - s);
      s += P;
      if (s >= w_hi) break;
    }
  }

  // Stage: 32x32 MFMA output, lane l / register r -> row 8*(r/4) + 4*(l/32)
  // + r%4, column l%32.
  if constexpr (ALIAS) __syncthreads();
  if (active)
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = mb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
        uint32_t bits;
        if constexpr (AK == A_I8)
          bits = static_cast<uint32_t>(acc[mb][b][r]);
        else
          bits = __float_as_uint(acc[mb][b][r]);
        lds[kw][row][(nw * NB + b) * 32 + li] = bits;
      }
    }
  }
  __syncthreads();

  if constexpr (QH) {
    // int8 query per (token, head): the tile is the head's whole Hckv
    // (N <= TN, one column tile).  TPR threads per row, each over 8-column
    // chunks c0 = 8*(part + TPR*i); the row's max |q^N| is a butterfly over
    // its TPR lanes (aligned, inside one wave); scale = max / 127, codes
    // round half to even in [-127, 127], 0 for an all-zero row.
    static_assert(EPI == EPI_UK && MB == 1 && KW == 1, "QH: one row block, whole-K waves");
    constexpr int NT = 64 * NW;
    constexpr int TPR = NT / 32;
    static_assert(TPR <= 64 && (TPR & (TPR - 1)) == 0, "QH: rows inside one wave");
    constexpr int CH = TN / 8 / TPR;  // chunks per thread
    const int row = threadIdx.x / TPR, part = threadIdx.x % TPR;
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int c0 = 8 * (part + TPR * i);
      if (c0 < N) {
#pragma unroll
        for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(__uint_as_float(lds[0][row][c0 + e])));
      }
    }
    amax = group_max<TPR>(amax);
    const float sc = amax / 127.0f;
    if (row < p.M) {
      const int64_t ob = static_cast<int64_t>(row) * p.q_ld + static_cast<int64_t>(bz) * p.q_bstride;
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        const int c0 = 8 * (part + TPR * i);
        if (c0 < N) {
          int q[8];
#pragma unroll
          for (int e = 0; e < 8; ++e)
            q[e] = sc > 0.f ? sat_rne(__uint_as_float(lds[0][row][c0 + e]) / sc, -127, 127) : 0;
          st8(p.q8_out + ob + c0,
              make_uint2(pack_i8x4(q[0], q[1], q[2], q[3]), pack_i8x4(q[4], q[5], q[6], q[7])));
        }
      }
      if (part == 0) gst(p.q8_scale + static_cast<int64_t>(row) * (p.q_ld / p.q_bstride) + bz, sc);
    }
    return;
  }

  // Epilogue: 8-column groups of the (MB*32) x TN tile.
  GemmParams pe = p;
  if constexpr (EPI == EPI_PARTIAL) pe.part += static_cast<int64_t>(by) * p.M * p.part_ld;
  for (int it = threadIdx.x; it < GROUPS; it += NALL) {
    const int row = it / (TN / 8);
    const int c0 = (it % (TN / 8)) * 8;
    const int64_t m = row;
    const int64_t gcol = n0 + c0;
    if (m >= p.M || gcol >= N) continue;
    uint32_t raw[8], rawp[8];
    const int poff = Epi::partner_offset(p, gcol);
    typename Epi::Pre pre = pre0;
    if (it != static_cast<int>(threadIdx.x)) pre = Epi::prefetch(p, m, gcol);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if constexpr (AK == A_I8) {
        int si = 0, sp = 0;
#pragma unroll
        for (int k = 0; k < KW; ++k) {
          si += static_cast<int>(lds[k][row][c0 + e]);
          if (poff) sp += static_cast<int>(lds[k][row][c0 + poff + e]);
        }
        raw[e] = static_cast<uint32_t>(si);
        rawp[e] = static_cast<uint32_t>(sp);
      } else {
        float sf = 0.f, spf = 0.f;
#pragma unroll
        for (int k = 0; k < KW; ++k) {
          sf += __uint_as_float(lds[k][row][c0 + e]);
          if (poff) spf += __uint_as_float(lds[k][row][c0 + poff + e]);
        }
        raw[e] = __float_as_uint(sf);
        rawp[e] = __float_as_uint(spf);
      }
    }
    Epi::apply(pe, m, gcol, ocol0 + gcol, z, raw, rawp, pre);
  }
}

template <int AK, int MB, int NB, int NW, int KW, int EPI,
          int P = SkinnyDepth<AK, MB, NB>::value, int ALDS = ALDS_NONE, int ACAP = A_LDS_STEPS,
          bool QH = false>
__global__ __launch_bounds__(64 * NW * KW) void k_skinny(GemmParams p) {
  if (p.zero_words != nullptr && blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0)
    for (int i = threadIdx.x; i < p.zero_count; i += blockDim.x)
      gst(p.zero_words + i * SYNC_STRIDE, 0u);
  skinny_tile<AK, MB, NB, NW, KW, EPI, P, ALDS, ACAP, QH>(p, static_cast<int>(blockIdx.x),
                                                     static_cast<int>(blockIdx.y),
                                                     static_cast<int>(blockIdx.z));
}

// ---------------------------------------------------------------------------
// W^UK tiles of the merged decode launch (k_decode_tail, after the finish
// kernel below): head h, 128 columns of Hckv, one 32-column block per wave.
// A tile loads its whole W^UK slice (D/16 k-steps, 16 bytes per lane each)
// into registers as soon as it is dispatched, waits until every
// up-projection tile covering head h's q^C columns has counted itself done,
// reads the head's q^C once per workgroup into LDS (device-scope loads: the
// producers wrote it through to the level every XCD shares, and these never
// hit a stale copy in this XCD's L2), and ends with D/16 MFMAs and the q^N
// stores.  Each XCD dispatches its workgroups in index order, so every
// up-projection tile is dispatched before any W^UK tile of its XCD and never
// waits itself: the wait always ends (it is bounded all the same).
// ---------------------------------------------------------------------------
constexpr int UK_TILE_COLS = 128;  // 4 waves x 32 columns of Hckv
constexpr int UK_MAX_STEPS = 8;    // D <= 128
constexpr int kA6Cols = 96;  // decode A6 tile: three waves across, one column block each

// Up-projection tiles of kA6Cols columns that cover head h's q^C columns
// [h*D, (h+1)*D): the count its W^UK tiles wait for.
__device__ __forceinline__ unsigned up_tiles_of_head(int h, int D, int tw = kA6Cols) {
  return static_cast<unsigned>(((h + 1) * D - 1) / tw - (h * D) / tw + 1);
}

template <int KS>
__device__ __forceinline__ void uk_tile_after_up(const GemmParams& p, const int h, const int ct,
                                                 const unsigned* ready, const unsigned need) {
  static_assert(KS <= UK_MAX_STEPS, "the W^UK slice is held in registers");
  __shared__ uint32_t stage[32][UK_TILE_COLS + 4];
  __shared__ uint4 qcs[UK_MAX_STEPS * 64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int li = lane & 31, g = lane >> 5;
  const int KC = static_cast<int>(p.K / 8);  // 16-byte chunk rows per column block
  const int64_t nblk = (p.N0 + 31) / 32;
  int64_t nb = static_cast<int64_t>(ct) * (UK_TILE_COLS / 32) + wave;
  nb = nb < nblk ? nb : nblk - 1;  // clamped blocks are computed, never stored
  const rsrc_t rb = make_rsrc(p.B0 + static_cast<int64_t>(h) * p.b_bstride + nb * KC * 32,
                              static_cast<uint32_t>(KC) * 512u);
  const uint32_t vl = static_cast<uint32_t>(lane) * 16u;
  uint4 w[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) w[s] = bld16_nt(rb, vl, static_cast<uint32_t>(s) * 1024u);

  if (threadIdx.x == 0) {
    uint32_t n = 0;
    while (__hip_atomic_load(ready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < need &&
           ++n < SYNC_SPIN_LIMIT)
      __builtin_amdgcn_s_sleep(4);
  }
  __syncthreads();

  // Head h's q^C in fragment layout: k-step s is 64 lanes x 16 bytes at s KB.
  const rsrc_t ra = make_rsrc(static_cast<const char*>(p.A) + static_cast<int64_t>(h) * p.a_zs,
                              static_cast<uint32_t>(KS) * 1024u);
  constexpr int PER = (KS * 64 + 255) / 256;
  uint4 q[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int c = static_cast<int>(threadIdx.x) + 256 * i;
    q[i] = bld16_dev(ra, static_cast<uint32_t>(c < KS * 64 ? c : KS * 64 - 1) * 16u, 0u);
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int c = static_cast<int>(threadIdx.x) + 256 * i;
    if (c < KS * 64) qcs[c] = q[i];
  }
  __syncthreads();
  f32x16_t acc = {};
#pragma unroll
  for (int s = 0; s < KS; ++s) mfma_step<A_BF16>(acc, qcs[s * 64 + lane], w[s]);

  // 32x32 block -> LDS (row 8*(r/4) + 4*g + r%4, column li), then each
  // thread stores 8 consecutive columns of one row.
#pragma unroll
  for (int r = 0; r < 16; ++r)
    stage[8 * (r >> 2) + 4 * g + (r & 3)][wave * 32 + li] = __float_as_uint(acc[r]);
  __syncthreads();
  for (int it = threadIdx.x; it < 32 * (UK_TILE_COLS / 8); it += 256) {
    const int row = it / (UK_TILE_COLS / 8);
    const int c0 = (it % (UK_TILE_COLS / 8)) * 8;
    const int64_t gcol = static_cast<int64_t>(ct) * UK_TILE_COLS + c0;
    if (row >= p.M || gcol >= p.N0) continue;
    const uint32_t* v = &stage[row][c0];
    st16_nt(p.q_out + row * p.q_ld + static_cast<int64_t>(h) * p.q_bstride + gcol,
            make_uint4(pack_bf16x2(__uint_as_float(v[0]), __uint_as_float(v[1])),
                       pack_bf16x2(__uint_as_float(v[2]), __uint_as_float(v[3])),
                       pack_bf16x2(__uint_as_float(v[4]), __uint_as_float(v[5])),
                       pack_bf16x2(__uint_as_float(v[6]), __uint_as_float(v[7]))));
  }
}

// An up-projection tile of the merged launch that holds q^C columns: once
// its q^C stores are complete, it bumps the counter of each head it covers.
__device__ __forceinline__ void up_tile_signal(const GemmParams& up, const int b,
                                               unsigned* ready, const int tw = kA6Cols) {
  const int64_t n0 = static_cast<int64_t>(b) * tw;
  if (n0 >= up.ND) return;  // q^R columns only
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this thread's q^C stores are complete
  __syncthreads();
  if (threadIdx.x == 0) {
    const int64_t n1 = n0 + tw < up.ND ? n0 + tw : up.ND;
    const int D = static_cast<int>(up.qc_D);
    for (int h = static_cast<int>(n0 / D); h <= static_cast<int>((n1 - 1) / D); ++h)
      __hip_atomic_fetch_add(ready + h * SYNC_STRIDE, 1u, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ---------------------------------------------------------------------------
// Large-M GEMM (T > 128, every mode): one TM x 256 output tile per
// workgroup, bf16 or int8 operands (16 or 32 k per 16-byte fragment), waves
// as rows x 2 of 64 x 128, each a 2 x 4 grid of 32x32 MFMA blocks: 4 waves
// for TM = 128 (two workgroups per CU), 8 waves for TM = 256 (one workgroup
// per CU, two waves per SIMD).  One stage covers two k-steps: for each, TM/32
// A blocks and 8 B blocks of 1 KB each in MFMA operand (lane) order, so
// every LDS read is one conflict-free ds_read_b128 per lane.  Stages are
// filled by direct buffer->LDS loads and rotate through NBUF LDS buffers:
// the loads of the next stages fly during the MFMAs of the current one, and
// before reading a stage a wave waits only for its own loads of it, then one
// barrier publishes all of them.
// ---------------------------------------------------------------------------
// (G_TN = 256 columns, plan.h.)
// 128-row tiles (three stage buffers, 72 KB of LDS) let two workgroups share
// a CU, so one's epilogue stores overlap the other's main loop; the prefill
// q^R GEMM and the quantised up projection and W^UK product use them.  The
// down projection and the fused q^C + W^UK tiles use 256 rows: the fused
// tiles load their two heads' W^UK per tile, and 128-row tiles double that
// traffic (437 vs 320 us).  (G_TM_HALF = 128, plan.h.)

// One wave's 16-byte-per-lane buffer -> LDS load (buffer_load_dwordx4 ...
// lds): lane l's 16 bytes land at lds + 16*l.  Issued from inline assembly
// so that the compiler does not track it as an LDS write: it cannot tell
// this kernel's many stage arrays apart and would otherwise drain every load
// in flight before each LDS access.  The GEMM orders these loads itself:
// before reading a stage (or reusing LDS) a wave waits for its own loads
// with an explicit vmcnt and then a barrier.  Untracked loads only make the
// compiler's own vmcnt waits stricter (they count in the same in-order
// counter), never looser.  The asm sets M0; no compiler-generated code in
// these kernels uses M0.
__device__ __forceinline__ void dma16(rsrc_t r, uint32_t voff, uint32_t soff, const uint4* lds) {
  const uint32_t l = __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds)));
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds" ::"s"(l), "v"(voff),
               "s"(r), "s"(soff)
               : "memory");
}

// Wait until at most N of this wave's loads are in flight and all of its
// LDS reads have returned, then barrier.  The "memory" clobber keeps LDS
// accesses on their side of it; lgkmcnt(0) also covers reads whose
// consumers (MFMAs, which touch no memory) the compiler placed after the
// barrier: once every wave has passed it, a buffer may be refilled by
// buffer->LDS loads while such a read would still be pending.
template <int N>
__device__ __forceinline__ void vm_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Tile order.  Workgroups are dealt to the 8 XCDs round-robin by linear id;
// when the tiles of one z-slice divide evenly, consecutive chunks of tiles go
// to one XCD, ordered in groups of G_GROUP tile rows (column index slowest
// within a group), so the ~32 tiles an XCD runs at once share A and B tiles
// in its L2.
constexpr int G_GROUP = 4;
// l: the workgroup's linear index within this set of nx x ny tiles (its XCD
// is l % 8 when the set starts at a multiple of 8 in the launch).
__device__ __forceinline__ void gemm_tile(int nx, int ny, int l, int& tx, int& ty) {
  const int n = nx * ny;
  if (n % 8 == 0) l = (l % 8) * (n / 8) + l / 8;
  const int gsz = G_GROUP * nx;
  const int grp = l / gsz;
  const int rows = min(G_GROUP, ny - grp * G_GROUP);
  const int in = l - grp * gsz;
  ty = grp * G_GROUP + in % rows;
  tx = in / rows;
}

// EPI_PARTIAL: blockIdx.z is the split-K index (k-steps [z*steps_per_split,
// ...), partials at part + z*M*part_ld).  Otherwise blockIdx.z is the batch
// (head) index.  K must be a multiple of 32 and steps_per_split even.
//
// EPI_QN (TM = 256, DH = the head dim D = 128): the tile is q^C columns
// only (two heads), and the W^UK product follows in the epilogue.  The main
// loop then swaps the MFMA operands, so the accumulators hold q^C
// transposed: lane l of block (i, j) holds token 32*(4wm+i) + l%32 and, in
// registers r, q^C columns 32*(4wn+j) + 8(r/4) + 4(l/32) + r%4.  Rounded to
// bf16, registers 8h..8h+7 are then directly the token-side operand of a
// 16-k step of the W^UK product -- in exactly the k order mla_pack_weight_uk
// gives W^UK -- so q^C never leaves the registers.
// Waves of a k_gemm workgroup: 2 x 2 of 64 x 128 for 128-row tiles (two
// workgroups per CU), 4 x 2 of 64 x 128 for 256-row tiles (one workgroup
// per CU, two waves per SIMD: 128 accumulators each, so one wave's MFMAs
// run while the other waits on LDS or a barrier).
template <int TM>
constexpr int gemm_waves() { return TM == 256 ? 8 : 4; }

// One tile (tx, ty) of batch / split z, run by the calling workgroup on the
// stage arrays its kernel declares (k_gemm, k_up_fused).  NJ: the 32-column
// blocks this wave computes of its 4 (fewer only where the rest lie past N:
// a ragged last column tile; the wave still loads and waits like the others).
template <int EPI, int TM, int NBUF, int DH, int AK, int MA, int NJ = 4>
__device__ __forceinline__ void gemm_tile_run(
    const GemmParams& p, const int tx, const int ty, const int z, uint4 (&sa0)[2][MA][64],
    uint4 (&sa1)[2][MA][64], uint4 (&sa2)[2][MA][64], uint4 (&sa3)[2][MA][64],
    uint4 (&sb0)[2][8][64], uint4 (&sb1)[2][8][64], uint4 (&sb2)[2][8][64],
    uint4 (&sb3)[2][8][64]) {
  typedef Epilogue<AK, EPI == EPI_QN ? EPI_UQQR : EPI> Epi;
  typedef typename AccT<AK>::type Acc;
  static_assert(AK == A_BF16 || AK == A_I8, "bf16 or int8 operands (16 or 32 k per 16 bytes)");
  constexpr bool SWAP = EPI == EPI_QN;
  static_assert(NJ == 4 || (EPI == EPI_PARTIAL && NJ >= 0 && NJ < 4), "ragged tiles: partials only");
  constexpr int NJA = NJ > 0 ? NJ : 1;  // accumulator blocks allocated
  static_assert(!SWAP || (TM == 256 && DH == 128 && NBUF == 4),
                "fused W^UK product: 256-row tiles, one 128-wide head per wave");
  static_assert(TM != 256 || NBUF == 4, "256-row tiles: the double-buffered pipeline");
  constexpr int NWV = gemm_waves<TM>();  // waves per workgroup
  constexpr int WR = NWV / 2;             // wave rows (two wave columns of 128)
  constexpr int TPW = TM / WR;            // tokens (rows) per wave
  static_assert(MA == TM / 32, "A blocks per k-step");
  constexpr int MI = TPW / 32;  // m-blocks per wave
  constexpr int AW = MA / NWV;  // A blocks loaded per wave per k-step
  constexpr int BW = 8 / NWV;   // B blocks loaded per wave per k-step
  static_assert(AW >= 1 && BW >= 1, "every wave loads A and B blocks");
  constexpr int LPW = 2 * (AW + BW);  // loads per wave per stage
  static_assert(TM == 256 || TM == 128, "tile height");
  static_assert(NBUF >= 3 && NBUF <= 4, "stage buffers");
  // Stage t: A blocks in sa<t>, B blocks in sb<t>, per k-step.
  auto SA = [&](auto bufc) -> uint4 (&)[2][MA][64] {
    constexpr int B = decltype(bufc)::value;
    static_assert(B < NBUF, "stage buffer");
    if constexpr (B == 0) return sa0;
    else if constexpr (B == 1) return sa1;
    else if constexpr (B == 2) return sa2;
    else return sa3;
  };
  auto SB = [&](auto bufc) -> uint4 (&)[2][8][64] {
    constexpr int B = decltype(bufc)::value;
    static_assert(B < NBUF, "stage buffer");
    if constexpr (B == 0) return sb0;
    else if constexpr (B == 1) return sb1;
    else if constexpr (B == 2) return sb2;
    else return sb3;
  };

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int wm = w >> 1, wn = w & 1;
  const int g = lane >> 5, li = lane & 31;
  const int zb = EPI == EPI_PARTIAL ? 0 : z;  // batch index

  const uint4* B;
  int64_t N, n0, ocol0;
  if (tx < p.ntiles0) {
    B = p.B0;
    N = p.N0;
    n0 = static_cast<int64_t>(tx) * G_TN;
    ocol0 = 0;
  } else {
    B = p.B1;
    N = p.N1;
    n0 = static_cast<int64_t>(tx - p.ntiles0) * G_TN;
    ocol0 = p.N0;
  }
  B += static_cast<int64_t>(zb) * p.b_bstride;
  const int64_t m0 = static_cast<int64_t>(ty) * TM;
  // 16-byte chunk rows per column of B, and MFMA k-steps (16 bf16 or 32
  // int8 k) of A and of B
  const int64_t KB = p.KB > 0 ? p.KB : p.K;
  const int KC = static_cast<int>(KB / (AK == A_I8 ? 16 : 8));
  const int nsteps = static_cast<int>(p.K / (AK == A_I8 ? 32 : 16));
  const uint32_t bsteps = static_cast<uint32_t>(KB / (AK == A_I8 ? 32 : 16));
  int s_lo = 0, s_hi = nsteps;
  if constexpr (EPI == EPI_PARTIAL) {
    s_lo = z * static_cast<int>(p.steps_per_split);
    s_hi = min(s_lo + static_cast<int>(p.steps_per_split), nsteps);
  }
  const int nst = s_hi > s_lo ? (s_hi - s_lo) / 2 : 0;

  // B: the tile's 8 column blocks; blocks past N read as zeros.  Wave w
  // loads blocks BW*w .. BW*w+BW-1 of each k-step.
  // (Both resources span this tile only, so their byte ranges fit 32 bits.)
  const int64_t nblk = (N + 31) / 32;
  const int64_t nb0 = n0 / 32;
  const int64_t nbt = nblk - nb0 < 8 ? nblk - nb0 : 8;
  const rsrc_t rb = make_rsrc(B + nb0 * KC * 32, static_cast<uint32_t>(nbt * KC * 512));
  uint32_t vb[BW], va[AW];
#pragma unroll
  for (int j = 0; j < BW; ++j) vb[j] = lane * 16u + static_cast<uint32_t>((BW * w + j) * KC) * 512u;
  // A in fragment layout (1 KB per 32-row block and k-step); wave w loads
  // blocks AW*w .. AW*w+AW-1.  Blocks past the buffer read as zeros.
  // (Gathering row-major A with the same loads, 32 rows per load, made the
  // T = 4096 down projection 38 us slower: more than the 21 us repack into
  // this layout.)
  const int64_t mb0 = m0 / 32, mbt = (p.M + 31) / 32;
  const int64_t nmb = mbt - mb0 < MA ? mbt - mb0 : MA;
  const rsrc_t ra = make_rsrc(static_cast<const char*>(p.A) + zb * p.a_zs + mb0 * p.a_mbs,
                              static_cast<uint32_t>(nmb * p.a_mbs));
#pragma unroll
  for (int j = 0; j < AW; ++j) va[j] = lane * 16u + static_cast<uint32_t>((AW * w + j) * p.a_mbs);

  // Loads of stage t (clamped to the last stage: the pipeline always issues
  // NBUF-1 stages ahead, and a repeated last stage lands in a buffer nobody
  // reads again).
  auto issue = [&](auto bufc, int t) {
    t = t < nst ? t : nst - 1;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const uint32_t s = static_cast<uint32_t>(s_lo + 2 * t + ks);
      const uint32_t sb = EPI == EPI_UK ? s % bsteps : s;
#pragma unroll
      for (int j = 0; j < AW; ++j) dma16(ra, va[j], s * 1024u, &SA(bufc)[ks][AW * w + j][0]);
#pragma unroll
      for (int j = 0; j < BW; ++j) dma16(rb, vb[j], sb * 1024u, &SB(bufc)[ks][BW * w + j][0]);
    }
  };

  Acc acc[MI][NJA];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJA; ++j) acc[i][j] = Acc{};

  auto compute = [&](auto bufc) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      uint4 a[MI], b[NJA];
#pragma unroll
      for (int i = 0; i < MI; ++i) a[i] = SA(bufc)[ks][MI * wm + i][lane];
#pragma unroll
      for (int j = 0; j < NJ; ++j) b[j] = SB(bufc)[ks][4 * wn + j][lane];
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          if constexpr (SWAP)
            mfma_step<AK>(acc[i][j], b[j], a[i]);
          else
            mfma_step<AK>(acc[i][j], a[i], b[j]);
        }
    }
  };

  // One pipeline step: stage t is in buffer BUF.  Every step has issued the
  // LPW loads per wave of each of the NBUF-2 stages after t, so waiting
  // until at most that many loads are in flight means this wave's loads of
  // stage t have landed; the barrier then covers every wave's, and also
  // tells that all waves are done reading the buffer the step refills
  // (stage t-1's).  The main loop is branch-free: branches inside it split
  // the accumulators' live ranges and the register allocator then spills.
  using C0 = std::integral_constant<int, 0>;
  using C1 = std::integral_constant<int, 1>;
  using C2 = std::integral_constant<int, 2>;
  using C3 = std::integral_constant<int, 3>;
  auto step = [&](auto bufc, int t) {
    constexpr int BUF = decltype(bufc)::value;
    vm_barrier<LPW*(NBUF - 2)>();
    issue(std::integral_constant<int, (BUF + NBUF - 1) % NBUF>{}, t + NBUF - 1);
    compute(bufc);
  };

  // 256-row tiles run one wave per SIMD, so nothing else hides the LDS
  // read latency of a k-step's fragments or the stage barrier.  Their
  // pipeline double-buffers the fragments: each step reads k-step 1 of its
  // stage while k-step 0's MFMAs run, and its barrier sits between the two
  // k-steps (after it, all of the stage's fragments are in registers, so
  // the stage's buffer is refilled at once and the next stage's k-step 0
  // fragments load under k-step 1's MFMAs).  One stage more is in flight:
  // the buffer refilled at step t is stage t's own, with stage t + NBUF.
  if constexpr (TM == 256) {
    uint4 fa0[MI], fb0[4], fa1[MI], fb1[4];
    auto rd = [&](auto bufc, int ks, uint4 (&fa)[MI], uint4 (&fb)[4]) {
#pragma unroll
      for (int i = 0; i < MI; ++i) fa[i] = SA(bufc)[ks][MI * wm + i][lane];
#pragma unroll
      for (int j = 0; j < NJ; ++j) fb[j] = SB(bufc)[ks][4 * wn + j][lane];
    };
    auto mm = [&](const uint4 (&fa)[MI], const uint4 (&fb)[4]) {
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          if constexpr (SWAP)
            mfma_step<AK>(acc[i][j], fb[j], fa[i]);
          else
            mfma_step<AK>(acc[i][j], fa[i], fb[j]);
        }
    };
    // Stage t in buffer BUF = t % NBUF; on entry fa0/fb0 hold its k-step 0.
    // The barrier's vmcnt allows the NBUF - 2 stages issued after stage
    // t + 1 to stay in flight; its lgkmcnt(0) also covers this stage's
    // k-step 1 reads, so every wave is done with buffer BUF after it.
    auto step2 = [&](auto bufc, int t) {
      constexpr int BUF = decltype(bufc)::value;
      // (sched_barrier pins each group in place: the compiler would sink
      // the MFMAs, which touch no memory, below the barrier)
      rd(bufc, 1, fa1, fb1);
      __builtin_amdgcn_sched_barrier(0);
      mm(fa0, fb0);
      __builtin_amdgcn_sched_barrier(0);
      vm_barrier<LPW*(NBUF - 2)>();
      issue(bufc, t + NBUF);
      rd(std::integral_constant<int, (BUF + 1) % NBUF>{}, 0, fa0, fb0);  // stage t + 1
      __builtin_amdgcn_sched_barrier(0);
      mm(fa1, fb1);
      __builtin_amdgcn_sched_barrier(0);
    };
    if (nst > 0) {
      issue(C0{}, 0);
      issue(C1{}, 1);
      issue(C2{}, 2);
      issue(C3{}, 3);
      vm_barrier<LPW*(NBUF - 1)>();  // stage 0 landed
      rd(C0{}, 0, fa0, fb0);
      const int nstb = nst / NBUF * NBUF;
      for (int t = 0; t < nstb; t += NBUF) {
        step2(C0{}, t);
        step2(C1{}, t + 1);
        step2(C2{}, t + 2);
        step2(C3{}, t + 3);
      }
      const int rem = nst - nstb;
      if (rem >= 1) step2(C0{}, nstb);
      if (rem >= 2) step2(C1{}, nstb + 1);
      if (rem >= 3) step2(C2{}, nstb + 2);
    }
  } else if (nst > 0) {
    issue(C0{}, 0);
    issue(C1{}, 1);
    if constexpr (NBUF == 4) issue(C2{}, 2);
    const int nstb = nst / NBUF * NBUF;
    for (int t = 0; t < nstb; t += NBUF) {
      step(C0{}, t);
      step(C1{}, t + 1);
      step(C2{}, t + 2);
      if constexpr (NBUF == 4) step(C3{}, t + 3);
    }
    // the remaining stages sit in buffers 0.. with q later stages issued
    const int rem = nst - nstb;
    if (rem >= 1) {
      vm_barrier<LPW*(NBUF - 2)>();
      compute(C0{});
    }
    if (rem >= 2) {
      vm_barrier<LPW*(NBUF - 3)>();
      compute(C1{});
    }
    if constexpr (NBUF == 4) {
      if (rem >= 3) {
        vm_barrier<0>();
        compute(C2{});
      }
    }
  }
  // No load into LDS outlives the loop, and every wave is done reading the
  // stage buffers before they hold the epilogue's staging.
  vm_barrier<0>();

  if constexpr (EPI == EPI_QN) {
    // q^C as bf16 operand fragments in registers: qc[0][i][k] = 16-k step k
    // of the wave's 128 q^C columns (its head) for m-block i.  With int8
    // operands the accumulators are integer sums, dequantised as the
    // unfused epilogue does (sum * s_t * dq_c: the token's c^Q scale, the
    // column's dequant scale, both staged in LDS) and carried as bf16 hi
    // (qc[0]) and lo = bf16(q^C - hi) (qc[1]); the W^UK product then
    // multiplies both, as the decode kernels' fp32-split operand does.
    constexpr int NQ = AK == A_I8 ? 2 : 1;
    uint4 qc[NQ][MI][8];
    if constexpr (AK == A_I8) {
      // stage buffer 3's A array (free until the passes' output staging)
      float* scl = reinterpret_cast<float*>(&SA(C3{})[0][0][0]);
      for (int t = threadIdx.x; t < TM + G_TN; t += 64 * NWV) {
        float v = 0.f;
        if (t < TM) {
          if (m0 + t < p.M) v = gld(p.cq_scale + m0 + t);
        } else {
          v = gld(p.dq + n0 + (t - TM));  // the tile's columns are all q^C columns
        }
        scl[t] = v;
      }
      lds_barrier();
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        // registers 8(k&1) .. +7 of block k>>1: columns cb + 16(k&1) + {0..3, 8..11}
        const int cb = TM + 32 * (4 * wn + (k >> 1)) + 4 * g + 16 * (k & 1);
        const float4 d0 = *reinterpret_cast<const float4*>(scl + cb);
        const float4 d1 = *reinterpret_cast<const float4*>(scl + cb + 8);
        const float dq[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
#pragma unroll
        for (int i = 0; i < MI; ++i) {
          const float cs = scl[TPW * wm + 32 * i + li];
          const int o = 8 * (k & 1);
          uint32_t hw[4], lw[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float a = static_cast<float>(acc[i][k >> 1][o + 2 * e]) * cs * dq[2 * e];
            const float b = static_cast<float>(acc[i][k >> 1][o + 2 * e + 1]) * cs * dq[2 * e + 1];
            const uint16_t ha = f32_to_bf16(a), hb = f32_to_bf16(b);
            hw[e] = static_cast<uint32_t>(ha) | (static_cast<uint32_t>(hb) << 16);
            lw[e] = pack_bf16x2(a - bf16_to_f32(ha), b - bf16_to_f32(hb));
          }
          qc[0][i][k] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
          qc[NQ - 1][i][k] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const Acc& c = acc[i][k >> 1];
          const int o = 8 * (k & 1);
          qc[0][i][k] = make_uint4(pack_bf16x2(c[o], c[o + 1]), pack_bf16x2(c[o + 2], c[o + 3]),
                                   pack_bf16x2(c[o + 4], c[o + 5]), pack_bf16x2(c[o + 6], c[o + 7]));
        }
    }
    // The tile's two heads (wn = 0, 1) run the W^UK product over passes of
    // PB = 2 column blocks (32 columns each) of Hckv (MI m-blocks x PB
    // column blocks of accumulators: the rest of the AGPRs and the VGPRs
    // hold qc).  A pass's W^UK operands (2 heads x 8 k-steps x PB column
    // blocks of 1 KB) are loaded into LDS by buffer->LDS loads two passes
    // ahead, as [head*8 + k-step][lane] per column block: pass buffer b
    // (0-2) is stage b's arrays, sa<b> for the first column block and sb<b>
    // for the second (16 KB each).
    constexpr int PB = 2;
    constexpr int SPP = MI * 2 * PB;  // stores per wave per full pass
    const int KC2 = DH / 8;
    const int64_t nblk2 = (p.uk_N + 31) / 32;
    const int npass = static_cast<int>((nblk2 + PB - 1) / PB);
    const int64_t head0 = n0 / DH;
    // this wave's load share of a pass: head hs, k-steps kw .. kw+KPW-1
    constexpr int KPW = 8 / (NWV / 2);
    const int hs = w / (NWV / 2), kw = KPW * (w % (NWV / 2));
    const rsrc_t ruk = make_rsrc(p.Buk + (head0 + hs) * p.uk_bstride,
                                 static_cast<uint32_t>(nblk2 * KC2 * 512));
    auto pbuf = [&](auto bc, int jb) -> uint4* {
      return jb == 0 ? &SA(bc)[0][0][0] : &SB(bc)[0][0][0];
    };
    auto issue_uk = [&](auto bc, int pp) {
#pragma unroll
      for (int jb = 0; jb < PB; ++jb) {
        int64_t nb2 = PB * pp + jb;
        nb2 = nb2 < nblk2 ? nb2 : nblk2 - 1;  // clamped blocks are never stored
        const uint32_t vo = lane * 16u + static_cast<uint32_t>(nb2 * KC2) * 512u;
        uint4* dst = pbuf(bc, jb);  // jb is static
#pragma unroll
        for (int k4 = 0; k4 < KPW; ++k4)
          dma16(ruk, vo, static_cast<uint32_t>(kw + k4) * 1024u, dst + (hs * 8 + kw + k4) * 64);
      }
    };
    const int64_t head = head0 + wn;
    // Output staging: a 4 KB slice per wave of stage buffer 3's arrays
    // (the passes use buffers 0-2; every load into LDS has landed).
    static_assert(sizeof(sa3) == 4 * 4096 && sizeof(sb3) == 4 * 4096,
                  "staging: four waves per array");
    char* stg = reinterpret_cast<char*>(w < 4 ? &sa3[0][0][0] : &sb3[0][0][0]) + (w & 3) * 4096;
    const bool rows_in = m0 + TPW * wm + TPW - 1 < p.M;  // all of this wave's tokens are rows
    // Returns whether the pass issued exactly SPP stores (all in range).
    auto pass_uk = [&](auto bc, int pp) -> bool {
      f32x16_t o[MI][PB];
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int jb = 0; jb < PB; ++jb) o[i][jb] = f32x16_t{};
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        uint4 wf[PB];
#pragma unroll
        for (int jb = 0; jb < PB; ++jb) wf[jb] = pbuf(bc, jb)[(wn * 8 + ks) * 64 + lane];
#pragma unroll
        for (int q = 0; q < NQ; ++q)
#pragma unroll
          for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int jb = 0; jb < PB; ++jb)
              o[i][jb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                  as_bf16x8(wf[jb]), as_bf16x8(qc[q][i][ks]), o[i][jb], 0, 0, 0);
      }
      // o[i][jb]: lane l holds token 32*(MI*wm+i) + l%32, registers r the
      // output columns 32*(PB*pp+jb) + 8(r/4) + 4g + r%4.  Transpose each
      // m-block through the wave's staging slice (32 tokens x 32*PB columns
      // bf16: CPR 16-byte chunks per row, chunk c of row t stored at chunk
      // c ^ (t % CPR)); then each store instruction writes 64/CPR whole rows.
      constexpr int CPR = 4 * PB;
      const int cc = lane & (CPR - 1);
      const int64_t nc = 32 * PB * pp + 8 * cc;
      const bool full = rows_in && 32 * PB * (pp + 1) <= p.uk_N;  // uniform per wave
#pragma unroll
      for (int i = 0; i < MI; ++i) {
#pragma unroll
        for (int jb = 0; jb < PB; ++jb)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int c = (4 * jb + q) ^ (li & (CPR - 1));
            *reinterpret_cast<uint2*>(stg + li * (16 * CPR) + c * 16 + g * 8) =
                make_uint2(pack_bf16x2(o[i][jb][4 * q], o[i][jb][4 * q + 1]),
                           pack_bf16x2(o[i][jb][4 * q + 2], o[i][jb][4 * q + 3]));
          }
#pragma unroll
        for (int k = 0; k < 2 * PB; ++k) {
          const int tr = (64 / CPR) * k + lane / CPR;
          const uint4 v = *reinterpret_cast<const uint4*>(stg + tr * (16 * CPR) +
                                                          ((cc ^ (tr & (CPR - 1))) * 16));
          const int64_t m = m0 + TPW * wm + 32 * i + tr;
          if (full || (m < p.M && nc < p.uk_N))
            // plain stores: streaming ones measured 27 us slower here
            st16(p.q_out + m * p.q_ld + head * p.q_bstride + nc, v);
        }
      }
      return full;
    };
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    using P2 = std::integral_constant<int, 2>;
    // Three pass buffers: pass pp's W^UK loads are issued two passes ahead,
    // so a pass's stores have two passes to complete before any wait needs
    // them.  Before pass pp a wave waits until its loads of pass pp have
    // landed: with in-order completion, until no more than the vector-memory
    // operations it issued after those loads are in flight.  after[b] counts
    // them for the pass in buffer b (a lower bound: a pass whose stores were
    // not all issued counts none).  The barrier then covers every wave's
    // loads, and every wave is done reading the buffer refilled next (pass
    // pp - 1's).
    constexpr int LPP = PB * KPW;  // W^UK loads per wave per pass
    int after[3] = {0, 0, 0};
    auto note = [&](int n) {
      after[0] += n;
      after[1] += n;
      after[2] += n;
    };
    auto issue_pass = [&](auto bc, int pp) {
      if (pp >= npass) return;
      note(LPP);
      issue_uk(bc, pp);
      after[decltype(bc)::value] = 0;
    };
    auto wait_loads = [&](int n) {  // n: a multiple of 4 (LPP and SPP are)
      static_assert(LPP % 4 == 0 && SPP % 4 == 0, "wait counts");
      if (n >= 20) vm_barrier<20>();
      else if (n >= 16) vm_barrier<16>();
      else if (n >= 12) vm_barrier<12>();
      else if (n >= 8) vm_barrier<8>();
      else if (n >= 4) vm_barrier<4>();
      else vm_barrier<0>();
    };
    auto run_pass = [&](auto bc, auto nextbc, int pp) {
      wait_loads(after[decltype(bc)::value]);
      issue_pass(nextbc, pp + 2);
      note(pass_uk(bc, pp) ? SPP : 0);
    };
    issue_pass(P0{}, 0);
    issue_pass(P1{}, 1);
    for (int pp = 0; pp < npass; pp += 3) {
      run_pass(P0{}, P2{}, pp);
      if (pp + 1 >= npass) break;
      run_pass(P1{}, P0{}, pp + 1);
      if (pp + 2 >= npass) break;
      run_pass(P2{}, P1{}, pp + 2);
    }
    return;
  }

  // Epilogue.  Wave w stages 32-row pieces of its tile (32 x 128 fp32) in
  // two 8 KB halves (rows 0-15 and 16-31) of B stage buffer sb<w> (with
  // three buffers, wave 3 uses sa0 and sa1; with eight waves, waves 4-7 use
  // the 16 KB A buffers sa<w-4>), 128 words
  // per row with 32-word halves swapped on every other 4-row group (so the
  // two lane halves of an accumulator write hit different banks).  Then
  // each lane takes 8 groups of 8 consecutive columns: 16 lanes cover one
  // row's 128 columns, so a wave's stores are 4 rows x 256 contiguous bytes
  // (bf16).  RoPE partners lie in the same 32-column block, so in the same
  // row.
  static_assert(sizeof(sb0) >= 16384 && sizeof(sa0) >= 8192, "staging space");
  static_assert(NWV == 4 || (NBUF == 4 && sizeof(sa0) >= 16384), "eight staging slices");
  uint32_t* se_lo;
  uint32_t* se_hi;
  switch (w) {
    case 0: se_lo = &sb0[0][0][0].x; se_hi = se_lo + 2048; break;
    case 1: se_lo = &sb1[0][0][0].x; se_hi = se_lo + 2048; break;
    case 2: se_lo = &sb2[0][0][0].x; se_hi = se_lo + 2048; break;
    case 3:
      if constexpr (NBUF == 4) {
        se_lo = &SB(std::integral_constant<int, 3>{})[0][0][0].x;
        se_hi = se_lo + 2048;
      } else {
        se_lo = &sa0[0][0][0].x;
        se_hi = &sa1[0][0][0].x;
      }
      break;
    case 4: se_lo = &sa0[0][0][0].x; se_hi = se_lo + 2048; break;
    case 5: se_lo = &sa1[0][0][0].x; se_hi = se_lo + 2048; break;
    case 6: se_lo = &sa2[0][0][0].x; se_hi = se_lo + 2048; break;
    default:
      if constexpr (NBUF == 4) {
        se_lo = &SA(std::integral_constant<int, 3>{})[0][0][0].x;
      } else {
        se_lo = &sa2[0][0][0].x;  // not reached: three buffers run four waves
      }
      se_hi = se_lo + 2048;
      break;
  }
  auto sep = [&](int row, int col) -> uint32_t& {
    uint32_t* base = row < 16 ? se_lo : se_hi;
    return base[(row & 15) * 128 + (col ^ (((row >> 2) & 1) << 5))];
  };
  // Only tiles holding q^R columns need the RoPE tables (uniform per tile).
  // (int8 tiles also need every column's dequant scale and every token's)
  const bool need_pre = EPI == EPI_UQQR && (AK == A_I8 || n0 + G_TN > p.ND);
  GemmParams pe = p;
  if constexpr (EPI == EPI_PARTIAL) pe.part += static_cast<int64_t>(z) * p.M * p.part_ld;
#pragma unroll
  for (int i = 0; i < MI; ++i) {
#pragma unroll
    for (int j = 0; j < NJ; ++j)  // (blocks past NJ lie past N: never stored)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        sep(8 * (r >> 2) + 4 * g + (r & 3), 32 * j + li) =
            AK == A_I8 ? static_cast<uint32_t>(acc[i][j][r]) : __float_as_uint(acc[i][j][r]);
    // Rolled over 2 batches of 4 groups: the accumulators must stay
    // statically indexed, which needs the unrolled loop above to stay
    // small.  A batch issues its RoPE-table loads together.
#pragma unroll 1
    for (int k = 0; k < 8; k += 4) {
      typename Epi::Pre pre[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int it = lane + 64 * (k + u);
        const int64_t m = m0 + TPW * wm + 32 * i + (it >> 4);
        const int64_t gcol = n0 + 128 * wn + (it & 15) * 8;
        pre[u] = typename Epi::Pre{};
        if (need_pre && m < p.M && gcol < N) pre[u] = Epi::prefetch(p, m, gcol);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int it = lane + 64 * (k + u);
        const int row = it >> 4;
        const int c0 = (it & 15) * 8;
        const int64_t m = m0 + TPW * wm + 32 * i + row;
        const int64_t gcol = n0 + 128 * wn + c0;
        if (m >= p.M || gcol >= N) continue;
        uint32_t raw[8], rawp[8];
        const int poff = Epi::partner_offset(p, gcol);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          raw[e] = sep(row, c0 + e);
          rawp[e] = poff ? sep(row, c0 + poff + e) : 0u;
        }
        Epi::apply(pe, m, gcol, ocol0 + gcol, zb, raw, rawp, pre[u]);
      }
    }
  }
}

template <int EPI, int TM, int NBUF, int DH = 0, int AK = A_BF16>
__global__ __launch_bounds__(64 * gemm_waves<TM>(), TM == 256 ? 1 : 2) void k_gemm(GemmParams p) {
  // Stage t: A blocks in sa<t>, B blocks in sb<t>, per k-step.  (Separate
  // arrays: with A and B in one array per stage the compiler drains the
  // loads in flight before each stage's second k-step.  Three-buffer
  // instances never name sa3/sb3, so they do not allocate them.)
  constexpr int MA = TM / 32;
  __shared__ uint4 sa0[2][MA][64], sa1[2][MA][64], sa2[2][MA][64], sa3[2][MA][64];
  __shared__ uint4 sb0[2][8][64], sb1[2][8][64], sb2[2][8][64], sb3[2][8][64];
  int tx, ty;
  gemm_tile(static_cast<int>(gridDim.x), static_cast<int>(gridDim.y),
            static_cast<int>(blockIdx.x + gridDim.x * blockIdx.y), tx, ty);
  const int z = static_cast<int>(blockIdx.z);
  if constexpr (NBUF == 4 && EPI == EPI_PARTIAL) {
    // A ragged last column tile (e.g. c^KV + k^R = 576 columns: 2.25 tiles):
    // a wave whose 128 columns reach past N by 64 or more computes only
    // the blocks before it (2 or none of its 4).  Same loads and barriers.
    const int64_t n0 = static_cast<int64_t>(tx < p.ntiles0 ? tx : tx - p.ntiles0) * G_TN;
    const int64_t valid = (tx < p.ntiles0 ? p.N0 : p.N1) - n0 -
                          128 * (__builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6)) & 1);
    if (valid > 64)
      gemm_tile_run<EPI, TM, NBUF, DH, AK, MA>(p, tx, ty, z, sa0, sa1, sa2, sa3, sb0, sb1, sb2, sb3);
    else if (valid > 0)
      gemm_tile_run<EPI, TM, NBUF, DH, AK, MA, 2>(p, tx, ty, z, sa0, sa1, sa2, sa3, sb0, sb1, sb2, sb3);
    else
      gemm_tile_run<EPI, TM, NBUF, DH, AK, MA, 0>(p, tx, ty, z, sa0, sa1, sa2, sa3, sb0, sb1, sb2, sb3);
  } else if constexpr (NBUF == 4) {
    gemm_tile_run<EPI, TM, NBUF, DH, AK, MA>(p, tx, ty, z, sa0, sa1, sa2, sa3, sb0, sb1, sb2, sb3);
  } else {  // (the fourth buffer is never touched)
    gemm_tile_run<EPI, TM, NBUF, DH, AK, MA>(p, tx, ty, z, sa0, sa1, sa2, sa2, sb0, sb1, sb2, sb2);
  }
}

// Prefill up projection in one launch (D = 128): workgroups [0, nq) are the
// q^C tiles with the fused W^UK product (nqx x ny tiles), the rest the q^R
// column tiles (nrx x ny), both 256 x 256 with eight waves on one set of
// stage arrays.  The shorter q^R tiles come last and fill the final round.
template <int AK>
__global__ __launch_bounds__(64 * gemm_waves<256>(), 1) void k_up_fused(GemmParams pq, GemmParams pr,
                                                                       int nqx, int nrx, int ny) {
  __shared__ uint4 sa0[2][8][64], sa1[2][8][64], sa2[2][8][64], sa3[2][8][64];
  __shared__ uint4 sb0[2][8][64], sb1[2][8][64], sb2[2][8][64], sb3[2][8][64];
  const int b = static_cast<int>(blockIdx.x), nq = nqx * ny;
  int tx, ty;
  if (b < nq) {
    gemm_tile(nqx, ny, b, tx, ty);
    gemm_tile_run<EPI_QN, 256, 4, 128, AK, 8>(pq, tx, ty, 0, sa0, sa1, sa2, sa3, sb0, sb1, sb2, sb3);
  } else {
    gemm_tile(nrx, ny, b - nq, tx, ty);
    gemm_tile_run<EPI_UQQR, 256, 4, 0, AK, 8>(pr, tx, ty, 0, sa0, sa1, sa2, sa3, sb0, sb1, sb2, sb3);
  }
}

// ---------------------------------------------------------------------------
// Down-projection finish: one workgroup per token, each thread owning 8
// consecutive columns of the token's Hcq + Hckv + Dr outputs.  Sums the
// split-K partials in split order, RmsNorms c^Q (and quantises it per token
// in the partial-quant scenarios), RmsNorms c^KV, rotates k^R and writes both
// cache rows at the token's slot.  A thread's global loads for its first
// chunk (partials, gammas, scales, cos/sin) and the slot are all issued at
// the start, so the kernel waits on memory once.
// ---------------------------------------------------------------------------
struct FinishParams {
  const float* part;
  int ksplit;
  int64_t T;
  int Hcq, Hckv, Dr;
  float eps_cq, eps_ckv;
  const uint16_t* gamma_cq;
  const uint16_t* gamma_ckv;
  const float* smooth;
  const float* qs_ckv;
  const float* qs_ckr;
  const uint16_t* cosb;
  const uint16_t* sinb;
  const int64_t* index;
  int64_t slots;
  void* kv_cache;
  void* kr_cache;
  uint16_t* cq_bf16;
  int8_t* cq_i8;
  int cq_frag;  // write c^Q in the skinny kernels' A fragment layout
  float* cq_scale;
  int8_t* dbg_cq_i8;
  float* dbg_cq_scale;
  // Full quantisation: the partials are int8 x int8 sums, dequantised per
  // token (sx) and per channel (sw_dq for c^Q's columns, sw_dkv for the
  // c^KV / k^R columns) once the splits are summed.  NULL otherwise.
  const float* sx;
  const float* sw_dq;
  const float* sw_dkv;
  // MlaPreprocessV2 (QM = 4): c^Q codes = sat(rne((RmsNorm(h) + bias) * qs_cq))
  // with the bias in `smooth`; the per-token scale the up projection applies
  // is 1.
  float qs_cq;
};

constexpr int FIN_MAX_THREADS = 1024;
// (FIN_MAXSPLIT and FIN_SPLIT_SMALL, the split-K bounds, are in plan.h.)

// Workgroup size of the finish kernel for ntot columns: one thread per
// 8-column chunk, whole waves, at most FIN_MAX_THREADS (more chunks loop).
inline int fin_threads(int64_t ntot) {
  const int64_t t = (ntot / 8 + 63) / 64 * 64;
  return static_cast<int>(t < 64 ? 64 : (t > FIN_MAX_THREADS ? FIN_MAX_THREADS : t));
}

// Sum (op = 0) or max (op = 1) of two values over the workgroup.
template <int OP>
__device__ __forceinline__ float2 block_reduce2(float2 v, float2* red) {
  if (OP == 0) {
    v.x = group_sum<64>(v.x);
    v.y = group_sum<64>(v.y);
  } else {
    v.x = group_max<64>(v.x);
    v.y = group_max<64>(v.y);
  }
  const int wave = threadIdx.x >> 6;
  __syncthreads();  // red[] free from an earlier reduction
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  float2 t = red[0];
  for (int w = 1; w < static_cast<int>(blockDim.x >> 6); ++w) {
    t.x = OP == 0 ? t.x + red[w].x : fmaxf(t.x, red[w].x);
    t.y = OP == 0 ? t.y + red[w].y : fmaxf(t.y, red[w].y);
  }
  return t;
}

__device__ __forceinline__ void unpack_bf16x8(uint4 w, float* f) {
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f[2 * e] = bf16lo(u[e]);
    f[2 * e + 1] = bf16hi(u[e]);
  }
}

// QM: 0 none, 1 c^Q quantised with bf16 caches (partial or full
// quantisation), 2 c^Q quantised with int8 kv and kr caches (partial),
// 3 c^Q quantised with an int8 kv cache and a bf16 kr cache (full),
// 4 c^Q quantised statically (MlaPreprocessV2's RmsNormQuant: bias, then
// one per-tensor scale) with bf16 caches.
// MAXS: most splits summed (ksplit <= MAXS); fewer keep more workgroups
// resident (the large-T plan splits at most 4 ways).
template <int QM, int MAXS = FIN_MAXSPLIT>
__global__ __launch_bounds__(FIN_MAX_THREADS) void k_down_finish(FinishParams p) {
  extern __shared__ float row[];  // Hcq + Hckv + Dr summed values
  __shared__ float2 red[FIN_MAX_THREADS / 64];
  const int64_t t = blockIdx.x;
  const int ntot = p.Hcq + p.Hckv + p.Dr;
  // With two workgroups per token (gridDim.y = 2), y = 0 takes the c^Q
  // chunks and y = 1 the c^KV and k^R chunks: their norms are independent.
  const int jlo = gridDim.y == 2 && blockIdx.y == 1 ? p.Hcq / 8 : 0;
  const int nch = gridDim.y == 2 && blockIdx.y == 0 ? p.Hcq / 8 : ntot / 8;
  const int half = p.Dr >> 1;
  const int64_t slot = gld(p.index + t);

  // Parameters of one chunk: pa = its gammas (c^Q, c^KV) or cos (k^R), pb =
  // sin (k^R), pf = smooth scales (c^Q) or int8 cache scales (c^KV, k^R).
  // Every pointer formed is valid whatever the region.
  uint4 pa, pb;
  float pf[8];
  auto load_params = [&](int j) {
    const int c0 = 8 * j;
    const bool cq = c0 < p.Hcq, ckv = !cq && c0 < p.Hcq + p.Hckv;
    const int i0 = cq || ckv ? 0 : c0 - p.Hcq - p.Hckv;
    pa = ld16(cq ? p.gamma_cq + c0
                 : (ckv ? p.gamma_ckv + (c0 - p.Hcq) : p.cosb + t * p.Dr + i0));
    pb = ld16(p.sinb + t * p.Dr + i0);
    if (QM != 0) {
      const float* f = p.smooth + (cq ? c0 : 0);
      if ((QM == 2 || QM == 3) && ckv) f = p.qs_ckv + (c0 - p.Hcq);
      if (QM == 2 && !cq && !ckv) f = p.qs_ckr + i0;
      ld8f(f, pf);
    }
  };
  // The first chunk's parameters load together with its partials; with one
  // round of chunks (the DeepSeek-V3 shapes) nothing is loaded later.
  if (jlo + static_cast<int>(threadIdx.x) < nch) load_params(jlo + threadIdx.x);

  // Pass 1: per chunk, sum the partials in split order into row[].
  float sq = 0.f, skv = 0.f, amax = 0.f;
  for (int j = jlo + threadIdx.x; j < nch; j += blockDim.x) {
    const int c0 = 8 * j;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float v[MAXS][8];
#pragma unroll
    for (int s = 0; s < MAXS; ++s) {
      const int se = s < p.ksplit ? s : p.ksplit - 1;
      ld8f(p.part + (static_cast<int64_t>(se) * p.T + t) * ntot + c0, v[s]);
    }
#pragma unroll
    for (int s = 0; s < MAXS; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += s < p.ksplit ? v[s][e] : 0.f;
    if (QM != 0 && p.sx != nullptr) {
      // full quantisation: integer sums times the token's and the
      // channels' dequant scales
      float sw[8];
      ld8f(c0 < p.Hcq ? p.sw_dq + c0 : p.sw_dkv + (c0 - p.Hcq), sw);
      const float sxt = gld(p.sx + t);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = acc[e] * sxt * sw[e];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      row[c0 + e] = acc[e];
      if (c0 < p.Hcq)
        sq += acc[e] * acc[e];
      else if (c0 < p.Hcq + p.Hckv)
        skv += acc[e] * acc[e];
    }
  }
  const float2 ss = block_reduce2<0>(make_float2(sq, skv), red);  // barrier: row[] complete
  const float rq = 1.0f / __builtin_sqrtf(ss.x / static_cast<float>(p.Hcq) + p.eps_cq);
  const float rkv = 1.0f / __builtin_sqrtf(ss.y / static_cast<float>(p.Hckv) + p.eps_ckv);

  // c^Q fragment layout: element (t, c) of a K-step of `ks` values sits at
  // ((mb*(Hcq/ks) + c/ks)*64 + g*32 + t%32)*(ks/2) + c%(ks/2),
  // g = (c%ks)/(ks/2); 8 consecutive c (c % 8 == 0) are contiguous.
  auto cq_off = [&](int c, int ks) -> int64_t {
    if (!p.cq_frag) return t * p.Hcq + c;
    const int h = ks / 2;
    return ((static_cast<int64_t>(t / 32) * (p.Hcq / ks) + c / ks) * 64 + ((c % ks) / h) * 32 +
            (t % 32)) * h + c % h;
  };
  const bool write_cache = slot >= 0 && slot < p.slots;

  // Pass 2: outputs.
  for (int j = jlo + threadIdx.x; j < nch; j += blockDim.x) {
    const int c0 = 8 * j;
    if (j != jlo + static_cast<int>(threadIdx.x)) load_params(j);
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = row[c0 + e];
    if (c0 < p.Hcq) {
      float g[8];
      unpack_bf16x8(pa, g);
      if (QM == 4) {
        // aclnnMlaPreprocessV2 RmsNormQuant: (RmsNorm(h) + bias) * scale
        int q[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) q[e] = sat_rne((x[e] * rq * g[e] + pf[e]) * p.qs_cq, -128, 127);
        const uint2 w = make_uint2(pack_i8x4(q[0], q[1], q[2], q[3]), pack_i8x4(q[4], q[5], q[6], q[7]));
        st8(p.cq_i8 + cq_off(c0, 32), w);
        if (p.dbg_cq_i8) st8(p.dbg_cq_i8 + t * p.Hcq + c0, w);
      } else if (QM == 0) {
        st16(p.cq_bf16 + cq_off(c0, 16),
             make_uint4(pack_bf16x2(x[0] * rq * g[0], x[1] * rq * g[1]),
                        pack_bf16x2(x[2] * rq * g[2], x[3] * rq * g[3]),
                        pack_bf16x2(x[4] * rq * g[4], x[5] * rq * g[5]),
                        pack_bf16x2(x[6] * rq * g[6], x[7] * rq * g[7])));
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float u = x[e] * rq * g[e] * pf[e];
          row[c0 + e] = u;  // this thread's own columns: no barrier needed
          amax = fmaxf(amax, fabsf(u));
        }
      }
    } else if (c0 < p.Hcq + p.Hckv) {
      if (!write_cache) continue;
      const int c = c0 - p.Hcq;
      float g[8], o[8];
      unpack_bf16x8(pa, g);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = x[e] * rkv * g[e];
      if (QM == 2 || QM == 3) {
        int q[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) q[e] = sat_rne(o[e] / pf[e], -128, 127);
        st8_nt(static_cast<int8_t*>(p.kv_cache) + slot * p.Hckv + c,
            make_uint2(pack_i8x4(q[0], q[1], q[2], q[3]), pack_i8x4(q[4], q[5], q[6], q[7])));
      } else {
        st16_nt(static_cast<uint16_t*>(p.kv_cache) + slot * p.Hckv + c,
             make_uint4(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]),
                        pack_bf16x2(o[4], o[5]), pack_bf16x2(o[6], o[7])));
      }
    } else {
      // k^R: half-and-half RoPE with the token's (cos, sin); the partner
      // chunk lies Dr/2 columns away in row[].
      if (!write_cache) continue;
      const int i0 = c0 - p.Hcq - p.Hckv;
      const float* kr = row + p.Hcq + p.Hckv;
      float cs[8], sn[8], o[8];
      unpack_bf16x8(pa, cs);
      unpack_bf16x8(pb, sn);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        o[e] = i0 < half ? x[e] * cs[e] - kr[i0 + half + e] * sn[e]
                         : x[e] * cs[e] + kr[i0 - half + e] * sn[e];
      if (QM == 2) {
        int q[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) q[e] = sat_rne(o[e] / pf[e], -128, 127);
        st8_nt(static_cast<int8_t*>(p.kr_cache) + slot * p.Dr + i0,
            make_uint2(pack_i8x4(q[0], q[1], q[2], q[3]), pack_i8x4(q[4], q[5], q[6], q[7])));
      } else {
        st16_nt(static_cast<uint16_t*>(p.kr_cache) + slot * p.Dr + i0,
             make_uint4(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]),
                        pack_bf16x2(o[4], o[5]), pack_bf16x2(o[6], o[7])));
      }
    }
  }
  if (QM == 0 || jlo > 0) return;  // (the c^Q quant below: the c^Q workgroup)
  if (QM == 4) {
    if (threadIdx.x == 0) gst(p.cq_scale + t, 1.0f);  // static quant: no per-token scale
    return;
  }

  // Partial quant: per-token dynamic int8 of the smoothed c^Q (max-abs/127).
  const float am = block_reduce2<1>(make_float2(amax, 0.f), red).x;
  const float sc = am / 127.0f;
  for (int j = threadIdx.x; 8 * j < p.Hcq; j += blockDim.x) {
    const int c0 = 8 * j;
    int q[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) q[e] = sc > 0.f ? sat_rne(row[c0 + e] / sc, -127, 127) : 0;
    const uint2 w = make_uint2(pack_i8x4(q[0], q[1], q[2], q[3]), pack_i8x4(q[4], q[5], q[6], q[7]));
    st8(p.cq_i8 + cq_off(c0, 32), w);
    if (p.dbg_cq_i8) st8(p.dbg_cq_i8 + t * p.Hcq + c0, w);
  }
  if (threadIdx.x == 0) {
    gst(p.cq_scale + t, sc);
    if (p.dbg_cq_scale) gst(p.dbg_cq_scale + t, sc);
  }
}

// ---------------------------------------------------------------------------
// Decode up projection and W^UK product in one launch (bf16, one 32-row
// block, D <= 128): k_decode_tail<KS>.  Workgroups [0, up_tiles) are the up
// projection's kA6Cols-column tiles (three streaming waves and a fourth
// that joins the epilogue); q^C leaves with device-scope stores and the
// tile then counts itself done for each head it covers (up_tile_signal).
// The others are W^UK tiles (uk_tile_after_up), which load their W^UK
// slices while the up projection streams and wait only for their head.
// Measured at the DeepSeek-V3 decode shape: 20.2 us for the launch against
// 15.0 + 5.7 us for two launches (step 35.9 vs 37.1 us); the up-projection
// tiles and the W^UK loads together stream at about 5.9 TB/s, and the W^UK
// tiles end 2.5 us after the last up-projection tile.  (Running the
// down-projection finish as more workgroups of this launch, with the
// up-projection tiles loading weight while they wait for c^Q, measured
// 1 us slower: under the launch's load the finish took 6-7 us.)
// ---------------------------------------------------------------------------
struct DecodeTailParams {
  GemmParams up, uk;
  unsigned* ready;  // per head, SYNC_STRIDE words apart: up-projection tiles done
  int up_tiles, uk_tiles;
};

template <int KS>
__global__ __launch_bounds__(256) void k_decode_tail(DecodeTailParams p) {
  const int b = static_cast<int>(blockIdx.x);
  if (b < p.up_tiles) {
    skinny_tile<A_BF16, 1, 1, 3, 1, EPI_UQQR, 4, ALDS_NONE, A_LDS_STEPS, false, 1>(p.up, b, 0, 0);
    up_tile_signal(p.up, b, p.ready);
    return;
  }
  const int u = b - p.up_tiles;
  const int h = u / p.uk_tiles, ct = u % p.uk_tiles;
  uk_tile_after_up<KS>(p.uk, h, ct, p.ready + h * SYNC_STRIDE,
                       up_tiles_of_head(h, static_cast<int>(p.up.qc_D)));
}

// W^UK tile of the quantised merged decode launch: as uk_tile_after_up, with
// q^C in fp32 (fragment layout, 32 bytes per lane and k-step: the dequantised
// int8 up projection) split into bf16 hi + lo = bf16(q^C - hi) for two MFMAs
// per k-step, and MB 32-row blocks of tokens.  The head's q^C is staged in
// LDS once; the same LDS then stages the output tile for whole-row stores.
template <int KS, int MB>
__device__ __forceinline__ void uk_tile_f32_after_up(const GemmParams& p, const int h,
                                                     const int ct, const unsigned* ready,
                                                     const unsigned need) {
  static_assert(KS <= UK_MAX_STEPS, "the W^UK slice is held in registers");
  constexpr int OPITCH = UK_TILE_COLS + 4;
  constexpr int QC_CH = MB * KS * 128;                // 16-byte chunks of q^C
  constexpr int OUT_CH = (MB * 32 * OPITCH + 3) / 4;  // 16-byte chunks of the output stage
  __shared__ uint4 area[QC_CH > OUT_CH ? QC_CH : OUT_CH];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int li = lane & 31, g = lane >> 5;
  const int KC = static_cast<int>(p.K / 8);  // 16-byte chunk rows per column block
  const int64_t nblk = (p.N0 + 31) / 32;
  int64_t nb = static_cast<int64_t>(ct) * (UK_TILE_COLS / 32) + wave;
  nb = nb < nblk ? nb : nblk - 1;  // clamped blocks are computed, never stored
  const rsrc_t rb = make_rsrc(p.B0 + static_cast<int64_t>(h) * p.b_bstride + nb * KC * 32,
                              static_cast<uint32_t>(KC) * 512u);
  const uint32_t vl = static_cast<uint32_t>(lane) * 16u;
  uint4 w[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) w[s] = bld16_nt(rb, vl, static_cast<uint32_t>(s) * 1024u);

  if (threadIdx.x == 0) {
    uint32_t n = 0;
    while (__hip_atomic_load(ready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < need &&
           ++n < SYNC_SPIN_LIMIT)
      __builtin_amdgcn_s_sleep(4);
  }
  __syncthreads();

  // Head h's fp32 q^C: row block mb, k-step s is 64 lanes x 32 bytes at
  // (mb * KS + s) * 2 KB; copied as is.
  const rsrc_t ra = make_rsrc(static_cast<const char*>(p.A) + static_cast<int64_t>(h) * p.a_zs,
                              static_cast<uint32_t>(QC_CH) * 16u);
  constexpr int PER = (QC_CH + 255) / 256;
  uint4 q[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int c = static_cast<int>(threadIdx.x) + 256 * i;
    q[i] = bld16_dev(ra, static_cast<uint32_t>(c < QC_CH ? c : QC_CH - 1) * 16u, 0u);
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int c = static_cast<int>(threadIdx.x) + 256 * i;
    if (c < QC_CH) area[c] = q[i];
  }
  __syncthreads();
  f32x16_t acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x16_t{};
#pragma unroll
  for (int s = 0; s < KS; ++s)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const uint4 r0 = area[((mb * KS + s) * 64 + lane) * 2];
      const uint4 r1 = area[((mb * KS + s) * 64 + lane) * 2 + 1];
      uint4 hi, lo;
      split8(make_float4(__uint_as_float(r0.x), __uint_as_float(r0.y), __uint_as_float(r0.z),
                         __uint_as_float(r0.w)),
             make_float4(__uint_as_float(r1.x), __uint_as_float(r1.y), __uint_as_float(r1.z),
                         __uint_as_float(r1.w)),
             hi, lo);
      mfma_step<A_BF16>(acc[mb], hi, w[s]);
      mfma_step<A_BF16>(acc[mb], lo, w[s]);
    }
  __syncthreads();  // every wave is done with the staged q^C

  // MB 32x32 blocks -> LDS (row 32*mb + 8*(r/4) + 4*g + r%4, column
  // 32*wave + li), then each thread stores 8 consecutive columns of a row.
  uint32_t* stage = reinterpret_cast<uint32_t*>(area);
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      stage[(32 * mb + 8 * (r >> 2) + 4 * g + (r & 3)) * OPITCH + wave * 32 + li] =
          __float_as_uint(acc[mb][r]);
  __syncthreads();
  for (int it = threadIdx.x; it < MB * 32 * (UK_TILE_COLS / 8); it += 256) {
    const int row = it / (UK_TILE_COLS / 8);
    const int c0 = (it % (UK_TILE_COLS / 8)) * 8;
    const int64_t gcol = static_cast<int64_t>(ct) * UK_TILE_COLS + c0;
    if (row >= p.M || gcol >= p.N0) continue;
    const uint32_t* v = &stage[row * OPITCH + c0];
    st16_nt(p.q_out + row * p.q_ld + static_cast<int64_t>(h) * p.q_bstride + gcol,
            make_uint4(pack_bf16x2(__uint_as_float(v[0]), __uint_as_float(v[1])),
                       pack_bf16x2(__uint_as_float(v[2]), __uint_as_float(v[3])),
                       pack_bf16x2(__uint_as_float(v[4]), __uint_as_float(v[5])),
                       pack_bf16x2(__uint_as_float(v[6]), __uint_as_float(v[7]))));
  }
}

// Quantised decode (int8 c^Q and W^UQ_QR, bf16 query; T <= 32 * MB, D <=
// 128): the up projection's 32-column tiles (K over four waves) and the W^UK
// product in one launch, handed over per head as in k_decode_tail.  The up
// tiles write fp32 q^C with device-scope stores; the W^UK tiles wait for the
// D/32 tiles that cover their head.
constexpr int kA6ColsQ = 32;
template <int KS, int MB>
__global__ __launch_bounds__(256) void k_decode_tail_q(DecodeTailParams p) {
  const int b = static_cast<int>(blockIdx.x);
  if (b < p.up_tiles) {
    skinny_tile<A_I8, MB, 1, 1, 4, EPI_UQQR>(p.up, b, 0, 0);
    up_tile_signal(p.up, b, p.ready, kA6ColsQ);
    return;
  }
  const int u = b - p.up_tiles;
  const int h = u / p.uk_tiles, ct = u % p.uk_tiles;
  uk_tile_f32_after_up<KS, MB>(p.uk, h, ct, p.ready + h * SYNC_STRIDE,
                               up_tiles_of_head(h, static_cast<int>(p.up.qc_D), kA6ColsQ));
}

// ---------------------------------------------------------------------------
// MlaPreprocessV2 first step (aclnnMlaPreprocessV2: x is processed by
// RmsNormQuant before the W^DQKV product; formula block): per token,
// codes = sat(rne((gamma * x / RMS(x) + bias) * scale)) in [-128, 127],
// written row-major (T, He) for the int8 down projection, which reads the
// token's dequant scale from sx: 1 here (the per-channel dequant scales of
// W^DQKV carry the step).  One 256-thread workgroup per token, He a
// multiple of 64; x is read twice (the second pass hits the cache).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_rmsnorm_quant_x(const uint16_t* __restrict__ x,
                                                         const uint16_t* __restrict__ gamma,
                                                         const float* __restrict__ bias,
                                                         float qs, float eps, int He,
                                                         int8_t* __restrict__ x8,
                                                         float* __restrict__ sx,
                                                         int8_t* __restrict__ dbg) {
  __shared__ float2 red[4];
  const int64_t t = blockIdx.x;
  const uint16_t* row = x + t * He;
  float ss = 0.f;
  for (int c = 8 * static_cast<int>(threadIdx.x); c < He; c += 8 * 256) {
    float v[8];
    unpack_bf16x8(ld16(row + c), v);
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += v[e] * v[e];
  }
  const float tot = block_reduce2<0>(make_float2(ss, 0.f), red).x;
  const float r = 1.0f / __builtin_sqrtf(tot / static_cast<float>(He) + eps);
  for (int c = 8 * static_cast<int>(threadIdx.x); c < He; c += 8 * 256) {
    float v[8], g[8], b[8];
    unpack_bf16x8(ld16(row + c), v);
    unpack_bf16x8(ld16(gamma + c), g);
    ld8f(bias + c, b);
    int q[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) q[e] = sat_rne((v[e] * r * g[e] + b[e]) * qs, -128, 127);
    const uint2 w = make_uint2(pack_i8x4(q[0], q[1], q[2], q[3]), pack_i8x4(q[4], q[5], q[6], q[7]));
    st8(x8 + t * He + c, w);
    if (dbg) st8(dbg + t * He + c, w);
  }
  if (threadIdx.x == 0) gst(sx + t, 1.0f);
}

// ---------------------------------------------------------------------------
// int8 query per (token, head) for full quantisation with an int8 kv_cache
// (MlaPrologV2 README: query quantised per token and head, its scales in
// dequant_scale_q_nope (T, N, 1)).  One wave per row of H = Hckv fp32 q^N
// values: scale = max|q| / 127, codes round half to even in [-127, 127];
// an all-zero row gets scale 0 and zero codes.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_quant_query(const float* __restrict__ qn,
                                                     int8_t* __restrict__ q8,
                                                     float* __restrict__ qscale, int64_t rows,
                                                     int H) {
  const int lane = threadIdx.x & 63;
  const int64_t r = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;  // whole wave leaves together
  const float* src = qn + r * H;
  float amax = 0.f;
  for (int c = 8 * lane; c < H; c += 512) {
    float v[8];
    ld8f(src + c, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[e]));
  }
  amax = group_max<64>(amax);
  const float sc = amax / 127.0f;
  for (int c = 8 * lane; c < H; c += 512) {
    float v[8];
    ld8f(src + c, v);
    int q[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) q[e] = sc > 0.f ? sat_rne(v[e] / sc, -127, 127) : 0;
    st8(q8 + r * H + c,
        make_uint2(pack_i8x4(q[0], q[1], q[2], q[3]), pack_i8x4(q[4], q[5], q[6], q[7])));
  }
  if (lane == 0) gst(qscale + r, sc);
}

// ---------------------------------------------------------------------------
// Activation packing for the 256-tile GEMM: bf16 rows (M, K) into the MFMA
// fragment layout, where chunk (32-row block mb, k-step s, lane (g, i))
// holds row 32*mb + i, k in [16s + 8g, 16s + 8g + 8).  One workgroup moves a
// 32-row x (16*PA_STEPS)-k block through LDS: thread c reads 16 bytes at
// (row c/CPR, chunk c%CPR), CPR = 2*PA_STEPS chunks of contiguous row bytes,
// into LDS slot (chunk)*32 + row, which is exactly the block's fragment
// order, so the writes are contiguous.  Rows past M are zeros.
// ---------------------------------------------------------------------------
constexpr int PA_STEPS = 32;  // k-steps per workgroup (512 k)
__global__ __launch_bounds__(256) void k_pack_a(const uint16_t* __restrict__ src,
                                                uint4* __restrict__ dst, int64_t M, int64_t K) {
  constexpr int CPR = 2 * PA_STEPS;       // 16-byte chunks per row of the block
  constexpr int PER = 32 * CPR / 256;     // chunks per thread
  __shared__ uint4 blk[PA_STEPS * 64];
  const int64_t steps = K / 16;
  const int64_t mb = blockIdx.y;
  const int64_t s0 = static_cast<int64_t>(blockIdx.x) * PA_STEPS;
  const int ns = static_cast<int>(min<int64_t>(PA_STEPS, steps - s0));
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int c = threadIdx.x + 256 * u;
    const int row = c / CPR, q = c % CPR;
    const int64_t m = mb * 32 + row;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (q < 2 * ns && m < M) {  // x is read once: streaming loads (10 us faster at T = 4096)
      const u32x4_t w = __builtin_nontemporal_load(
          (const QKVNR_GLOBAL u32x4_t*)(src + m * K + (s0 * 16 + 8 * q)));
      v = make_uint4(w.x, w.y, w.z, w.w);
    }
    blk[q * 32 + row] = v;
  }
  __syncthreads();
  uint4* out = dst + (mb * steps + s0) * 64;
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int o = threadIdx.x + 256 * u;
    if (o < ns * 64) st16(out + o, blk[o]);
  }
}

// ---------------------------------------------------------------------------
// Weight packing into the N32-blocked K16 layout, one thread per 16-byte
// output chunk (block nb, chunk row kc, column j): the G = 16/eb consecutive
// k values of column 32*nb + j.  Columns past N (the last block's padding)
// are zero.  Columns from rope_col0 on are rope heads of rope_dim columns;
// when rope_dim > 32 they are reordered so that packed block b of a head
// holds natural columns [16b, 16b + 16) then [rope_dim/2 + 16b, ... + 16).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_pack(const char* __restrict__ src, uint4* __restrict__ dst,
                                              int64_t batch, int64_t K, int64_t N, int eb,
                                              int64_t rope_col0, int64_t rope_dim, int kperm) {
  const int G = 16 / eb;
  const int64_t KC = K / G;
  const int64_t nblk = (N + 31) / 32;
  const int64_t per = nblk * KC * 32;
  const int64_t total = batch * per;
  for (int64_t c = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; c < total;
       c += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t b = c / per;
    const int64_t r = c % per;
    const int64_t nb = r / (KC * 32);
    const int64_t kc = (r / 32) % KC;
    const int64_t n = nb * 32 + (r % 32);
    uint32_t w[4] = {0, 0, 0, 0};
    if (n < N) {
      int64_t ns = n;  // source column
      if (n >= rope_col0 && rope_dim > 32) {
        const int64_t rr = n - rope_col0;
        const int64_t pj = rr % rope_dim, bb = pj / 32, ww = pj % 32;
        ns = rope_col0 + (rr - pj) + (ww < 16 ? 16 * bb + ww : rope_dim / 2 + 16 * bb + ww - 16);
      }
      const char* s = src + ((b * K + kc * G) * N + ns) * eb;
      if (eb == 2) {
        // kperm: chunk kc = 2*step + h holds k = 16*step + {4h..4h+3, 8+4h..8+4h+3}
        const char* s2 = src + ((b * K + (kc & ~int64_t(1)) * G) * N + ns) * eb;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int64_t ke = kperm ? ((e < 4 ? 0 : 8) + 4 * (kc & 1) + (e & 3)) : e;
          const uint32_t v =
              *reinterpret_cast<const uint16_t*>((kperm ? s2 : s) + ke * N * 2);
          w[e >> 1] |= v << (16 * (e & 1));
        }
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const uint32_t v = static_cast<uint8_t>(s[static_cast<int64_t>(e) * N]);
          w[e >> 2] |= v << (8 * (e & 3));
        }
      }
    }
    dst[c] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// One launch: the stream and, when the caller asked for per-kernel timing,
// the start and stop events (hipExtLaunchKernel takes them at the kernel's
// own dispatch, so they bracket exactly its execution).
struct Launch {
  hipStream_t st;
  hipEvent_t start;
  hipEvent_t stop;
};
template <typename F, typename... Args>
void launch(const Launch& L, F kernel, dim3 grid, dim3 block, uint32_t shmem, Args... args) {
  if (L.start != nullptr)
    hipExtLaunchKernelGGL(kernel, grid, block, shmem, L.st, L.start, L.stop, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, shmem, L.st, args...);
}

template <int AK, int MB, int NB, int NW, int KW, int EPI>
void skinny(const GemmParams& p, dim3 grid, const Launch& L) {
  launch(L, k_skinny<AK, MB, NB, NW, KW, EPI>, grid, dim3(64 * NW * KW), 0, p);
}


// Decode plan: three weight-streaming launches plus the down-projection
// finish (launched between A1 and A6).  Many short per-wave weight runs keep
// the most bytes in flight.  A1: 64-column tiles with the K range split over
// ksplit workgroups and, inside one, over 8 waves (fewer when more 32-row
// blocks fill the registers); with one or two row blocks, x is staged in LDS
// and two waves across take one column block each.  A6: 96-column tiles, three waves
// across with one column block each (256 tiles for the DeepSeek-V3 shape:
// one per CU); with one row block each wave streams the whole K in batches
// of 4 k-steps, otherwise K is split over waves.  A8: 4 waves on different
// column blocks of one head, the head's q^C staged in LDS.
template <int MB>
constexpr int a1_kw() { return MB >= 4 ? 2 : (MB == 2 ? 4 : 8); }
template <int MB>
constexpr int a6_kw() { return MB >= 4 ? 1 : 2; }
template <int MB>
constexpr int a8_nw() { return 4; }
// A1 tiles are kA1Cols = 64 columns wide (plan.h): two column blocks, one
// per wave across when x is staged in LDS, both in each wave otherwise.

// A1 reads x row-major: with one or two 32-row blocks each workgroup stages
// its split of x in LDS (fragment order; bf16 x up to 64 k-steps, int8 x up
// to A1_I8_LDS_STEPS), otherwise lanes load rows directly.
constexpr int A1_I8_LDS_STEPS = 32;
template <int MB>
void skinny_a1(const GemmParams& g1, const MlaPlan& pl, bool xq, const Launch& L) {
  const dim3 grid(static_cast<unsigned>(g1.ntiles0 + (g1.N1 + kA1Cols - 1) / kA1Cols),
                  static_cast<unsigned>(pl.ksplit), 1);
  constexpr int KW = a1_kw<MB>();
  if (xq) {
    // full quantisation: int8 x . int8 weights (32-k steps), int32 sums;
    // staged like the bf16 x below (a split of at most 32 steps: 4 per wave)
    if constexpr (MB <= 2) {
      if (pl.steps_per_split <= A1_I8_LDS_STEPS) {
        launch(L, k_skinny<A_I8, MB, 1, 2, 8, EPI_PARTIAL, 4, ALDS_ROWMAJOR, A1_I8_LDS_STEPS>,
               grid, dim3(64 * 2 * 8), 0, g1);
        return;
      }
    }
    skinny<A_I8, MB, 2, 1, KW, EPI_PARTIAL>(g1, grid, L);
    return;
  }
  if constexpr (MB == 1) {
    if (pl.steps_per_split <= A_LDS_STEPS) {
      // one column block per wave, two waves across, K over 8 waves
      launch(L, k_skinny<A_BF16, 1, 1, 2, KW, EPI_PARTIAL, 8, ALDS_ROWMAJOR>, grid,
             dim3(64 * 2 * KW), 0, g1);
      return;
    }
  } else if constexpr (MB == 2) {
    if (pl.steps_per_split <= A_LDS_STEPS) {
      // the same shape over two row blocks (x split staged once: 128 KB)
      launch(L, k_skinny<A_BF16, 2, 1, 2, 8, EPI_PARTIAL, 8, ALDS_ROWMAJOR>, grid,
             dim3(64 * 2 * 8), 0, g1);
      return;
    }
  }
  skinny<A_BF16, MB, 2, 1, KW, EPI_PARTIAL>(g1, grid, L);
}
template <int MB>
void skinny_a6(const GemmParams& g6, bool quant, const Launch& L) {
  const unsigned nt = static_cast<unsigned>((g6.N0 + kA6Cols - 1) / kA6Cols);
  if (quant && nt < 128) {
    // few columns (e.g. 32 heads): 32-column tiles with K over 4 waves fill
    // more CUs than 96-column tiles (T = 64, N = 32: 7.4 vs 12.4 us)
    skinny<A_I8, MB, 1, 1, 4, EPI_UQQR>(g6, dim3(static_cast<unsigned>((g6.N0 + 31) / 32), 1, 1),
                                        L);
  } else if (quant)
    skinny<A_I8, MB, 1, 3, a6_kw<MB>(), EPI_UQQR>(g6, dim3(nt, 1, 1), L);
  else if constexpr (MB == 1)
    // each wave streams its column block over the whole K, 4 k-steps per batch
    launch(L, k_skinny<A_BF16, 1, 1, 3, 1, EPI_UQQR, 4>, dim3(nt, 1, 1), dim3(64 * 3), 0, g6);
  else
    skinny<A_BF16, MB, 1, 3, a6_kw<MB>(), EPI_UQQR>(g6, dim3(nt, 1, 1), L);
}
// A8 stages a head's q^C (K = D <= 16 k-steps) in LDS once per workgroup;
// the one-workgroup-per-head query-quant variant stages fp32 q^C (<= 8
// k-steps).  (Staging fp32 q^C in the four-wave quantised tiles below made
// them slower, 5.4 -> 6.7 us at T = 64: the staging latency comes before
// the first MFMA, and the lockstep waves' re-reads hit L1.)
constexpr int A8_LDS_STEPS = 16;
constexpr int A8_LDS_STEPS_F32 = 8;
template <int MB>
void skinny_a8(const GemmParams& g8, int nheads, bool quant, const Launch& L) {
  constexpr int NW = a8_nw<MB>();
  const unsigned nt = static_cast<unsigned>((g8.N0 + 32 * NW - 1) / (32 * NW));
  const dim3 grid(nt, 1, static_cast<unsigned>(nheads));
  if (quant && MB <= 2 && grid.x * grid.z < 256) {
    // few heads (e.g. 32): 64-column tiles with K over 2 waves give more
    // workgroups (T = 64, N = 32: 4.9 vs 5.8 us)
    const dim3 g2(static_cast<unsigned>((g8.N0 + 63) / 64), 1, static_cast<unsigned>(nheads));
    skinny<A_F32SPLIT, MB, 1, 2, 2, EPI_UK>(g8, g2, L);
  } else if (quant)
    skinny<A_F32SPLIT, MB, 1, NW, 1, EPI_UK>(g8, grid, L);
  else if (MB == 1 && g8.K / 16 <= A8_LDS_STEPS && g8.a_frag)
    launch(L, k_skinny<A_BF16, 1, 1, NW, 1, EPI_UK, 4, ALDS_FRAG, A8_LDS_STEPS>, grid,
           dim3(64 * NW), 0, g8);
  else
    skinny<A_BF16, MB, 1, NW, 1, EPI_UK>(g8, grid, L);
}

}  // namespace

int launch_pack_weight(const void* src, void* dst, int64_t batch, int64_t K, int64_t N,
                       int elem_bytes, int64_t rope_col0, int64_t rope_dim, void* stream_v,
                       bool kperm) {
  const hipStream_t stream = static_cast<hipStream_t>(stream_v);
  const int G = 16 / elem_bytes;
  const int64_t total = batch * (K / G) * ((N + 31) / 32) * 32;
  if (total == 0) return QKVNR_OK;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(k_pack, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                     static_cast<const char*>(src), static_cast<uint4*>(dst), batch, K, N,
                     elem_bytes, rope_col0, rope_dim, kperm ? 1 : 0);
  return hipGetLastError() == hipSuccess ? QKVNR_OK : QKVNR_ERR_LAUNCH_FAILED;
}

int launch_mla_prolog_v2(const MlaPrologV2Args* a, const MlaPlan& pl, void* workspace,
                         void* stream, const PreprocessExtra* pre) {
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t T = a->B * a->S;
  if (T == 0) return QKVNR_OK;
  const bool quant = a->quant_mode != MLA_QUANT_NONE;
  const bool xq = a->quant_mode == MLA_QUANT_FULL_KV_BF16 || a->quant_mode == MLA_QUANT_FULL_KV_INT8;
  const bool q8out = a->quant_mode == MLA_QUANT_FULL_KV_INT8;
  // finish variant: 0 none, 1 c^Q quant + bf16 caches, 2 + int8 kv / kr,
  // 3 + int8 kv and bf16 kr (k_down_finish's QM)
  const int qm = pre != nullptr                              ? 4
                 : a->quant_mode == MLA_QUANT_FULL_KV_BF16 ? 1
                 : a->quant_mode == MLA_QUANT_FULL_KV_INT8 ? 3
                                                           : a->quant_mode;
  char* ws = static_cast<char*>(workspace);
  const int64_t NDR = a->N * (a->D + a->Dr);
  const int64_t ntot = a->Hcq + a->Hckv + a->Dr;

  const uint4 *wdq, *wdkvkr, *wuqqr, *wuk;
  // MlaPreprocessV2's merged W^DQKV packs as one matrix: with Hcq a whole
  // number of 32-column blocks, its W^DKV | W^KR columns start at block
  // Hcq / 32, the layout of two separately packed matrices back to back.
  const int64_t dkv_chunks = (a->Hcq / 32) * (a->He / (xq ? 16 : 8)) * 32;
  if (a->weight_layout == MLA_WEIGHT_ND) {
    const int eb_down = xq ? 1 : 2;
    int rc = pre != nullptr
                 ? launch_pack_weight(a->weight_dq, ws + pl.off_wdq, 1, a->He, ntot, 1, ntot, 0, st)
                 : launch_pack_weight(a->weight_dq, ws + pl.off_wdq, 1, a->He, a->Hcq, eb_down,
                                      a->Hcq, 0, st);
    if (rc == QKVNR_OK && pre == nullptr)
      rc = launch_pack_weight(a->weight_dkv_kr, ws + pl.off_wdkvkr, 1, a->He, a->Hckv + a->Dr,
                              eb_down,
                              a->Hckv + a->Dr, 0, st);
    if (rc == QKVNR_OK)
      rc = launch_pack_weight(a->weight_uq_qr, ws + pl.off_wuqqr, 1, a->Hcq, NDR, quant ? 1 : 2,
                              a->N * a->D, a->Dr, st);
    if (rc == QKVNR_OK)
      rc = launch_pack_weight(a->weight_uk, ws + pl.off_wuk, a->N, a->D, a->Hckv, 2, a->Hckv, 0,
                              st, /*kperm=*/true);
    if (rc != QKVNR_OK) return rc;
    wdq = reinterpret_cast<const uint4*>(ws + pl.off_wdq);
    wdkvkr = pre != nullptr ? wdq + dkv_chunks : reinterpret_cast<const uint4*>(ws + pl.off_wdkvkr);
    wuqqr = reinterpret_cast<const uint4*>(ws + pl.off_wuqqr);
    wuk = reinterpret_cast<const uint4*>(ws + pl.off_wuk);
  } else {
    wdq = static_cast<const uint4*>(a->weight_dq);
    wdkvkr = pre != nullptr ? wdq + dkv_chunks : static_cast<const uint4*>(a->weight_dkv_kr);
    wuqqr = static_cast<const uint4*>(a->weight_uq_qr);
    wuk = static_cast<const uint4*>(a->weight_uk);
  }
  // Phase events (instrumentation only).
  auto mark = [&](int i) {
    if (i < a->n_phase_events && a->phase_events[i] != nullptr)
      (void)hipEventRecord(static_cast<hipEvent_t>(a->phase_events[i]), st);
  };

  float* part = reinterpret_cast<float*>(ws + pl.off_part);
  void* cq = ws + pl.off_cq;
  float* cq_scale = reinterpret_cast<float*>(ws + pl.off_cq_scale);
  void* qc = ws + pl.off_qc;

  // ---- A1: x . [W^DQ | W^DKV_KR] -> fp32 (partials) ----
  // The skinny and 256-tile plans read c^Q and q^C in fragment layout
  // (written so by the finish kernel and A6's epilogue); x is read
  // row-major.
  const bool frag = pl.skinny || pl.gemm256;
  const int64_t mblocks = pl.rows / 32;
  GemmParams g1{};
  g1.A = pre != nullptr ? static_cast<const void*>(ws + pl.off_prex8) : a->token_x;
  g1.lda = a->He;
  g1.B0 = wdq;
  g1.N0 = a->Hcq;
  g1.B1 = wdkvkr;
  g1.N1 = a->Hckv + a->Dr;
  g1.M = T;
  g1.K = a->He;
  g1.steps_per_split = pl.steps_per_split;
  g1.part = part;
  g1.part_ld = ntot;

  // ---- A6: c^Q . [W^UQ | W^QR] -> q^C (workspace) and RoPE'd q^R ----
  GemmParams g6{};
  g6.A = cq;
  g6.lda = a->Hcq;
  g6.B0 = wuqqr;
  g6.N0 = NDR;
  g6.M = T;
  g6.K = a->Hcq;
  g6.ntiles0 = 1 << 30;  // every tile reads B0
  g6.steps_per_split = a->Hcq / (quant ? 32 : 16);
  g6.ND = a->N * a->D;
  g6.Dr = static_cast<int>(a->Dr);
  g6.cosb = static_cast<const uint16_t*>(a->rope_cos);
  g6.sinb = static_cast<const uint16_t*>(a->rope_sin);
  g6.cq_scale = cq_scale;
  g6.dq = a->dequant_scale_w_uq_qr;
  g6.qc_out = qc;
  g6.qc_f32 = quant ? 1 : 0;
  g6.qr_out = static_cast<uint16_t*>(a->query_rope);
  g6.qr_ld = a->N * a->Dr;
  if (frag) {
    g6.a_frag = 1;
    g6.a_mbs = a->Hcq * (quant ? 32 : 64);  // 32 rows x Hcq int8 / bf16
    g6.qc_frag = 1;
    g6.qc_D = a->D;
    g6.qc_mblocks = mblocks;
  }

  // ---- A8: per head q^C[:, n] . W^UK[n] -> query ----
  GemmParams g8{};
  g8.A = qc;
  g8.lda = a->N * a->D;
  g8.a_bstride = a->D;
  g8.B0 = wuk;
  g8.N0 = a->Hckv;
  g8.b_bstride = ((a->Hckv + 31) / 32) * (a->D / 8) * 32;  // chunks per packed head
  g8.M = T;
  g8.K = a->D;
  g8.ntiles0 = 1 << 30;
  g8.steps_per_split = a->D / 16;
  g8.q_out = static_cast<uint16_t*>(a->query);
  g8.q_ld = a->N * a->Hckv;
  g8.q_bstride = a->Hckv;
  // FULL_KV_INT8: one workgroup per head quantises the query in its
  // epilogue when a head's Hckv fits one tile of at most 16 waves and T fits
  // one row block (the plan's qh); otherwise q^N goes out in fp32 for
  // k_quant_query.
  const bool qh = pl.qh;
  if (q8out && !qh) g8.q_f32 = reinterpret_cast<float*>(ws + pl.off_qn);
  if (qh) {
    g8.q8_out = static_cast<int8_t*>(a->query);
    g8.q8_scale = a->dequant_scale_q_nope;
  }
  if (frag) {
    g8.a_frag = 1;
    g8.a_mbs = a->D * (quant ? 128 : 64);  // 32 rows x D fp32 / bf16
    g8.a_zs = mblocks * g8.a_mbs;
  }

  // ---- finish of A1 ----
  FinishParams f{};
  f.part = part;
  f.ksplit = pl.ksplit;
  f.T = T;
  f.Hcq = static_cast<int>(a->Hcq);
  f.Hckv = static_cast<int>(a->Hckv);
  f.Dr = static_cast<int>(a->Dr);
  f.eps_cq = static_cast<float>(a->rmsnorm_epsilon_cq);
  f.eps_ckv = static_cast<float>(a->rmsnorm_epsilon_ckv);
  f.gamma_cq = static_cast<const uint16_t*>(a->rmsnorm_gamma_cq);
  f.gamma_ckv = static_cast<const uint16_t*>(a->rmsnorm_gamma_ckv);
  f.smooth = a->smooth_scales_cq;
  f.qs_ckv = a->quant_scale_ckv;
  f.qs_ckr = a->quant_scale_ckr;
  f.cosb = static_cast<const uint16_t*>(a->rope_cos);
  f.sinb = static_cast<const uint16_t*>(a->rope_sin);
  f.index = a->cache_index;
  f.slots = a->block_num * a->block_size;
  f.kv_cache = a->kv_cache;
  f.kr_cache = a->kr_cache;
  f.cq_bf16 = static_cast<uint16_t*>(cq);
  f.cq_i8 = static_cast<int8_t*>(cq);
  f.cq_scale = cq_scale;
  f.cq_frag = frag ? 1 : 0;
  f.dbg_cq_i8 = a->dbg_cq_int8;
  f.dbg_cq_scale = a->dbg_cq_scale;
  if (xq) {
    f.sx = pre != nullptr ? reinterpret_cast<const float*>(ws + pl.off_presx) : a->dequant_scale_x;
    f.sw_dq = a->dequant_scale_w_dq;
    f.sw_dkv = a->dequant_scale_w_dkv_kr;
  }
  if (pre != nullptr) f.qs_cq = pre->qs_cq;
  // Merged decode tail: the down projection zeroes its handoff counters.
  unsigned* ready = reinterpret_cast<unsigned*>(ws + pl.off_sync);
  if (pl.merge_uk || pl.merge_uk_q) {
    g1.zero_words = ready;
    g1.zero_count = static_cast<int>(a->N);
    g6.qc_coherent = 1;
  }
  const size_t fin_smem = static_cast<size_t>(ntot) * sizeof(float);
  // Two workgroups per token (c^Q; c^KV and k^R), sized for the larger
  // part.
  const int fin_y = 2;
  const dim3 fin_block(static_cast<unsigned>(fin_threads(std::max<int64_t>(a->Hcq, a->Hckv + a->Dr))));

  // Launch contexts of the main kernels (optional per-kernel timing).
  Launch Lk[MLA_KERNEL_COUNT];
  for (int i = 0; i < MLA_KERNEL_COUNT; ++i) {
    Lk[i] = {st, nullptr, nullptr};
    if (a->n_kernel_events > 2 * i + 1) {
      Lk[i].start = static_cast<hipEvent_t>(a->kernel_events[2 * i]);
      Lk[i].stop = static_cast<hipEvent_t>(a->kernel_events[2 * i + 1]);
    }
  }
  const Launch L0{st, nullptr, nullptr};
  const Launch& L1 = Lk[MLA_KERNEL_DOWN];
  const Launch& Lf = Lk[MLA_KERNEL_NORM];
  const Launch& L6 = Lk[MLA_KERNEL_UQQR];
  const Launch& L8 = Lk[MLA_KERNEL_UK];

  // The large-T plan splits at most FIN_SPLIT_SMALL ways: its instances
  // hold fewer partials per thread and keep more workgroups resident.
  auto finish = [&]() {
    const dim3 grid(static_cast<unsigned>(T), static_cast<unsigned>(fin_y));
    const uint32_t sm = static_cast<uint32_t>(fin_smem);
    if (pl.ksplit <= FIN_SPLIT_SMALL) {
      switch (qm) {
        case 0: launch(Lf, k_down_finish<0, FIN_SPLIT_SMALL>, grid, fin_block, sm, f); break;
        case 1: launch(Lf, k_down_finish<1, FIN_SPLIT_SMALL>, grid, fin_block, sm, f); break;
        case 2: launch(Lf, k_down_finish<2, FIN_SPLIT_SMALL>, grid, fin_block, sm, f); break;
        case 3: launch(Lf, k_down_finish<3, FIN_SPLIT_SMALL>, grid, fin_block, sm, f); break;
        default: launch(Lf, k_down_finish<4, FIN_SPLIT_SMALL>, grid, fin_block, sm, f); break;
      }
      return;
    }
    switch (qm) {
      case 0: launch(Lf, k_down_finish<0>, grid, fin_block, sm, f); break;
      case 1: launch(Lf, k_down_finish<1>, grid, fin_block, sm, f); break;
      case 2: launch(Lf, k_down_finish<2>, grid, fin_block, sm, f); break;
      case 3: launch(Lf, k_down_finish<3>, grid, fin_block, sm, f); break;
      default: launch(Lf, k_down_finish<4>, grid, fin_block, sm, f); break;
    }
  };

  const int nh = static_cast<int>(a->N);
  if (pre != nullptr)  // RmsNormQuant of x: the down projection's int8 input
    launch(L0, k_rmsnorm_quant_x, dim3(static_cast<unsigned>(T)), dim3(256), 0,
           static_cast<const uint16_t*>(a->token_x), static_cast<const uint16_t*>(pre->gamma_x),
           pre->bias_x, pre->qs_x, static_cast<float>(a->rmsnorm_epsilon_cq),
           static_cast<int>(a->He), reinterpret_cast<int8_t*>(ws + pl.off_prex8),
           reinterpret_cast<float*>(ws + pl.off_presx), pre->dbg_x_int8);
  mark(MLA_PHASE_START);
  if (pl.skinny) {
    g1.ntiles0 = static_cast<int>((g1.N0 + kA1Cols - 1) / kA1Cols);
    switch (pl.mb) {
      case 1: skinny_a1<1>(g1, pl, xq, L1); break;
      case 2: skinny_a1<2>(g1, pl, xq, L1); break;
      default: skinny_a1<4>(g1, pl, xq, L1); break;
    }
    mark(MLA_PHASE_AFTER_DOWN);
    finish();
    mark(MLA_PHASE_AFTER_NORM);
    if (pl.merge_uk) {
      DecodeTailParams u{};
      u.up = g6;
      u.uk = g8;
      u.ready = ready;
      u.up_tiles = static_cast<int>((g6.N0 + kA6Cols - 1) / kA6Cols);
      u.uk_tiles = static_cast<int>((a->Hckv + UK_TILE_COLS - 1) / UK_TILE_COLS);
      const dim3 grid(static_cast<unsigned>(u.up_tiles + nh * u.uk_tiles));
      switch (a->D / 16) {
        case 2: launch(L6, k_decode_tail<2>, grid, dim3(256), 0, u); break;
        case 4: launch(L6, k_decode_tail<4>, grid, dim3(256), 0, u); break;
        case 6: launch(L6, k_decode_tail<6>, grid, dim3(256), 0, u); break;
        default: launch(L6, k_decode_tail<8>, grid, dim3(256), 0, u); break;
      }
      mark(MLA_PHASE_AFTER_UQQR);
    } else if (pl.merge_uk_q) {
      DecodeTailParams u{};
      u.up = g6;
      u.uk = g8;
      u.ready = ready;
      u.up_tiles = static_cast<int>((g6.N0 + kA6ColsQ - 1) / kA6ColsQ);
      u.uk_tiles = static_cast<int>((a->Hckv + UK_TILE_COLS - 1) / UK_TILE_COLS);
      const dim3 grid(static_cast<unsigned>(u.up_tiles + nh * u.uk_tiles));
      // (D a multiple of 32, at most 128: 2, 4, 6 or 8 k-steps)
      const int ks = static_cast<int>(a->D / 16);
      if (pl.mb == 1) {
        switch (ks) {
          case 2: launch(L6, k_decode_tail_q<2, 1>, grid, dim3(256), 0, u); break;
          case 4: launch(L6, k_decode_tail_q<4, 1>, grid, dim3(256), 0, u); break;
          case 6: launch(L6, k_decode_tail_q<6, 1>, grid, dim3(256), 0, u); break;
          default: launch(L6, k_decode_tail_q<8, 1>, grid, dim3(256), 0, u); break;
        }
      } else {
        switch (ks) {
          case 2: launch(L6, k_decode_tail_q<2, 2>, grid, dim3(256), 0, u); break;
          case 4: launch(L6, k_decode_tail_q<4, 2>, grid, dim3(256), 0, u); break;
          case 6: launch(L6, k_decode_tail_q<6, 2>, grid, dim3(256), 0, u); break;
          default: launch(L6, k_decode_tail_q<8, 2>, grid, dim3(256), 0, u); break;
        }
      }
      mark(MLA_PHASE_AFTER_UQQR);
    } else {
      switch (pl.mb) {
        case 1: skinny_a6<1>(g6, quant, L6); break;
        case 2: skinny_a6<2>(g6, quant, L6); break;
        default: skinny_a6<4>(g6, quant, L6); break;
      }
      mark(MLA_PHASE_AFTER_UQQR);
    }
    if (pl.merge_uk || pl.merge_uk_q) {
      // the W^UK product ran inside k_decode_tail(_q)
    } else if (qh) {
      // one workgroup per head; its fp32 q^C (D <= 128) staged in LDS once
      // (16 waves re-reading it: 11.2 -> 9.9 us at the DeepSeek-V3 shape)
      const dim3 grid(1, 1, static_cast<unsigned>(nh));
      const bool stage = a->D / 16 <= A8_LDS_STEPS_F32;
      if (a->Hckv <= 128 && stage)
        launch(L8, k_skinny<A_F32SPLIT, 1, 1, 4, 1, EPI_UK, 2, ALDS_FRAG, A8_LDS_STEPS_F32, true>,
               grid, dim3(64 * 4), 0, g8);
      else if (a->Hckv <= 128)
        launch(L8, k_skinny<A_F32SPLIT, 1, 1, 4, 1, EPI_UK, 2, ALDS_NONE, A_LDS_STEPS, true>,
               grid, dim3(64 * 4), 0, g8);
      else if (a->Hckv <= 256 && stage)
        launch(L8, k_skinny<A_F32SPLIT, 1, 1, 8, 1, EPI_UK, 2, ALDS_FRAG, A8_LDS_STEPS_F32, true>,
               grid, dim3(64 * 8), 0, g8);
      else if (a->Hckv <= 256)
        launch(L8, k_skinny<A_F32SPLIT, 1, 1, 8, 1, EPI_UK, 2, ALDS_NONE, A_LDS_STEPS, true>,
               grid, dim3(64 * 8), 0, g8);
      else if (stage)
        launch(L8, k_skinny<A_F32SPLIT, 1, 1, 16, 1, EPI_UK, 2, ALDS_FRAG, A8_LDS_STEPS_F32, true>,
               grid, dim3(64 * 16), 0, g8);
      else
        launch(L8, k_skinny<A_F32SPLIT, 1, 1, 16, 1, EPI_UK, 2, ALDS_NONE, A_LDS_STEPS, true>,
               grid, dim3(64 * 16), 0, g8);
    } else {
      switch (pl.mb) {
        case 1: skinny_a8<1>(g8, nh, quant, L8); break;
        case 2: skinny_a8<2>(g8, nh, quant, L8); break;
        default: skinny_a8<4>(g8, nh, quant, L8); break;
      }
    }
  } else {
    // Large T (pl.gemm256).  x into fragment layout first: the GEMM's A
    // loads are then 1 KB contiguous per wave (row-major x costs 32 cache
    // lines per load).  int8 x (full quantisation, MlaPreprocessV2's codes)
    // moves as 16-bit pairs: a 32-byte k-step is 32 int8 k or 16 bf16 k.
    const int64_t xk = xq ? a->He / 2 : a->He;  // row length in 16-bit units
    launch(L0, k_pack_a,
           dim3(static_cast<unsigned>((xk / 16 + PA_STEPS - 1) / PA_STEPS),
                static_cast<unsigned>(mblocks)),
           dim3(256), 0, static_cast<const uint16_t*>(g1.A),
           reinterpret_cast<uint4*>(ws + pl.off_xfrag), T, xk);
    g1.A = ws + pl.off_xfrag;
    g1.a_frag = 1;
    g1.a_mbs = xk * 64;
    // A6's q^R columns (bf16) and the quantised A6 and W^UK product:
    // 128x256 tiles and three buffers, two workgroups per CU so one's
    // epilogue stores overlap the other's main loop (256-row tiles measured
    // the same for q^R).  A1 and the fused q^C + W^UK tiles: 256x256, eight
    // waves, four buffers (A1 at T = 4096: 157 vs 167 us).
    const unsigned mt2 = static_cast<unsigned>((T + G_TM_HALF - 1) / G_TM_HALF);
    g1.ntiles0 = static_cast<int>((g1.N0 + G_TN - 1) / G_TN);
    const unsigned nt1 = static_cast<unsigned>(g1.ntiles0 + (g1.N1 + G_TN - 1) / G_TN);
    const dim3 grid1(nt1, static_cast<unsigned>((T + 255) / 256), static_cast<unsigned>(pl.ksplit));
    if (xq)
      launch(L1, k_gemm<EPI_PARTIAL, 256, 4, 0, A_I8>, grid1, dim3(64 * gemm_waves<256>()), 0, g1);
    else
      launch(L1, k_gemm<EPI_PARTIAL, 256, 4>, grid1, dim3(64 * gemm_waves<256>()), 0, g1);
    mark(MLA_PHASE_AFTER_DOWN);
    finish();
    mark(MLA_PHASE_AFTER_NORM);
    if (pl.fuse_uk) {
      // One launch: the q^C tiles with the W^UK product in their epilogue,
      // then the q^R tiles.  q^R: the W^QR columns alone (packed columns
      // from N*D on; with the rope region at column 0 every column is a
      // rope column).
      const int64_t ND = a->N * a->D;
      GemmParams gr = g6;
      gr.B0 = wuqqr + (ND / 32) * (a->Hcq / (quant ? 16 : 8)) * 32;
      gr.N0 = a->N * a->Dr;
      gr.ND = 0;
      if (quant) gr.dq = g6.dq + ND;  // the W^QR columns' dequant scales
      GemmParams gq = g6;
      gq.N0 = ND;
      gq.Buk = wuk;
      gq.uk_bstride = g8.b_bstride;
      gq.uk_N = a->Hckv;
      gq.q_out = g8.q_out;
      gq.q_ld = g8.q_ld;
      gq.q_bstride = g8.q_bstride;
      const int nqx = static_cast<int>(ND / G_TN);
      const int nrx = static_cast<int>((gr.N0 + G_TN - 1) / G_TN);
      const int ny = static_cast<int>((T + 255) / 256);
      const dim3 grid(static_cast<unsigned>((nqx + nrx) * ny));
      if (quant)
        launch(L8, k_up_fused<A_I8>, grid, dim3(64 * gemm_waves<256>()), 0, gq, gr, nqx, nrx, ny);
      else
        launch(L8, k_up_fused<A_BF16>, grid, dim3(64 * gemm_waves<256>()), 0, gq, gr, nqx, nrx, ny);
      mark(MLA_PHASE_AFTER_UQQR);
    } else {
      const unsigned nt6 = static_cast<unsigned>((g6.N0 + G_TN - 1) / G_TN);
      if (quant) {
        // int8 c^Q . int8 [W^UQ | W^QR]; q^C leaves as bf16 hi and lo
        // fragments so that the W^UK product runs as one bf16 GEMM over
        // K = 2D (q^C hi | lo against W^UK twice): the fp32 q^C of the
        // quantised modes, to about 16 bits, as the decode kernels' hi + lo
        // split keeps it.
        g6.qc_f32 = 0;
        g6.qc_split = 1;
        launch(L6, k_gemm<EPI_UQQR, G_TM_HALF, 3, 0, A_I8>, dim3(nt6, mt2, 1), dim3(256), 0, g6);
        g8.K = 2 * a->D;
        g8.KB = a->D;
      } else {
        launch(L6, k_gemm<EPI_UQQR, G_TM_HALF, 3>, dim3(nt6, mt2, 1), dim3(256), 0, g6);
      }
      mark(MLA_PHASE_AFTER_UQQR);
      const unsigned nt8 = static_cast<unsigned>((g8.N0 + G_TN - 1) / G_TN);
      launch(L8, k_gemm<EPI_UK, 128, 3>,
             dim3(nt8, static_cast<unsigned>((T + 127) / 128), static_cast<unsigned>(nh)),
             dim3(256), 0, g8);
    }
  }
  if (q8out && !qh) {
    const int64_t rows = T * a->N;
    launch(L0, k_quant_query, dim3(static_cast<unsigned>((rows + 3) / 4)), dim3(256), 0,
           static_cast<const float*>(g8.q_f32), static_cast<int8_t*>(a->query),
           a->dequant_scale_q_nope, rows, static_cast<int>(a->Hckv));
  }
  mark(MLA_PHASE_AFTER_UK);
  return hipGetLastError() == hipSuccess ? QKVNR_OK : QKVNR_ERR_LAUNCH_FAILED;
}

}  // namespace qkvnr
