// Fused decode path of MlaPrologV2 ("MlaPrologV2" README: formulas;
// non-quantised scenario) for T <= 32 tokens: one persistent kernel with one
// workgroup per CU runs the four steps as phases separated by grid
// barriers, and keeps HBM busy across the barriers by issuing each phase's
// weight loads before waiting for the previous phase's results.
//
//   phase A  h, g = x . [W^DQ | W^DKV_KR]        split-K partials (fp32)
//   phase B  c^Q = RmsNorm(h); c^KV = RmsNorm(g_kv) -> kv_cache;
//            k^R = RoPE(g_r) -> kr_cache          one workgroup per token;
//            every workgroup first issues loads for its phase-C weights
//   phase C  y = c^Q . [W^UQ | W^QR]; q^C -> fragment layout, q^R (pre-RoPE)
//            -> workspace; phase-D weights are requested before the barrier
//   phase D  q^N = q^C . W^UK per head -> query; RoPE(q^R) -> query_rope
//
// A small prologue kernel packs x into the MFMA fragment layout and zeroes
// the barrier counter.  The barrier spins with s_sleep on an agent-scope
// counter and gives up after a bounded time (setting a flag in the
// workspace), so a workgroup that never arrives cannot hang the GPU.
#include "device_common.h"
#include "launch.h"
#include "mla_device.h"

namespace qkvnr {

namespace {

constexpr int FT = 256;       // threads per workgroup: one wave per SIMD,
constexpr int FW = FT / 64;   // so each wave may hold 512 registers
constexpr int NB1 = 2;        // column blocks per wave, phase A
constexpr int NB6 = 3;        // column blocks per wave, phase C
constexpr int NB8 = 2;        // column blocks per wave, phase D
constexpr int PB1 = 4;        // k-steps per register batch, phase A
constexpr int PB6 = 6;        // phase C (two batches are prefetched in phase B)
constexpr int PB8 = 4;        // phase D (both batches prefetched in phase C)
constexpr int FIN_COLS = 9;   // finish: columns per thread per pass
constexpr int LDS_WORDS = FW * 32 * (NB6 * 32 + 4);  // 51200 bytes
// ~0.25 s of the 100 MHz constant clock
constexpr uint64_t kBarrierTimeout = 25000000ull;

struct FusedParams {
  int T, He, Hcq, N, D, Hckv, Dr;
  int64_t slots;
  float eps_cq, eps_ckv;
  const uint4* xfrag;  // x in fragment layout (one 32-row block)
  const uint4* wdq;
  const uint4* wdkvkr;
  const uint4* wuqqr;
  const uint4* wuk;
  const uint16_t* gamma_cq;
  const uint16_t* gamma_ckv;
  const uint16_t* cosb;
  const uint16_t* sinb;
  const int64_t* index;
  uint16_t* kv_cache;
  uint16_t* kr_cache;
  uint16_t* query;
  uint16_t* query_rope;
  float* part;        // [ks1][T][Hcq + Hckv + Dr]
  uint16_t* cqfrag;   // c^Q, fragment layout
  uint16_t* qcfrag;   // q^C, per-head fragment layout
  float* yrope;       // [T][N*Dr] pre-RoPE q^R
  unsigned* bar;      // [0] barrier arrivals, [1] timeout flag,
                      // [2..17] workgroup-0 phase timestamps (8 x u64)
  int ks1;            // phase-A K splits
  int steps1;         // phase-A k-steps per split
};

__device__ __forceinline__ void grid_barrier(unsigned* bar, unsigned nblocks) {
  __syncthreads();
  if (threadIdx.x == 0) {
    __threadfence();
    const unsigned old = __hip_atomic_fetch_add(bar, 1u, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
    const unsigned target = (old / nblocks + 1u) * nblocks;
    const uint64_t t0 = wall_clock64();
    while (__hip_atomic_load(bar, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
      __builtin_amdgcn_s_sleep(1);
      if (static_cast<uint64_t>(wall_clock64()) - t0 > kBarrierTimeout) {
        __hip_atomic_fetch_or(bar + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
    __threadfence();
  }
  __syncthreads();
}

// Register batches of PB k-steps: B chunks of NB column blocks and the A
// chunk (one 32-row block).
template <int NB, int PB>
struct Batch {
  uint4 b[PB][NB];
  uint4 a[PB];
};

template <int NB, int PB>
__device__ __forceinline__ void load_b(Batch<NB, PB>& x, const uint4* const* bptr, int64_t s0,
                                       int64_t s_last) {
#pragma unroll
  for (int u = 0; u < PB; ++u) {
    const int64_t s = (s0 + u) < s_last ? (s0 + u) : s_last;
#pragma unroll
    for (int b = 0; b < NB; ++b) x.b[u][b] = ld16(bptr[b] + s * 64);
  }
}
template <int NB, int PB>
__device__ __forceinline__ void load_a(Batch<NB, PB>& x, const uint4* aptr, int64_t s0,
                                       int64_t s_last) {
#pragma unroll
  for (int u = 0; u < PB; ++u) {
    const int64_t s = (s0 + u) < s_last ? (s0 + u) : s_last;
    x.a[u] = ld16(aptr + s * 64);
  }
}
template <int NB, int PB>
__device__ __forceinline__ void compute(f32x16_t* acc, const Batch<NB, PB>& x, int64_t count) {
#pragma unroll
  for (int u = 0; u < PB; ++u) {
    if (u >= count) break;  // wave-uniform; only MFMAs are skipped
#pragma unroll
    for (int b = 0; b < NB; ++b) mfma_step<A_BF16>(acc[b], x.a[u], x.b[u][b]);
  }
}

// Stream k-steps [lo, hi) of NB column blocks.  X and Y hold the first two
// batches' B chunks already (issued by the caller, possibly long before);
// their A chunks are loaded here.  Loads are unconditional (clamped) so the
// compiler waits only for the batch being consumed.
template <int NB, int PB>
__device__ __forceinline__ void stream(f32x16_t* acc, Batch<NB, PB>& X, Batch<NB, PB>& Y,
                                       const uint4* const* bptr, const uint4* aptr, int64_t lo,
                                       int64_t hi) {
  if (lo >= hi) return;
  const int64_t last = hi - 1;
  int64_t s = lo;
  load_a(X, aptr, s, last);
  load_a(Y, aptr, s + PB, last);
  for (;;) {
    compute(acc, X, hi - s);
    s += PB;
    if (s >= hi) break;
    load_b(X, bptr, s + PB < hi ? s + PB : s, last);
    load_a(X, aptr, s + PB < hi ? s + PB : s, last);
    compute(acc, Y, hi - s);
    s += PB;
    if (s >= hi) break;
    load_b(Y, bptr, s + PB < hi ? s + PB : s, last);
    load_a(Y, aptr, s + PB < hi ? s + PB : s, last);
  }
}

// Stage a wave's NB 32x32 accumulators into its LDS slot: lane l / register
// r holds row 8*(r/4) + 4*(l/32) + r%4, column l%32.
template <int NB, int PITCH>
__device__ __forceinline__ void stage(float* slot, const f32x16_t* acc, int lane) {
  const int g = lane >> 5, li = lane & 31;
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      slot[(8 * (r >> 2) + 4 * g + (r & 3)) * PITCH + b * 32 + li] = acc[b][r];
}

__device__ __forceinline__ float block_sum_f(float v, float* red) {
  v = group_sum<64>(v);
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int w = 0; w < FW; ++w) t += red[w];
  return t;
}

// Workgroup 0 records the 100 MHz constant clock at each phase boundary
// (start, after A, after barrier 1, after B, after barrier 2, after C, after
// barrier 3, end) into workspace words [2, 18) for profiling.
__device__ __forceinline__ void stamp(unsigned* bar, int i) {
  if (blockIdx.x == 0 && threadIdx.x == 0)
    gst(reinterpret_cast<uint64_t*>(bar + 2) + i, static_cast<uint64_t>(wall_clock64()));
}

__global__ __launch_bounds__(FT, 1) void k_mla_decode_fused(FusedParams p) {
  __shared__ float lds[LDS_WORDS];
  __shared__ float red[FW];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const unsigned G = gridDim.x;
  const int ntot = p.Hcq + p.Hckv + p.Dr;
  stamp(p.bar, 0);

  // ------------------------------- phase A --------------------------------
  {
    const int64_t KC = p.He / 8;
    const int64_t S1 = p.He / 16;
    const int nbq = p.Hcq / 32, nbk = (p.Hckv + p.Dr + 31) / 32;
    const int ntq = (nbq + NB1 - 1) / NB1, ntk = (nbk + NB1 - 1) / NB1;
    const int items = (ntq + ntk) * p.ks1;
    constexpr int PITCH = NB1 * 32 + 4;
    for (int item = blockIdx.x; item < items; item += G) {
      const int tile = item % (ntq + ntk);
      const int sp = item / (ntq + ntk);
      const uint4* B;
      int nblk, blk0, ncols, colbase;
      if (tile < ntq) {
        B = p.wdq; nblk = nbq; blk0 = tile * NB1; ncols = p.Hcq; colbase = 0;
      } else {
        B = p.wdkvkr; nblk = nbk; blk0 = (tile - ntq) * NB1; ncols = p.Hckv + p.Dr;
        colbase = p.Hcq;
      }
      const uint4* bptr[NB1];
#pragma unroll
      for (int b = 0; b < NB1; ++b) {
        const int blk = blk0 + b < nblk ? blk0 + b : nblk - 1;
        bptr[b] = B + static_cast<int64_t>(blk) * KC * 32 + lane;
      }
      const int64_t s_lo = static_cast<int64_t>(sp) * p.steps1;
      const int64_t s_hi = min(s_lo + p.steps1, S1);
      const int64_t cnt = s_hi - s_lo;
      const int64_t lo = s_lo + cnt * wave / FW, hi = s_lo + cnt * (wave + 1) / FW;
      f32x16_t acc[NB1];
#pragma unroll
      for (int b = 0; b < NB1; ++b) acc[b] = f32x16_t{};
      if (lo < hi) {
        Batch<NB1, PB1> X, Y;
        load_b(X, bptr, lo, hi - 1);
        load_b(Y, bptr, lo + PB1, hi - 1);
        stream(acc, X, Y, bptr, p.xfrag + lane, lo, hi);
      }
      stage<NB1, PITCH>(lds + wave * 32 * PITCH, acc, lane);
      __syncthreads();
      // 32 rows x (NB1*32/8) column groups, summed over waves in order
      for (int it = tid; it < 32 * NB1 * 4; it += FT) {
        const int row = it / (NB1 * 4);
        const int c0 = (it % (NB1 * 4)) * 8;
        const int col = blk0 * 32 + c0;
        if (row >= p.T || col >= ncols) continue;
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float a = 0.f;
#pragma unroll
          for (int w = 0; w < FW; ++w) a += lds[(w * 32 + row) * PITCH + c0 + e];
          v[e] = a;
        }
        st8f(p.part + (static_cast<int64_t>(sp) * p.T + row) * ntot + colbase + col, v);
      }
      __syncthreads();
    }
  }
  stamp(p.bar, 1);
  grid_barrier(p.bar, G);
  stamp(p.bar, 2);

  // ------------------------------- phase B --------------------------------
  // This workgroup's phase-C work: passes of NB6 column blocks, K split over
  // the waves.  The first two batches of the first pass are requested now.
  const int64_t NDR = static_cast<int64_t>(p.N) * (p.D + p.Dr);
  const int nb6 = static_cast<int>((NDR + 31) / 32);
  const int64_t KC6 = p.Hcq / 8;
  const int64_t S6 = p.Hcq / 16;
  const int64_t lo6 = S6 * wave / FW, hi6 = S6 * (wave + 1) / FW;
  auto bptr6 = [&](int pass, const uint4** bp) {
    const int blk0 = (pass * static_cast<int>(G) + static_cast<int>(blockIdx.x)) * NB6;
#pragma unroll
    for (int b = 0; b < NB6; ++b) {
      const int blk = blk0 + b < nb6 ? blk0 + b : nb6 - 1;
      bp[b] = p.wuqqr + static_cast<int64_t>(blk) * KC6 * 32 + lane;
    }
  };
  Batch<NB6, PB6> X6, Y6;
  const uint4* bp6[NB6];
  bptr6(0, bp6);
  auto prefetch6 = [&]() {
    if (lo6 < hi6) {
      load_b(X6, bp6, lo6, hi6 - 1);
      load_b(Y6, bp6, lo6 + PB6, hi6 - 1);
    }
  };
  const bool finisher = static_cast<int>(blockIdx.x) < p.T;
  if (!finisher) prefetch6();
  if (finisher) {
    const int t = blockIdx.x;
    float* row = lds;  // ntot floats
    // split-K partial sums, in split order; a thread's FIN_COLS columns x 8
    // splits are all in flight together (clamped, unconditional loads)
    for (int c0 = 0; c0 < ntot; c0 += FIN_COLS * FT) {
      float v[FIN_COLS][8];
#pragma unroll
      for (int i = 0; i < FIN_COLS; ++i) {
        int c = c0 + tid + i * FT;
        c = c < ntot ? c : ntot - 1;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const int se = s < p.ks1 ? s : p.ks1 - 1;
          v[i][s] = gld(p.part + (static_cast<int64_t>(se) * p.T + t) * ntot + c);
        }
      }
#pragma unroll
      for (int i = 0; i < FIN_COLS; ++i) {
        const int c = c0 + tid + i * FT;
        float a = 0.f;
#pragma unroll
        for (int s = 0; s < 8; ++s) a += s < p.ks1 ? v[i][s] : 0.f;
        if (c < ntot) row[c] = a;
      }
    }
    __syncthreads();
    float sq = 0.f, skv = 0.f;
    for (int c = tid; c < p.Hcq; c += FT) sq += row[c] * row[c];
    for (int c = tid; c < p.Hckv; c += FT) skv += row[p.Hcq + c] * row[p.Hcq + c];
    sq = block_sum_f(sq, red);
    skv = block_sum_f(skv, red);
    const float rq = 1.0f / __builtin_sqrtf(sq / static_cast<float>(p.Hcq) + p.eps_cq);
    const float rkv = 1.0f / __builtin_sqrtf(skv / static_cast<float>(p.Hckv) + p.eps_ckv);
    // c^Q in fragment layout: ((c/16)*64 + ((c%16)/8)*32 + t)*8 + c%8
    for (int c = tid; c < p.Hcq; c += FT) {
      const int64_t off = ((c / 16) * 64 + ((c % 16) / 8) * 32 + t) * 8 + c % 8;
      gst(p.cqfrag + off, f32_to_bf16(row[c] * rq * bf16_to_f32(gld(p.gamma_cq + c))));
    }
    const int64_t slot = gld(p.index + t);
    if (slot >= 0 && slot < p.slots) {
      for (int c = tid; c < p.Hckv; c += FT)
        gst(p.kv_cache + slot * p.Hckv + c,
            f32_to_bf16(row[p.Hcq + c] * rkv * bf16_to_f32(gld(p.gamma_ckv + c))));
      const int half = p.Dr >> 1;
      const float* kr = row + p.Hcq + p.Hckv;
      for (int i = tid; i < p.Dr; i += FT) {
        const float cs = bf16_to_f32(gld(p.cosb + static_cast<int64_t>(t) * p.Dr + i));
        const float sn = bf16_to_f32(gld(p.sinb + static_cast<int64_t>(t) * p.Dr + i));
        const float o = i < half ? kr[i] * cs - kr[i + half] * sn : kr[i] * cs + kr[i - half] * sn;
        gst(p.kr_cache + slot * p.Dr + i, f32_to_bf16(o));
      }
    }
    prefetch6();
  }
  stamp(p.bar, 3);
  grid_barrier(p.bar, G);
  stamp(p.bar, 4);

  // ------------------------------- phase C --------------------------------
  // A8 work of this workgroup: NB8 column blocks of one head per wave.
  const int nb8 = (p.Hckv + 31) / 32;
  const int grp8 = (nb8 + FW * NB8 - 1) / (FW * NB8);  // workgroup items per head
  const int items8 = p.N * grp8;
  const int64_t KC8 = p.D / 8;
  const int64_t S8 = p.D / 16;
  auto bptr8 = [&](int item, const uint4** bp) {
    const int head = item / grp8;
#pragma unroll
    for (int b = 0; b < NB8; ++b) {
      int blk = ((item % grp8) * FW + wave) * NB8 + b;
      blk = blk < nb8 ? blk : nb8 - 1;
      bp[b] = p.wuk + static_cast<int64_t>(head) * nb8 * KC8 * 32 +
              static_cast<int64_t>(blk) * KC8 * 32 + lane;
    }
  };
  Batch<NB8, PB8> X8, Y8;
  const uint4* bp8[NB8];
  bool pre8 = false;
  // phase-D weights of this workgroup's first item, requested before the
  // last phase-C epilogue and the barrier (or right after the phase-C loop
  // when this workgroup has no phase-C block)
  auto prefetch8 = [&]() {
    if (!pre8 && static_cast<int>(blockIdx.x) < items8) {
      bptr8(blockIdx.x, bp8);
      load_b(X8, bp8, 0, S8 - 1);
      load_b(Y8, bp8, PB8, S8 - 1);
      pre8 = true;
    }
  };
  {
    constexpr int PITCH = NB6 * 32 + 4;
    for (int pass = 0;; ++pass) {
      const int blk0 = (pass * static_cast<int>(G) + static_cast<int>(blockIdx.x)) * NB6;
      if (blk0 >= nb6) break;
      if (pass > 0) {
        bptr6(pass, bp6);
        prefetch6();
      }
      f32x16_t acc[NB6];
#pragma unroll
      for (int b = 0; b < NB6; ++b) acc[b] = f32x16_t{};
      stream(acc, X6, Y6, bp6, reinterpret_cast<const uint4*>(p.cqfrag) + lane, lo6, hi6);
      const bool last_pass = (blk0 + static_cast<int>(G) * NB6) >= nb6;
      if (last_pass) prefetch8();
      stage<NB6, PITCH>(lds + wave * 32 * PITCH, acc, lane);
      __syncthreads();
      for (int it = tid; it < 32 * NB6 * 4; it += FT) {
        const int row = it / (NB6 * 4);
        const int c0 = (it % (NB6 * 4)) * 8;
        const int64_t col = static_cast<int64_t>(blk0) * 32 + c0;
        if (row >= p.T || col >= NDR) continue;
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float a = 0.f;
#pragma unroll
          for (int w = 0; w < FW; ++w) a += lds[(w * 32 + row) * PITCH + c0 + e];
          v[e] = a;
        }
        const int64_t ND = static_cast<int64_t>(p.N) * p.D;
        if (col < ND) {
          const int64_t head = col / p.D, d = col % p.D;
          const int64_t off =
              ((head * (p.D / 16) + d / 16) * 64 + ((d % 16) / 8) * 32 + row) * 8;
          st16(p.qcfrag + off, make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                          pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])));
        } else {
          st8f(p.yrope + static_cast<int64_t>(row) * p.N * p.Dr + (col - ND), v);
        }
      }
      __syncthreads();
    }
    prefetch8();
  }
  stamp(p.bar, 5);
  grid_barrier(p.bar, G);
  stamp(p.bar, 6);

  // ------------------------------- phase D --------------------------------
  {
    constexpr int PITCH = NB8 * 32 + 4;
    for (int pass = 0;; ++pass) {
      const int item = pass * static_cast<int>(G) + static_cast<int>(blockIdx.x);
      if (item >= items8) break;
      const int head = item / grp8;
      const int blk0 = ((item % grp8) * FW + wave) * NB8;
      if (pass > 0 || !pre8) {
        bptr8(item, bp8);
        load_b(X8, bp8, 0, S8 - 1);
        load_b(Y8, bp8, PB8, S8 - 1);
      }
      f32x16_t acc[NB8];
#pragma unroll
      for (int b = 0; b < NB8; ++b) acc[b] = f32x16_t{};
      const uint4* aptr =
          reinterpret_cast<const uint4*>(p.qcfrag) + static_cast<int64_t>(head) * S8 * 64 + lane;
      stream(acc, X8, Y8, bp8, aptr, 0, S8);
      float* slot = lds + wave * 32 * PITCH;
      stage<NB8, PITCH>(slot, acc, lane);
      // this wave's own 32 x (NB8*32) tile: groups of 8 columns per row
      for (int it = lane; it < 32 * NB8 * 4; it += 64) {
        const int row = it / (NB8 * 4);
        const int c0 = (it % (NB8 * 4)) * 8;
        const int col = blk0 * 32 + c0;
        if (row >= p.T || col >= p.Hckv) continue;
        const float* v = slot + row * PITCH + c0;
        st16(p.query + (static_cast<int64_t>(row) * p.N + head) * p.Hckv + col,
             make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                        pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])));
      }
      __syncthreads();
    }
    // RoPE of q^R: 8 consecutive rotation pairs per thread.
    const int half = p.Dr >> 1;
    const int64_t groups = static_cast<int64_t>(p.T) * p.N * (half / 8);
    for (int64_t gi = static_cast<int64_t>(blockIdx.x) * FT + tid; gi < groups;
         gi += static_cast<int64_t>(G) * FT) {
      const int64_t t = gi / (static_cast<int64_t>(p.N) * (half / 8));
      const int64_t rem = gi % (static_cast<int64_t>(p.N) * (half / 8));
      const int64_t head = rem / (half / 8);
      const int i0 = static_cast<int>(rem % (half / 8)) * 8;
      float a[8], b[8];
      const float* y = p.yrope + t * p.N * p.Dr + head * p.Dr;
      ld8f(y + i0, a);
      ld8f(y + i0 + half, b);
      const uint4 c1 = ld16(p.cosb + t * p.Dr + i0), s1 = ld16(p.sinb + t * p.Dr + i0);
      const uint4 c2 = ld16(p.cosb + t * p.Dr + i0 + half), s2 = ld16(p.sinb + t * p.Dr + i0 + half);
      const uint32_t cw1[4] = {c1.x, c1.y, c1.z, c1.w}, sw1[4] = {s1.x, s1.y, s1.z, s1.w};
      const uint32_t cw2[4] = {c2.x, c2.y, c2.z, c2.w}, sw2[4] = {s2.x, s2.y, s2.z, s2.w};
      float o1[8], o2[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float ca = (e & 1) ? bf16hi(cw1[e >> 1]) : bf16lo(cw1[e >> 1]);
        const float sa = (e & 1) ? bf16hi(sw1[e >> 1]) : bf16lo(sw1[e >> 1]);
        const float cb = (e & 1) ? bf16hi(cw2[e >> 1]) : bf16lo(cw2[e >> 1]);
        const float sb = (e & 1) ? bf16hi(sw2[e >> 1]) : bf16lo(sw2[e >> 1]);
        o1[e] = a[e] * ca - b[e] * sa;  // first half: y*cos - partner*sin
        o2[e] = b[e] * cb + a[e] * sb;  // second half: y*cos + partner*sin
      }
      uint16_t* q = p.query_rope + (t * p.N + head) * p.Dr;
      st16(q + i0, make_uint4(pack_bf16x2(o1[0], o1[1]), pack_bf16x2(o1[2], o1[3]),
                              pack_bf16x2(o1[4], o1[5]), pack_bf16x2(o1[6], o1[7])));
      st16(q + i0 + half, make_uint4(pack_bf16x2(o2[0], o2[1]), pack_bf16x2(o2[2], o2[3]),
                                     pack_bf16x2(o2[4], o2[5]), pack_bf16x2(o2[6], o2[7])));
    }
  }
  stamp(p.bar, 7);
}

// Prologue: x rows into the fragment layout (rows past T are zero) and the
// barrier words cleared.  One thread per 16 bytes of x.
__global__ __launch_bounds__(256) void k_fused_prologue(const uint16_t* __restrict__ x,
                                                        uint4* __restrict__ xfrag, int64_t T,
                                                        int64_t He, unsigned* bar) {
  const int64_t steps = He / 16;
  const int64_t per_row = He / 8;
  const int64_t total = 32 * per_row;
  if (blockIdx.x == 0 && threadIdx.x < 18) gst(bar + threadIdx.x, 0u);
  for (int64_t c = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; c < total;
       c += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t m = c / per_row;
    const int64_t q = c % per_row;
    const int64_t chunk = (q / 2) * 64 + (q % 2) * 32 + m;
    (void)steps;
    st16(xfrag + chunk, m < T ? ld16(x + m * He + 8 * q) : make_uint4(0, 0, 0, 0));
  }
}

}  // namespace

bool mla_fused_supported(const MlaPrologV2Args* a) {
  const int64_t T = a->B * a->S;
  return T >= 1 && T <= 32 && a->quant_mode == MLA_QUANT_NONE &&
         a->Dr % 16 == 0 && (a->Hcq + a->Hckv + a->Dr) * 4 <= LDS_WORDS * 4;
}

void mla_fused_layout(const MlaPrologV2Args* a, int64_t ks1, FusedLayout* L) {
  const int64_t T = a->B * a->S;
  const int64_t ntot = a->Hcq + a->Hckv + a->Dr;
  auto al = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  size_t off = 0;
  L->off_bar = off;
  off += 256;
  L->off_part = off;
  off += al(static_cast<size_t>(ks1 * T * ntot) * 4);
  L->off_cq = off;
  off += al(static_cast<size_t>(32 * a->Hcq) * 2);
  L->off_qc = off;
  off += al(static_cast<size_t>(a->N * 32 * a->D) * 2);
  L->off_yrope = off;
  off += al(static_cast<size_t>(T * a->N * a->Dr) * 4);
  L->off_xfrag = off;
  off += al(static_cast<size_t>(32 * a->He) * 2);
  L->total = off;
}

int launch_mla_decode_fused(const MlaPrologV2Args* a, const MlaPlan& pl, void* workspace,
                            const void* wdq, const void* wdkvkr, const void* wuqqr,
                            const void* wuk, hipStream_t st) {
  auto mark = [&](int i) {
    if (i < a->n_phase_events && a->phase_events[i] != nullptr)
      (void)hipEventRecord(static_cast<hipEvent_t>(a->phase_events[i]), st);
  };
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    return QKVNR_ERR_LAUNCH_FAILED;
  char* ws = static_cast<char*>(workspace) + pl.off_fused;
  FusedLayout L;
  mla_fused_layout(a, pl.ksplit, &L);
  FusedParams p{};
  p.T = static_cast<int>(a->B * a->S);
  p.He = static_cast<int>(a->He);
  p.Hcq = static_cast<int>(a->Hcq);
  p.N = static_cast<int>(a->N);
  p.D = static_cast<int>(a->D);
  p.Hckv = static_cast<int>(a->Hckv);
  p.Dr = static_cast<int>(a->Dr);
  p.slots = a->block_num * a->block_size;
  p.eps_cq = static_cast<float>(a->rmsnorm_epsilon_cq);
  p.eps_ckv = static_cast<float>(a->rmsnorm_epsilon_ckv);
  p.xfrag = reinterpret_cast<const uint4*>(ws + L.off_xfrag);
  p.wdq = static_cast<const uint4*>(wdq);
  p.wdkvkr = static_cast<const uint4*>(wdkvkr);
  p.wuqqr = static_cast<const uint4*>(wuqqr);
  p.wuk = static_cast<const uint4*>(wuk);
  p.gamma_cq = static_cast<const uint16_t*>(a->rmsnorm_gamma_cq);
  p.gamma_ckv = static_cast<const uint16_t*>(a->rmsnorm_gamma_ckv);
  p.cosb = static_cast<const uint16_t*>(a->rope_cos);
  p.sinb = static_cast<const uint16_t*>(a->rope_sin);
  p.index = a->cache_index;
  p.kv_cache = static_cast<uint16_t*>(a->kv_cache);
  p.kr_cache = static_cast<uint16_t*>(a->kr_cache);
  p.query = static_cast<uint16_t*>(a->query);
  p.query_rope = static_cast<uint16_t*>(a->query_rope);
  p.part = reinterpret_cast<float*>(ws + L.off_part);
  p.cqfrag = reinterpret_cast<uint16_t*>(ws + L.off_cq);
  p.qcfrag = reinterpret_cast<uint16_t*>(ws + L.off_qc);
  p.yrope = reinterpret_cast<float*>(ws + L.off_yrope);
  p.bar = reinterpret_cast<unsigned*>(ws + L.off_bar);
  p.ks1 = pl.ksplit;
  p.steps1 = static_cast<int>(pl.steps_per_split);

  const int64_t chunks = 32 * (a->He / 8);
  mark(MLA_PHASE_START);
  hipLaunchKernelGGL(k_fused_prologue, dim3(static_cast<unsigned>((chunks + 255) / 256)),
                     dim3(256), 0, st, static_cast<const uint16_t*>(a->token_x),
                     reinterpret_cast<uint4*>(ws + L.off_xfrag), static_cast<int64_t>(p.T),
                     a->He, p.bar);
  mark(MLA_PHASE_AFTER_DOWN);
  mark(MLA_PHASE_AFTER_NORM);
  mark(MLA_PHASE_AFTER_UQQR);
  hipLaunchKernelGGL(k_mla_decode_fused, dim3(static_cast<unsigned>(cus)), dim3(FT), 0, st, p);
  mark(MLA_PHASE_AFTER_UK);
  return hipGetLastError() == hipSuccess ? QKVNR_OK : QKVNR_ERR_LAUNCH_FAILED;
}

}  // namespace qkvnr
