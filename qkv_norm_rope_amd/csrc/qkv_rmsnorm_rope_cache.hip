// Fused qkv split / RmsNorm / half-and-half RoPE / int8 quant / paged
// scatter for gfx950 ("aclnnQkvRmsNormRopeCache": formulas (1) SplitVD,
// (2) RmsNorm, (3) RoPE half-and-half, (4) Quant; index rule from its other
// restrictions).
//
// One pass over HBM.  Each wavefront owns one token; its 64 lanes form four
// row slots of 16 lanes, and lane j of a slot holds the 8 consecutive
// elements [8j, 8j+8) of a 128-wide head row (one 16-byte load).  A row's
// sum of squares is a butterfly over its 16 lanes; the RoPE partner of
// element i (i +/- 64) sits in lane j ^ 8 of the same slot, fetched with one
// cross-lane exchange.  Rows are loaded four slots-iterations at a time so
// several 1 KB wave loads are in flight before any arithmetic.
#include "device_common.h"
#include "launch.h"

namespace qkvnr {

namespace {

constexpr int kD = 128;
constexpr int kChunk = 4;  // row iterations loaded before processing

struct QkvParams {
  const uint16_t* __restrict__ qkv;
  const uint16_t* __restrict__ gq;
  const uint16_t* __restrict__ gk;
  const uint16_t* __restrict__ cosb;
  const uint16_t* __restrict__ sinb;
  const int64_t* __restrict__ index;
  const float* __restrict__ ks;
  const float* __restrict__ vs;
  const float* __restrict__ ko;
  const float* __restrict__ vo;
  void* __restrict__ kc;
  void* __restrict__ vc;
  uint16_t* __restrict__ q_out;
  uint16_t* __restrict__ qbq;
  uint16_t* __restrict__ kbq;
  uint16_t* __restrict__ vbq;
  int64_t T;
  int Nq, Nk, Nv;
  int64_t slots;
  float eps;
};

template <class ET>
__device__ __forceinline__ void unpack8(uint4 w, float* f) {
  f[0] = ET::lo(w.x); f[1] = ET::hi(w.x);
  f[2] = ET::lo(w.y); f[3] = ET::hi(w.y);
  f[4] = ET::lo(w.z); f[5] = ET::hi(w.z);
  f[6] = ET::lo(w.w); f[7] = ET::hi(w.w);
}

template <class ET>
__device__ __forceinline__ uint4 pack8(const float* f) {
  return make_uint4(ET::pack(f[0], f[1]), ET::pack(f[2], f[3]), ET::pack(f[4], f[5]),
                    ET::pack(f[6], f[7]));
}


// v / scale (+ offset), round half to even, saturate to int8; 8 lanes' worth
// packed into 8 bytes.
template <int QM>
__device__ __forceinline__ uint2 quant8(const float* v, const float* __restrict__ sc,
                                        const float* __restrict__ off) {
  float s[8], o[8];
  ld8f(sc, s);
  if (QM == 2) ld8f(off, o);
  int c[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float q = v[i] / s[i];
    if (QM == 2) q += o[i];
    c[i] = sat_rne(q, -128, 127);
  }
  return make_uint2(pack_i8x4(c[0], c[1], c[2], c[3]), pack_i8x4(c[4], c[5], c[6], c[7]));
}

// QM: 0 = no quant (caches in the input type), 1 = symmetric, 2 = asymmetric.
template <class ET, int QM>
__global__ __launch_bounds__(256) void k_qkv_rmsnorm_rope_cache(QkvParams p) {
  const int lane = threadIdx.x & 63;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= p.T) return;  // whole wave leaves together
  const int rs = lane >> 4;  // row slot
  const int j = lane & 15;   // element slice [8j, 8j+8)
  const int jp = j ^ 8;      // RoPE partner slice
  const int H = p.Nq + p.Nk + p.Nv;
  const bool first_half = j < 8;

  float cs[8], sn[8], gq[8], gqp[8], gk[8], gkp[8];
  unpack8<ET>(ld16(p.cosb + t * kD + 8 * j), cs);
  unpack8<ET>(ld16(p.sinb + t * kD + 8 * j), sn);
  unpack8<ET>(ld16(p.gq + 8 * j), gq);
  unpack8<ET>(ld16(p.gq + 8 * jp), gqp);
  unpack8<ET>(ld16(p.gk + 8 * j), gk);
  unpack8<ET>(ld16(p.gk + 8 * jp), gkp);

  const int64_t slot = gld(p.index + t);
  const bool write_cache = slot >= 0 && slot < p.slots;

  const uint16_t* __restrict__ src = p.qkv + t * static_cast<int64_t>(H) * kD + 8 * j;

  for (int h0 = 0; h0 < H; h0 += 4 * kChunk) {
    uint4 raw[kChunk];
#pragma unroll
    for (int c = 0; c < kChunk; ++c) {
      const int h = h0 + 4 * c + rs;
      raw[c] = h < H ? ld16(src + static_cast<int64_t>(h) * kD) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int c = 0; c < kChunk; ++c) {
      const int h = h0 + 4 * c + rs;
      float x[8];
      unpack8<ET>(raw[c], x);
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) ss += x[i] * x[i];
      ss = group_sum<16>(ss);
      const float rinv = 1.0f / __builtin_sqrtf(ss * (1.0f / kD) + p.eps);
      // partner slice of the same row (all lanes take part in the exchange)
      uint4 pr;
      pr.x = __shfl_xor(raw[c].x, 8);
      pr.y = __shfl_xor(raw[c].y, 8);
      pr.z = __shfl_xor(raw[c].z, 8);
      pr.w = __shfl_xor(raw[c].w, 8);
      if (h >= H) continue;
      if (h < p.Nq + p.Nk) {
        const bool is_q = h < p.Nq;
        float xp[8], y[8];
        unpack8<ET>(pr, xp);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float g = is_q ? gq[i] : gk[i];
          const float gp = is_q ? gqp[i] : gkp[i];
          const float a = x[i] * rinv * g;
          const float b = xp[i] * rinv * gp;
          // cat(-y2, y1): first half takes -partner, second half +partner
          y[i] = first_half ? (a * cs[i] - b * sn[i]) : (a * cs[i] + b * sn[i]);
        }
        const uint4 packed = pack8<ET>(y);
        if (is_q) {
          const int64_t o = (t * p.Nq + h) * kD + 8 * j;
          st16_nt(p.q_out + o, packed);
          if (p.qbq) st16_nt(p.qbq + o, packed);
        } else {
          const int hk = h - p.Nq;
          if (p.kbq) st16_nt(p.kbq + (t * p.Nk + hk) * kD + 8 * j, packed);
          if (write_cache) {
            const int64_t o = (slot * p.Nk + hk) * kD + 8 * j;
            if (QM == 0) {
              st16_nt(static_cast<uint16_t*>(p.kc) + o, packed);
            } else {
              const uint2 q8 = quant8<QM>(y, p.ks + hk * kD + 8 * j, p.ko + hk * kD + 8 * j);
              st8_nt(static_cast<int8_t*>(p.kc) + o, q8);
            }
          }
        }
      } else {
        const int hv = h - p.Nq - p.Nk;
        if (p.vbq) st16_nt(p.vbq + (t * p.Nv + hv) * kD + 8 * j, raw[c]);
        if (write_cache) {
          const int64_t o = (slot * p.Nv + hv) * kD + 8 * j;
          if (QM == 0) {
            st16_nt(static_cast<uint16_t*>(p.vc) + o, raw[c]);
          } else {
            const uint2 q8 = quant8<QM>(x, p.vs + hv * kD + 8 * j, p.vo + hv * kD + 8 * j);
            st8_nt(static_cast<int8_t*>(p.vc) + o, q8);
          }
        }
      }
    }
  }
}

template <class ET, int QM>
void launch_t(const QkvParams& p, hipStream_t stream) {
  const unsigned blocks = static_cast<unsigned>((p.T + 3) / 4);
  hipLaunchKernelGGL((k_qkv_rmsnorm_rope_cache<ET, QM>), dim3(blocks), dim3(256), 0, stream, p);
}

}  // namespace

int launch_qkv_rmsnorm_rope_cache(const QkvRmsNormRopeCacheArgs* a, void* stream_v) {
  const hipStream_t stream = static_cast<hipStream_t>(stream_v);
  QkvParams p;
  p.qkv = static_cast<const uint16_t*>(a->qkv);
  p.gq = static_cast<const uint16_t*>(a->gamma_q);
  p.gk = static_cast<const uint16_t*>(a->gamma_k);
  p.cosb = static_cast<const uint16_t*>(a->cos);
  p.sinb = static_cast<const uint16_t*>(a->sin);
  p.index = a->index;
  p.ks = a->k_scale;
  p.vs = a->v_scale;
  p.ko = a->k_offset;
  p.vo = a->v_offset;
  p.kc = a->k_cache;
  p.vc = a->v_cache;
  p.q_out = static_cast<uint16_t*>(a->q_out);
  p.qbq = static_cast<uint16_t*>(a->q_before_quant);
  p.kbq = static_cast<uint16_t*>(a->k_before_quant);
  p.vbq = static_cast<uint16_t*>(a->v_before_quant);
  p.T = a->B * a->S;
  p.Nq = static_cast<int>(a->Nq);
  p.Nk = static_cast<int>(a->Nk);
  p.Nv = static_cast<int>(a->Nv);
  p.slots = a->block_num * a->block_size;
  p.eps = static_cast<float>(a->epsilon);
  if (p.T == 0) return QKVNR_OK;
  const bool bf = a->dtype == QKV_DTYPE_BF16;
  switch (a->quant_mode) {
    case QKV_QUANT_NONE:
      bf ? launch_t<Bf16T, 0>(p, stream) : launch_t<F16T, 0>(p, stream);
      break;
    case QKV_QUANT_SYMMETRIC:
      bf ? launch_t<Bf16T, 1>(p, stream) : launch_t<F16T, 1>(p, stream);
      break;
    default:
      bf ? launch_t<Bf16T, 2>(p, stream) : launch_t<F16T, 2>(p, stream);
      break;
  }
  return hipGetLastError() == hipSuccess ? QKVNR_OK : QKVNR_ERR_LAUNCH_FAILED;
}

}  // namespace qkvnr
