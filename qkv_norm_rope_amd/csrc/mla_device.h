// Device pieces shared by the MLA prolog kernels: MFMA operand kinds and
// the one-step MFMA helpers on 16-byte operands.
#pragma once

#include "device_common.h"

namespace qkvnr {

// A-operand kinds: bf16, int8, or fp32 split into bf16 hi + lo (two MFMAs).
enum AKind { A_BF16 = 0, A_I8 = 1, A_F32SPLIT = 2 };

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }
__device__ __forceinline__ i32x4_t as_i32x4(uint4 v) { return __builtin_bit_cast(i32x4_t, v); }

// Split 8 fp32 values into bf16 hi + bf16 lo (hi + lo carries ~16 bits).
__device__ __forceinline__ void split8(const float4 a, const float4 b, uint4& hi, uint4& lo) {
  const float f[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint32_t h[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint16_t h0 = f32_to_bf16(f[2 * i]), h1 = f32_to_bf16(f[2 * i + 1]);
    const float r0 = f[2 * i] - bf16_to_f32(h0), r1 = f[2 * i + 1] - bf16_to_f32(h1);
    h[i] = static_cast<uint32_t>(h0) | (static_cast<uint32_t>(h1) << 16);
    l[i] = pack_bf16x2(r0, r1);
  }
  hi = make_uint4(h[0], h[1], h[2], h[3]);
  lo = make_uint4(l[0], l[1], l[2], l[3]);
}

template <int AK>
struct AccT {
  typedef f32x16_t type;
};
template <>
struct AccT<A_I8> {
  typedef i32x16_t type;
};

// acc += A(16B/lane) x B(16B/lane) for one MFMA k-step.
template <int AK>
__device__ __forceinline__ void mfma_step(typename AccT<AK>::type& acc, uint4 a, uint4 b) {
  if constexpr (AK == A_I8) {
    acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(as_i32x4(a), as_i32x4(b), acc, 0, 0, 0);
  } else {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), acc, 0, 0, 0);
  }
}


}  // namespace qkvnr
