// Device helpers shared by the gfx950 kernels: vector types, 16-bit float
// conversions, int8 saturation and wavefront reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qkvnr {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) int i32x4_t;
typedef __attribute__((ext_vector_type(16))) int i32x16_t;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;

// ---- bf16 -----------------------------------------------------------------
// bf16 is the upper half of an fp32 bit pattern.
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Two packed bf16 in a 32-bit word: low half is the lower address.
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

// ---- fp16 -----------------------------------------------------------------
__device__ __forceinline__ float f16lo(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w & 0xffffu)));
}
__device__ __forceinline__ float f16hi(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w >> 16)));
}
// fp32 -> fp16 uses the hardware conversion (round to nearest even).
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  uint16_t a = __builtin_bit_cast(uint16_t, static_cast<_Float16>(lo));
  uint16_t b = __builtin_bit_cast(uint16_t, static_cast<_Float16>(hi));
  return static_cast<uint32_t>(a) | (static_cast<uint32_t>(b) << 16);
}

// Element-type traits for the 16-bit float inputs.
struct Bf16T {
  static __device__ __forceinline__ float lo(uint32_t w) { return bf16lo(w); }
  static __device__ __forceinline__ float hi(uint32_t w) { return bf16hi(w); }
  static __device__ __forceinline__ uint32_t pack(float a, float b) { return pack_bf16x2(a, b); }
};
struct F16T {
  static __device__ __forceinline__ float lo(uint32_t w) { return f16lo(w); }
  static __device__ __forceinline__ float hi(uint32_t w) { return f16hi(w); }
  static __device__ __forceinline__ uint32_t pack(float a, float b) { return pack_f16x2(a, b); }
};

// ---- int8 -------------------------------------------------------------------
// Round half to even, then saturate to [lo, hi].
__device__ __forceinline__ int sat_rne(float x, int lo, int hi) {
  float r = __builtin_rintf(x);
  r = fminf(fmaxf(r, static_cast<float>(lo)), static_cast<float>(hi));
  return static_cast<int>(r);
}
__device__ __forceinline__ uint32_t pack_i8x4(int a, int b, int c, int d) {
  return (static_cast<uint32_t>(a) & 0xffu) | ((static_cast<uint32_t>(b) & 0xffu) << 8) |
         ((static_cast<uint32_t>(c) & 0xffu) << 16) | ((static_cast<uint32_t>(d) & 0xffu) << 24);
}

// ---- reductions ----------------------------------------------------------------
// Butterfly sums over aligned groups of `W` lanes (W a power of two <= 64).
// Every lane of a group ends with the bitwise-identical total.
template <int W>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int m = 1; m < W; m <<= 1) v += __shfl_xor(v, m);
  return v;
}
template <int W>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int m = 1; m < W; m <<= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}

// 16-byte global load/store helpers.
__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void st16(void* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }

}  // namespace qkvnr
