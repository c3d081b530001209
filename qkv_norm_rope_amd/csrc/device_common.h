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

// fp32 -> bf16 with the hardware conversion (v_cvt_pk_bf16_f32: round to
// nearest even, NaN stays NaN).
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Two packed bf16 in a 32-bit word: low half is the lower address.
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
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

// Global-memory accessors.  Pointers reach the kernels inside by-value
// argument structs, where the compiler cannot always prove they address
// global memory; it then emits flat instructions, which count against the
// LDS counter too and force full waits that serialise the load pipeline.
// Casting to address space 1 makes every access a global_load / store.
#define QKVNR_GLOBAL __attribute__((address_space(1)))
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 ld16(const void* p) {
  const u32x4_t v = *(const QKVNR_GLOBAL u32x4_t*)p;
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st16(void* p, uint4 v) {
  const u32x4_t w = {v.x, v.y, v.z, v.w};
  *(QKVNR_GLOBAL u32x4_t*)p = w;
}
// Streaming stores for outputs that no later kernel of the call reads:
// nontemporal, so they do not displace reused lines from the caches.
__device__ __forceinline__ void st16_nt(void* p, uint4 v) {
  const u32x4_t w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, (QKVNR_GLOBAL u32x4_t*)p);
}
__device__ __forceinline__ void st8_nt(void* p, uint2 v) {
  const u32x2_t w = {v.x, v.y};
  __builtin_nontemporal_store(w, (QKVNR_GLOBAL u32x2_t*)p);
}
__device__ __forceinline__ void st8(void* p, uint2 v) {
  const u32x2_t w = {v.x, v.y};
  *(QKVNR_GLOBAL u32x2_t*)p = w;
}
template <class T>
__device__ __forceinline__ T gld(const T* p) {
  return *(const QKVNR_GLOBAL T*)p;
}
template <class T>
__device__ __forceinline__ void gst(T* p, T v) {
  *(QKVNR_GLOBAL T*)p = v;
}
// 8 fp32 values from / to 32 bytes of global memory.
__device__ __forceinline__ void ld8f(const float* p, float* f) {
  const uint4 a = ld16(p), b = ld16(p + 4);
  f[0] = __uint_as_float(a.x); f[1] = __uint_as_float(a.y);
  f[2] = __uint_as_float(a.z); f[3] = __uint_as_float(a.w);
  f[4] = __uint_as_float(b.x); f[5] = __uint_as_float(b.y);
  f[6] = __uint_as_float(b.z); f[7] = __uint_as_float(b.w);
}
__device__ __forceinline__ void st8f(float* p, const float* f) {
  st16(p, make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                     __float_as_uint(f[3])));
  st16(p + 4, make_uint4(__float_as_uint(f[4]), __float_as_uint(f[5]), __float_as_uint(f[6]),
                         __float_as_uint(f[7])));
}

// Workgroup barrier ordering LDS accesses only: waits for this wave's LDS
// (and scalar) operations, then s_barrier.  Unlike __syncthreads it does not
// drain the wave's global loads in flight.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// ---- buffer loads -------------------------------------------------------------
// A raw buffer resource over [base, base + bytes): loads through it take a
// per-lane VGPR offset plus a wave-uniform SGPR offset, so a stream's
// per-step address is one scalar add, and a load whose offset falls outside
// the range returns zeros instead of touching memory.  base must be
// wave-uniform.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;  // raw 32-bit data format (gfx9 family)

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), kRsrcWord3);
}
__device__ __forceinline__ uint4 bld16(rsrc_t r, uint32_t voff, uint32_t soff) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(voff),
                                                          static_cast<int>(soff), 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}
// Streaming variant (nontemporal: cache policy bit 1) for data read once.
__device__ __forceinline__ uint4 bld16_nt(rsrc_t r, uint32_t voff, uint32_t soff) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(voff),
                                                          static_cast<int>(soff), 2);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Device-scope accesses (cache policy bit 4, sc1) for data handed from one
// workgroup to another within a launch: the store writes through to the
// level shared by every XCD before it counts as complete, and the load is
// served from that level, never from a stale copy in this XCD's L2.
constexpr int kDeviceScope = 16;
__device__ __forceinline__ uint4 bld16_dev(rsrc_t r, uint32_t voff, uint32_t soff) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(voff),
                                                          static_cast<int>(soff), kDeviceScope);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void bst8_dev(rsrc_t r, uint32_t voff, uint2 v) {
  const u32x2_t w = {v.x, v.y};
  __builtin_amdgcn_raw_buffer_store_b64(w, r, static_cast<int>(voff), 0, kDeviceScope);
}
__device__ __forceinline__ void bst16_dev(rsrc_t r, uint32_t voff, uint4 v) {
  const u32x4_t w = {v.x, v.y, v.z, v.w};
  __builtin_amdgcn_raw_buffer_store_b128(w, r, static_cast<int>(voff), 0, kDeviceScope);
}

}  // namespace qkvnr
