// HIP runtime helpers behind the C ABI that are not kernels of the hot path:
// the stream-ordered host copy used by the debug input checks.
#include <hip/hip_runtime.h>

#include "launch.h"

namespace qkvnr {

int copy_to_host_sync(void* host_dst, const void* dev_src, size_t bytes, void* stream) {
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (hipMemcpyAsync(host_dst, dev_src, bytes, hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess) {
    (void)hipGetLastError();
    return QKVNR_ERR_LAUNCH_FAILED;
  }
  return QKVNR_OK;
}


// ---------------------------------------------------------------------------
// Measurement probes: the achievable HBM read rate and dense bf16 MFMA rate
// of the GPU they run on, the reference points the benchmark reports beside
// the published peaks.  Neither is part of either operator.
// ---------------------------------------------------------------------------
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 probe_bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float probe_f32x16_t;

// Streams n16 16-byte chunks once (grid-stride, nontemporal) and folds them
// into a per-thread value that is stored only if it equals `never`, so the
// loads cannot be dropped and nothing is written in practice.
typedef __attribute__((ext_vector_type(4))) unsigned int probe_u32x4_t;

__device__ __forceinline__ uint32_t fold(probe_u32x4_t v) { return v.x ^ v.y ^ v.z ^ v.w; }

__global__ __launch_bounds__(256) void k_probe_read(const probe_u32x4_t* __restrict__ src,
                                                    int64_t n16, uint32_t never,
                                                    uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
  int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const probe_u32x4_t a = __builtin_nontemporal_load(src + i);
    const probe_u32x4_t b = __builtin_nontemporal_load(src + i + stride);
    const probe_u32x4_t c = __builtin_nontemporal_load(src + i + 2 * stride);
    const probe_u32x4_t d = __builtin_nontemporal_load(src + i + 3 * stride);
    acc ^= fold(a) ^ fold(b) ^ fold(c) ^ fold(d);
  }
  for (; i < n16; i += stride) acc ^= fold(__builtin_nontemporal_load(src + i));
  if (acc == never) sink[0] = acc;
}

// Four independent 32x32x16 bf16 MFMA chains per wave, `iters` steps each:
// 4 * iters * 32768 flop per wave, no memory traffic in the loop.
__global__ __launch_bounds__(256) void k_probe_mfma(int64_t iters, float never,
                                                    float* __restrict__ sink) {
  const uint32_t l = threadIdx.x;
  probe_bf16x8_t a, b;
  for (int e = 0; e < 8; ++e) {
    a[e] = static_cast<__bf16>(static_cast<float>((l + e) & 7) * 0.125f);
    b[e] = static_cast<__bf16>(static_cast<float>((l * 3 + e) & 7) * 0.0625f);
  }
  probe_f32x16_t c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int64_t i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, b, c3, 0, 0, 0);
  }
  float s = 0.f;
  for (int e = 0; e < 16; ++e) s += c0[e] + c1[e] + c2[e] + c3[e];
  if (s == never) sink[0] = s;
}

}  // namespace

int probe_read(const void* src, size_t bytes, void* sink, void* stream) {
  const int64_t n16 = static_cast<int64_t>(bytes / 16);
  hipLaunchKernelGGL(k_probe_read, dim3(4096), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const probe_u32x4_t*>(src), n16, 0x9e3779b9u,
                     static_cast<uint32_t*>(sink));
  return hipGetLastError() == hipSuccess ? QKVNR_OK : QKVNR_ERR_LAUNCH_FAILED;
}

int probe_mfma(int64_t iters, void* sink, void* stream) {
  // two workgroups of four waves per CU on 256 CUs: two waves per SIMD
  hipLaunchKernelGGL(k_probe_mfma, dim3(512), dim3(256), 0, static_cast<hipStream_t>(stream),
                     iters, -1.0f, static_cast<float*>(sink));
  return hipGetLastError() == hipSuccess ? QKVNR_OK : QKVNR_ERR_LAUNCH_FAILED;
}

}  // namespace qkvnr
