// The no-allocation variant of mla_prolog_v2: the workspace is a fixed
// device array of this library instead of caller memory.
//
// `scratch` below is a file-scope __device__ array: every GPU the library
// runs on holds its own copy at its own address until the process ends.  In
// host code its name is only a stand-in, so the device address is looked up
// once per device with hipGetSymbolAddress (that device current) and kept;
// only that address is ever passed to kernels.  The prolog's kernels need no
// part of the workspace cleared (it is fully written before it is read
// within one call), and calls that overlap on one GPU share the array and
// race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.h"

namespace qkvnr {

static __device__ __align__(256) unsigned char scratch[MLA_NO_ALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch`, per device

// The device address of `scratch` on device `dev` (looked up on the first
// call for that device, with it current).  nullptr on a HIP error.
void* scratch_on(int dev) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[dev] != nullptr) return g_scratch[dev];
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return nullptr;
  if (cur != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
  void* p = nullptr;
  const hipError_t rc = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (cur != dev) (void)hipSetDevice(cur);
  if (rc != hipSuccess) return nullptr;
  g_scratch[dev] = p;
  return p;
}

}  // namespace

int launch_mla_prolog_v2_no_alloc(const MlaPrologV2Args* a, const MlaPlan& plan, void* stream) {
  int dev = -1;
  const hipError_t rc = stream != nullptr
                            ? hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev)
                            : hipGetDevice(&dev);
  if (rc != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return QKVNR_ERR_LAUNCH_FAILED;
  }
  void* ws = scratch_on(dev);
  if (ws == nullptr) {
    (void)hipGetLastError();
    return QKVNR_ERR_LAUNCH_FAILED;
  }
  return launch_mla_prolog_v2(a, plan, ws, stream);
}

}  // namespace qkvnr
