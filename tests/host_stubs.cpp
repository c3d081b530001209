// Launcher stand-ins for the host-only build of the C ABI layer (host.cpp)
// that the sanitizer test links: no HIP, every launch reports a failure.
// The CPU boundary tests never get past validation, so none is reached.
#include "launch.h"

namespace qkvnr {

int launch_qkv_rmsnorm_rope_cache(const QkvRmsNormRopeCacheArgs*, void*) {
  return QKVNR_ERR_LAUNCH_FAILED;
}

int launch_pack_weight(const void*, void*, int64_t, int64_t, int64_t, int, int64_t, int64_t,
                       void*, bool) {
  return QKVNR_ERR_LAUNCH_FAILED;
}

int launch_mla_prolog_v2(const MlaPrologV2Args*, const MlaPlan&, void*, void*,
                         const PreprocessExtra*) {
  return QKVNR_ERR_LAUNCH_FAILED;
}

int launch_mla_prolog_v2_no_alloc(const MlaPrologV2Args*, const MlaPlan&, void*) {
  return QKVNR_ERR_LAUNCH_FAILED;
}

int copy_to_host_sync(void*, const void*, size_t, void*) { return QKVNR_ERR_LAUNCH_FAILED; }

int probe_read(const void*, size_t, void*, void*) { return QKVNR_ERR_LAUNCH_FAILED; }

int probe_mfma(int64_t, void*, void*) { return QKVNR_ERR_LAUNCH_FAILED; }

}  // namespace qkvnr
