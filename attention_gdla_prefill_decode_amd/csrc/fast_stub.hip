// Placeholder until the MFMA kernels land: every size is served by the generic kernels.
#include "fast_paths.h"

namespace gdla {
int32_t fast_decode_splits(int32_t, int32_t) { return 1; }
bool fast_decode_supported(const LayerDims &, gdla_dtype) { return false; }
gdla_status run_fast_decode(const LayerDims &, const gdla_weights *, int32_t, const int32_t *, const int32_t *,
                            void *, int32_t, const float *, const float *, float *, const FastDecodeLayout &,
                            void *, hipStream_t, StageEvents &) {
  return GDLA_ERR_UNSUPPORTED;
}
}  // namespace gdla
