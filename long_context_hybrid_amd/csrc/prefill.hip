// Prefill kernels (placeholder until the MFMA prefill path lands).
#include "hys_common.h"
#include "hys_internal.h"

namespace hys {

size_t prefill_full_ws_bytes(const Geom& g, int /*score_block*/) {
  return align_up((size_t)g.B * g.Hq * g.Tq * sizeof(float));
}
hipError_t launch_full_prefill(const Geom&, const void*, const void*, const void*, int, void*, float*, float*, void*,
                               hipStream_t) {
  return hipErrorNotSupported;
}
size_t sparse_block_ws_bytes(const Geom&, int, int) { return 0; }
hipError_t launch_sparse_block(const Geom&, const void*, const void*, const void*, const int32_t*, int, int, int,
                               const float*, void*, void*, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace hys
