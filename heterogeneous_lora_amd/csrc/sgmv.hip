// SGMV: the prefill path (segment tiles on MFMA). Not built yet.
#include "device_common.h"

namespace slora {

hipError_t launch_sgmv_shrink(const Geom&, const int32_t*, const SgTile*, int32_t n_tiles,
                              const void*, float*, hipStream_t) {
  return n_tiles > 0 ? hipErrorNotSupported : hipSuccess;
}

hipError_t launch_sgmv_expand(const Geom&, const int32_t*, const SgTile*, int32_t n_tiles,
                              const float*, void*, hipStream_t) {
  return n_tiles > 0 ? hipErrorNotSupported : hipSuccess;
}

}  // namespace slora
