#include "hs_internal.h"
namespace hs {
hipError_t launch_prefill(const Dims &, const CacheView &, const uint16_t *, uint16_t *, float *,
                          float, bool, hipStream_t) {
  return hipErrorNotSupported;
}
}  // namespace hs
