// Stand-ins for the kernel launchers, for a host-only build of the ABI layer
// (flh_api.cpp) under AddressSanitizer and UndefinedBehaviorSanitizer.  The ABI
// tests only make calls that fail validation, so none of these runs; if one did,
// the call would report FLH_E_HIP.
#include "flh_internal.h"

namespace flh {
hipError_t launch_gemm(int, GemmKind, const GemmArgs &, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_spans(const uint8_t *, int64_t, int32_t, int32_t, int64_t, int32_t *, int32_t *, uint32_t *,
                        int32_t *, hipStream_t) {
  return hipErrorInvalidValue;
}
hipError_t launch_lists(int64_t, const uint32_t *, const int32_t *, const int32_t *, int64_t, int32_t *, int32_t *,
                        int32_t *, int64_t, hipStream_t, uint32_t *) {
  return hipErrorInvalidValue;
}
hipError_t launch_target_logit(int, int64_t, int64_t, int64_t, const void *, const void *, const int64_t *,
                               float *, hipStream_t, const uint32_t *) {
  return hipErrorInvalidValue;
}
hipError_t launch_combine(int64_t, int64_t, const float *, float *, float *, float *, hipStream_t,
                          const uint32_t *) {
  return hipErrorInvalidValue;
}
hipError_t launch_transpose(int, const void *, int64_t, int64_t, void *, int64_t, int64_t, hipStream_t,
                            const int32_t *, const int32_t *) {
  return hipErrorInvalidValue;
}
hipError_t launch_finalize(int, int64_t, int64_t, const float *, const uint8_t *, const uint32_t *, void *,
                           hipStream_t) {
  return hipErrorInvalidValue;
}
}  // namespace flh

