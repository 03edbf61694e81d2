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
                               float *, hipStream_t, const uint32_t *, float) {
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
                           hipStream_t, float) {
  return hipErrorInvalidValue;
}
}  // namespace flh

// The no-allocation forward without its device array: the same checks, then the error
// the real call returns when the scratch address cannot be looked up.
extern "C" flh_status flh_forward_noalloc(flh_dtype dt, const void *h, const void *W, const int64_t *targets,
                                          int64_t T, int64_t H, int64_t V, float *logprob, float *entropy,
                                          float *lse, const flh_active_meta *meta, void *, uint32_t flags) {
  if (dt == FLH_FP8_E4M3) return FLH_E_UNSUPPORTED;
  const flh_status chk = flh::forward_check(dt, h, W, targets, T, H, V, logprob, entropy, lse, meta, flags);
  if (chk != FLH_OK) return chk;
  if (flh_workspace_bytes(FLH_OP_FORWARD, dt, T, H, V, 0) > FLH_NOALLOC_SCRATCH_BYTES) return FLH_E_SCRATCH;
  return FLH_E_HIP;
}
