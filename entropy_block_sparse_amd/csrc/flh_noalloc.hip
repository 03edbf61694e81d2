// flh_forward_noalloc: the forward with its scratch in a static device array, for
// callers that cannot allocate device memory (include/flh.h).
//
// The array lives in this file; each GPU holds its own copy at its own address.  In
// host code the array's name only stands in for it (it is not a device address), so
// the address is looked up with hipGetSymbolAddress once per device, with that device
// current, and only that address is ever handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "flh.h"
#include "flh_internal.h"

namespace {

constexpr size_t kScratchBytes = FLH_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch is handed out 256-byte aligned");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_lock;
void *g_scratch[kMaxDevices] = {};

// Device address of `scratch` on the current device, or null on a HIP error.
void *scratch_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> guard(g_lock);
  if (!g_scratch[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch[dev] = p;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" flh_status flh_forward_noalloc(flh_dtype dt, const void *h, const void *W, const int64_t *targets,
                                          int64_t T, int64_t H, int64_t V, float *logprob, float *entropy,
                                          float *lse, const flh_active_meta *meta, void *stream,
                                          uint32_t flags) {
  if (dt == FLH_FP8_E4M3) return FLH_E_UNSUPPORTED;  // fp8 inputs need their scales
  const flh_status chk = flh::forward_check(dt, h, W, targets, T, H, V, logprob, entropy, lse, meta, flags);
  if (chk != FLH_OK) return chk;
  if (flh_workspace_bytes(FLH_OP_FORWARD, dt, T, H, V, 0) > kScratchBytes) return FLH_E_SCRATCH;
  void *ws = scratch_address();
  if (!ws) return FLH_E_HIP;
  return flh_forward_ex(dt, h, W, targets, T, H, V, logprob, entropy, lse, meta, ws, kScratchBytes, stream,
                        flags);
}
