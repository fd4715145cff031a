// tri_evict_step_noalloc: the whole pass with its control words (per-unit tickets, score ranges, chunk flags) in a
// library-owned device array instead of a caller-allocated workspace, for callers that cannot allocate device
// memory at the time of the call.
#include <hip/hip_runtime.h>

#include <mutex>

#include "tri_internal.h"

namespace {

constexpr size_t kScratchBytes = (size_t)TRI_NOALLOC_SCRATCH_BYTES;

// The control words of tri_evict_step_noalloc.  In host code `scratch` names a host-side stand-in, not device
// memory: the kernels receive the device address that hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 256;
std::mutex g_mu;
void *g_scratch[kMaxDevices];   // device address of `scratch` on each device, looked up once per device

// Device address of `scratch` on the current device (looked up on the first call made on that device).
hipError_t scratch_on_current_device(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[dev] == nullptr) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace

extern "C" tri_status tri_evict_step_noalloc(const tri_cache *cache, const tri_params *params, float *scores,
                                             int32_t *keep, int32_t *new_lengths, int32_t *block_table_out,
                                             int32_t *freed, int32_t *n_freed, hipStream_t stream) {
  if (!scores || !keep) return tri::fail_status(TRI_ERR_INVALID_ARG, "scores and keep must be non-NULL");
  const size_t need = tri::control_bytes(cache, params);
  if (need == 0)   // invalid cache or parameters: the full validation reports which
    return tri::evict_step(cache, params, scores, keep, new_lengths, block_table_out, freed, n_freed, nullptr, 0,
                           stream, nullptr, true);
  if (need > kScratchBytes) {
    char msg[160];
    snprintf(msg, sizeof msg, "these shapes need %zu bytes of control words, more than the %zu of the library's array",
             need, kScratchBytes);
    return tri::fail_status(TRI_ERR_UNSUPPORTED, msg);
  }
  void *ws = nullptr;
  const hipError_t e = scratch_on_current_device(&ws);
  if (e != hipSuccess) {
    char msg[160];
    snprintf(msg, sizeof msg, "device address of the control-word array: %s", hipGetErrorString(e));
    return tri::fail_status(TRI_ERR_HIP, msg);
  }
  return tri::evict_step(cache, params, scores, keep, new_lengths, block_table_out, freed, n_freed, ws,
                         kScratchBytes, stream, nullptr, true);
}
