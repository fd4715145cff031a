// Host-only stand-ins for the kernel launchers and the two HIP runtime calls of api.cpp, so that the C ABI's
// argument validation can be built with the host sanitizers (g++ -fsanitize=address,undefined) and driven without
// a GPU.  Every launcher records that it was reached and launches nothing.  Test infrastructure only.
#include <hip/hip_runtime_api.h>

#include "tri_internal.h"

int g_launches = 0;   // how many launchers the validation let through

extern "C" const char *hipGetErrorString(hipError_t) { return "stubbed HIP error"; }
extern "C" hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return hipSuccess; }

namespace tri {
hipError_t launch_prepare(const float *, const float *, int, int, int, int, double, int, const int32_t *, int, float *,
                          float *, hipStream_t) { return ++g_launches, hipSuccess; }
hipError_t launch_prepare_variant(const float *, int, int, int, int, double, int, const int32_t *, int, float *,
                                  hipStream_t) { return ++g_launches, hipSuccess; }
hipError_t launch_score(const CacheView &, const PassView &, float *, int64_t, uint32_t *, hipStream_t) {
  return ++g_launches, hipSuccess;
}
hipError_t launch_select(const CacheView &, const PassView &, const float *, int64_t, int32_t *, int32_t *, uint32_t *,
                         uint32_t *, uint32_t *, hipStream_t) { return ++g_launches, hipSuccess; }
bool select_moves_fit(const CacheView &, const PassView &pv) { return pv.budget <= 8192; }
hipError_t launch_select_move(const CacheView &, const PassView &, const float *, int64_t, int32_t *, int32_t *,
                              uint32_t *, int32_t *, int32_t *, int32_t *, hipStream_t) {
  return ++g_launches, hipSuccess;
}
bool fused_fits(const CacheView &cv) { return cv.capacity <= kFusedMax; }
hipError_t launch_fused(const CacheView &, const PassView &, float *, int64_t, int32_t *, int32_t *, int32_t *,
                        int32_t *, int32_t *, hipStream_t) { return ++g_launches, hipSuccess; }
hipError_t launch_calibrate(const QueryView &, double *, float *, float *, hipStream_t) {
  return ++g_launches, hipSuccess;
}
int decode_split(int64_t, int) { return 512; }
hipError_t launch_decode(const CacheView &, const PassView &, const DecodeView &, float *, float *, hipStream_t) {
  return ++g_launches, hipSuccess;
}
hipError_t launch_check(const CacheView &, const PassView &, int32_t, int32_t, int32_t, uint32_t *, uint32_t *,
                        hipStream_t) { return ++g_launches, hipSuccess; }
hipError_t launch_reset(uint32_t *, int64_t, uint32_t *, int64_t, hipStream_t) { return ++g_launches, hipSuccess; }
hipError_t launch_compact(const CacheView &, const PassView &, const int32_t *, int32_t *, int32_t *, int32_t *,
                          uint32_t *, uint32_t *, hipStream_t) { return ++g_launches, hipSuccess; }
}  // namespace tri
