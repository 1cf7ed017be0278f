// moe_timing_arm / moe_timing_read: per-kernel execution times of the library's own launches.
//
// Armed launches go through hipExtLaunchKernel with a start/stop event pair, which the runtime
// stamps at the kernel's own start and end (the interval a kernel trace reports), so the times
// exclude the dispatch gaps that events recorded between launches would include.
#include "launch.hpp"

#include "moe_mx4.h"

namespace {

hipEvent_t g_start[MOE_TIMING_MAX];
hipEvent_t g_stop[MOE_TIMING_MAX];
bool g_created = false;
int g_armed = 0;   // launches to time since the last arm
int g_used = 0;    // of which already launched

}  // namespace

bool moe::timing_next(hipEvent_t* start, hipEvent_t* stop) {
  if (g_used >= g_armed) return false;
  *start = g_start[g_used];
  *stop = g_stop[g_used];
  ++g_used;
  return true;
}

extern "C" int moe_timing_arm(int n) {
  if (n < 0 || n > MOE_TIMING_MAX) return MOE_EINVAL;
  if (n > 0 && !g_created) {
    for (int i = 0; i < MOE_TIMING_MAX; ++i) {
      if (hipEventCreate(&g_start[i]) != hipSuccess || hipEventCreate(&g_stop[i]) != hipSuccess)
        return MOE_ELAUNCH;
    }
    g_created = true;
  }
  g_armed = n;
  g_used = 0;
  return MOE_OK;
}

extern "C" int moe_timing_read(float* ms, int n) {
  if (!ms || n < 0) return MOE_EINVAL;
  if (n > g_used) return MOE_ESHAPE;
  for (int i = 0; i < n; ++i) {
    if (hipEventSynchronize(g_stop[i]) != hipSuccess ||
        hipEventElapsedTime(&ms[i], g_start[i], g_stop[i]) != hipSuccess)
      return MOE_ELAUNCH;
  }
  return MOE_OK;
}
