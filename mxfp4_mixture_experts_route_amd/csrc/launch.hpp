// Kernel launch used by every entry point: a plain launch, or, when kernel timing is armed
// (moe_timing_arm), a launch that records the runtime's per-kernel start/stop events.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

namespace moe {

// Set-up a device keeps (a kernel's dynamic-LDS opt-in) is done once per device: call sites keep
// a flag per device slot. Slot of the current device, or -1 (then the set-up simply repeats).
constexpr int kMaxDevices = 64;
inline int device_slot() {
  int dev = 0;
  return (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < kMaxDevices) ? dev : -1;
}

// Next pair of timing events, or false when timing is not armed (timing.hip).
bool timing_next(hipEvent_t* start, hipEvent_t* stop);

// The runtime's last-error state is cleared first: entry points report MOE_ELAUNCH from
// hipGetLastError() after the launch, and an error left by an earlier, unrelated runtime call
// (the caller's, or a framework's start-up) must not be reported as this launch's.
template <typename Kernel, typename... Args>
inline void launch(Kernel kernel, dim3 grid, dim3 block, size_t lds, hipStream_t stream,
                   Args... args) {
  (void)hipGetLastError();
  hipEvent_t start, stop;
  if (timing_next(&start, &stop))
    hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)lds, stream, start, stop, 0u, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, lds, stream, args...);
}

}  // namespace moe
