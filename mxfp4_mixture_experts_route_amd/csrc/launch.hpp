// Kernel launch used by every entry point: a plain launch, or, when kernel timing is armed
// (moe_timing_arm), a launch that records the runtime's per-kernel start/stop events.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

namespace moe {

// Next pair of timing events, or false when timing is not armed (timing.hip).
bool timing_next(hipEvent_t* start, hipEvent_t* stop);

template <typename Kernel, typename... Args>
inline void launch(Kernel kernel, dim3 grid, dim3 block, size_t lds, hipStream_t stream,
                   Args... args) {
  hipEvent_t start, stop;
  if (timing_next(&start, &stop))
    hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)lds, stream, start, stop, 0u, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, lds, stream, args...);
}

}  // namespace moe
