// Kernel launches of the library.  Every launch goes through launch(): a
// measurement hook (ce_debug_time_next_launch) can ask that the next launch
// made on the calling thread record a pair of HIP events at that kernel's
// own start and end (hipExtLaunchKernel), so a caller can time one kernel
// without event packets of its own between kernels on the stream.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ce_host {

// The events set by ce_debug_time_next_launch on this thread, if any; a
// launch that takes them clears them.
bool take_launch_events(hipEvent_t* start, hipEvent_t* stop);

template <typename F, typename... Args>
void launch(F kernel, dim3 grid, dim3 block, uint32_t shmem, hipStream_t st, Args... args) {
  hipEvent_t a = nullptr, b = nullptr;
  if (take_launch_events(&a, &b))
    hipExtLaunchKernelGGL(kernel, grid, block, shmem, st, a, b, 0u, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, shmem, st, args...);
}

}  // namespace ce_host
