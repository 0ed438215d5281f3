// launch.h -- the library's kernel launches, which a timed forward can
// bracket with events of each kernel's own execution.
//
// moe::launch(kernel, grid, block, lds, stream, args...) is an ordinary
// launch.  While a KernelTimer is installed on the calling host thread (only
// moe_forward_timed does so, for the duration of its call), each launch asks
// it for a start and a stop event and goes through hipExtLaunchKernel, which
// records the two events at the kernel's own begin and end: their elapsed
// time is the kernel's execution, with no launch gap or event packet inside.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstdint>
#include <utility>

namespace moe {

struct KernelTimer {
  // Events for the next kernel; false when none are left (plain launch).
  virtual bool next_events(hipEvent_t *start, hipEvent_t *stop) = 0;
  virtual ~KernelTimer() = default;
};

// The timer of the calling thread (null outside moe_forward_timed).
KernelTimer *&kernel_timer();

template <typename F, typename... Args>
inline void launch(F kernel, dim3 grid, dim3 block, uint32_t lds, hipStream_t stream, Args &&...args) {
  hipEvent_t e0, e1;
  KernelTimer *t = kernel_timer();
  if (t && t->next_events(&e0, &e1))
    hipExtLaunchKernelGGL(kernel, grid, block, lds, stream, e0, e1, 0u, std::forward<Args>(args)...);
  else
    hipLaunchKernelGGL(kernel, grid, block, lds, stream, std::forward<Args>(args)...);
}

}  // namespace moe
