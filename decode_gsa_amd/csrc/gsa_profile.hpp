// Optional timing hook of libgsa: caller-owned HIP events attached to each
// kernel launch of a call (see gsa_profile_events in gsa.h).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

namespace gsa {

// Start of a library call.
void prof_begin_call();
// Events for the call's next kernel launch: the first launch gets armed
// event 0 as its start event; launch i (from 0) gets armed event i + 1 as its
// stop event; null where nothing is armed. The runtime stamps them with the
// kernel's own start and end, so the caller's event pairs time the kernels
// rather than the dispatch around them.
void prof_launch_events(hipEvent_t* start, hipEvent_t* stop);

// Launch a kernel with this thread's armed events attached.
template <typename F, typename... Args>
inline void prof_launch(F kernel, dim3 grid, dim3 block, uint32_t shm, hipStream_t st, Args... args) {
  hipEvent_t e0, e1;
  prof_launch_events(&e0, &e1);
  hipExtLaunchKernelGGL(kernel, grid, block, shm, st, e0, e1, 0u, args...);
}

}  // namespace gsa
