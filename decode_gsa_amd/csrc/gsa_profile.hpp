// Optional timing hook of libgsa: caller-owned HIP events recorded on the
// call's stream around each kernel launch (see gsa_profile_events in gsa.h).
#pragma once

#include <hip/hip_runtime.h>

namespace gsa {

// Start of a library call: the next mark is the call's first.
void prof_begin_call();
// Record the next armed event of this thread, if any, on stream s.
void prof_mark(hipStream_t s);

}  // namespace gsa
