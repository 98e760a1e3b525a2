// Timing hook of libgsa (see gsa_profile_events in gsa.h): a per-thread list
// of caller-owned hipEvent_t handles, recorded in order around the kernel
// launches of each later call on that thread.
#include "gsa_profile.hpp"

#include "gsa.h"
#include "gsa_plan.hpp"

namespace gsa {
namespace {
constexpr int kMaxEvents = 8;
thread_local hipEvent_t g_events[kMaxEvents];
thread_local int g_n = 0;
thread_local int g_next = 0;
}  // namespace

void prof_begin_call() { g_next = 0; }

void prof_mark(hipStream_t s) {
  if (g_next < g_n) (void)hipEventRecord(g_events[g_next], s);
  ++g_next;
}

}  // namespace gsa

extern "C" gsa_status_t gsa_profile_events(void* const* events, int32_t n) {
  gsa::clear_error();
  if (n < 0 || n > gsa::kMaxEvents)
    return gsa::fail(GSA_ERR_INVALID_ARG, "n=%d outside [0, %d]", n, gsa::kMaxEvents);
  if (n > 0 && events == nullptr) return gsa::fail(GSA_ERR_INVALID_ARG, "events is NULL");
  for (int i = 0; i < n; ++i)
    if (events[i] == nullptr) return gsa::fail(GSA_ERR_INVALID_ARG, "events[%d] is NULL", i);
  for (int i = 0; i < n; ++i) gsa::g_events[i] = reinterpret_cast<hipEvent_t>(events[i]);
  gsa::g_n = n;
  gsa::g_next = 0;
  return GSA_OK;
}

extern "C" gsa_status_t gsa_profile_marks(int32_t* n) {
  gsa::clear_error();
  if (n == nullptr) return gsa::fail(GSA_ERR_INVALID_ARG, "n is NULL");
  *n = gsa::g_next;
  return GSA_OK;
}
