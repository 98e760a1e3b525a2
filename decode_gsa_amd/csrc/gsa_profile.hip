// Timing hook of libgsa (see gsa_profile_events in gsa.h): a per-thread list
// of caller-owned hipEvent_t handles, attached in order to the kernel
// launches of each later call on that thread.
#include "gsa_profile.hpp"

#include "gsa.h"
#include "gsa_plan.hpp"

namespace gsa {
namespace {
constexpr int kMaxEvents = 8;
thread_local hipEvent_t g_events[kMaxEvents];
thread_local int g_n = 0;
thread_local int g_launches = 0;   // launches of the current (or last) call
}  // namespace

void prof_begin_call() { g_launches = 0; }

void prof_launch_events(hipEvent_t* start, hipEvent_t* stop) {
  *start = (g_launches == 0 && g_n > 0) ? g_events[0] : nullptr;
  *stop = g_launches + 1 < g_n ? g_events[g_launches + 1] : nullptr;
  ++g_launches;
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
  return GSA_OK;
}

extern "C" gsa_status_t gsa_profile_marks(int32_t* n) {
  gsa::clear_error();
  if (n == nullptr) return gsa::fail(GSA_ERR_INVALID_ARG, "n is NULL");
  *n = gsa::g_launches + 1;
  return GSA_OK;
}
