// Opt-in kernel timing hook (msa_set_profile_events): when a caller has
// registered HIP events, every public call records event i on its stream
// right after its i-th kernel launch.  Thread-local; off by default.
#include <hip/hip_runtime.h>

#include "launch.hpp"
#include "msa.h"

namespace {
thread_local void *const *g_events = nullptr;
thread_local int g_num_events = 0;
thread_local int g_next = 0;
}  // namespace

namespace msa {

void profile_begin_call() { g_next = 0; }

void profile_mark(hipStream_t s) {
  if (g_events != nullptr && g_next < g_num_events) {
    (void)hipEventRecord(reinterpret_cast<hipEvent_t>(g_events[g_next]), s);
  }
  ++g_next;
}

}  // namespace msa

extern "C" void msa_set_profile_events(void *const *events, int num_events) {
  g_events = num_events > 0 ? events : nullptr;
  g_num_events = num_events > 0 ? num_events : 0;
  g_next = 0;
}
