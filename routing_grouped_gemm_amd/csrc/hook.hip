// Per-kernel timing hook (see moe_set_kernel_events in include/moe.h).
#include "../../include/moe.h"
#include "hook.h"

namespace {
struct Hook {
  hipEvent_t const* events = nullptr;
  const char** names = nullptr;
  int capacity = 0;
  int* count = nullptr;
  int n = 0;
};
thread_local Hook g_hook;
}  // namespace

namespace moe {
// A failed record switches the hook off and reports -(HIP error) through
// *count; the error is cleared so that it cannot be mistaken for a failure of
// the kernel launch that precedes it.
void note_launch(const char* name, hipStream_t stream) {
  Hook& h = g_hook;
  if (!h.events || h.n >= h.capacity) return;
  if (h.names) h.names[h.n] = name;
  hipError_t e = hipEventRecord(h.events[h.n], stream);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    if (h.count) *h.count = -static_cast<int>(e);
    h.events = nullptr;
    return;
  }
  ++h.n;
  if (h.count) *h.count = h.n;
}
}  // namespace moe

extern "C" int moe_set_kernel_events(void* const* events, const char** names, int capacity,
                                     int* count) {
  if (events && capacity <= 0) return MOE_ERR_SHAPE;
  g_hook.events = reinterpret_cast<hipEvent_t const*>(events);
  g_hook.names = names;
  g_hook.capacity = events ? capacity : 0;
  g_hook.count = count;
  g_hook.n = 0;
  if (count) *count = 0;
  return MOE_OK;
}
