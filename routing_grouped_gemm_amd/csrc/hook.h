// Per-kernel timing hook: an event recorded after every launch while a
// caller has set one (moe_set_kernel_events); with a name filter set
// (moe_set_kernel_filter), an event before and one after each launch of the
// named kernel only.
#pragma once

#include <hip/hip_runtime.h>

namespace moe {
// called right before a kernel launch (it records only under a filter)
void note_prelaunch(const char* name, hipStream_t stream);
// called right after a kernel launch
void note_launch(const char* name, hipStream_t stream);
}  // namespace moe
