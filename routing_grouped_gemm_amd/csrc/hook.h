// Per-kernel timing hook: an event recorded after every launch while a
// caller has set one (moe_set_kernel_events).
#pragma once

#include <hip/hip_runtime.h>

namespace moe {
void note_launch(const char* name, hipStream_t stream);
}  // namespace moe
