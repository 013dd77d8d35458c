// Per-kernel timing hook (see moe_set_kernel_events and moe_set_kernel_filter
// in include/moe.h).
#include <string.h>

#include "../../include/moe.h"
#include "hook.h"

namespace {
constexpr int kFilterMax = 64;  // longest filter name, with its terminating 0
struct Hook {
  hipEvent_t const* events = nullptr;
  const char** names = nullptr;
  int capacity = 0;
  int* count = nullptr;
  int n = 0;
  char only[kFilterMax] = {};  // empty: every kernel
  bool pending = false;        // filter: events[n] holds a start not yet closed
};
thread_local Hook g_hook;

// A failed record switches the hook off and reports -(HIP error) through
// *count; the error is cleared so that it cannot be mistaken for a failure of
// the kernel launch around it.
bool record(Hook& h, int i, const char* name, hipStream_t stream) {
  if (h.names) h.names[i] = name;
  hipError_t e = hipEventRecord(h.events[i], stream);
  if (e == hipSuccess) return true;
  (void)hipGetLastError();
  if (h.count) *h.count = -static_cast<int>(e);
  h.events = nullptr;
  h.pending = false;
  return false;
}
}  // namespace

namespace moe {
void note_prelaunch(const char* name, hipStream_t stream) {
  Hook& h = g_hook;
  if (!h.events || !h.only[0] || strcmp(name, h.only) != 0 || h.n + 2 > h.capacity) return;
  // a start left open (a launch that returned early) is overwritten
  h.pending = record(h, h.n, name, stream);
}

void note_launch(const char* name, hipStream_t stream) {
  Hook& h = g_hook;
  if (!h.events) return;
  if (h.only[0]) {
    if (!h.pending || strcmp(name, h.only) != 0) return;
    h.pending = false;
    if (!record(h, h.n + 1, name, stream)) return;
    h.n += 2;
  } else {
    if (h.n >= h.capacity || !record(h, h.n, name, stream)) return;
    ++h.n;
  }
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
  g_hook.pending = false;
  if (count) *count = 0;
  return MOE_OK;
}

extern "C" int moe_set_kernel_filter(const char* name) {
  if (name && strlen(name) >= static_cast<size_t>(kFilterMax)) return MOE_ERR_SHAPE;
  if (name)
    strcpy(g_hook.only, name);
  else
    g_hook.only[0] = 0;
  g_hook.pending = false;
  return MOE_OK;
}

// ---------------------------------------------------------------------------
// Clock probe (observability): MFMA-only work on every CU, so that the clock
// is read under the load the expert GEMMs put on the chip.
// ---------------------------------------------------------------------------
namespace {
typedef __attribute__((ext_vector_type(8))) __bf16 pbf16x8_t;
typedef __attribute__((ext_vector_type(16))) float pf32x16_t;

__global__ __launch_bounds__(256) void clock_probe_kernel(unsigned long long* __restrict__ ticks,
                                                          int iters) {
  const int tid = threadIdx.x;
  pbf16x8_t a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(1.0f + 0.001f * (float)((tid + i) & 7));
    b[i] = (__bf16)(1.0f - 0.001f * (float)((tid * 3 + i) & 7));
  }
  pf32x16_t acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = pf32x16_t{};
  __syncthreads();
  unsigned long long t0 = 0, r0 = 0;
  if (tid == 0) {
    t0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += acc[j][tid & 15];
  __syncthreads();
  if (tid == 0) {
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    unsigned long long* o = ticks + 4 * (long)blockIdx.x;
    o[0] = t0;
    o[1] = t1;
    o[2] = r0;
    o[3] = r1;
  }
  // keeps the MFMA results alive; never true for the inputs above
  if (s == -1.0f) ticks[0] = 0;
}
}  // namespace

extern "C" int moe_probe_clock(unsigned long long* ticks, int grid, int iters, void* stream) {
  if (!ticks) return MOE_ERR_NULL;
  if (grid <= 0 || iters <= 0) return MOE_ERR_SHAPE;
  if ((reinterpret_cast<uintptr_t>(ticks) & 15u) != 0) return MOE_ERR_ALIGN;
  (void)hipGetLastError();
  hipLaunchKernelGGL(clock_probe_kernel, dim3(grid), dim3(256), 0,
                     static_cast<hipStream_t>(stream), ticks, iters);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}
