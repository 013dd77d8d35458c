// Routing, dispatch and combine for small batches (a few dozen tokens, as in
// token-by-token generation).
//
// At a handful of tokens every kernel of the layer is a few microseconds of
// launch and drain, so the number of kernels sets the latency.  Here the
// router is two kernels (partial logits over slices of Wr's rows, then their
// sum, softmax and top-k); the routing
// metadata (counts, offsets, each slot's row, each row's token) and the row
// copies are one kernel, every workgroup recomputing the (small) metadata in
// LDS so that no workgroup waits for another; and the combine spreads one
// token over a whole workgroup.  Results are those of the general kernels:
// the same slot order, ranks and sums.
#include "hook.h"
#include "moe_common.h"
#include "route.h"
#include "topk_dev.h"

namespace moe {

// ---------------------------------------------------------------------------
// router: partial logits over slices of 128 k-rows (one workgroup per slice
// and 4 tokens), then per token the sum of the slices in order, softmax and
// top-k
// ---------------------------------------------------------------------------
// Thread (g, o) of a slice sums k-rows g, g + G, ... of Wr's expert octet o
// (16-byte loads of a Wr row, all in flight together) for each token; the G
// partial sums are added in order of g.
__global__ __launch_bounds__(256) void route_part_kernel(const bf16_t* __restrict__ x,
                                                         const bf16_t* __restrict__ Wr, int T,
                                                         int d, int E,
                                                         float* __restrict__ part) {
  __shared__ float red[2048 * 4];                  // [G][4 tokens][E], G * E <= 2048
  const int tid = threadIdx.x;
  const int slice = blockIdx.x, t0 = blockIdx.y * 4;
  const int nt = min(4, T - t0);
  const int kb = slice * kRouteSlice;
  const int oct = E >> 3;                 // expert octets
  const int G = 256 / oct;                // k-row groups
  const int g = tid / oct, o = tid - g * oct;
  float acc[4][8];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[t][q] = 0.0f;
  if (g < G) {
    const int kend = min(d, kb + kRouteSlice);
    constexpr int U = 8;
    for (int k0 = kb + g; k0 < kend; k0 += U * G) {
      float w[U][8], xv[U][4];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int kk = k0 + u * G;
        if (kk < kend) {
          load8(Wr + (long)kk * E + 8 * o, w[u]);
#pragma unroll
          for (int t = 0; t < 4; ++t)
            xv[u][t] = (t < nt) ? bf16_to_f32(x[(long)(t0 + t) * d + kk]) : 0.0f;
        } else {
#pragma unroll
          for (int q = 0; q < 8; ++q) w[u][q] = 0.0f;
#pragma unroll
          for (int t = 0; t < 4; ++t) xv[u][t] = 0.0f;
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int q = 0; q < 8; ++q) acc[t][q] = fmaf(xv[u][t], w[u][q], acc[t][q]);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int q = 0; q < 8; ++q) red[(g * 4 + t) * E + 8 * o + q] = acc[t][q];
  }
  __syncthreads();
  for (int i = tid; i < nt * E; i += 256) {
    const int t = i / E, e = i - t * E;
    float sum = 0.0f;
    for (int gg = 0; gg < G; ++gg) sum += red[(gg * 4 + t) * E + e];
    part[((long)slice * T + t0 + t) * E + e] = sum;
  }
}

// logits[t] = sum over slices in order; then softmax and top-k (one wave per
// token).
__global__ __launch_bounds__(256) void route_final_kernel(const float* __restrict__ part, int P,
                                                          int T, int E, int k, int renorm,
                                                          float* __restrict__ logits,
                                                          int32_t* __restrict__ topk_idx,
                                                          float* __restrict__ topk_w) {
  __shared__ __attribute__((aligned(16))) float lg[4][256];
  __shared__ float ps[4][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * 4;
  const int nt = min(4, T - t0);
  for (int i = tid; i < nt * E; i += 256) {
    const int t = i / E, e = i - t * E;
    float sum = 0.0f;
#pragma unroll 16
    for (int p = 0; p < P; ++p) sum += part[((long)p * T + t0 + t) * E + e];
    lg[t][e] = sum;
    logits[(long)(t0 + t) * E + e] = sum;
  }
  __syncthreads();
  if (wave < nt) {
    if (E <= 64)
      topk_rank64(lg[wave], E, k, renorm, lane, ps[wave], topk_idx + (long)(t0 + wave) * k,
                  topk_w + (long)(t0 + wave) * k);
    else
      topk_row(lg[wave], E, k, renorm, lane, topk_idx + (long)(t0 + wave) * k,
               topk_w + (long)(t0 + wave) * k);
  }
}

// ---------------------------------------------------------------------------
// dispatch: metadata in LDS (every workgroup), rows copied by slot ranges
// ---------------------------------------------------------------------------
// rank of slot s among the slots of its expert = number of earlier slots
// (token-major order) routed to the same expert, i.e. rows in ascending
// token order within each expert, as the general kernels place them.
template <typename TS>
__global__ __launch_bounds__(256) void dispatch_small_kernel(
    const TS* __restrict__ x, const int32_t* __restrict__ idx, int T, int d, int E, int k,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ dest_row,
    int32_t* __restrict__ src_token, TS* __restrict__ Xs) {
  __shared__ int ex[kSmallMaxRows];
  __shared__ int dst[kSmallMaxRows];
  __shared__ int cnt[256];
  __shared__ int off[257];
  __shared__ int run[256];
  __shared__ int cw[4 * 256];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int R = T * k;
  for (int e = tid; e < E; e += 256) { cnt[e] = 0; run[e] = 0; }
  for (int s = tid; s < R; s += 256) {
    const int e = idx[s];
    ex[s] = (e >= 0 && e < E) ? e : -1;
  }
  __syncthreads();
  for (int s = tid; s < R; s += 256)
    if (ex[s] >= 0) atomicAdd(&cnt[ex[s]], 1);
  __syncthreads();
  if (tid < 64) {
    int c[4], sum = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = tid * 4 + q;
      c[q] = (e < E) ? cnt[e] : 0;
      sum += c[q];
    }
    int incl = sum;
#pragma unroll
    for (int sh = 1; sh < 64; sh <<= 1) {
      const int v = __shfl_up(incl, sh, 64);
      if (tid >= sh) incl += v;
    }
    int r = incl - sum;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = tid * 4 + q;
      if (e <= E) off[e] = r;
      r += c[q];
    }
    if (tid == 63 && E == 256) off[256] = incl;
  }
  __syncthreads();
  // ranks, 256 slots at a time: slots of the same expert in earlier waves
  // (per-wave counts) plus earlier lanes of this wave (lane scan)
  for (int c0 = 0; c0 < R; c0 += 256) {
    const int s = c0 + tid;
    const int e = (s < R) ? ex[s] : -1;
    for (int i = tid; i < 4 * E; i += 256) cw[i] = 0;
    __syncthreads();
    if (e >= 0) atomicAdd(&cw[wave * E + e], 1);
    int rin = 0;
    for (int l = 0; l < 64; ++l) {
      const int el = __builtin_amdgcn_readlane(e, l);
      rin += (l < lane && el == e) ? 1 : 0;
    }
    __syncthreads();
    if (e >= 0) {
      int b = run[e] + rin;
      for (int w = 0; w < wave; ++w) b += cw[w * E + e];
      dst[s] = off[e] + b;
    } else if (s < R) {
      dst[s] = -1;
    }
    __syncthreads();
    for (int i = tid; i < E; i += 256) run[i] += cw[i] + cw[E + i] + cw[2 * E + i] + cw[3 * E + i];
    __syncthreads();
  }
  if (blockIdx.x == 0) {
    for (int e = tid; e < E; e += 256) counts[e] = cnt[e];
    for (int e = tid; e <= E; e += 256) offsets[e] = off[e];
    for (int s = tid; s < R; s += 256) {
      dest_row[s] = dst[s];
      if (dst[s] >= 0) src_token[dst[s]] = s / k;
    }
  }
  // rows: one wave per slot of this workgroup's range
  const int per = (R + gridDim.x - 1) / gridDim.x;
  const int s1 = min(R, (int)(blockIdx.x + 1) * per);
  for (int s = blockIdx.x * per + wave; s < s1; s += 4) {
    const int r = dst[s];
    if (r < 0) continue;
    const TS* src = x + (long)(s / k) * d;
    TS* out = Xs + (long)r * d;
    for (int c = lane * 8; c < d; c += 64 * 8) {
      if constexpr (sizeof(TS) == 2) {
        *reinterpret_cast<uint4*>(out + c) = *reinterpret_cast<const uint4*>(src + c);
      } else {
        *reinterpret_cast<float4*>(out + c) = *reinterpret_cast<const float4*>(src + c);
        *reinterpret_cast<float4*>(out + c + 4) = *reinterpret_cast<const float4*>(src + c + 4);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// combine: y[t] = sum_j w[t,j] Ys[dest_row[t,j]], one workgroup per token and
// 2048 columns, the k rows' loads in flight together; a slot whose row lies
// outside [0, R) adds nothing (its load goes to a clamped row)
// ---------------------------------------------------------------------------
template <typename TS>
__global__ __launch_bounds__(256) void combine_small_kernel(const TS* __restrict__ Ys,
                                                            const float* __restrict__ w,
                                                            const int32_t* __restrict__ dest_row,
                                                            int T, int d, int k,
                                                            TS* __restrict__ y) {
  const long t = blockIdx.y;
  const int c = (blockIdx.x * 256 + threadIdx.x) * 8;
  if (c >= d) return;
  const int R = T * k;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  int j = 0;
  for (; j + 4 <= k; j += 4) {
    float v[4][8];
    float wj[4];
    bool ok[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int rr = dest_row[t * k + j + u];
      const int r = min(max(rr, 0), R - 1);
      ok[u] = (unsigned)rr < (unsigned)R;
      wj[u] = w[t * k + j + u];
      load8(Ys + (long)r * d + c, v[u]);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (ok[u])
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] = fmaf(wj[u], v[u][q], acc[q]);
  }
  for (; j < k; ++j) {
    const int rr = dest_row[t * k + j];
    if ((unsigned)rr >= (unsigned)R) continue;
    const float wj = w[t * k + j];
    float v[8];
    load8(Ys + (long)rr * d + c, v);
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = fmaf(wj, v[q], acc[q]);
  }
  store8(y + t * d + c, acc);
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
bool route_small_applies(int T, int d, int E) {
  return T <= kSmallMaxTokens && E % 8 == 0 && E <= 256 && d % 8 == 0;
}

size_t route_small_workspace(int T, int d, int E) {
  return (size_t)((d + kRouteSlice - 1) / kRouteSlice) * T * E * sizeof(float);
}

hipError_t launch_route_small(const uint16_t* x, const uint16_t* Wr, int T, int d, int E, int k,
                              int renorm, float* part, float* logits, int32_t* idx, float* w,
                              hipStream_t s) {
  const int P = (d + kRouteSlice - 1) / kRouteSlice;
  note_prelaunch("route_small_part", s);
  hipLaunchKernelGGL(route_part_kernel, dim3(P, (T + 3) / 4), dim3(256), 0, s, x, Wr, T, d, E,
                     part);
  note_launch("route_small_part", s);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  note_prelaunch("route_small_final", s);
  hipLaunchKernelGGL(route_final_kernel, dim3((T + 3) / 4), dim3(256), 0, s, part, P, T, E, k,
                     renorm, logits, idx, w);
  note_launch("route_small_final", s);
  return hipGetLastError();
}

bool dispatch_small_applies(int T, int k) { return (long long)T * k <= kSmallMaxRows; }

hipError_t launch_dispatch_small(int dtype, const void* x, const int32_t* idx, int T, int d, int E,
                                 int k, int32_t* counts, int32_t* offsets, int32_t* dest_row,
                                 int32_t* src_token, void* Xs, hipStream_t s) {
  const int R = T * k;
  const int blocks = max(1, min(256, (R + 7) / 8));
  note_prelaunch("dispatch_small", s);
  if (dtype)
    hipLaunchKernelGGL(dispatch_small_kernel<bf16_t>, dim3(blocks), dim3(256), 0, s,
                       static_cast<const bf16_t*>(x), idx, T, d, E, k, counts, offsets, dest_row,
                       src_token, static_cast<bf16_t*>(Xs));
  else
    hipLaunchKernelGGL(dispatch_small_kernel<float>, dim3(blocks), dim3(256), 0, s,
                       static_cast<const float*>(x), idx, T, d, E, k, counts, offsets, dest_row,
                       src_token, static_cast<float*>(Xs));
  note_launch("dispatch_small", s);
  return hipGetLastError();
}

bool combine_small_applies(int T) { return T <= kSmallMaxTokens; }

hipError_t launch_combine_small(int dtype, const void* Ys, const float* w, const int32_t* dest,
                                int T, int d, int k, void* y, hipStream_t s) {
  dim3 grid((d + 2047) / 2048, T);
  note_prelaunch("combine_small", s);
  if (dtype)
    hipLaunchKernelGGL(combine_small_kernel<bf16_t>, grid, dim3(256), 0, s,
                       static_cast<const bf16_t*>(Ys), w, dest, T, d, k, static_cast<bf16_t*>(y));
  else
    hipLaunchKernelGGL(combine_small_kernel<float>, grid, dim3(256), 0, s,
                       static_cast<const float*>(Ys), w, dest, T, d, k, static_cast<float*>(y));
  note_launch("combine_small", s);
  return hipGetLastError();
}

}  // namespace moe
