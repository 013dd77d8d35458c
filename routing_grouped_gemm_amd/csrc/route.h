// Launchers of the routing, dispatch and combine kernels (route.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// Small batches: the router runs as two kernels (partial logits over slices
// of kRouteSlice rows of Wr, then sum, softmax and top-k), the dispatch
// (metadata and copies) and the combine as one kernel each.
constexpr int kSmallMaxTokens = 64;     // router and combine
constexpr int kSmallMaxRows = 1024;     // dispatch: tokens * top_k
constexpr int kRouteSlice = 128;

bool route_small_applies(int T, int d, int E);
// part: float workspace of route_small_workspace(T, d, E) bytes
size_t route_small_workspace(int T, int d, int E);
hipError_t launch_route_small(const uint16_t* x, const uint16_t* Wr, int T, int d, int E, int k,
                              int renorm, float* part, float* logits, int32_t* idx, float* w,
                              hipStream_t s);
bool dispatch_small_applies(int T, int k);
hipError_t launch_dispatch_small(int dtype, const void* x, const int32_t* idx, int T, int d, int E,
                                 int k, int32_t* counts, int32_t* offsets, int32_t* dest_row,
                                 int32_t* src_token, void* Xs, hipStream_t s);
bool combine_small_applies(int T);
hipError_t launch_combine_small(int dtype, const void* Ys, const float* w, const int32_t* dest,
                                int T, int d, int k, void* y, hipStream_t s);

// Router logits of a bf16 batch on the thin-product MFMA kernel (router.hip):
// E % 8 == 0, E <= 256, d % 64 == 0.
bool router_logits_applies(int d, int E);
hipError_t launch_router_logits(const uint16_t* x, const uint16_t* Wr, int T, int d, int E,
                                float* logits, hipStream_t s);

// Router input gradient dx += dl16 . Wr^T on MFMAs (router.hip): dl16 [T][ld]
// bf16 with a zero tail, ld = 64 * ceil(E / 64); E % 8 == 0, E <= 256, d % 64 == 0.
bool router_dx_applies(int d, int E);
hipError_t launch_router_dx(const uint16_t* dl16, int ld, const uint16_t* Wr, int T, int d, int E,
                            uint16_t* dx, hipStream_t s);

// Router weight-gradient partials on MFMAs (router.hip): part[s][d][E] float
// over S token slices (router_dwr_launch_slices picks S <= max_slices), to be
// added in slice order; dl16 as for launch_router_dx; E % 8 == 0, E <= 256,
// d % 64 == 0.
bool router_dwr_applies(int d, int E);
int router_dwr_launch_slices(int T, int d, int E, int max_slices);
hipError_t launch_router_dwr(const uint16_t* x, const uint16_t* dl16, int ld, int T, int d, int E,
                             int S, float* part, hipStream_t s);

// renorm: divide the k chosen probabilities by their sum.
hipError_t launch_topk_softmax(const float* logits, int T, int E, int k, int renorm, int32_t* idx,
                               float* w, hipStream_t s);
// hist and base: E * ceil(T/64) int32 each (workspace).
hipError_t launch_dispatch_meta(const int32_t* idx, int T, int E, int k, int32_t* hist,
                                int32_t* base, int32_t* counts, int32_t* offsets,
                                int32_t* dest_row, int32_t* src_token, hipStream_t s);
// Xs[dest_row[t,j]] = x[t].
hipError_t launch_dispatch_copy(int dtype, const void* x, const int32_t* dest_row, int T, int d,
                                int k, void* Xs, hipStream_t s);
hipError_t launch_combine(int dtype, const void* Ys, const float* w, const int32_t* dest, int T,
                          int d, int k, void* y, hipStream_t s);
// dYs_q / dYs_q_scale (optional, bf16 only): the stored dYs rows block-quantised
// along d (e4m3 codes; E8M0 scales in the dispatch's Xq_scale layout, pitch
// roundup(T*k, 16)).
hipError_t launch_combine_bwd(int dtype, const void* dY, const void* Ys, const float* w,
                              const int32_t* dest, int T, int d, int k, void* dYs, float* dw,
                              void* dYs_q, uint8_t* dYs_q_scale, hipStream_t s);
hipError_t launch_gather_sum(int dtype, const void* dXs, const int32_t* dest, int T, int d, int k,
                             int accumulate, void* dx, hipStream_t s);
// out[i] = (accumulate ? out[i] : 0) + sum over s of part[s*n + i], summed in
// float32 in order of s; out has the dtype.
hipError_t launch_split_reduce(int dtype, const float* part, int S, long n, int accumulate,
                               void* out, hipStream_t s);
// dl16 (optional): bf16 copy of dl as rows of ld16 >= E entries, tail zeroed.
// renorm: the weights were renormalised; aux_dp (optional, [E]): a per-expert
// gradient with respect to every token's probabilities (load-balancing loss).
hipError_t launch_router_bwd_softmax(const float* logits, const int32_t* idx, const float* dw,
                                     int T, int E, int k, int renorm, const float* aux_dp,
                                     float* dl, uint16_t* dl16, int ld16, hipStream_t s);
// Load-balancing loss and its per-expert probability gradient; part: float
// workspace of E * ceil(T/64).
hipError_t launch_router_aux(const float* logits, const int32_t* counts, int T, int E, int k,
                             float coef, float* part, float* loss, float* dp, hipStream_t s);
// report[0] = entries of idx[T][k] outside [0, E); report[1] = tokens with a
// repeated expert (device, written after the launch completes).
hipError_t launch_check_routing(const int32_t* idx, int T, int E, int k, int32_t* report,
                                hipStream_t s);

}  // namespace moe
