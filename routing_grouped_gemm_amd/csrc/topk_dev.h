// Softmax and top-k of one token's router logits, by one wave (shared by the
// general and the small-batch router kernels).
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "moe_common.h"

namespace moe {

// One token's softmax and top-k, by one wave: row = its float32 logits (global
// memory or LDS).  Slots are ordered by (logit desc, expert asc); weights are
// the softmax probabilities of the chosen experts, divided by their sum when
// renorm is set.  Lane 0 writes idx_out[0..k) and w_out[0..k).
__device__ __forceinline__ void topk_row(const float* row, int E, int k, int renorm, int lane,
                         int32_t* __restrict__ idx_out, float* __restrict__ w_out) {
  float v[4];
  int taken = 0;  // bit q: logit q of this lane already chosen
  float mx = -INFINITY;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    int e = lane + 64 * q;
    v[q] = (e < E) ? row[e] : -INFINITY;
    if (e < E) mx = fmaxf(mx, v[q]);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
  float se = 0.0f;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    if (lane + 64 * q < E) se += expf(v[q] - mx);
  se = wave_sum(se);
  float wsum = 0.0f;
  for (int j = 0; j < k; ++j) {
    // lane-local best among the untaken: larger logit, then lower index
    float bv = -INFINITY;
    int be = 0x7fffffff;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      int e = lane + 64 * q;
      if (e < E && !((taken >> q) & 1)) {
        if (v[q] > bv || (v[q] == bv && e < be) || be == 0x7fffffff) {
          bv = v[q];
          be = e;
        }
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      float ov = __shfl_xor(bv, o, 64);
      int oe = __shfl_xor(be, o, 64);
      bool better = (oe != 0x7fffffff) &&
                    (be == 0x7fffffff || ov > bv || (ov == bv && oe < be));
      if (better) { bv = ov; be = oe; }
    }
    if ((be & 63) == lane) taken |= 1 << (be >> 6);
    const float p = expf(bv - mx) / se;
    wsum += p;
    if (lane == 0) {
      idx_out[j] = be;
      w_out[j] = p;
    }
  }
  if (renorm && lane == 0) {
    // optional top-k renormalisation: the chosen probabilities over their sum
    for (int j = 0; j < k; ++j) w_out[j] = w_out[j] / wsum;
  }
}

}  // namespace moe
