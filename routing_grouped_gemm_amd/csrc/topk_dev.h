// Softmax and top-k of one token's router logits, by one wave (shared by the
// general and the small-batch router kernels).
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "moe_common.h"

namespace moe {

// (value, expert) candidate o replaces the current one when it is present
// and has the larger value, or the same value and the lower expert.
__device__ __forceinline__ void take_better(float& bv, int& be, float ov, int oe) {
  const bool better = (oe != 0x7fffffff) &&
                      (be == 0x7fffffff || ov > bv || (ov == bv && oe < be));
  if (better) { bv = ov; be = oe; }
}
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ void argmax_step(float& bv, int& be) {
  const float ov = dpp_f<CTRL, ROWS>(bv, bv);
  const int oe = dpp_i<CTRL, ROWS>(be, be);
  take_better(bv, be, ov, oe);
}
// Best (value, expert) of the wave, returned to every lane (DPP reduction in
// the pattern of wave_sum; lanes outside a step's row mask compare with
// themselves).
__device__ __forceinline__ void wave_argmax(float& bv, int& be) {
  argmax_step<kDppQuad1032>(bv, be);
  argmax_step<kDppQuad2301>(bv, be);
  argmax_step<kDppRowHalfMirror>(bv, be);
  argmax_step<kDppRowMirror>(bv, be);
  argmax_step<kDppRowBcast15, 0xA>(bv, be);
  argmax_step<kDppRowBcast31, 0xC>(bv, be);
  bv = lane63_f(bv);
  be = __builtin_amdgcn_readlane(be, 63);
}

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
  mx = wave_max(mx);
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
    wave_argmax(bv, be);
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

// The same for E <= 64 experts with one logit per lane and no serial rounds:
// a chosen expert's slot is its rank among the E logits by (logit desc,
// expert asc), counted against the row held in LDS (sv: the E logits,
// 16-byte aligned, readable by the wave); ps: k floats of wave-private LDS
// for the renormalising sum, which is taken in slot order.  Choice, order and
// weights are those of topk_row, bit for bit.
__device__ __forceinline__ void topk_rank64(const float* sv, int E, int k, int renorm, int lane,
                                            float* ps, int32_t* __restrict__ idx_out,
                                            float* __restrict__ w_out) {
  const bool act = lane < E;
  const float v = act ? sv[lane] : -INFINITY;
  const float mx = wave_max(v);
  const float se = wave_sum(act ? expf(v - mx) : 0.0f);
  int rank = 0;
  int f = 0;
  for (; f + 4 <= E; f += 4) {
    const float4 u = *reinterpret_cast<const float4*>(sv + f);
    rank += (u.x > v || (u.x == v && f < lane)) ? 1 : 0;
    rank += (u.y > v || (u.y == v && f + 1 < lane)) ? 1 : 0;
    rank += (u.z > v || (u.z == v && f + 2 < lane)) ? 1 : 0;
    rank += (u.w > v || (u.w == v && f + 3 < lane)) ? 1 : 0;
  }
  for (; f < E; ++f) {
    const float u = sv[f];
    rank += (u > v || (u == v && f < lane)) ? 1 : 0;
  }
  const bool chosen = act && rank < k;
  const float p = expf(v - mx) / se;
  if (renorm) {
    if (chosen) ps[rank] = p;
    // the wave's own LDS writes are seen by its later reads
    __builtin_amdgcn_wave_barrier();
    float wsum = 0.0f;
    if (lane == 0)
      for (int j = 0; j < k; ++j) wsum += ps[j];
    wsum = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(wsum)));
    __builtin_amdgcn_wave_barrier();
    if (chosen) {
      idx_out[rank] = lane;
      w_out[rank] = p / wsum;
    }
  } else if (chosen) {
    idx_out[rank] = lane;
    w_out[rank] = p;
  }
}

}  // namespace moe
