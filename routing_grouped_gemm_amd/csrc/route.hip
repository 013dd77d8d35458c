// Router, routing metadata, row-wise dispatch, combine and their backwards.
//
// Router (HF OLMoE walkthrough, section 2): softmax of the float32 logits
// over the experts and the top_k experts per token, weights = the chosen
// probabilities (no renormalisation).  One wave per token; every lane holds
// up to four logits; the k winners are taken by k wave-wide arg-max rounds
// ordered by (logit desc, index asc), so ties go to the lower expert index.
//
// Metadata and dispatch (olmoforge README: row-wise expert parallel writes
// every token row straight into its expert's input buffer; the routing table
// stays on the GPU): a per-64-token histogram, one scan workgroup per expert
// that turns the histograms into counts and per-block bases, a rank kernel that
// gives every (token, slot) its row (stable: ascending token order inside an
// expert, by ballot masks and popcount, no atomics on the result), and a copy
// kernel that writes each row of Xs from its source token with 16-byte loads
// and stores.  The combine and the gathers of the backward run one wave per
// token and sum in float32 in slot order.
#include "moe_common.h"
#include "mx_codec.h"
#include "hook.h"
#include "route.h"
#include "topk_dev.h"

namespace moe {

// ---------------------------------------------------------------------------
// softmax + top-k
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void topk_softmax_kernel(const float* __restrict__ logits, int T,
                                                           int E, int k, int renorm,
                                                           int32_t* __restrict__ topk_idx,
                                                           float* __restrict__ topk_w) {
  __shared__ __attribute__((aligned(16))) float row[4][64];
  __shared__ float ps[4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;
  if (E <= 64) {
    if (lane < E) row[wave][lane] = logits[(long)t * E + lane];
    __builtin_amdgcn_wave_barrier();
    topk_rank64(row[wave], E, k, renorm, lane, ps[wave], topk_idx + (long)t * k, topk_w + (long)t * k);
  } else {
    topk_row(logits + (long)t * E, E, k, renorm, lane, topk_idx + (long)t * k, topk_w + (long)t * k);
  }
}

// ---------------------------------------------------------------------------
// metadata: histogram per 64-token block, scan, rank
// ---------------------------------------------------------------------------
// hist[e][b]: rows of expert e among the (token, slot) pairs of block b.
__global__ __launch_bounds__(64) void block_hist_kernel(const int32_t* __restrict__ idx, int T,
                                                        int E, int k, int nblk,
                                                        int32_t* __restrict__ hist) {
  __shared__ int cnt[256];
  const int lane = threadIdx.x;
  for (int e = lane; e < E; e += 64) cnt[e] = 0;
  __syncthreads();
  const int t = blockIdx.x * 64 + lane;
  if (t < T)
    for (int j = 0; j < k; ++j) {
      int e = idx[(long)t * k + j];
      if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
    }
  __syncthreads();
  for (int e = lane; e < E; e += 64) hist[(long)e * nblk + blockIdx.x] = cnt[e];
}

// One workgroup per expert: exclusive scan of its block counts into
// base[e][b]; the total is counts[e].
__global__ __launch_bounds__(256) void scan_kernel(const int32_t* __restrict__ hist, int nblk,
                                                   int32_t* __restrict__ base,
                                                   int32_t* __restrict__ counts) {
  __shared__ int wsum[4];
  const int e = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int32_t* h = hist + (long)e * nblk;
  int32_t* bo = base + (long)e * nblk;
  int carry = 0;
  for (int b0 = 0; b0 < nblk; b0 += 256) {
    const int b = b0 + tid;
    const int c = (b < nblk) ? h[b] : 0;
    int incl = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      int v = __shfl_up(incl, o, 64);
      if (lane >= o) incl += v;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int wbase = 0;
    for (int w = 0; w < wave; ++w) wbase += wsum[w];
    const int total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
    if (b < nblk) bo[b] = carry + wbase + incl - c;
    carry += total;
    __syncthreads();
  }
  if (tid == 0) counts[e] = carry;
}

// Row of every (token, slot): offsets[e] + base[e][block] + rank of the token
// among the block's tokens routed to e.  The workgroup also forms offsets
// from counts (block 0 writes them out for the grouped GEMMs).
__global__ __launch_bounds__(64) void rank_kernel(const int32_t* __restrict__ idx, int T, int E,
                                                  int k, int nblk,
                                                  const int32_t* __restrict__ base,
                                                  const int32_t* __restrict__ counts,
                                                  int32_t* __restrict__ offsets,
                                                  int32_t* __restrict__ dest_row,
                                                  int32_t* __restrict__ src_token) {
  __shared__ unsigned long long mask[256];
  __shared__ int off[257];
  const int lane = threadIdx.x;
  {
    int c[4], sum = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      int e = lane * 4 + q;
      c[q] = (e < E) ? counts[e] : 0;
      sum += c[q];
    }
    int incl = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      int v = __shfl_up(incl, o, 64);
      if (lane >= o) incl += v;
    }
    int run = incl - sum;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      int e = lane * 4 + q;
      if (e <= E) off[e] = run;
      run += c[q];
    }
    if (lane == 63 && E == 256) off[256] = incl;
  }
  for (int e = lane; e < E; e += 64) mask[e] = 0ull;
  __syncthreads();
  if (blockIdx.x == 0)
    for (int e = lane; e <= E; e += 64) offsets[e] = off[e];
  const int t = blockIdx.x * 64 + lane;
  if (t < T)
    for (int j = 0; j < k; ++j) {
      int e = idx[(long)t * k + j];
      if (e >= 0 && e < E) atomicOr(&mask[e], 1ull << lane);
    }
  __syncthreads();
  if (t >= T) return;
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int j = 0; j < k; ++j) {
    int e = idx[(long)t * k + j];
    if (e < 0 || e >= E) { dest_row[(long)t * k + j] = -1; continue; }
    int r = off[e] + base[(long)e * nblk + blockIdx.x] + __popcll(mask[e] & below);
    dest_row[(long)t * k + j] = r;
    src_token[r] = t;
  }
}

// ---------------------------------------------------------------------------
// row copies
// ---------------------------------------------------------------------------
// Xs[r] = x[src_token[r]]: one wave per row, 8 elements per lane per step.
// ---------------------------------------------------------------------------
// row kernels: one wave per token.  A pass covers kPassCols columns, each lane
// kPassChunks chunks of 8 consecutive elements 512 columns apart.  A lane
// whose chunk lies past the row end reads the row's last chunk instead (in
// bounds, result discarded), so that every load of a pass is issued without
// a branch and the loads of two rows are in flight together.
// ---------------------------------------------------------------------------
constexpr int kPassChunks = 4;
constexpr int kPassCols = kPassChunks * 512;

__device__ __forceinline__ int clamp_row(int r, int R) { return min(max(r, 0), R - 1); }
__device__ __forceinline__ int chunk_col(int c0, int u, int d) { return min(c0 + 512 * u, d - 8); }

// 8 raw elements (one or two 16-byte words).
template <typename TS>
struct Raw8 {
  uint4 w[sizeof(TS) / 2];
  __device__ __forceinline__ void load_nt(const TS* p) {
#pragma unroll
    for (int i = 0; i < (int)(sizeof(TS) / 2); ++i) {
      const u32x4_t x = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p) + i);
      w[i] = uint4{x[0], x[1], x[2], x[3]};
    }
  }
  // Non-temporal stores: the dispatch copy measured 28% faster with them; the
  // combine backward's dYs rows measured slower and keep plain stores.
  __device__ __forceinline__ void store_nt(TS* p) const {
#pragma unroll
    for (int i = 0; i < (int)(sizeof(TS) / 2); ++i) {
      const u32x4_t x = {w[i].x, w[i].y, w[i].z, w[i].w};
      __builtin_nontemporal_store(x, reinterpret_cast<u32x4_t*>(p) + i);
    }
  }
};

// Xs[dest_row[t,j]] = x[t] for every slot j: each token row is read once and
// written k times.  Rows of Xs that no slot names are left as they are (the
// rank kernel makes dest_row a permutation of [0, T*k)).
template <typename TS>
__global__ __launch_bounds__(256) void dispatch_scatter_kernel(const TS* __restrict__ x,
                                                               const int32_t* __restrict__ dest_row,
                                                               int T, int d, int k,
                                                               TS* __restrict__ Xs) {
  const int lane = threadIdx.x & 63;
  const long t = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int R = T * k;
  for (int c0 = lane * 8; c0 < d; c0 += kPassCols) {
    Raw8<TS> v[kPassChunks];
#pragma unroll
    for (int u = 0; u < kPassChunks; ++u) v[u].load_nt(x + t * d + chunk_col(c0, u, d));
    for (int j = 0; j < k; ++j) {
      const int r = dest_row[t * k + j];
      if (r < 0 || r >= R) continue;
#pragma unroll
      for (int u = 0; u < kPassChunks; ++u)
        if (c0 + 512 * u < d) v[u].store_nt(Xs + (long)r * d + c0 + 512 * u);
    }
  }
}

// 8 elements as floats through a non-temporal 16-byte load (rows read once:
// measured 10-20% faster for the gathers than plain loads).
__device__ __forceinline__ void load8_nt(const bf16_t* p, float (&v)[8]) {
  const u32x4_t u = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  unpack8(uint4{u[0], u[1], u[2], u[3]}, v);
}
__device__ __forceinline__ void load8_nt(const float* p, float (&v)[8]) {
  const f32x4_t a = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
  const f32x4_t b = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p + 4));
  v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
  v[4] = b[0]; v[5] = b[1]; v[6] = b[2]; v[7] = b[3];
}

// y[t] = sum_j w[t,j] Ys[dest_row[t,j]], in float32 in slot order.
// dXs gather (W == false): dx[t] (+)= sum_j dXs[dest_row[t,j]].
// A slot whose row lies outside [0, R) (the rank kernel marks a slot with an
// expert index outside [0, E) by -1) adds nothing; its load still goes to a
// clamped row so that every load of a pass is issued without a branch.
template <typename TS, bool W>
__device__ __forceinline__ void gather_rows(const TS* __restrict__ src, const float* __restrict__ w,
                                            const int32_t* __restrict__ dest_row, long t, int T,
                                            int d, int k, int accumulate, TS* __restrict__ out,
                                            int lane) {
  const int R = T * k;
  const int32_t* dr = dest_row + t * k;
  for (int c0 = lane * 8; c0 < d; c0 += kPassCols) {
    float acc[kPassChunks][8];
#pragma unroll
    for (int u = 0; u < kPassChunks; ++u)
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[u][q] = 0.0f;
    auto add = [&](const float (&v)[kPassChunks][8], float wj) {
#pragma unroll
      for (int u = 0; u < kPassChunks; ++u)
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[u][q] = W ? fmaf(wj, v[u][q], acc[u][q]) : acc[u][q] + v[u][q];
    };
    int j = 0;
    for (; j + 2 <= k; j += 2) {
      const TS* p0 = src + (long)clamp_row(dr[j], R) * d;
      const TS* p1 = src + (long)clamp_row(dr[j + 1], R) * d;
      float v0[kPassChunks][8], v1[kPassChunks][8];
#pragma unroll
      for (int u = 0; u < kPassChunks; ++u) load8_nt(p0 + chunk_col(c0, u, d), v0[u]);
#pragma unroll
      for (int u = 0; u < kPassChunks; ++u) load8_nt(p1 + chunk_col(c0, u, d), v1[u]);
      if ((unsigned)dr[j] < (unsigned)R) add(v0, W ? w[t * k + j] : 1.0f);
      if ((unsigned)dr[j + 1] < (unsigned)R) add(v1, W ? w[t * k + j + 1] : 1.0f);
    }
    if (j < k) {
      const TS* p0 = src + (long)clamp_row(dr[j], R) * d;
      float v0[kPassChunks][8];
#pragma unroll
      for (int u = 0; u < kPassChunks; ++u) load8_nt(p0 + chunk_col(c0, u, d), v0[u]);
      if ((unsigned)dr[j] < (unsigned)R) add(v0, W ? w[t * k + j] : 1.0f);
    }
#pragma unroll
    for (int u = 0; u < kPassChunks; ++u) {
      const int c = c0 + 512 * u;
      if (c < d) {
        if (accumulate) {
          float o[8];
          load8(out + t * d + c, o);
#pragma unroll
          for (int q = 0; q < 8; ++q) acc[u][q] += o[q];
        }
        store8(out + t * d + c, acc[u]);
      }
    }
  }
}

template <typename TS>
__global__ __launch_bounds__(256) void combine_kernel(const TS* __restrict__ Ys,
                                                      const float* __restrict__ w,
                                                      const int32_t* __restrict__ dest_row, int T,
                                                      int d, int k, TS* __restrict__ y) {
  const long t = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  gather_rows<TS, true>(Ys, w, dest_row, t, T, d, k, 0, y, threadIdx.x & 63);
}

template <typename TS>
__global__ __launch_bounds__(256) void gather_sum_kernel(const TS* __restrict__ dXs,
                                                         const int32_t* __restrict__ dest_row,
                                                         int T, int d, int k, int accumulate,
                                                         TS* __restrict__ dx) {
  const long t = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  gather_rows<TS, false>(dXs, nullptr, dest_row, t, T, d, k, accumulate, dx, threadIdx.x & 63);
}

// dYs[dest] = w * dY[t]; dw[t,j] = <dY[t], Ys[dest]>.  Each lane sums its
// products in column order, then the wave sums the lanes.  A slot whose row
// lies outside [0, R) stores no dYs row and gets dw = 0.
template <typename TS, bool MXQ>
__device__ __forceinline__ void combine_bwd_slot(const float (&g)[8], const float (&v)[8], float wj,
                                                 long r, int c, TS* __restrict__ dYs,
                                                 uint8_t* __restrict__ q, uint8_t* __restrict__ qs,
                                                 long pitch, int d, int lane, float& dot) {
  float o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    dot = fmaf(g[i], v[i], dot);
    o[i] = wj * g[i];
  }
  store8(dYs + r * d + c, o);
  if constexpr (MXQ) {
    // the stored (bf16) row, block-quantised along d for the down dgrad
    float ro[8];
    round_bf16_8(o, ro);
    quant8_store(ro, q + r * d + c, qs + mx_scale_at(r, c, pitch), lane);
  }
}

template <typename TS, bool MXQ>
__global__ __launch_bounds__(256) void combine_bwd_kernel(const TS* __restrict__ dY,
                                                          const TS* __restrict__ Ys,
                                                          const float* __restrict__ w,
                                                          const int32_t* __restrict__ dest_row,
                                                          int T, int d, int k,
                                                          TS* __restrict__ dYs,
                                                          float* __restrict__ dw,
                                                          uint8_t* __restrict__ q,
                                                          uint8_t* __restrict__ qs, long pitch) {
  const int lane = threadIdx.x & 63;
  const long t = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int R = T * k;
  if (d <= kPassCols) {
    // one pass: the dY row stays in registers and two slots' rows are read together
    const int c0 = lane * 8;
    float g[kPassChunks][8];
#pragma unroll
    for (int u = 0; u < kPassChunks; ++u) load8(dY + t * d + chunk_col(c0, u, d), g[u]);
    int j = 0;
    auto slot = [&](int jj, const float (&v)[kPassChunks][8]) {
      const int rr = dest_row[t * k + jj];
      if ((unsigned)rr >= (unsigned)R) {
        if (lane == 0) dw[t * k + jj] = 0.0f;
        return;
      }
      const long r = rr;
      const float wj = w[t * k + jj];
      float dot = 0.0f;
#pragma unroll
      for (int u = 0; u < kPassChunks; ++u)
        if (c0 + 512 * u < d)
          combine_bwd_slot<TS, MXQ>(g[u], v[u], wj, r, c0 + 512 * u, dYs, q, qs, pitch, d, lane, dot);
      dot = wave_sum(dot);
      if (lane == 0) dw[t * k + jj] = dot;
    };
    for (; j + 2 <= k; j += 2) {
      const TS* p0 = Ys + (long)clamp_row(dest_row[t * k + j], R) * d;
      const TS* p1 = Ys + (long)clamp_row(dest_row[t * k + j + 1], R) * d;
      float v0[kPassChunks][8], v1[kPassChunks][8];
#pragma unroll
      for (int u = 0; u < kPassChunks; ++u) load8_nt(p0 + chunk_col(c0, u, d), v0[u]);
#pragma unroll
      for (int u = 0; u < kPassChunks; ++u) load8_nt(p1 + chunk_col(c0, u, d), v1[u]);
      slot(j, v0);
      slot(j + 1, v1);
    }
    if (j < k) {
      const TS* p0 = Ys + (long)clamp_row(dest_row[t * k + j], R) * d;
      float v0[kPassChunks][8];
#pragma unroll
      for (int u = 0; u < kPassChunks; ++u) load8_nt(p0 + chunk_col(c0, u, d), v0[u]);
      slot(j, v0);
    }
    return;
  }
  for (int j = 0; j < k; ++j) {
    const int rr = dest_row[t * k + j];
    if ((unsigned)rr >= (unsigned)R) {
      if (lane == 0) dw[t * k + j] = 0.0f;
      continue;
    }
    const long r = rr;
    const float wj = w[t * k + j];
    float dot = 0.0f;
    for (int c = lane * 8; c < d; c += 64 * 8) {
      float g[8], v[8];
      load8(dY + t * d + c, g);
      load8_nt(Ys + r * d + c, v);
      combine_bwd_slot<TS, MXQ>(g, v, wj, r, c, dYs, q, qs, pitch, d, lane, dot);
    }
    dot = wave_sum(dot);
    if (lane == 0) dw[t * k + j] = dot;
  }
}

// Router backward, softmax part: dl = p * (dp - <p, dp>), one wave per token.
// Also writes dl rounded to bf16 when dl16 is given (GEMM operand), as rows
// of ld16 >= E entries whose tail is zero.
__global__ __launch_bounds__(256) void router_bwd_softmax_kernel(
    const float* __restrict__ logits, const int32_t* __restrict__ idx,
    const float* __restrict__ dw, int T, int E, int k, int renorm,
    const float* __restrict__ aux_dp, float* __restrict__ dl, bf16_t* __restrict__ dl16,
    int ld16) {
  const int lane = threadIdx.x & 63;
  const long t = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* row = logits + t * E;
  float v[4], dp[4];
  float mx = -INFINITY;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    int e = lane + 64 * q;
    v[q] = (e < E) ? row[e] : -INFINITY;
    if (e < E) mx = fmaxf(mx, v[q]);
    dp[q] = 0.0f;
  }
  mx = wave_max(mx);
  float se = 0.0f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    int e = lane + 64 * q;
    v[q] = (e < E) ? expf(v[q] - mx) : 0.0f;
    se += v[q];
  }
  se = wave_sum(se);
#pragma unroll
  for (int q = 0; q < 4; ++q) v[q] = v[q] / se;  // p
  float S = 1.0f, wdot = 0.0f;
  if (renorm) {
    // w_j = p_j / S over the chosen experts: dp_m = (dw_m - sum_j dw_j w_j) / S
    float ps = 0.0f, pd = 0.0f;
    for (int j = 0; j < k; ++j) {
      const int e = idx[t * k + j];
      if (e >= 0 && e < E && (e & 63) == lane) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if ((e >> 6) == q) { ps += v[q]; pd = fmaf(dw[t * k + j], v[q], pd); }
      }
    }
    S = wave_sum(ps);
    wdot = wave_sum(pd) / S;
  }
  for (int j = 0; j < k; ++j) {
    int e = idx[t * k + j];
    float g = renorm ? (dw[t * k + j] - wdot) / S : dw[t * k + j];
    if (e >= 0 && e < E && (e & 63) == lane) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if ((e >> 6) == q) dp[q] = g;
    }
  }
  if (aux_dp) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane + 64 * q;
      if (e < E) dp[q] += aux_dp[e];
    }
  }
  float inner = 0.0f;
#pragma unroll
  for (int q = 0; q < 4; ++q) inner = fmaf(v[q], dp[q], inner);
  inner = wave_sum(inner);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    int e = lane + 64 * q;
    if (e < E) {
      float g = v[q] * (dp[q] - inner);
      dl[t * E + e] = g;
      if (dl16) dl16[t * ld16 + e] = f32_to_bf16(g);
    } else if (dl16 && e < ld16) {
      dl16[t * ld16 + e] = 0;
    }
  }
}

// ---------------------------------------------------------------------------
// load-balancing loss: per-expert mean router probability P_e (partial sums
// per block of 64 tokens, then an ordered sum over blocks), then
// L = coef * E * sum_e f_e P_e with f_e = counts[e] / T (the fraction of
// tokens that route a slot to e; the per-slot frequencies summed), and its gradient
// with respect to every token's probabilities, coef * E * f_e / T.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void aux_partial_kernel(const float* __restrict__ logits, int T,
                                                          int E, float* __restrict__ part) {
  __shared__ float acc[4][256];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float s[4] = {0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < 16; ++i) {
    const long t = (long)blockIdx.x * 64 + wave * 16 + i;
    if (t >= T) break;
    const float* row = logits + t * E;
    float v[4], mx = -INFINITY;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane + 64 * q;
      v[q] = (e < E) ? row[e] : -INFINITY;
      mx = fmaxf(mx, v[q]);
    }
    mx = wave_max(mx);
    float se = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[q] = (lane + 64 * q < E) ? expf(v[q] - mx) : 0.0f;
      se += v[q];
    }
    se = wave_sum(se);
#pragma unroll
    for (int q = 0; q < 4; ++q) s[q] += v[q] / se;
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) acc[wave][lane + 64 * q] = s[q];
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256)
    part[(long)blockIdx.x * E + e] = ((acc[0][e] + acc[1][e]) + acc[2][e]) + acc[3][e];
}

__global__ __launch_bounds__(256) void aux_final_kernel(const float* __restrict__ part, int nblk,
                                                        const int32_t* __restrict__ counts, int T,
                                                        int E, int k, float coef,
                                                        float* __restrict__ loss,
                                                        float* __restrict__ dp) {
  __shared__ float contrib[256];
  const int e = threadIdx.x;
  float term = 0.0f;
  if (e < E) {
    float P = 0.0f;
    for (int b = 0; b < nblk; ++b) P += part[(long)b * E + e];
    P /= (float)T;
    const float f = (float)counts[e] / (float)T;
    term = f * P;
    dp[e] = coef * (float)E * f / (float)T;
  }
  contrib[e] = term;
  __syncthreads();
  if (e == 0) {
    float sum = 0.0f;
    for (int i = 0; i < E; ++i) sum += contrib[i];
    *loss = coef * (float)E * sum;
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
#define MOE_LAUNCH_CHECK() \
  do {                     \
    hipError_t e_ = hipGetLastError(); if (e_ != hipSuccess) return e_; \
  } while (0)

hipError_t launch_topk_softmax(const float* logits, int T, int E, int k, int renorm, int32_t* idx,
                               float* w, hipStream_t s) {
  if (T == 0) return hipSuccess;
  note_prelaunch("topk_softmax", s);
  hipLaunchKernelGGL(topk_softmax_kernel, dim3((T + 3) / 4), dim3(256), 0, s, logits, T, E, k,
                     renorm, idx, w);
  note_launch("topk_softmax", s);
  return hipGetLastError();
}

hipError_t launch_dispatch_meta(const int32_t* idx, int T, int E, int k, int32_t* hist,
                                int32_t* base, int32_t* counts, int32_t* offsets,
                                int32_t* dest_row, int32_t* src_token, hipStream_t s) {
  const int nblk = (T + 63) / 64;
  note_prelaunch("block_hist", s);
  hipLaunchKernelGGL(block_hist_kernel, dim3(nblk), dim3(64), 0, s, idx, T, E, k, nblk, hist);
  note_launch("block_hist", s);
  MOE_LAUNCH_CHECK();
  note_prelaunch("expert_scan", s);
  hipLaunchKernelGGL(scan_kernel, dim3(E), dim3(256), 0, s, hist, nblk, base, counts);
  note_launch("expert_scan", s);
  MOE_LAUNCH_CHECK();
  note_prelaunch("rank", s);
  hipLaunchKernelGGL(rank_kernel, dim3(nblk), dim3(64), 0, s, idx, T, E, k, nblk, base, counts,
                     offsets, dest_row, src_token);
  note_launch("rank", s);
  return hipGetLastError();
}

template <typename TS>
static hipError_t copy_impl(const void* x, const int32_t* dest, int T, int d, int k, void* Xs,
                            hipStream_t s) {
  note_prelaunch("dispatch_copy", s);
  hipLaunchKernelGGL(dispatch_scatter_kernel<TS>, dim3((T + 3) / 4), dim3(256), 0, s,
                     static_cast<const TS*>(x), dest, T, d, k, static_cast<TS*>(Xs));
  note_launch("dispatch_copy", s);
  return hipGetLastError();
}

hipError_t launch_dispatch_copy(int dtype, const void* x, const int32_t* dest_row, int T, int d,
                                int k, void* Xs, hipStream_t s) {
  if (T == 0) return hipSuccess;
  return dtype ? copy_impl<bf16_t>(x, dest_row, T, d, k, Xs, s)
               : copy_impl<float>(x, dest_row, T, d, k, Xs, s);
}

hipError_t launch_combine(int dtype, const void* Ys, const float* w, const int32_t* dest, int T,
                          int d, int k, void* y, hipStream_t s) {
  dim3 grid((T + 3) / 4);
  note_prelaunch("combine", s);
  if (dtype)
    hipLaunchKernelGGL(combine_kernel<bf16_t>, grid, dim3(256), 0, s,
                       static_cast<const bf16_t*>(Ys), w, dest, T, d, k, static_cast<bf16_t*>(y));
  else
    hipLaunchKernelGGL(combine_kernel<float>, grid, dim3(256), 0, s,
                       static_cast<const float*>(Ys), w, dest, T, d, k, static_cast<float*>(y));
  note_launch("combine", s);
  return hipGetLastError();
}

hipError_t launch_combine_bwd(int dtype, const void* dY, const void* Ys, const float* w,
                              const int32_t* dest, int T, int d, int k, void* dYs, float* dw,
                              void* dYs_q, uint8_t* dYs_q_scale, hipStream_t s) {
  dim3 grid((T + 3) / 4);
  const long pitch = ((long)T * k + 15) / 16 * 16;
  note_prelaunch("combine_bwd", s);
  if (dtype && dYs_q)
    hipLaunchKernelGGL((combine_bwd_kernel<bf16_t, true>), grid, dim3(256), 0, s,
                       static_cast<const bf16_t*>(dY), static_cast<const bf16_t*>(Ys), w, dest,
                       T, d, k, static_cast<bf16_t*>(dYs), dw, static_cast<uint8_t*>(dYs_q),
                       dYs_q_scale, pitch);
  else if (dtype)
    hipLaunchKernelGGL((combine_bwd_kernel<bf16_t, false>), grid, dim3(256), 0, s,
                       static_cast<const bf16_t*>(dY), static_cast<const bf16_t*>(Ys), w, dest,
                       T, d, k, static_cast<bf16_t*>(dYs), dw, nullptr, nullptr, 0L);
  else
    hipLaunchKernelGGL((combine_bwd_kernel<float, false>), grid, dim3(256), 0, s,
                       static_cast<const float*>(dY), static_cast<const float*>(Ys), w, dest, T,
                       d, k, static_cast<float*>(dYs), dw, nullptr, nullptr, 0L);
  note_launch("combine_bwd", s);
  return hipGetLastError();
}

// out[i] (+)= sum over s of part[s][i], in order of s; each thread four
// consecutive outputs with eight partials in flight (16-byte loads: n is a
// multiple of 4, as d * E is).
template <typename TS>
__global__ __launch_bounds__(64) void split_reduce_kernel(const float* __restrict__ part, int S,
                                                          long n, int accumulate,
                                                          TS* __restrict__ out) {
  const long i = ((long)blockIdx.x * 64 + threadIdx.x) * 4;
  if (i >= n) return;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  if (accumulate)
    for (int q = 0; q < 4; ++q) acc[q] = (i + q < n) ? St<TS>::load(out + i + q) : 0.f;
  if (i + 4 <= n) {
    const float* p = part + i;
    int s = 0;
    for (; s + 8 <= S; s += 8) {
      float4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = *reinterpret_cast<const float4*>(p + (long)(s + u) * n);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        acc[0] += v[u].x; acc[1] += v[u].y; acc[2] += v[u].z; acc[3] += v[u].w;
      }
    }
    for (; s < S; ++s) {
      const float4 v = *reinterpret_cast<const float4*>(p + (long)s * n);
      acc[0] += v.x; acc[1] += v.y; acc[2] += v.z; acc[3] += v.w;
    }
  } else {
    for (int s = 0; s < S; ++s)
      for (int q = 0; q < 4 && i + q < n; ++q) acc[q] += part[(long)s * n + i + q];
  }
  for (int q = 0; q < 4 && i + q < n; ++q) St<TS>::store(out + i + q, acc[q]);
}

hipError_t launch_split_reduce(int dtype, const float* part, int S, long n, int accumulate,
                               void* out, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const dim3 grid((unsigned)((n + 255) / 256));
  note_prelaunch("router_dwr_reduce", s);
  if (dtype)
    hipLaunchKernelGGL(split_reduce_kernel<bf16_t>, grid, dim3(64), 0, s, part, S, n, accumulate,
                       static_cast<bf16_t*>(out));
  else
    hipLaunchKernelGGL(split_reduce_kernel<float>, grid, dim3(64), 0, s, part, S, n, accumulate,
                       static_cast<float*>(out));
  note_launch("router_dwr_reduce", s);
  return hipGetLastError();
}

hipError_t launch_gather_sum(int dtype, const void* dXs, const int32_t* dest, int T, int d, int k,
                             int accumulate, void* dx, hipStream_t s) {
  dim3 grid((T + 3) / 4);
  note_prelaunch("gather_sum", s);
  if (dtype)
    hipLaunchKernelGGL(gather_sum_kernel<bf16_t>, grid, dim3(256), 0, s,
                       static_cast<const bf16_t*>(dXs), dest, T, d, k, accumulate,
                       static_cast<bf16_t*>(dx));
  else
    hipLaunchKernelGGL(gather_sum_kernel<float>, grid, dim3(256), 0, s,
                       static_cast<const float*>(dXs), dest, T, d, k, accumulate,
                       static_cast<float*>(dx));
  note_launch("gather_sum", s);
  return hipGetLastError();
}

hipError_t launch_router_bwd_softmax(const float* logits, const int32_t* idx, const float* dw,
                                     int T, int E, int k, int renorm, const float* aux_dp,
                                     float* dl, bf16_t* dl16, int ld16, hipStream_t s) {
  note_prelaunch("router_bwd_softmax", s);
  hipLaunchKernelGGL(router_bwd_softmax_kernel, dim3((T + 3) / 4), dim3(256), 0, s, logits, idx,
                     dw, T, E, k, renorm, aux_dp, dl, dl16, ld16);
  note_launch("router_bwd_softmax", s);
  return hipGetLastError();
}

}  // namespace moe

namespace moe {

// ---------------------------------------------------------------------------
// routing check: pre-routed expert indices outside [0, E) and tokens whose
// experts repeat (one thread per token, a 256-bit set of the experts seen)
// ---------------------------------------------------------------------------
__global__ void check_init_kernel(int32_t* __restrict__ report) {
  report[0] = 0;
  report[1] = 0;
}

__global__ __launch_bounds__(256) void check_routing_kernel(const int32_t* __restrict__ idx, int T,
                                                            int E, int k,
                                                            int32_t* __restrict__ report) {
  int bad = 0, dup = 0;
  for (long t = (long)blockIdx.x * 256 + threadIdx.x; t < T; t += (long)gridDim.x * 256) {
    uint32_t seen[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    bool rep = false;
    for (int j = 0; j < k; ++j) {
      const int e = idx[t * k + j];
      if (e < 0 || e >= E) {
        ++bad;
        continue;
      }
      const uint32_t bit = 1u << (e & 31);
#pragma unroll
      for (int w = 0; w < 8; ++w)
        if (w == (e >> 5)) {
          rep = rep || (seen[w] & bit) != 0;
          seen[w] |= bit;
        }
    }
    dup += rep ? 1 : 0;
  }
  const float b = wave_sum((float)bad), d = wave_sum((float)dup);
  if ((threadIdx.x & 63) == 0) {
    if (b > 0.0f) atomicAdd(&report[0], (int)b);
    if (d > 0.0f) atomicAdd(&report[1], (int)d);
  }
}

hipError_t launch_check_routing(const int32_t* idx, int T, int E, int k, int32_t* report,
                                hipStream_t s) {
  note_prelaunch("check_init", s);
  hipLaunchKernelGGL(check_init_kernel, dim3(1), dim3(1), 0, s, report);
  note_launch("check_init", s);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  const long nb = ((long)T + 255) / 256;
  note_prelaunch("check_routing", s);
  hipLaunchKernelGGL(check_routing_kernel, dim3((unsigned)(nb < 1024 ? nb : 1024)), dim3(256), 0, s,
                     idx, T, E, k, report);
  note_launch("check_routing", s);
  return hipGetLastError();
}

hipError_t launch_router_aux(const float* logits, const int32_t* counts, int T, int E, int k,
                             float coef, float* part, float* loss, float* dp, hipStream_t s) {
  const int nblk = (T + 63) / 64;
  note_prelaunch("router_aux_partial", s);
  hipLaunchKernelGGL(aux_partial_kernel, dim3(nblk), dim3(256), 0, s, logits, T, E, part);
  note_launch("router_aux_partial", s);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  note_prelaunch("router_aux_final", s);
  hipLaunchKernelGGL(aux_final_kernel, dim3(1), dim3(256), 0, s, part, nblk, counts, T, E, k, coef,
                     loss, dp);
  note_launch("router_aux_final", s);
  return hipGetLastError();
}

}  // namespace moe
