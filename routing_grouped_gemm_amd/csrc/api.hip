// C ABI of the MoE expert layer: host-side validation, workspace carving and
// launch order.  Declarations and argument meanings: include/moe.h.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <mutex>

#include "../../include/moe.h"
#include "gemm.h"
#include "mx.h"
#include "route.h"
#include "skinny.h"

using namespace moe;

namespace {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t v) { return (v + kAlign - 1) & ~(kAlign - 1); }

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int num_cu() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

thread_local hipError_t g_last_launch_error = hipSuccess;

inline int status_of(hipError_t e) {
  if (e == hipSuccess) return MOE_OK;
  g_last_launch_error = e;
  return MOE_ERR_LAUNCH;
}

#define MOE_TRY(expr)                                    \
  do {                                                   \
    hipError_t e_ = (expr);                              \
    if (e_ != hipSuccess) return status_of(e_);          \
  } while (0)

// hipGetLastError reports the last error of any earlier runtime call on this
// thread (for example a not-ready event query made by another library);
// every entry point clears it once its arguments are valid, so that the
// check after each of its own launches sees only that launch.
inline void clear_stale_error() { (void)hipGetLastError(); }

inline int check_dtype(int dtype) { return (dtype == MOE_F32 || dtype == MOE_BF16) ? MOE_OK : MOE_ERR_DTYPE; }

inline int check_prec(int dtype, int prec) {
  if (check_dtype(dtype) != MOE_OK) return MOE_ERR_DTYPE;
  if (prec == MOE_PREC_F32) return dtype == MOE_F32 ? MOE_OK : MOE_ERR_DTYPE;
  if (prec == MOE_PREC_BF16) return dtype == MOE_BF16 ? MOE_OK : MOE_ERR_DTYPE;
  if (prec == MOE_PREC_MXFP8) return dtype == MOE_BF16 ? MOE_OK : MOE_ERR_DTYPE;
  return MOE_ERR_DTYPE;
}

// T, k, E shape rules shared by the routed entry points.
inline int check_route_shape(int T, int E, int k) {
  if (T <= 0 || E <= 0 || k <= 0) return MOE_ERR_SHAPE;
  if ((long long)T * k > 0x7fffffffLL) return MOE_ERR_SHAPE;
  if (E > 256 || k > E) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

inline int check_width(int v) {
  if (v <= 0) return MOE_ERR_SHAPE;
  return (v % 64) ? MOE_ERR_UNSUPPORTED : MOE_OK;
}

// Element counts of the largest tensors must stay below 2^31 * 2^31; row
// indices are int32, element offsets are 64-bit.
inline int check_elems(long long rows, long long cols) {
  return (rows * cols > (1LL << 46)) ? MOE_ERR_SHAPE : MOE_OK;
}

// The GEMM engines address their operands through buffer resources with
// 32-bit byte offsets from a per-tile or per-expert base.  A larger problem
// is refused (MOE_ERR_UNSUPPORTED) instead of wrapping:
//  * one expert's weight matrix, gate/up panels padded to 128 columns
//    included: d * (f + 128) * 2 bytes below 2^32;
//  * the bf16 weight gradients stream one expert's rows of Xs [n_e][d],
//    A [n_e][f], dH [n_e][2f] and dYs [n_e][d] along K = n_e from one base:
//    R * max(d, 2f) * 2 bytes below 2^32 (n_e <= R);
//  * the MXFP8 weight gradients read codes [features][Kp] (Kp = R padded per
//    expert): 256 rows of a tile span 256 * Kp bytes, below 2^32;
//  * every MXFP8 scale array a GEMM reads through one resource stays below
//    2^30 bytes (offsets past it mark lanes and loads that read nothing):
//    the token-quantised scales (Kp / 32) * max(d, 2f), the activation
//    scales ceil(max(d, 2f) / 128) * 4 * Rp (Rp = R rounded up to 16).
constexpr long long kOff32 = 1LL << 32;
constexpr long long kScaleRange = 1LL << 30;
inline int check_weight_offsets(int d, int f) {
  return ((long long)d * (f + 128) * 2 >= kOff32) ? MOE_ERR_UNSUPPORTED : MOE_OK;
}
inline int check_wgrad_offsets(long long R, int d, int f) {
  const long long w = d > 2LL * f ? d : 2LL * f;
  return (R * w * 2 >= kOff32) ? MOE_ERR_UNSUPPORTED : MOE_OK;
}
inline int check_mx_wgrad_offsets(long long R, int d, int f, int E) {
  const long long kp = (R + 127LL * E + 127) / 128 * 128;
  const long long w = d > 2LL * f ? d : 2LL * f;
  return (256 * kp >= kOff32 || (kp / 32) * w >= kScaleRange) ? MOE_ERR_UNSUPPORTED : MOE_OK;
}
inline int check_mx_scale_offsets(long long R, int d, int f) {
  const long long w = d > 2LL * f ? d : 2LL * f;
  const long long rp = (R + 15) / 16 * 16;
  return ((w + 127) / 128 * 4 * rp >= kScaleRange) ? MOE_ERR_UNSUPPORTED : MOE_OK;
}

template <typename... P>
inline bool all_nonnull(P... p) { return ((p != nullptr) && ...); }
template <typename... P>
inline bool all_aligned(P... p) { return ((p == nullptr || aligned16(p)) && ...); }

inline size_t dispatch_ws(int T, int E) {
  const size_t nblk = (size_t)(T + 63) / 64;
  return 2 * align_up(nblk * (size_t)E * sizeof(int32_t));
}

// Width of the bf16 copy of dlogits: E rounded up to the MFMA engine's K step.
inline int router_ld16(int E) { return (E + 63) / 64 * 64; }

// Router weight gradient on the MFMA engine: K = T is split into chunks of
// at least 256 tokens (at most 64 chunks) whose float32 partials
// [S][d][E] are summed in chunk order.
inline int router_splits(int T) {
  const int s = (T + 255) / 256;
  return s < 1 ? 1 : (s > 64 ? 64 : s);
}
inline size_t route_bwd_ws(int T, int d, int E, int dtype) {
  if (dtype != MOE_BF16) return 0;
  size_t n = align_up((size_t)T * router_ld16(E) * 2);
  if (E % 8 == 0) n += align_up((size_t)router_splits(T) * d * E * 4);
  return n;
}

inline int gemm_engine(int dtype, int router_E = 8) {
  if (dtype == MOE_F32) return GEMM_F32_SIMT;
  return (router_E % 8 == 0) ? GEMM_BF16_MFMA : GEMM_BF16_SIMT;
}

}  // namespace

extern "C" {

const char* moe_last_launch_error(void) {
  return g_last_launch_error == hipSuccess ? "none" : hipGetErrorName(g_last_launch_error);
}

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "a required pointer is NULL";
    case MOE_ERR_SHAPE: return "invalid shape (non-positive size or int32 overflow)";
    case MOE_ERR_DTYPE: return "unknown dtype/precision or invalid dtype/precision pair";
    case MOE_ERR_ALIGN: return "pointer not 16-byte aligned";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_UNSUPPORTED:
      return "unsupported shape (E > 256, k > E, d/f not a multiple of 64, or an operand beyond "
             "the GEMM engines' 32-bit offsets)";
    case MOE_ERR_LAUNCH: return "HIP kernel launch failed";
    case MOE_ERR_SCRATCH:
      return "problem larger than the static scratch of a no-allocation entry point";
  }
  return "unknown status";
}

int moe_workspace_size(int op, int T, int d, int E, int f, int k, int dtype, int prec,
                       size_t* bytes) {
  if (!bytes) return MOE_ERR_NULL;
  *bytes = 0;
  if (T <= 0 || d <= 0 || E <= 0 || f <= 0 || k <= 0) return MOE_ERR_SHAPE;
  if (int s = check_prec(dtype, prec)) return s;
  const size_t R = (size_t)T * k;
  switch (op) {
    case MOE_OP_ROUTE:
      if (dtype == MOE_BF16 && route_small_applies(T, d, E))
        *bytes = align_up(route_small_workspace(T, d, E));
      return MOE_OK;
    case MOE_OP_COMBINE:
    case MOE_OP_COMBINE_BWD:
    case MOE_OP_DISPATCH_BWD:
      return MOE_OK;
    case MOE_OP_DISPATCH:
      *bytes = dispatch_ws(T, E);
      return MOE_OK;
    case MOE_OP_FFN_FWD:
      if (prec == MOE_PREC_MXFP8)
        *bytes = mx_fwd_workspace(R, d, f, E);
      else if (prec == MOE_PREC_BF16 && R <= (size_t)kSkinnyMaxRows)
        *bytes = align_up(skinny_workspace((int)R, E, d, f));
      return MOE_OK;
    case MOE_OP_FFN_BWD:
      *bytes = (prec == MOE_PREC_MXFP8) ? mx_bwd_workspace(R, d, f, E) : 0;
      return MOE_OK;
    case MOE_OP_ROUTE_BWD:
      *bytes = route_bwd_ws(T, d, E, dtype);
      return MOE_OK;
    case MOE_OP_ROUTE_AUX:
      *bytes = align_up((size_t)((T + 63) / 64) * E * sizeof(float));
      return MOE_OK;
    case MOE_OP_FFN_BWD_MXW:
      if (prec != MOE_PREC_MXFP8) return MOE_ERR_DTYPE;
      *bytes = mx_wgrad_workspace(R, d, f, E);
      return MOE_OK;
    case MOE_OP_FFN_FWD_KEEP:
      if (prec != MOE_PREC_MXFP8) return MOE_ERR_DTYPE;
      *bytes = mx_fwd_workspace(R, d, f, E, true);
      return MOE_OK;
  }
  return MOE_ERR_SHAPE;
}

int moe_route(const void* x, const void* Wr, int T, int d, int E, int k, int dtype,
              unsigned flags, float* logits, int32_t* topk_idx, float* topk_w, void* ws,
              size_t ws_bytes, void* stream) {
  const bool lin = (flags & MOE_ROUTE_LOGITS_IN) != 0;
  if (!all_nonnull(logits, topk_idx, topk_w)) return MOE_ERR_NULL;
  if (!lin && !all_nonnull(x, Wr)) return MOE_ERR_NULL;
  if (int s = check_dtype(dtype)) return s;
  if (int s = check_route_shape(T, E, k)) return s;
  if (!lin) {
    if (int s = check_width(d)) return s;
    if (int s = check_elems(T, d)) return s;
  }
  if (!all_aligned(x, Wr, logits, topk_idx, topk_w, ws)) return MOE_ERR_ALIGN;
  hipStream_t st = static_cast<hipStream_t>(stream);
  clear_stale_error();
  const int renorm = (flags & MOE_ROUTE_RENORM) ? 1 : 0;
  if (!lin && dtype == MOE_BF16 && route_small_applies(T, d, E) && ws &&
      ws_bytes >= route_small_workspace(T, d, E))
    return status_of(launch_route_small(static_cast<const uint16_t*>(x),
                                        static_cast<const uint16_t*>(Wr), T, d, E, k, renorm,
                                        static_cast<float*>(ws), logits, topk_idx, topk_w, st));
  if (!lin && dtype == MOE_BF16 && router_logits_applies(d, E)) {
    MOE_TRY(launch_router_logits(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(Wr),
                                 T, d, E, logits, st));
  } else if (!lin) {
    GemmArgs g{};
    g.E = 1; g.offsets = nullptr; g.rows_total = T; g.ragged = RAG_M;
    g.M = T; g.N = E; g.K = d;
    g.a = x; g.lda = d;
    g.b0 = Wr; g.ldb = E;
    g.c0 = logits; g.ldc = E;
    MOE_TRY(launch_grouped_gemm(GK_ROUTER_LOGITS, gemm_engine(dtype, E), g, num_cu(), st));
  }
  return status_of(launch_topk_softmax(logits, T, E, k, renorm, topk_idx, topk_w, st));
}

}  // extern "C"

namespace {

// moe_dispatch's validation and launches; ws is device memory of ws_bytes.
int dispatch_impl(const void* x, const int32_t* topk_idx, int T, int d, int E, int k, int dtype,
                  int prec, int32_t* counts, int32_t* offsets, int32_t* dest_row,
                  int32_t* src_token, void* Xs, void* Xq, uint8_t* Xq_scale, void* ws,
                  size_t ws_bytes, hipStream_t st) {
  const bool mx = prec == MOE_PREC_MXFP8;
  if (!dispatch_small_applies(T, k) || mx) {
    if (ws_bytes < dispatch_ws(T, E)) return MOE_ERR_WORKSPACE;
  }
  clear_stale_error();
  if (!mx && dispatch_small_applies(T, k))
    return status_of(launch_dispatch_small(dtype, x, topk_idx, T, d, E, k, counts, offsets,
                                           dest_row, src_token, Xs, st));
  const size_t nblk = (size_t)(T + 63) / 64;
  int32_t* hist = static_cast<int32_t*>(ws);
  int32_t* base = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + align_up(nblk * E * 4));
  MOE_TRY(launch_dispatch_meta(topk_idx, T, E, k, hist, base, counts, offsets, dest_row,
                               src_token, st));
  const int R = T * k;
  if (mx) return status_of(launch_mx_dispatch_copy(x, dest_row, T, d, k, Xs, Xq, Xq_scale, st));
  return status_of(launch_dispatch_copy(dtype, x, dest_row, T, d, k, Xs, st));
}

// Argument checks of moe_dispatch that need no workspace.
int dispatch_args(const void* x, const int32_t* topk_idx, int T, int d, int E, int k, int dtype,
                  int prec, const int32_t* counts, const int32_t* offsets,
                  const int32_t* dest_row, const int32_t* src_token, const void* Xs,
                  const void* Xq, const uint8_t* Xq_scale) {
  if (!all_nonnull(x, topk_idx, counts, offsets, dest_row, src_token, Xs)) return MOE_ERR_NULL;
  if (int s = check_prec(dtype, prec)) return s;
  const bool mx = prec == MOE_PREC_MXFP8;
  if (mx && !all_nonnull(Xq, Xq_scale)) return MOE_ERR_NULL;
  if (int s = check_route_shape(T, E, k)) return s;
  if (int s = check_width(d)) return s;
  if (int s = check_elems((long long)T * k, d)) return s;
  if (!all_aligned(x, topk_idx, counts, offsets, dest_row, src_token, Xs)) return MOE_ERR_ALIGN;
  if (mx && !all_aligned(Xq, Xq_scale)) return MOE_ERR_ALIGN;
  return MOE_OK;
}

// ---------------------------------------------------------------------------
// Static scratch of moe_dispatch_noalloc: the dispatch's per-block expert
// histograms and their scanned bases, in device memory that the library
// holds from load to process end (one copy per GPU).  Every table is fully
// written by the kernels before it is read, so nothing needs clearing.  In
// host code `scratch` is only a stand-in for the symbol: its device address,
// per device, comes from hipGetSymbolAddress and is what the kernels get.
// ---------------------------------------------------------------------------
constexpr size_t kNoAllocScratchBytes = size_t(4) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch (looked up once per device).
int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return status_of(e);
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) return status_of(e != hipSuccess ? e : hipErrorUnknown);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_dispatch(const void* x, const int32_t* topk_idx, int T, int d, int E, int k, int dtype,
                 int prec, int32_t* counts, int32_t* offsets, int32_t* dest_row,
                 int32_t* src_token, void* Xs, void* Xq, uint8_t* Xq_scale, void* ws,
                 size_t ws_bytes, void* stream) {
  if (int s = dispatch_args(x, topk_idx, T, d, E, k, dtype, prec, counts, offsets, dest_row,
                            src_token, Xs, Xq, Xq_scale))
    return s;
  if (!ws) return MOE_ERR_NULL;
  if (!aligned16(ws)) return MOE_ERR_ALIGN;
  if (ws_bytes < dispatch_ws(T, E)) return MOE_ERR_WORKSPACE;
  return dispatch_impl(x, topk_idx, T, d, E, k, dtype, prec, counts, offsets, dest_row, src_token,
                       Xs, Xq, Xq_scale, ws, ws_bytes, static_cast<hipStream_t>(stream));
}

int moe_dispatch_noalloc(const void* x, const int32_t* topk_idx, int T, int d, int E, int k,
                         int dtype, int prec, int32_t* counts, int32_t* offsets,
                         int32_t* dest_row, int32_t* src_token, void* Xs, void* Xq,
                         uint8_t* Xq_scale, void* stream) {
  if (int s = dispatch_args(x, topk_idx, T, d, E, k, dtype, prec, counts, offsets, dest_row,
                            src_token, Xs, Xq, Xq_scale))
    return s;
  const size_t need = dispatch_ws(T, E);
  if (need > kNoAllocScratchBytes) return MOE_ERR_SCRATCH;
  void* ws = nullptr;
  if (int s = scratch_address(&ws)) return s;
  return dispatch_impl(x, topk_idx, T, d, E, k, dtype, prec, counts, offsets, dest_row, src_token,
                       Xs, Xq, Xq_scale, ws, kNoAllocScratchBytes,
                       static_cast<hipStream_t>(stream));
}

int moe_grouped_ffn_fwd(const void* Xs, const uint8_t* Xs_scale, const int32_t* offsets, int T,
                        int k, int d, int f, int E, const void* Wg, const void* Wu,
                        const void* Wd, int dtype, int prec, unsigned flags, void* Hg, void* Hu,
                        void* A, void* Ys, void* ws, size_t ws_bytes, void* stream) {
  if (!all_nonnull(Xs, offsets, Wg, Wu, Wd, Hg, Hu, A, Ys)) return MOE_ERR_NULL;
  if (int s = check_prec(dtype, prec)) return s;
  const bool keep = (flags & MOE_MX_KEEP_WEIGHTS) != 0;
  if (keep && prec != MOE_PREC_MXFP8) return MOE_ERR_DTYPE;
  if (prec == MOE_PREC_MXFP8 && !all_nonnull(Xs_scale, ws)) return MOE_ERR_NULL;
  if (int s = check_route_shape(T, E, k)) return s;
  if (int s = check_width(d)) return s;
  if (int s = check_width(f)) return s;
  const long long R = (long long)T * k;
  if (int s = check_elems(R, 2LL * (d > f ? d : f))) return s;
  if (int s = check_elems(E, (long long)d * f)) return s;
  if (int s = check_weight_offsets(d, f)) return s;
  if (prec == MOE_PREC_MXFP8)
    if (int s = check_mx_scale_offsets(R, d, f)) return s;
  if (!all_aligned(Xs, offsets, Wg, Wu, Wd, Hg, Hu, A, Ys, ws)) return MOE_ERR_ALIGN;
  if (prec == MOE_PREC_MXFP8 && !aligned16(Xs_scale)) return MOE_ERR_ALIGN;
  hipStream_t st = static_cast<hipStream_t>(stream);
  clear_stale_error();
  if (prec == MOE_PREC_MXFP8) {
    if (ws_bytes < mx_fwd_workspace(R, d, f, E, keep)) return MOE_ERR_WORKSPACE;
    return status_of(mx_ffn_fwd(Xs, Xs_scale, offsets, (int)R, d, f, E, Wg, Wu, Wd, Hg, Hu, A,
                                Ys, ws, keep, num_cu(), st));
  }
  if (prec == MOE_PREC_BF16 && skinny_applies((int)R, E, d, f)) {
    // a few rows per expert: the weight-streaming small-batch engine
    const size_t need = skinny_workspace((int)R, E, d, f);
    if (need && !ws) return MOE_ERR_NULL;
    if (ws_bytes < need) return MOE_ERR_WORKSPACE;
    return status_of(launch_skinny_ffn_fwd(
        offsets, E, (int)R, d, f, static_cast<const bf16_t*>(Xs), static_cast<const bf16_t*>(Wg),
        static_cast<const bf16_t*>(Wu), static_cast<const bf16_t*>(Wd), static_cast<bf16_t*>(Hg),
        static_cast<bf16_t*>(Hu), static_cast<bf16_t*>(A), static_cast<bf16_t*>(Ys),
        static_cast<float*>(ws), st));
  }
  const int eng = gemm_engine(dtype);
  GemmArgs g{};
  g.E = E; g.offsets = offsets; g.rows_total = (int)R; g.ragged = RAG_M;
  g.N = f; g.K = d;
  g.a = Xs; g.lda = d;
  g.b0 = Wg; g.b1 = Wu; g.ldb = f; g.b_es = (long)d * f;
  g.c0 = Hg; g.c1 = Hu; g.c2 = A; g.ldc = f;
  g.m_fast = 1;
  MOE_TRY(launch_grouped_gemm(GK_FWD_GATEUP, eng, g, num_cu(), st));
  GemmArgs h{};
  h.E = E; h.offsets = offsets; h.rows_total = (int)R; h.ragged = RAG_M;
  h.N = d; h.K = f;
  h.a = A; h.lda = f;
  h.b0 = Wd; h.ldb = d; h.b_es = (long)f * d;
  h.c0 = Ys; h.ldc = d;
  h.m_fast = 1;
  return status_of(launch_grouped_gemm(GK_FWD_DOWN, eng, h, num_cu(), st));
}

int moe_combine(const void* Ys, const float* topk_w, const int32_t* dest_row, int T, int d, int k,
                int dtype, void* y, void* stream) {
  if (!all_nonnull(Ys, topk_w, dest_row, y)) return MOE_ERR_NULL;
  if (int s = check_dtype(dtype)) return s;
  if (T <= 0 || k <= 0 || (long long)T * k > 0x7fffffffLL) return MOE_ERR_SHAPE;
  if (int s = check_width(d)) return s;
  if (!all_aligned(Ys, topk_w, dest_row, y)) return MOE_ERR_ALIGN;
  clear_stale_error();
  if (combine_small_applies(T))
    return status_of(launch_combine_small(dtype, Ys, topk_w, dest_row, T, d, k, y,
                                          static_cast<hipStream_t>(stream)));
  return status_of(launch_combine(dtype, Ys, topk_w, dest_row, T, d, k, y,
                                  static_cast<hipStream_t>(stream)));
}

int moe_combine_bwd(const void* dY, const void* Ys, const float* topk_w, const int32_t* dest_row,
                    int T, int d, int k, int dtype, void* dYs, float* dtopk_w, void* dYs_q,
                    uint8_t* dYs_q_scale, void* stream) {
  if (!all_nonnull(dY, Ys, topk_w, dest_row, dYs, dtopk_w)) return MOE_ERR_NULL;
  if (int s = check_dtype(dtype)) return s;
  if ((dYs_q == nullptr) != (dYs_q_scale == nullptr)) return MOE_ERR_NULL;
  if (dYs_q && dtype != MOE_BF16) return MOE_ERR_DTYPE;
  if (T <= 0 || k <= 0 || (long long)T * k > 0x7fffffffLL) return MOE_ERR_SHAPE;
  if (int s = check_width(d)) return s;
  if (!all_aligned(dY, Ys, topk_w, dest_row, dYs, dtopk_w, dYs_q, dYs_q_scale)) return MOE_ERR_ALIGN;
  clear_stale_error();
  return status_of(launch_combine_bwd(dtype, dY, Ys, topk_w, dest_row, T, d, k, dYs, dtopk_w,
                                      dYs_q, dYs_q_scale, static_cast<hipStream_t>(stream)));
}

int moe_grouped_ffn_bwd(const void* dYs, const void* dYs_q, const uint8_t* dYs_q_scale,
                        const void* Xs, const void* Hg, const void* Hu, const void* A,
                        const int32_t* offsets, int T, int k, int d, int f, int E, const void* Wg,
                        const void* Wu, const void* Wd, int dtype, int prec, unsigned flags,
                        void* dH, void* dXs, void* dWg, void* dWu, void* dWd, void* ws,
                        size_t ws_bytes, void* stream) {
  if (!all_nonnull(dYs, Xs, Hg, Hu, A, offsets, Wg, Wu, Wd, dH, dXs, dWg, dWu, dWd))
    return MOE_ERR_NULL;
  if (int s = check_prec(dtype, prec)) return s;
  if (prec == MOE_PREC_MXFP8 && !all_nonnull(ws, dYs_q, dYs_q_scale)) return MOE_ERR_NULL;
  if (int s = check_route_shape(T, E, k)) return s;
  if (int s = check_width(d)) return s;
  if (int s = check_width(f)) return s;
  const long long R = (long long)T * k;
  if (int s = check_elems(R, 2LL * (d > f ? d : f))) return s;
  if (int s = check_elems(E, (long long)d * f)) return s;
  if (int s = check_weight_offsets(d, f)) return s;
  if (prec == MOE_PREC_MXFP8)
    if (int s = check_mx_scale_offsets(R, d, f)) return s;
  if (flags & MOE_WGRAD_MX) {
    if (int s = check_mx_wgrad_offsets(R, d, f, E)) return s;
  } else if (int s = check_wgrad_offsets(R, d, f)) {
    return s;
  }
  if (!all_aligned(dYs, Xs, Hg, Hu, A, offsets, Wg, Wu, Wd, dH, dXs, dWg, dWu, dWd, ws))
    return MOE_ERR_ALIGN;
  if (prec == MOE_PREC_MXFP8 && !all_aligned(dYs_q, dYs_q_scale)) return MOE_ERR_ALIGN;
  hipStream_t st = static_cast<hipStream_t>(stream);
  clear_stale_error();
  const int acc = (flags & MOE_ACCUMULATE) ? 1 : 0;
  const int eng = gemm_engine(dtype);
  const bool mxw = (flags & MOE_WGRAD_MX) != 0;
  const bool kept = (flags & MOE_MX_KEEP_WEIGHTS) != 0;
  if ((mxw || kept) && prec != MOE_PREC_MXFP8) return MOE_ERR_DTYPE;
  // kept: ws = the forward's workspace (with the backward's weight codes),
  // then the backward's own
  const size_t kept_bytes = kept ? mx_fwd_workspace(R, d, f, E, true) : 0;
  if (ws_bytes < kept_bytes) return MOE_ERR_WORKSPACE;
  void* own = static_cast<char*>(ws) + kept_bytes;
  const size_t own_bytes = ws_bytes - kept_bytes;
  if (mxw && own_bytes < mx_wgrad_workspace(R, d, f, E)) return MOE_ERR_WORKSPACE;
  if (prec == MOE_PREC_MXFP8) {
    if (own_bytes < mx_bwd_workspace(R, d, f, E)) return MOE_ERR_WORKSPACE;
    MOE_TRY(mx_ffn_dgrad(dYs_q, dYs_q_scale, Hg, Hu, offsets, (int)R, d, f, E, Wg, Wu, Wd, dH,
                         dXs, own, kept ? ws : nullptr, num_cu(), st));
  } else {
    GemmArgs g{};
    g.E = E; g.offsets = offsets; g.rows_total = (int)R; g.ragged = RAG_M;
    g.N = f; g.K = d;
    g.a = dYs; g.lda = d;
    g.b0 = Wd; g.ldb = d; g.b_es = (long)f * d;
    g.c0 = dH; g.ldc = 2L * f; g.c_split = f;
    g.h0 = Hg; g.h1 = Hu; g.ldh = f;
    MOE_TRY(launch_grouped_gemm(GK_DGRAD_DOWN, eng, g, num_cu(), st));
    GemmArgs h{};
    h.E = E; h.offsets = offsets; h.rows_total = (int)R; h.ragged = RAG_M;
    h.N = d; h.K = 2 * f;
    h.a = dH; h.lda = 2L * f;
    h.b0 = Wg; h.b1 = Wu; h.ldb = f; h.b_es = (long)d * f; h.b_split = f;
    h.c0 = dXs; h.ldc = d;
    MOE_TRY(launch_grouped_gemm(GK_DGRAD_GATEUP, eng, h, num_cu(), st));
  }
  if (mxw)
    return status_of(mx_ffn_wgrad(Xs, dH, A, dYs, offsets, (int)R, d, f, E,
                                  (flags & MOE_WGRAD_F32) ? 1 : 0, acc, dWg, dWu, dWd, own,
                                  num_cu(), st));
  // weight gradients: dWg|dWu = Xs^T . dH, dWd = A^T . dYs (ragged K = rows of e)
  const GemmKind wk =
      ((flags & MOE_WGRAD_F32) && dtype == MOE_BF16) ? GK_WGRAD_F32 : GK_WGRAD;
  GemmArgs w{};
  w.E = E; w.offsets = offsets; w.rows_total = (int)R; w.ragged = RAG_K;
  w.M = d; w.N = 2 * f;
  w.a = Xs; w.lda = d;
  w.b0 = dH; w.ldb = 2L * f;
  w.c0 = dWg; w.c1 = dWu; w.ldc = f; w.c_es = (long)d * f; w.c_split = f;
  w.accumulate = acc;
  MOE_TRY(launch_grouped_gemm(wk, eng, w, num_cu(), st));
  GemmArgs v{};
  v.E = E; v.offsets = offsets; v.rows_total = (int)R; v.ragged = RAG_K;
  v.M = f; v.N = d;
  v.a = A; v.lda = f;
  v.b0 = dYs; v.ldb = d;
  v.c0 = dWd; v.ldc = d; v.c_es = (long)f * d; v.c_split = d;
  v.accumulate = acc;
  return status_of(launch_grouped_gemm(wk, eng, v, num_cu(), st));
}

int moe_dispatch_bwd(const void* dXs, const int32_t* dest_row, int T, int d, int k, int dtype,
                     unsigned flags, void* dx, void* stream) {
  if (!all_nonnull(dXs, dest_row, dx)) return MOE_ERR_NULL;
  if (int s = check_dtype(dtype)) return s;
  if (T <= 0 || k <= 0 || (long long)T * k > 0x7fffffffLL) return MOE_ERR_SHAPE;
  if (int s = check_width(d)) return s;
  if (!all_aligned(dXs, dest_row, dx)) return MOE_ERR_ALIGN;
  clear_stale_error();
  return status_of(launch_gather_sum(dtype, dXs, dest_row, T, d, k,
                                     (flags & MOE_ACCUMULATE) ? 1 : 0, dx,
                                     static_cast<hipStream_t>(stream)));
}

int moe_route_bwd(const void* x, const void* Wr, const float* logits, const int32_t* topk_idx,
                  const float* dtopk_w, const float* aux_dp, int T, int d, int E, int k, int dtype,
                  unsigned flags, float* dlogits, void* dWr, void* dx, void* ws, size_t ws_bytes,
                  void* stream) {
  if (!all_nonnull(x, Wr, logits, topk_idx, dtopk_w, dlogits, dWr, dx)) return MOE_ERR_NULL;
  if (int s = check_dtype(dtype)) return s;
  if (int s = check_route_shape(T, E, k)) return s;
  if (int s = check_width(d)) return s;
  if (int s = check_elems(T, d)) return s;
  if (!all_aligned(x, Wr, logits, topk_idx, dtopk_w, aux_dp, dlogits, dWr, dx, ws))
    return MOE_ERR_ALIGN;
  const int ld16 = router_ld16(E);
  const size_t need = route_bwd_ws(T, d, E, dtype);
  if (need && !ws) return MOE_ERR_NULL;
  if (ws_bytes < need) return MOE_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  clear_stale_error();
  uint16_t* dl16 = (dtype == MOE_BF16) ? static_cast<uint16_t*>(ws) : nullptr;
  MOE_TRY(launch_router_bwd_softmax(logits, topk_idx, dtopk_w, T, E, k,
                                    (flags & MOE_ROUTE_RENORM) ? 1 : 0, aux_dp, dlogits, dl16,
                                    ld16, st));
  const void* dl = (dtype == MOE_BF16) ? static_cast<const void*>(dl16) : dlogits;
  const int ldl = (dtype == MOE_BF16) ? ld16 : E;
  const int eng = gemm_engine(dtype, E);
  const int acc = (flags & MOE_ACCUMULATE) ? 1 : 0;
  GemmArgs g{};
  g.E = 1; g.offsets = nullptr; g.rows_total = T; g.ragged = RAG_K;
  g.M = d; g.N = E;
  g.a = x; g.lda = d;
  g.b0 = dl; g.ldb = ldl;
  if (dtype == MOE_BF16 && router_dwr_applies(d, E)) {
    float* part = reinterpret_cast<float*>(static_cast<char*>(ws) + align_up((size_t)T * ld16 * 2));
    const int S = router_dwr_launch_slices(T, d, E, router_splits(T));
    MOE_TRY(launch_router_dwr(static_cast<const uint16_t*>(x), dl16, ld16, T, d, E, S, part, st));
    MOE_TRY(launch_split_reduce(dtype, part, S, (long)d * E, acc, dWr, st));
  } else if (eng == GEMM_BF16_MFMA) {
    // split K: d/256 output tiles alone would leave most of the chip idle
    const int S = router_splits(T);
    float* part = reinterpret_cast<float*>(static_cast<char*>(ws) + align_up((size_t)T * ld16 * 2));
    g.E = S; g.kchunk = (T + S - 1) / S;
    g.c0 = part; g.ldc = E; g.c_es = (long)d * E;
    MOE_TRY(launch_grouped_gemm(GK_ROUTER_DWR_SPLIT, eng, g, num_cu(), st));
    MOE_TRY(launch_split_reduce(dtype, part, S, (long)d * E, acc, dWr, st));
  } else {
    g.c0 = dWr; g.ldc = E;
    g.accumulate = acc;
    MOE_TRY(launch_grouped_gemm(GK_ROUTER_DWR, eng, g, num_cu(), st));
  }
  if (dtype == MOE_BF16 && router_dx_applies(d, E))
    return status_of(launch_router_dx(dl16, ld16, static_cast<const uint16_t*>(Wr), T, d, E,
                                      static_cast<uint16_t*>(dx), st));
  GemmArgs h{};
  h.E = 1; h.offsets = nullptr; h.rows_total = T; h.ragged = RAG_M;
  // the MFMA engine runs K over the zero-padded width; the SIMT engine over E
  h.M = T; h.N = d; h.K = (eng == GEMM_BF16_MFMA) ? ld16 : E;
  h.a = dl; h.lda = ldl;
  h.b0 = Wr; h.ldb = E;
  h.c0 = dx; h.ldc = d;
  h.accumulate = 1;
  return status_of(launch_grouped_gemm(GK_ROUTER_DX, eng, h, num_cu(), st));
}

int moe_check_routing(const int32_t* topk_idx, int T, int E, int k, int32_t* report,
                      void* stream) {
  if (!all_nonnull(topk_idx, report)) return MOE_ERR_NULL;
  if (T <= 0 || E <= 0 || k <= 0 || (long long)T * k > 0x7fffffffLL) return MOE_ERR_SHAPE;
  if (E > 256) return MOE_ERR_UNSUPPORTED;
  if (!all_aligned(topk_idx, report)) return MOE_ERR_ALIGN;
  clear_stale_error();
  return status_of(launch_check_routing(topk_idx, T, E, k, report,
                                        static_cast<hipStream_t>(stream)));
}

int moe_route_aux(const float* logits, const int32_t* counts, int T, int E, int k, float coef,
                  float* aux_loss, float* aux_dp, void* ws, size_t ws_bytes, void* stream) {
  if (!all_nonnull(logits, counts, aux_loss, aux_dp, ws)) return MOE_ERR_NULL;
  if (int s = check_route_shape(T, E, k)) return s;
  if (!(coef == coef)) return MOE_ERR_SHAPE;  // NaN coefficient
  if (!all_aligned(logits, counts, aux_loss, aux_dp, ws)) return MOE_ERR_ALIGN;
  if (ws_bytes < (size_t)((T + 63) / 64) * E * sizeof(float)) return MOE_ERR_WORKSPACE;
  clear_stale_error();
  return status_of(launch_router_aux(logits, counts, T, E, k, coef, static_cast<float*>(ws),
                                     aux_loss, aux_dp, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
