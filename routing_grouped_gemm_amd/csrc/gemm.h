// Grouped GEMM engine of the MoE expert layer: problem description shared by
// the host launchers and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// What the epilogue does with a finished tile.
enum EpiKind : int {
  EPI_STORE = 0,       // C[row][n] = acc (dtype), or += with accumulate
  EPI_STORE_F32 = 1,   // C[row][n] = acc as float32
  EPI_SWIGLU_FWD = 2,  // acc pair (gate, up): Hg, Hu and A = silu(Hg)*Hu
  EPI_SWIGLU_BWD = 3,  // acc = dA: dHg = dA*Hu*silu'(Hg), dHu = dA*silu(Hg) into dH[R,2f]
  EPI_WGRAD_SPLIT = 4,     // columns [0,c_split) -> c0, [c_split, N) -> c1 (dWg | dWu)
  EPI_WGRAD_SPLIT_F32 = 5  // as EPI_WGRAD_SPLIT into float32 outputs (float32 accumulation)
};

// How the B operand is assembled from two sources.
enum BSplit : int {
  BS_NONE = 0,
  BS_DUAL_N = 1,  // gate/up: tile columns alternate 64 from b0 (Wg), 64 from b1 (Wu)
  BS_SPLIT_K = 2  // k < b_split from b0, k >= b_split from b1 (shifted by b_split)
};

// Which dimension is ragged across groups (experts).
enum Ragged : int { RAG_M = 0, RAG_K = 1 };

struct GemmArgs {
  int E;               // number of groups
  const int* offsets;  // [E+1] device row offsets of the groups, or nullptr: see kchunk
  int kchunk;          // offsets == nullptr: 0 = one group; else (RAG_K) group e covers
                       // rows [e*kchunk, min((e+1)*kchunk, rows_total)) (split K)
  int rows_total;      // rows of the row-indexed operands (R, or T for router GEMMs)
  int ragged;          // RAG_M: group rows are GEMM rows; RAG_K: group rows are the K axis
  int M, N, K;         // the fixed dimensions (the ragged one is read from offsets)
  // A: RAG_M -> A[row][k] (K contiguous), row = global row; RAG_K -> A[krow][m]
  const void* a;
  long lda;
  long a_es;            // per-group element stride (0: rows are global)
  const int* a_gather;  // RAG_K only: source row of each global k-row, or nullptr
  // B: per-group matrix b + e*b_es, [N][K] (K contiguous) or [K][N] (N contiguous);
  // RAG_K: B[krow][n] with global k-rows.
  const void* b0;
  const void* b1;
  long ldb;
  long b_es;
  int b_split;
  // epilogue
  void* c0;
  void* c1;
  void* c2;
  long ldc;
  long c_es;  // RAG_K: per-group stride of C; RAG_M: 0 (C rows are global rows)
  int c_split;
  const void* h0;  // SWIGLU_BWD: Hg
  const void* h1;  // SWIGLU_BWD: Hu
  long ldh;
  int accumulate;
  // MXFP8 kinds: E8M0 scale bytes.  Block b (32 consecutive k) of B row n
  // of group e is sb[e * sb_es + b * sb_pitch + n] (block-major); of A row r
  // sa[b * sa_pitch + r] for the weight gradients (token-quantised operands)
  // and sa[((b / 4) * sa_pitch + r) * 4 + b % 4] otherwise (activation rows:
  // four blocks per group, mx_scale_at).  Operands a / b0 hold e4m3 codes,
  // and lda / ldb / b_es are in bytes (= elements).
  const uint8_t* sa;
  long sa_pitch;
  const uint8_t* sb;
  long sb_es;
  long sb_pitch;
  // MXFP8 kinds whose epilogue output feeds the next MX GEMM (gate/up: A,
  // down dgrad: dH): that output, as stored, block-quantised along its row:
  // codes at q0 (same layout as the output), scales at qs in the grouped
  // activation layout with pitch qs_pitch.
  uint8_t* q0;
  uint8_t* qs;
  long qs_pitch;
  // RAG_M tile order within a group: 0 = N-tiles fastest; 1 = M-tiles fastest
  // whenever the group has fewer M-tiles than N-tiles (sched_decode).
  int m_fast;
};

// Operand layouts of the five GEMM kinds of the layer and of the router.
enum GemmKind : int {
  GK_FWD_GATEUP = 0,    // Xs[R,d] . [Wg|Wu][e][d,f]  -> Hg, Hu, A    (ragged M)
  GK_FWD_DOWN = 1,      // A[R,f] . Wd[e][f,d]        -> Ys           (ragged M)
  GK_DGRAD_DOWN = 2,    // dYs[R,d] . Wd[e]^T         -> dHg, dHu     (ragged M)
  GK_DGRAD_GATEUP = 3,  // dH[R,2f] . [Wg|Wu][e]^T    -> dXs          (ragged M)
  GK_WGRAD = 4,         // P[rows,M]^T . Q[rows,N]    -> dW[e][M,N]   (ragged K)
  GK_WGRAD_F32 = 13,    // as GK_WGRAD, dW stored (or accumulated) as float32
  GK_ROUTER_LOGITS = 5, // x[T,d] . Wr[d,E]           -> logits f32   (one group)
  GK_ROUTER_DWR = 6,    // x[T,d]^T . dl[T,E]         -> dWr[d,E]     (one group, K = T)
  GK_ROUTER_DX = 7,     // dl[T,E] . Wr[d,E]^T        -> dx += [T,d]  (one group, K = E)
  GK_ROUTER_DWR_SPLIT = 12, // x^T . dl over K chunks     -> float32 partials [S][d][E]
  // MXFP8 kinds: both operands K-contiguous e4m3 codes with E8M0 block scales
  GK_MX_GATEUP = 8,       // Xq[R,d] . WguT[e][2f',d] (256-row panels: 128 gate rows, 128 up rows)
  GK_MX_DOWN = 9,         // Aq[R,f] . WdT[e][d,f]   -> Ys
  GK_MX_DGRAD_DOWN = 10,  // dYsq[R,d] . Wd[e][f,d]  -> dHg, dHu
  GK_MX_DGRAD_GATEUP = 11, // dHq[R,2f] . Wgu[e][d,2f] -> dXs
  // MXFP8 weight gradients: both operands transposed codes [rows][Kp] whose K
  // axis is every expert's tokens, each expert's segment padded to 128
  GK_MX_WGRAD = 14,       // P^T . Q over the expert's tokens -> dW[e] (bf16)
  GK_MX_WGRAD_F32 = 15    // as GK_MX_WGRAD into float32 gradients
};

// The weight-gradient kinds: ragged K over each expert's tokens, so their
// tiles' lengths follow the experts' loads.
constexpr bool wgrad_kind(int k) {
  return k == GK_WGRAD || k == GK_WGRAD_F32 || k == GK_MX_WGRAD || k == GK_MX_WGRAD_F32;
}

// Engines: float32 storage on the SIMT engine, bf16 on MFMA, and bf16 on the
// SIMT engine for router shapes the MFMA engine does not take (E % 8 != 0).
enum GemmEngine : int { GEMM_F32_SIMT = 0, GEMM_BF16_MFMA = 1, GEMM_BF16_SIMT = 2 };

// Number of groups of a GEMM: the offsets' groups, the K chunks, or one.
inline __host__ __device__ int ngroups(const GemmArgs& g) {
  return (g.offsets || g.kchunk > 0) ? g.E : 1;
}

// Launch a grouped GEMM of the given kind.  num_cu sizes the persistent grid.
hipError_t launch_grouped_gemm(GemmKind kind, int engine, const GemmArgs& g, int num_cu,
                               hipStream_t stream);

// Eight-wave form of the bf16 MFMA engine (gemm8.hip), launched for GK_WGRAD;
// grid: persistent workgroups.
hipError_t launch_gemm8(GemmKind kind, const GemmArgs& g, int grid, hipStream_t stream);

// Launch an MXFP8 grouped GEMM (kinds GK_MX_*).
hipError_t launch_grouped_gemm_mx(GemmKind kind, const GemmArgs& g, int num_cu, hipStream_t stream);

}  // namespace moe
