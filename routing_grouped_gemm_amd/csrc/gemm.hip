// Grouped GEMM engine of the MoE expert layer (gfx950).
//
// One launch runs every expert's GEMM ("merge the many small per-expert
// matmuls into one kernel", olmoforge README, grouped-GEMM module).  The
// groups are read on the device from the routing offsets, so the host never
// waits for routing metadata (GPU-resident routing table, same README).
//
// bf16 engine: persistent workgroups of 256 threads (4 waves, one per SIMD)
// walk a tile list over the ragged expert segments.  Tiles are 256x256
// outputs with a K step of 32 through a 4-stage LDS ring (128 KiB).  Each
// stage of both operands arrives by buffer->LDS DMA (16 bytes per lane, no
// register staging); the ring keeps three stages in flight.  Operands that
// are K-contiguous in HBM sit in LDS as rows of 32 k; operands that are
// contiguous along M or N (the weights in the forward GEMMs, both operands of
// the weight gradient) sit as rows of k and are read transposed by
// ds_read_b64_tr_b16.  Each wave owns a 128x128 sub-tile as 4x4 MFMA
// 32x32x16 bf16 blocks with float32 accumulators.  Buffer resources bound
// every operand, so rows past a ragged K or past the end of a tensor read as
// zeros.  Consecutive logical tiles go to workgroups of the same XCD, so tiles
// that share an activation or weight panel meet in the same L2.
//
// float32 engine (the fp32 layer and odd router shapes): a plain LDS-tiled
// SIMT kernel with the same tile schedule and the same epilogues.
#include "gemm.h"
#include "gemm_dev.h"
#include "hook.h"
#include "moe_common.h"

namespace moe {
namespace mf {

template <int KIND>
__global__ __launch_bounds__(NTHR, 1) void gemm_bf16_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(1024))) char smem[NST * STAGE];
  __shared__ Sched sch;
  constexpr bool DUAL = KT<KIND>::BSP == BS_DUAL_N;
  constexpr bool AMN = !KT<KIND>::AK, BMN = !KT<KIND>::BK_;
  constexpr int BNT = DUAL ? BN / 2 : BN;
  const int ntiles = sched_setup<BM, BNT>(g, sch);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform in the wave
  const int wm = wave >> 1, wn = wave & 1;
  const uint32_t lds0 = lds_u32(smem);

  for (int it = 0;; ++it) {
    const int L = logical_tile(it);
    if (L >= ntiles) break;
    const Tile t = sched_decode<BM, BNT>(g, sch, L);
    Plan pa, pb;
    plan_tile<KIND>(g, t, wave, lane, pa, pb);

    f32x16_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x16_t{};

    // Ring of NST = 4 buffers, prefetch distance 4.  Stage kt's two k16 steps
    // use fragment sets F0 (step 0) and F1 (step 1).  F1 is read while the
    // MFMAs of F0 run; then every wave has finished reading stage kt, and one
    // barrier both publishes stage kt+1 (each wave waited for its own DMA) and
    // frees stage kt's buffer for stage kt+4.  The MFMAs of F1 then run while
    // F0 of stage kt+1 is read.
    const int nk = (t.klen + BK - 1) / BK;
#pragma unroll
    for (int s = 0; s < NST; ++s)
      if (s < nk) {
        issue<AMN>(pa, s, lds0 + s * STAGE, wave);
        issue<BMN>(pb, s, lds0 + s * STAGE + OPB, wave);
      }
    bf16x8_t fa0[4], fb0[4], fa1[4], fb1[4];
    if (nk > 0) {
      wait_stage(0, min(nk - 1, NST - 1));
      barrier();
      load_frags<AMN, BMN, DUAL>(smem, 0, 0, wm, wn, lane, fa0, fb0);
    }
    for (int kt = 0; kt < nk; ++kt) {
      // F0 was read a whole phase ago: this wait is nearly free, and it lets
      // the compiler issue F0's MFMAs without waiting on the F1 reads that
      // are interleaved with them (lgkmcnt cannot count all 16 reads of a set).
      __builtin_amdgcn_s_waitcnt(kLgkm0);
      load_frags<AMN, BMN, DUAL>(smem, kt, 1, wm, wn, lane, fa1, fb1);
      mfma16(acc, fa0, fb0);
      interleave_mfma_ds();
      __builtin_amdgcn_s_waitcnt(kLgkm0);
      const bool more = kt + 1 < nk;
      if (more) wait_stage(kt + 1, min(nk - 1, kt + NST - 1));
      barrier();
      if (kt + NST < nk) {
        const uint32_t nb = lds0 + (kt & (NST - 1)) * STAGE;
        issue<AMN>(pa, kt + NST, nb, wave);
        issue<BMN>(pb, kt + NST, nb + OPB, wave);
      }
      if (more) load_frags<AMN, BMN, DUAL>(smem, kt + 1, 0, wm, wn, lane, fa0, fb0);
      mfma16(acc, fa1, fb1);
      interleave_mfma_ds();
    }
    // every wave is done reading the ring before the next tile refills it
    barrier();

    // Epilogue through LDS.  The ring is idle now: each wave takes a private
    // 32 KiB slice and, for each half of its 128 rows, writes its float32
    // accumulators there straight from the accumulator registers, then reads
    // back 8 consecutive columns of a row per lane and applies the epilogue
    // with 16-byte global accesses.
    epilogue_lds<KIND>(g, t, smem + wave * 32768, acc, wm, wn, lane);
    // the slices are ring buffers of the next tile
    barrier();
  }
}

}  // namespace mf

// ---------------------------------------------------------------------------
// SIMT engine (float32 layer; any storage type)
// ---------------------------------------------------------------------------
namespace st {

constexpr int BM = 64, BN = 64, BK = 16, NTHR = 256;

template <int KIND, typename TS>
__device__ __forceinline__ float a_elem(const GemmArgs& g, const Tile& t, int m, int k) {
  const TS* A = static_cast<const TS*>(g.a);
  if (k >= t.klen) return 0.0f;
  if constexpr (KT<KIND>::AK) {
    int r = min(m, t.mlim - 1);
    return St<TS>::to_f(A[((long)t.row0 + r) * g.lda + k]);
  } else {
    int mm = t.m0 + m;
    if (mm >= g.M) return 0.0f;
    long row = (long)t.row0 + k;
    if (g.a_gather) row = g.a_gather[row];
    return St<TS>::to_f(A[row * g.lda + mm]);
  }
}

// half: 0 = b0 side, 1 = b1 side (BS_DUAL_N); n is the output column.
template <int KIND, typename TS>
__device__ __forceinline__ float b_elem(const GemmArgs& g, const Tile& t, int k, int n, int half) {
  if (k >= t.klen || n >= g.N) return 0.0f;
  constexpr int BSP = KT<KIND>::BSP;
  const TS* base = static_cast<const TS*>(half ? g.b1 : g.b0);
  int kk = k;
  if constexpr (BSP == BS_SPLIT_K) {
    if (k >= g.b_split) { base = static_cast<const TS*>(g.b1); kk = k - g.b_split; }
  }
  if constexpr (KT<KIND>::BK_) {
    return St<TS>::to_f(base[(long)t.e * g.b_es + (long)n * g.ldb + kk]);
  } else {
    if (g.ragged == RAG_M) return St<TS>::to_f(base[(long)t.e * g.b_es + (long)kk * g.ldb + n]);
    return St<TS>::to_f(base[((long)t.row0 + kk) * g.ldb + n]);
  }
}

template <int KIND, typename TS>
__global__ __launch_bounds__(NTHR) void gemm_simt_kernel(GemmArgs g) {
  constexpr bool DUAL = KT<KIND>::BSP == BS_DUAL_N;
  __shared__ float As[BK][BM + 4];
  __shared__ float Bs[DUAL ? 2 : 1][BK][BN + 4];
  __shared__ Sched sch;
  const int ntiles = sched_setup<BM, BN>(g, sch);
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  for (int L = blockIdx.x; L < ntiles; L += gridDim.x) {
    const Tile t = sched_decode<BM, BN>(g, sch, L);
    float acc[2][4][4] = {};
    for (int k0 = 0; k0 < t.klen; k0 += BK) {
      for (int q = tid; q < BK * BM; q += NTHR) {
        int kk = q / BM, m = q % BM;
        As[kk][m] = a_elem<KIND, TS>(g, t, m, k0 + kk);
      }
      for (int h = 0; h < (DUAL ? 2 : 1); ++h)
        for (int q = tid; q < BK * BN; q += NTHR) {
          int kk = q / BN, n = q % BN;
          Bs[h][kk][n] = b_elem<KIND, TS>(g, t, k0 + kk, t.n0 + n, h);
        }
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < BK; ++kk) {
        float a[4], b[2][4];
#pragma unroll
        for (int r = 0; r < 4; ++r) a[r] = As[kk][ty * 4 + r];
#pragma unroll
        for (int h = 0; h < (DUAL ? 2 : 1); ++h)
#pragma unroll
          for (int c = 0; c < 4; ++c) b[h][c] = Bs[h][kk][tx * 4 + c];
#pragma unroll
        for (int h = 0; h < (DUAL ? 2 : 1); ++h)
#pragma unroll
          for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[h][r][c] = fmaf(a[r], b[h][c], acc[h][r][c]);
      }
      __syncthreads();
    }
    constexpr int EPI = KT<KIND>::EPI;
    const int n = t.n0 + tx * 4;
    if (n < g.N) {
      for (int r = 0; r < 4; ++r) {
        int m = ty * 4 + r;
        if (m >= t.mlim) continue;
        float v[4], u[4];
        for (int c = 0; c < 4; ++c) { v[c] = acc[0][r][c]; u[c] = acc[DUAL ? 1 : 0][r][c]; }
        epilogue4<EPI, TS>(g, t, m, n, v, u);
      }
    }
  }
}

}  // namespace st

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
namespace {

int tiles_upper_bound(const GemmArgs& g, int BM, int BNT) {
  const int ntn = (g.N + BNT - 1) / BNT;
  if (g.ragged == RAG_M) {
    const int E = g.offsets ? g.E : 1;
    long mt = (long)g.rows_total / BM + E;
    long ub = mt * ntn;
    return (int)(ub < (1L << 30) ? ub : (1L << 30));
  }
  const int E = g.offsets ? g.E : 1;
  return E * ((g.M + BM - 1) / BM) * ntn;
}

const char* kind_name(int kind, const GemmArgs& g) {
  switch (kind) {
    case GK_FWD_GATEUP: return "gemm_fwd_gateup_swiglu";
    case GK_FWD_DOWN: return "gemm_fwd_down";
    case GK_DGRAD_DOWN: return "gemm_dgrad_down_swiglu_bwd";
    case GK_DGRAD_GATEUP: return "gemm_dgrad_gateup";
    case GK_WGRAD: return g.c1 ? "gemm_wgrad_gateup" : "gemm_wgrad_down";
    case GK_ROUTER_LOGITS: return "gemm_router_logits";
    case GK_ROUTER_DWR: return "gemm_router_dwr";
    case GK_ROUTER_DX: return "gemm_router_dx";
  }
  return "gemm";
}

template <int KIND>
hipError_t launch_kind(int dtype, const GemmArgs& g, int num_cu, hipStream_t stream) {
  if (dtype == GEMM_BF16_MFMA) {
    constexpr int BNT = (KT<KIND>::BSP == BS_DUAL_N) ? mf::BN / 2 : mf::BN;
    int ub = tiles_upper_bound(g, mf::BM, BNT);
    int grid = min(num_cu, ub);
    if (grid <= 0) return hipSuccess;
    hipLaunchKernelGGL(mf::gemm_bf16_kernel<KIND>, dim3(grid), dim3(mf::NTHR), 0, stream, g);
  } else {
    int ub = tiles_upper_bound(g, st::BM, st::BN);
    int grid = min(num_cu * 8, ub);
    if (grid <= 0) return hipSuccess;
    if (dtype == GEMM_F32_SIMT)
      hipLaunchKernelGGL((st::gemm_simt_kernel<KIND, float>), dim3(grid), dim3(st::NTHR), 0, stream, g);
    else
      hipLaunchKernelGGL((st::gemm_simt_kernel<KIND, bf16_t>), dim3(grid), dim3(st::NTHR), 0, stream, g);
  }
  note_launch(kind_name(KIND, g), stream);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_grouped_gemm(GemmKind kind, int dtype, const GemmArgs& g, int num_cu,
                               hipStream_t stream) {
  switch (kind) {
    case GK_FWD_GATEUP: return launch_kind<GK_FWD_GATEUP>(dtype, g, num_cu, stream);
    case GK_FWD_DOWN: return launch_kind<GK_FWD_DOWN>(dtype, g, num_cu, stream);
    case GK_DGRAD_DOWN: return launch_kind<GK_DGRAD_DOWN>(dtype, g, num_cu, stream);
    case GK_DGRAD_GATEUP: return launch_kind<GK_DGRAD_GATEUP>(dtype, g, num_cu, stream);
    case GK_WGRAD: return launch_kind<GK_WGRAD>(dtype, g, num_cu, stream);
    case GK_ROUTER_LOGITS: return launch_kind<GK_ROUTER_LOGITS>(dtype, g, num_cu, stream);
    case GK_ROUTER_DWR: return launch_kind<GK_ROUTER_DWR>(dtype, g, num_cu, stream);
    case GK_ROUTER_DX: return launch_kind<GK_ROUTER_DX>(dtype, g, num_cu, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
