// Grouped GEMM engine of the MoE expert layer (gfx950).
//
// One launch runs every expert's GEMM ("merge the many small per-expert
// matmuls into one kernel", olmoforge README, grouped-GEMM module).  The
// groups are read on the device from the routing offsets, so the host never
// waits for routing metadata (GPU-resident routing table, same README).
//
// bf16 engine: persistent workgroups of 256 threads (4 waves, one per SIMD)
// walk a tile list over the ragged expert segments.  Tiles are 256x256
// outputs with a K step of 64 through two 64 KiB LDS stages; the next
// tile's first stage loads while the current tile's epilogue runs.  Each
// stage of both operands arrives by buffer->LDS DMA (16 bytes per lane, no
// register staging); one stage is in flight while the other is consumed.
// A wave that issues a DMA load stalls until the load path accepts it, and
// the MFMAs behind it in program order wait too; so each wave's 16 loads of
// a stage are spread over two k16 steps, one load after every two MFMAs.
// Operands that are K-contiguous in HBM sit in LDS as rows of 64 k (whole
// 128-byte lines); operands that are
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
  __shared__ __attribute__((aligned(256))) uint32_t pf_sink[64];
  constexpr bool DUAL = KT<KIND>::BSP == BS_DUAL_N;
  constexpr bool AMN = !KT<KIND>::AK, BMN = !KT<KIND>::BK_;
  constexpr int BNT = DUAL ? BN / 2 : BN;
  const int ntiles = sched_setup<BM, BNT, wgrad_kind(KIND)>(g, sch);
  const bool alt = wgrad_kind(KIND) && sch.alt;  // alternating rounds (logical_tile)

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform in the wave
  const int wm = wave >> 1, wn = wave & 1;
  const uint32_t lds0 = lds_u32(smem), sink = lds_u32(pf_sink);
  // L2 prefetch of a quarter of each K-contiguous operand's rows (wave 0:
  // A, wave 2: B); an operand that is contiguous along M or N is not
  // prefetched, as measured prefetching it does not pay.
  const bool pf_a = wave == 0 && !AMN, pf_b = wave == 2 && !BMN;
  const bool pf_on = pf_a || pf_b;
  // the lane's prefetch offset for tile tt (the quarter follows the tile)
  auto pf_plan = [&](const Tile& tt) -> uint32_t {
    return pf_a ? pf_quarter(tt.n0 / BNT, lane, (long)g.lda * 2)
                : pf_quarter(tt.m0 / BM, lane, (long)g.ldb * 2);
  };
  uint32_t pfv = 0;
  // DMA of stage s, then the prefetch of stage s + PF_AHEAD (issued even past
  // the last stage, where it touches no memory or a line of another row, so
  // that every stage adds the same number of loads to vmcnt)
  auto issue_stage = [&](const Plan& qa, const Plan& qb, int s) {
    issue<AMN>(qa, s, lds0 + (s & 1) * STAGE, wave);
    issue<BMN>(qb, s, lds0 + (s & 1) * STAGE + OPB, wave);
    if constexpr (!AMN) {
      if (pf_a) issue_pf(qa, pfv, s + PF_AHEAD, sink);
    }
    if constexpr (!BMN) {
      if (pf_b) issue_pf(qb, pfv, s + PF_AHEAD, sink);
    }
  };

  int it = 0;
  int L = logical_tile(it, alt);
  if (L >= ntiles) return;
  Tile t = sched_decode<BM, BNT, wgrad_kind(KIND)>(g, sch, L);
  Plan pa, pb;
  plan_tile<KIND>(g, t, wave, lane, pa, pb);
  pfv = pf_plan(t);
  int nk = (t.klen + BK - 1) / BK;
  if (nk > 0) issue_stage(pa, pb, 0);
  if (nk > 1) issue_stage(pa, pb, 1);

  for (;;) {
    // Stages 0 and 1 of tile t are in flight (as far as they exist).
    // The first k16 step of the tile writes the accumulators from a zero
    // operand, so they are not cleared first (256 register writes per tile);
    // a tile with no K stage (an expert without rows) clears them here.
    f32x16_t acc[4][4];
    if (nk == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x16_t{};
    }

    // Two stage buffers; stage kt+1 loads while stage kt is consumed in four
    // k16 steps with alternating fragment sets F0 / F1: the fragments of
    // step s+1 are read while the MFMAs of step s run.  After the reads of
    // step 3, one barrier publishes stage kt+1 (each wave waited for its own
    // DMA) and frees stage kt's buffer for stage kt+2, whose DMA then runs
    // under the MFMAs of step 3 and of the whole of stage kt+1.
    bf16x8_t fa0[4], fb0[4], fa1[4], fb1[4];
    if (nk > 0) {
      // stage 1 and both prefetches may still be in flight
      if (nk <= 1) wait_vmcnt<0>();
      else if (pf_on) wait_vmcnt<DMA_PER_OP * 2 + 2 * PF_PER_STAGE>();
      else wait_vmcnt<DMA_PER_OP * 2>();
      barrier();
      load_frags<AMN, BMN, DUAL>(smem, 0, 0, wm, wn, lane, fa0, fb0);
    }
    // The A loads of stage kt+2 go with the MFMAs of step 3 of stage kt, its
    // B loads and prefetches with step 0 of stage kt+1 (pend_b).
    bool pend_b = false;
    int pend_stage = 0;
    // The next tile's coordinates are decoded while this tile's first stage
    // lands (a binary search over the group table in LDS).
    L = logical_tile(it + 1, alt);
    const bool has_next = L < ntiles;
    Tile tn = t;
    if (has_next) tn = sched_decode<BM, BNT, wgrad_kind(KIND)>(g, sch, L);
    for (int kt = 0; kt < nk; ++kt) {
      // step 0 (set F0), reading F1 for step 1
      if (kt == 0) {
        kstep<AMN, BMN, DUAL, true>(acc, fa0, fb0, fa1, fb1, smem, kt, 1, wm, wn, lane);
      } else {
        // with the B loads (and prefetches) of stage kt+1 between MFMA pairs
        const bool dma = pend_b;
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          if (q == 2) {
            __builtin_amdgcn_s_waitcnt(kLgkm0);
            __builtin_amdgcn_sched_barrier(0);
          }
          mfma_pair(acc, fa0, fb0, q);
          if (dma) issue_one<BMN>(pb, pend_stage, lds0 + (pend_stage & 1) * STAGE + OPB, wave, q);
          if (q >= 2 && q < 6) {
            load_frag<AMN, BMN, DUAL>(smem, kt, 1, wm, wn, lane, fa1, fb1, 2 * (q - 2));
            load_frag<AMN, BMN, DUAL>(smem, kt, 1, wm, wn, lane, fa1, fb1, 2 * (q - 2) + 1);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        if (dma) {
          if constexpr (!AMN) {
            if (pf_a) issue_pf(pa, pfv, pend_stage + PF_AHEAD, sink);
          }
          if constexpr (!BMN) {
            if (pf_b) issue_pf(pb, pfv, pend_stage + PF_AHEAD, sink);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        pend_b = false;
      }
      kstep<AMN, BMN, DUAL, false>(acc, fa1, fb1, fa0, fb0, smem, kt, 2, wm, wn, lane);
      kstep<AMN, BMN, DUAL, false>(acc, fa0, fb0, fa1, fb1, smem, kt, 3, wm, wn, lane);
      __builtin_amdgcn_s_waitcnt(kLgkm0);
      const bool more = kt + 1 < nk;
      // stage kt+1 has landed once only its prefetch loads may be pending
      if (more) {
        if (pf_on) wait_vmcnt<PF_PER_STAGE>(); else wait_vmcnt<0>();
      }
      barrier();
      // step 3 (set F1) with the A loads of stage kt+2 between MFMA pairs,
      // reading F0 for step 0 of stage kt+1 (past the last stage the reads
      // land in the idle buffer and go unused)
      const bool dma = kt + 2 < nk;
      if (dma) pend_stage = kt + 2;
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        mfma_pair(acc, fa1, fb1, q);
        if (dma) issue_one<AMN>(pa, pend_stage, lds0 + (pend_stage & 1) * STAGE, wave, q);
        if (q < 4) {
          load_frag<AMN, BMN, DUAL>(smem, kt + 1, 0, wm, wn, lane, fa0, fb0, 2 * q);
          load_frag<AMN, BMN, DUAL>(smem, kt + 1, 0, wm, wn, lane, fa0, fb0, 2 * q + 1);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      pend_b = dma;
    }
    // every wave is done reading the ring
    __builtin_amdgcn_s_waitcnt(kLgkm0);
    barrier();

    // The next tile's stage 0 loads into buffer 0 while this tile's epilogue
    // stages through buffer 1 (one 16 KiB slice per wave); its stage 1
    // follows once the slices are read.  Loads complete in order, so the
    // stage waits of the next tile stay exact whatever the epilogue's own
    // global accesses do.
    ++it;
    Plan pan = pa, pbn = pb;
    int nkn = 0;
    if (has_next) {
      plan_tile<KIND>(g, tn, wave, lane, pan, pbn);
      nkn = (tn.klen + BK - 1) / BK;
      pfv = pf_plan(tn);
      if (nkn > 0) issue_stage(pan, pbn, 0);
    }
    epilogue_lds<KIND>(g, t, smem + STAGE + wave * EPI_SLICE, acc, wm, wn, lane);
    barrier();
    if (!has_next) break;
    if (nkn > 1) issue_stage(pan, pbn, 1);
    t = tn; pa = pan; pb = pbn; nk = nkn;
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
  const int ntiles = sched_setup<BM, BN, wgrad_kind(KIND)>(g, sch);
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  for (int L = blockIdx.x; L < ntiles; L += gridDim.x) {
    const Tile t = sched_decode<BM, BN, wgrad_kind(KIND)>(g, sch, L);
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
    const int E = ngroups(g);
    long mt = (long)g.rows_total / BM + E;
    long ub = mt * ntn;
    return (int)(ub < (1L << 30) ? ub : (1L << 30));
  }
  return ngroups(g) * ((g.M + BM - 1) / BM) * ntn;
}

const char* kind_name(int kind, const GemmArgs& g) {
  switch (kind) {
    case GK_FWD_GATEUP: return "gemm_fwd_gateup_swiglu";
    case GK_FWD_DOWN: return "gemm_fwd_down";
    case GK_DGRAD_DOWN: return "gemm_dgrad_down_swiglu_bwd";
    case GK_DGRAD_GATEUP: return "gemm_dgrad_gateup";
    case GK_WGRAD: return g.c1 ? "gemm_wgrad_gateup" : "gemm_wgrad_down";
    case GK_WGRAD_F32: return g.c1 ? "gemm_wgrad_gateup_f32" : "gemm_wgrad_down_f32";
    case GK_ROUTER_LOGITS: return "gemm_router_logits";
    case GK_ROUTER_DWR: return "gemm_router_dwr";
    case GK_ROUTER_DWR_SPLIT: return "gemm_router_dwr";
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
    note_prelaunch(kind_name(KIND, g), stream);
    if constexpr (KIND == GK_WGRAD) {  // eight-wave form (gemm8.hip)
      if (hipError_t e = launch_gemm8(static_cast<GemmKind>(KIND), g, grid, stream); e != hipSuccess)
        return e;
    } else {
      hipLaunchKernelGGL(mf::gemm_bf16_kernel<KIND>, dim3(grid), dim3(mf::NTHR), 0, stream, g);
    }
  } else {
    int ub = tiles_upper_bound(g, st::BM, st::BN);
    int grid = min(num_cu * 8, ub);
    if (grid <= 0) return hipSuccess;
    note_prelaunch(kind_name(KIND, g), stream);
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
    case GK_WGRAD_F32: return launch_kind<GK_WGRAD_F32>(dtype, g, num_cu, stream);
    case GK_ROUTER_LOGITS: return launch_kind<GK_ROUTER_LOGITS>(dtype, g, num_cu, stream);
    case GK_ROUTER_DWR: return launch_kind<GK_ROUTER_DWR>(dtype, g, num_cu, stream);
    case GK_ROUTER_DX: return launch_kind<GK_ROUTER_DX>(dtype, g, num_cu, stream);
    case GK_ROUTER_DWR_SPLIT: return launch_kind<GK_ROUTER_DWR_SPLIT>(dtype, g, num_cu, stream);
    default: break;
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
