// Grouped GEMM engine, eight-wave form (gfx950), used for the bf16 weight
// gradients dW[e] = P^T . Q over each expert's tokens (ragged K).
//
// Same tiles, stage ring, LDS layouts, buffer->LDS DMA and epilogues as the
// four-wave engine of gemm.hip, with eight waves per workgroup: two per SIMD,
// each owning a 128x64 sub-tile (wave = 4*wm + wn: rows wm*128.., columns
// wn*64..).  A wave that issues a buffer->LDS load stalls until the load path
// accepts it, and with one wave per SIMD the matrix core idles meanwhile; with
// two, the other wave's MFMAs can run.  Each wave moves half as many DMA
// blocks per stage (4 per operand) and keeps half the accumulators (128
// registers), so two waves fit one SIMD's register file.  Every output
// element is summed over the same k16 steps in the same order as in the
// four-wave engine, so the results are bitwise the same.
//
// Measured on the OLMoE-shaped layer (8192 tokens, d 2048, 64 experts, f
// 1024, top-8): the bf16 weight gradients, whose operands are both read
// transposed from LDS, run 5-8% faster in this form; the forward and
// input-gradient GEMMs ran up to 6% slower (each A fragment is now read by
// four waves instead of two) and the float32 weight gradients spill, so those
// keep the four-wave engine.  The kernel is written for every expert kind;
// only GK_WGRAD is launched in this form.
#include "gemm.h"
#include "gemm_dev.h"
#include "hook.h"
#include "moe_common.h"

namespace moe {
namespace mf8 {
using namespace mf;

constexpr int NW = 8, NTHR8 = 512, DPO8 = 4;
constexpr int PF8 = 1;                 // L2 prefetch loads per wave per stage
constexpr int SLICE8 = 32 * 64 * 4;    // epilogue staging per wave: 32 rows x 64 floats

// L2 prefetch of K-contiguous operands: waves 0-3 cover the 256 rows of A,
// waves 4-7 those of B, one line per wave per stage.
__device__ __forceinline__ uint32_t plan_pf8(long ld_bytes, int wave, int lane) {
  return (uint32_t)(((wave & 3) * 64 + lane) * ld_bytes);
}
__device__ __forceinline__ void issue_pf8(const Plan& P, uint32_t v, int kt, uint32_t sink) {
  const bool second = kt >= P.split_stage;
  const i32x4_t rs = second ? P.rs1 : P.rs0;
  const uint32_t soff = (uint32_t)(second ? kt - P.split_stage : kt) * P.kstep;
  pf4(rs, sink, v, soff);
}

// Fragments of one k16 step: 4 A fragments (rows wm*128 + 32i) and 2 B
// fragments (columns wn*64 + 32j; gate/up: gate wn*32.., up 128 + wn*32..).
template <bool AMN, bool BMN, bool DUAL>
__device__ __forceinline__ void load_frags8(const char* smem, int kt, int s, int wm, int wn,
                                            int lane, bf16x8_t (&fa)[4], bf16x8_t (&fb)[2]) {
  const char* As = smem + (kt & (NST - 1)) * STAGE;
  const char* Bs = As + OPB;
#pragma unroll
  for (int i = 0; i < 4; ++i) fa[i] = frag<AMN>(As, wm * 128 + i * 32, s, lane);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int col = DUAL ? (j * 128 + wn * 32) : (wn * 64 + j * 32);
    fb[j] = frag<BMN>(Bs, col, s, lane);
  }
}

// The two MFMAs of row block q.
__device__ __forceinline__ void mfma8_pair(f32x16_t (&acc)[4][2], const bf16x8_t (&fa)[4],
                                           const bf16x8_t (&fb)[2], int q) {
  acc[q][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[0], fa[q], acc[q][0], 0, 0, 0);
  acc[q][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[1], fa[q], acc[q][1], 0, 0, 0);
}
// One fragment of a k16 step: p = 0-1 the B fragments, p = 2-5 the A
// fragments.  B first: the MFMAs of row block 0 need both B fragments and
// only the first A fragment.
template <bool AMN, bool BMN, bool DUAL>
__device__ __forceinline__ void load_frag8(const char* smem, int kt, int s, int wm, int wn, int lane,
                                           bf16x8_t (&fa)[4], bf16x8_t (&fb)[2], int p) {
  const char* As = smem + (kt & (NST - 1)) * STAGE;
  const char* Bs = As + OPB;
  if (p < 2) {
    const int col = DUAL ? (p * 128 + wn * 32) : (wn * 64 + p * 32);
    fb[p] = frag<BMN>(Bs, col, s, lane);
  } else {
    fa[p - 2] = frag<AMN>(As, wm * 128 + (p - 2) * 32, s, lane);
  }
}
// The reads of a whole fragment set, B first.
template <bool AMN, bool BMN, bool DUAL>
__device__ __forceinline__ void load_set8(const char* smem, int kt, int s, int wm, int wn, int lane,
                                          bf16x8_t (&fa)[4], bf16x8_t (&fb)[2]) {
#pragma unroll
  for (int p = 0; p < 6; ++p) load_frag8<AMN, BMN, DUAL>(smem, kt, s, wm, wn, lane, fa, fb, p);
}
template <bool FIRST>
__device__ __forceinline__ void mfma8_row(f32x16_t (&acc)[4][2], const bf16x8_t (&fa)[4],
                                          const bf16x8_t (&fb)[2], int q) {
  acc[q][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[0], fa[q], FIRST ? f32x16_t{} : acc[q][0], 0, 0, 0);
  acc[q][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[1], fa[q], FIRST ? f32x16_t{} : acc[q][1], 0, 0, 0);
}
// A k16 step without DMA: the MFMAs of row block 0 of set (ca, cb) (they
// need only its first reads), one wait for the rest of the set, the reads of
// the next step's set into (na, nb), then the remaining MFMAs.  The next
// reads thus have most of a step to land before the next step's wait.
template <bool AMN, bool BMN, bool DUAL, bool FIRST>
__device__ __forceinline__ void kstep8(f32x16_t (&acc)[4][2], const bf16x8_t (&ca)[4],
                                       const bf16x8_t (&cb)[2], bf16x8_t (&na)[4], bf16x8_t (&nb)[2],
                                       const char* smem, int kt, int s, int wm, int wn, int lane) {
  __builtin_amdgcn_sched_barrier(0);
  mfma8_row<FIRST>(acc, ca, cb, 0);
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(kLgkm0);
  __builtin_amdgcn_sched_barrier(0);
  load_set8<AMN, BMN, DUAL>(smem, kt, s, wm, wn, lane, na, nb);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int q = 1; q < 4; ++q) mfma8_row<FIRST>(acc, ca, cb, q);
  __builtin_amdgcn_sched_barrier(0);
}


// Epilogue staging slice of one wave: 32 rows x 64 floats (256 bytes), the
// 16-byte chunks of a row XOR-permuted by the row.
__device__ __forceinline__ int stage8_off(int r, int chunk) { return r * 256 + ((chunk ^ (r & 15)) << 4); }
// bf16 staging of the same block: 128 bytes a row, chunk c of row r at c ^ (r & 7)
__device__ __forceinline__ int stage8_bf_off(int r, int chunk) { return r * 128 + ((chunk ^ (r & 7)) << 4); }

// One 32-row block (I) of a wave's 128x64 sub-tile.
template <int KIND, int I>
__device__ __forceinline__ void epilogue8_block(const GemmArgs& g, const Tile& t, char* slice,
                                                f32x16_t (&acc)[4][2], int wm, int wn, int lane) {
  constexpr int EPI = KT<KIND>::EPI;
  constexpr bool DUAL = KT<KIND>::BSP == BS_DUAL_N;
  static_assert(!qout_of<KIND>(), "bf16 kinds only");
  __builtin_amdgcn_sched_barrier(0);
  // lane's pieces outside the gate/up GEMM: row it*8 + lane/8, columns 8*(lane%8)
  const int cc = (lane & 7) * 8;
  uint4 hg[4], hu[4];
  // old output rows (accumulating stores) and Hg, Hu (SwiGLU backward) are
  // loaded before the staging so that their latency overlaps it
  constexpr bool PRE_ACC =
      EPI == EPI_STORE || EPI == EPI_WGRAD_SPLIT || EPI == EPI_WGRAD_SPLIT_F32;
  const bool pre_acc = PRE_ACC && g.accumulate;
  if constexpr (PRE_ACC) {
    if (pre_acc) {
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int m = wm * 128 + I * 32 + it * 8 + (lane >> 3);
        const int n = t.n0 + wn * 64 + cc;
        hg[it] = make_uint4(0, 0, 0, 0);
        hu[it] = make_uint4(0, 0, 0, 0);
        if (m < t.mlim && n < g.N) {
          const long row = (g.ragged == RAG_M) ? (long)t.row0 + m : (long)t.m0 + m;
          const uint4* p = reinterpret_cast<const uint4*>(epi_ptr<EPI>(g, t, row, n));
          hg[it] = p[0];
          if constexpr (EPI == EPI_WGRAD_SPLIT_F32) hu[it] = p[1];
        }
      }
    }
  }
  if constexpr (EPI == EPI_SWIGLU_BWD) {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int m = wm * 128 + I * 32 + it * 8 + (lane >> 3);
      const int n = t.n0 + wn * 64 + cc;
      hg[it] = hu[it] = make_uint4(0, 0, 0, 0);
      if (m < t.mlim && n < g.N) {
        const long off = ((long)t.row0 + m) * g.ldh + n;
        hg[it] = *reinterpret_cast<const uint4*>(static_cast<const bf16_t*>(g.h0) + off);
        hu[it] = *reinterpret_cast<const uint4*>(static_cast<const bf16_t*>(g.h1) + off);
      }
    }
  }
  // Plain bf16 stores that do not accumulate: rounded to bf16 in registers
  // and staged as bf16, 128 bytes a row (half the LDS traffic; the same
  // rounding, so the same bytes).
  constexpr bool BF_STAGE = EPI == EPI_STORE || EPI == EPI_WGRAD_SPLIT;
  if constexpr (BF_STAGE) {
    if (!g.accumulate) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int grp = 0; grp < 4; ++grp) {
          const int r = lane & 31;
          const uint2 w = make_uint2(pack_bf16x2(acc[I][j][4 * grp], acc[I][j][4 * grp + 1]),
                                     pack_bf16x2(acc[I][j][4 * grp + 2], acc[I][j][4 * grp + 3]));
          *reinterpret_cast<uint2*>(slice + stage8_bf_off(r, 4 * j + grp) + 8 * (lane >> 5)) = w;
        }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int r = it * 8 + (lane >> 3);
        const int m = wm * 128 + I * 32 + r;
        const int n = t.n0 + wn * 64 + cc;
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(slice + stage8_bf_off(r, lane & 7));
        if (m < t.mlim && n < g.N) {
          const long row = (g.ragged == RAG_M) ? (long)t.row0 + m : (long)t.m0 + m;
          __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(epi_ptr<EPI>(g, t, row, n)));
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      return;
    }
  }
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) {
      const int r = lane & 31;
      const int chunk = j * 8 + 2 * grp + (lane >> 5);
      f32x4_t v = {acc[I][j][4 * grp], acc[I][j][4 * grp + 1], acc[I][j][4 * grp + 2],
                   acc[I][j][4 * grp + 3]};
      *reinterpret_cast<f32x4_t*>(slice + stage8_off(r, chunk)) = v;
    }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  if constexpr (DUAL) {
    // slice columns 0..31: gate, 32..63: up, for f columns n0 + wn*32 + c
    static_assert(EPI == EPI_SWIGLU_FWD, "paired gate/up columns feed the SwiGLU forward");
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int r = it * 16 + (lane >> 2);
      const int c = (lane & 3) * 8;
      const int m = wm * 128 + I * 32 + r;
      const f32x4_t a0 = *reinterpret_cast<const f32x4_t*>(slice + stage8_off(r, c >> 2));
      const f32x4_t a1 = *reinterpret_cast<const f32x4_t*>(slice + stage8_off(r, (c >> 2) + 1));
      const f32x4_t b0 = *reinterpret_cast<const f32x4_t*>(slice + stage8_off(r, (c >> 2) + 8));
      const f32x4_t b1 = *reinterpret_cast<const f32x4_t*>(slice + stage8_off(r, (c >> 2) + 9));
      float v[8], u[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) { v[q] = a0[q]; v[q + 4] = a1[q]; u[q] = b0[q]; u[q + 4] = b1[q]; }
      const int n = t.n0 + wn * 32 + c;
      if (m < t.mlim && n < g.N) {
        float a[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) a[q] = silu_f(v[q]) * u[q];
        const long off = ((long)t.row0 + m) * g.ldc + n;
        store8_nt(static_cast<bf16_t*>(g.c0) + off, v);
        store8_nt(static_cast<bf16_t*>(g.c1) + off, u);
        store8_nt(static_cast<bf16_t*>(g.c2) + off, a);
      }
    }
  } else {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int r = it * 8 + (lane >> 3);
      const int m = wm * 128 + I * 32 + r;
      const int n = t.n0 + wn * 64 + cc;
      const f32x4_t a0 = *reinterpret_cast<const f32x4_t*>(slice + stage8_off(r, cc >> 2));
      const f32x4_t a1 = *reinterpret_cast<const f32x4_t*>(slice + stage8_off(r, (cc >> 2) + 1));
      float v[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) { v[q] = a0[q]; v[q + 4] = a1[q]; }
      if (m < t.mlim && n < g.N) {
        const long row = (g.ragged == RAG_M) ? (long)t.row0 + m : (long)t.m0 + m;
        if constexpr (EPI == EPI_SWIGLU_BWD) {
          float h0[8], h1[8], dg[8], du[8];
          unpack8(hg[it], h0);
          unpack8(hu[it], h1);
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const float sg = sigmoid_f(h0[q]);
            du[q] = v[q] * h0[q] * sg;
            dg[q] = v[q] * h1[q] * sg * (1.0f + h0[q] * (1.0f - sg));
          }
          bf16_t* p = static_cast<bf16_t*>(g.c0) + row * g.ldc + n;
          store8_nt(p, dg);
          store8_nt(p + g.c_split, du);
        } else if (pre_acc) {
          float o[8], w[8];
          if constexpr (EPI == EPI_WGRAD_SPLIT_F32) {
            const uint32_t* a = reinterpret_cast<const uint32_t*>(&hg[it]);
            const uint32_t* b = reinterpret_cast<const uint32_t*>(&hu[it]);
#pragma unroll
            for (int q = 0; q < 4; ++q) { o[q] = __uint_as_float(a[q]); o[q + 4] = __uint_as_float(b[q]); }
          } else {
            unpack8(hg[it], o);
          }
#pragma unroll
          for (int q = 0; q < 8; ++q) w[q] = v[q] + o[q];
          store8_nt(epi_ptr<EPI>(g, t, row, n), w);
        } else {
          epi8<EPI>(g, t, row, n, v, v);
        }
      }
    }
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

template <int KIND>
__device__ __forceinline__ void epilogue8_lds(const GemmArgs& g, const Tile& tile, char* slice,
                                              f32x16_t (&acc)[4][2], int wm, int wn, int lane_in) {
  // the tile's coordinates pass through an empty asm statement so that the
  // epilogue's address arithmetic is not hoisted above the K loop
  Tile t = tile;
  int lane = lane_in;
  asm volatile("" : "+v"(t.row0), "+v"(t.n0), "+v"(t.m0), "+v"(t.e), "+v"(t.mlim), "+v"(lane));
  epilogue8_block<KIND, 0>(g, t, slice, acc, wm, wn, lane);
  epilogue8_block<KIND, 1>(g, t, slice, acc, wm, wn, lane);
  epilogue8_block<KIND, 2>(g, t, slice, acc, wm, wn, lane);
  epilogue8_block<KIND, 3>(g, t, slice, acc, wm, wn, lane);
}

template <int KIND>
__global__ __launch_bounds__(NTHR8, 1) void gemm8_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(1024))) char smem[NST * STAGE];
  __shared__ Sched sch;
  __shared__ __attribute__((aligned(256))) uint32_t pf_sink[64];
  constexpr bool DUAL = KT<KIND>::BSP == BS_DUAL_N;
  constexpr bool AMN = !KT<KIND>::AK, BMN = !KT<KIND>::BK_;
  constexpr int BNT = DUAL ? BN / 2 : BN;
  constexpr bool SPLIT = KIND != GK_FWD_GATEUP;  // spread the stage DMA over two k16 steps
  const int ntiles = sched_setup<BM, BNT, wgrad_kind(KIND)>(g, sch);
  const bool alt = wgrad_kind(KIND) && sch.alt;  // alternating rounds (logical_tile)

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform in the wave
  const int wm = wave >> 2, wn = wave & 3;
  const uint32_t lds0 = lds_u32(smem), sink = lds_u32(pf_sink);
  // L2 prefetch of the K-contiguous operands (waves 0-3: A, 4-7: B)
  const bool pf_on = (wave < 4) ? !AMN : !BMN;
  const uint32_t pfv = plan_pf8((wave < 4 ? g.lda : g.ldb) * 2, wave, lane);
  // DMA of stage s, then the prefetch of stage s + PF_AHEAD (issued even past
  // the last stage, so that every stage adds the same number of loads to vmcnt)
  auto issue_stage = [&](const Plan& qa, const Plan& qb, int s) {
    issue<AMN, DPO8, NW>(qa, s, lds0 + (s & 1) * STAGE, wave);
    issue<BMN, DPO8, NW>(qb, s, lds0 + (s & 1) * STAGE + OPB, wave);
    if constexpr (!AMN) {
      if (wave < 4) issue_pf8(qa, pfv, s + PF_AHEAD, sink);
    }
    if constexpr (!BMN) {
      if (wave >= 4) issue_pf8(qb, pfv, s + PF_AHEAD, sink);
    }
  };

  int it = 0;
  int L = logical_tile(it, alt);
  if (L >= ntiles) return;
  Tile t = sched_decode<BM, BNT, wgrad_kind(KIND)>(g, sch, L);
  Plan pa, pb;
  plan_tile<KIND, DPO8, NW>(g, t, wave, lane, pa, pb);
  int nk = (t.klen + BK - 1) / BK;
  if (nk > 0) issue_stage(pa, pb, 0);
  if (nk > 1) issue_stage(pa, pb, 1);

  for (;;) {
    // stages 0 and 1 of tile t are in flight (as far as they exist)
    f32x16_t acc[4][2];
    if (nk == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x16_t{};
    }
    bf16x8_t fa0[4], fb0[2], fa1[4], fb1[2];
    if (nk > 0) {
      if (nk <= 1) wait_vmcnt<0>();
      else if (pf_on) wait_vmcnt<DPO8 * 2 + 2 * PF8>();
      else wait_vmcnt<DPO8 * 2>();
      barrier();
      load_frags8<AMN, BMN, DUAL>(smem, 0, 0, wm, wn, lane, fa0, fb0);
    }
    bool pend_b = false;
    int pend_stage = 0;
    L = logical_tile(it + 1, alt);
    const bool has_next = L < ntiles;
    Tile tn = t;
    if (has_next) tn = sched_decode<BM, BNT, wgrad_kind(KIND)>(g, sch, L);
    for (int kt = 0; kt < nk; ++kt) {
      // step 0 (set F0), reading F1 for step 1
      if (kt == 0) {
        kstep8<AMN, BMN, DUAL, true>(acc, fa0, fb0, fa1, fb1, smem, kt, 1, wm, wn, lane);
      } else if constexpr (SPLIT) {
        // with the B loads (and prefetches) of stage kt+1 between MFMA pairs
        const bool dma = pend_b;
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          mfma8_pair(acc, fa0, fb0, q);
          if (dma)
            issue_one<BMN, DPO8, NW>(pb, pend_stage, lds0 + (pend_stage & 1) * STAGE + OPB, wave, q);
          if (q == 0) {
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_waitcnt(kLgkm0);
            __builtin_amdgcn_sched_barrier(0);
            load_set8<AMN, BMN, DUAL>(smem, kt, 1, wm, wn, lane, fa1, fb1);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        if (dma) {
          if constexpr (!AMN) {
            if (wave < 4) issue_pf8(pa, pfv, pend_stage + PF_AHEAD, sink);
          }
          if constexpr (!BMN) {
            if (wave >= 4) issue_pf8(pb, pfv, pend_stage + PF_AHEAD, sink);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        pend_b = false;
      } else {
        kstep8<AMN, BMN, DUAL, false>(acc, fa0, fb0, fa1, fb1, smem, kt, 1, wm, wn, lane);
      }
      kstep8<AMN, BMN, DUAL, false>(acc, fa1, fb1, fa0, fb0, smem, kt, 2, wm, wn, lane);
      // step 2 (set F0), reading F1 for step 3
      kstep8<AMN, BMN, DUAL, false>(acc, fa0, fb0, fa1, fb1, smem, kt, 3, wm, wn, lane);
      __builtin_amdgcn_s_waitcnt(kLgkm0);
      const bool more = kt + 1 < nk;
      // stage kt+1 has landed once only its prefetch loads may be pending
      if (more) {
        if (pf_on) wait_vmcnt<PF8>(); else wait_vmcnt<0>();
      }
      barrier();
      // step 3 (set F1), reading F0 for step 0 of stage kt+1 (past the last
      // stage the reads land in the idle buffer and go unused)
      if constexpr (SPLIT) {
        const bool dma = kt + 2 < nk;
        if (dma) pend_stage = kt + 2;
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          mfma8_pair(acc, fa1, fb1, q);
          if (dma) issue_one<AMN, DPO8, NW>(pa, pend_stage, lds0 + (pend_stage & 1) * STAGE, wave, q);
          if (q == 0) load_set8<AMN, BMN, DUAL>(smem, kt + 1, 0, wm, wn, lane, fa0, fb0);
          __builtin_amdgcn_sched_barrier(0);
        }
        pend_b = dma;
      } else {
        if (kt + 2 < nk) issue_stage(pa, pb, kt + 2);
        __builtin_amdgcn_sched_barrier(0);
        mfma8_row<false>(acc, fa1, fb1, 0);
        __builtin_amdgcn_sched_barrier(0);
        load_set8<AMN, BMN, DUAL>(smem, kt + 1, 0, wm, wn, lane, fa0, fb0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 1; q < 4; ++q) mfma8_row<false>(acc, fa1, fb1, q);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // every wave is done reading the ring
    __builtin_amdgcn_s_waitcnt(kLgkm0);
    barrier();

    // the next tile's stage 0 loads into buffer 0 while this tile's epilogue
    // stages through buffer 1 (8 KiB per wave); its stage 1 follows
    ++it;
    Plan pan = pa, pbn = pb;
    int nkn = 0;
    if (has_next) {
      plan_tile<KIND, DPO8, NW>(g, tn, wave, lane, pan, pbn);
      nkn = (tn.klen + BK - 1) / BK;
      if (nkn > 0) issue_stage(pan, pbn, 0);
    }
    epilogue8_lds<KIND>(g, t, smem + STAGE + wave * SLICE8, acc, wm, wn, lane);
    barrier();
    if (!has_next) break;
    if (nkn > 1) issue_stage(pan, pbn, 1);
    t = tn; pa = pan; pb = pbn; nk = nkn;
  }
}

}  // namespace mf8

hipError_t launch_gemm8(GemmKind kind, const GemmArgs& g, int grid, hipStream_t stream) {
  if (kind != GK_WGRAD) return hipErrorInvalidValue;
  hipLaunchKernelGGL(mf8::gemm8_kernel<GK_WGRAD>, dim3(grid), dim3(mf8::NTHR8), 0, stream, g);
  return hipGetLastError();
}

}  // namespace moe
