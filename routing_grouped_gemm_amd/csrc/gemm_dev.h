// Device-side building blocks of the grouped GEMM engines (bf16 and MXFP8):
// tile schedule over ragged groups, buffer->LDS DMA ring, LDS layouts and
// fragment reads, and the LDS-staged epilogues.  Included by gemm.hip and
// mx.hip only.
#pragma once

#include <type_traits>

#include "gemm.h"
#include "moe_common.h"
#include "mx_codec.h"

namespace moe {

// ---------------------------------------------------------------------------
// kind traits
// ---------------------------------------------------------------------------
template <int KIND> struct KT;
template <> struct KT<GK_FWD_GATEUP> {
  static constexpr bool AK = true, BK_ = false;
  static constexpr int BSP = BS_DUAL_N, EPI = EPI_SWIGLU_FWD;
};
template <> struct KT<GK_FWD_DOWN> {
  static constexpr bool AK = true, BK_ = false;
  static constexpr int BSP = BS_NONE, EPI = EPI_STORE;
};
template <> struct KT<GK_DGRAD_DOWN> {
  static constexpr bool AK = true, BK_ = true;
  static constexpr int BSP = BS_NONE, EPI = EPI_SWIGLU_BWD;
};
template <> struct KT<GK_DGRAD_GATEUP> {
  static constexpr bool AK = true, BK_ = true;
  static constexpr int BSP = BS_SPLIT_K, EPI = EPI_STORE;
};
template <> struct KT<GK_WGRAD> {
  static constexpr bool AK = false, BK_ = false;
  static constexpr int BSP = BS_NONE, EPI = EPI_WGRAD_SPLIT;
};
template <> struct KT<GK_WGRAD_F32> {
  static constexpr bool AK = false, BK_ = false;
  static constexpr int BSP = BS_NONE, EPI = EPI_WGRAD_SPLIT_F32;
};
template <> struct KT<GK_ROUTER_LOGITS> {
  static constexpr bool AK = true, BK_ = false;
  static constexpr int BSP = BS_NONE, EPI = EPI_STORE_F32;
};
template <> struct KT<GK_ROUTER_DWR> {
  static constexpr bool AK = false, BK_ = false;
  static constexpr int BSP = BS_NONE, EPI = EPI_STORE;
};
template <> struct KT<GK_ROUTER_DX> {
  static constexpr bool AK = true, BK_ = true;
  static constexpr int BSP = BS_NONE, EPI = EPI_STORE;
};
template <> struct KT<GK_ROUTER_DWR_SPLIT> {
  static constexpr bool AK = false, BK_ = false;
  static constexpr int BSP = BS_NONE, EPI = EPI_STORE_F32;
};
// MXFP8 kinds: BS_DUAL_N only marks the gate/up tile layout for the epilogue
// (tile columns 0-127 gate, 128-255 up); the codes are one K-major matrix.
template <> struct KT<GK_MX_GATEUP> {
  static constexpr bool AK = true, BK_ = true;
  static constexpr int BSP = BS_DUAL_N, EPI = EPI_SWIGLU_FWD;
};
template <> struct KT<GK_MX_DOWN> {
  static constexpr bool AK = true, BK_ = true;
  static constexpr int BSP = BS_NONE, EPI = EPI_STORE;
};
template <> struct KT<GK_MX_DGRAD_DOWN> {
  static constexpr bool AK = true, BK_ = true;
  static constexpr int BSP = BS_NONE, EPI = EPI_SWIGLU_BWD;
};
template <> struct KT<GK_MX_DGRAD_GATEUP> {
  static constexpr bool AK = true, BK_ = true;
  static constexpr int BSP = BS_NONE, EPI = EPI_STORE;
};
template <> struct KT<GK_MX_WGRAD> {
  static constexpr bool AK = true, BK_ = true;
  static constexpr int BSP = BS_NONE, EPI = EPI_WGRAD_SPLIT;
};
template <> struct KT<GK_MX_WGRAD_F32> {
  static constexpr bool AK = true, BK_ = true;
  static constexpr int BSP = BS_NONE, EPI = EPI_WGRAD_SPLIT_F32;
};

// Kinds whose epilogue also writes the block-quantised output (MXFP8).
template <int KIND>
constexpr bool qout_of() { return KIND == GK_MX_GATEUP || KIND == GK_MX_DGRAD_DOWN; }

// One output tile of one group.
struct Tile {
  int e;      // group (expert)
  int m0;     // first row of the tile inside the group (RAG_M) or inside C (RAG_K)
  int n0;     // first column (for BS_DUAL_N: first f column of the gate/up pair)
  int mlim;   // rows of the tile that exist
  int row0;   // RAG_M: global row of tile row 0; RAG_K: global row of k = 0
  int klen;   // length of the K loop
};

// ---------------------------------------------------------------------------
// schedule: group offsets and per-group tile starts cached in LDS
// ---------------------------------------------------------------------------
struct Sched {
  int off[257];
  int ts[257];  // RAG_M: exclusive prefix of M tiles per group; RAG_K: group order
  int alt;      // RAG_K: groups taken longest first, rounds alternating (logical_tile)
};

// Fill the schedule; returns the number of tiles.  All threads must call it.
// SORT (the weight-gradient kinds): RAG_K groups are taken longest first.
template <int BM, int BNT, bool SORT = false>
__device__ int sched_setup(const GemmArgs& g, Sched& s) {
  const int tid = threadIdx.x;
  const int E = ngroups(g);
  if (g.offsets) {
    for (int e = tid; e <= E; e += blockDim.x) s.off[e] = g.offsets[e];
  } else if (g.kchunk > 0) {
    for (int e = tid; e <= E; e += blockDim.x) s.off[e] = min(e * g.kchunk, g.rows_total);
  } else if (tid == 0) {
    s.off[0] = 0;
    s.off[1] = g.rows_total;
  }
  __syncthreads();
  const int ntn = (g.N + BNT - 1) / BNT;
  if (g.ragged == RAG_M) {
    // wave 0 scans ceil(n_e / BM) over the groups, 4 groups per lane
    if (tid < kWave) {
      int c[4], sum = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        int e = tid * 4 + q;
        c[q] = (e < E) ? (s.off[e + 1] - s.off[e] + BM - 1) / BM : 0;
        sum += c[q];
      }
      int incl = sum;
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        int v = __shfl_up(incl, o, kWave);
        if (tid >= o) incl += v;
      }
      int run = incl - sum;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        int e = tid * 4 + q;
        if (e <= E) s.ts[e] = run;
        run += c[q];
      }
      if (tid == kWave - 1 && E == 256) s.ts[256] = incl;
    }
    __syncthreads();
    return s.ts[E] * ntn;
  }
  // RAG_K with skewed groups: every tile of a group costs about the same, and
  // when the longest group is more than twice the mean length (Zipf-like
  // expert loads) the groups are taken in order of decreasing length (ties
  // by index), so that the persistent workgroups start with the longest
  // tiles and the short ones fill in at the end; with the alternating rounds
  // of logical_tile this is close to a longest-first greedy schedule.  Group
  // e goes to place #{j: n_j > n_e, or n_j == n_e and j < e}.  Near-uniform
  // loads keep the index order (measured 0.4-1% faster there).
  if constexpr (SORT) {
    for (int e = tid; e < E; e += blockDim.x) {
      const int ne = s.off[e + 1] - s.off[e];
      int r = 0, mx = 0;
      long tot = 0;
      for (int j = 0; j < E; ++j) {
        const int nj = s.off[j + 1] - s.off[j];
        r += (nj > ne) | ((nj == ne) & (j < e));
        mx = max(mx, nj);
        tot += nj;
      }
      const bool skew = (long)mx * E > 2 * tot;
      s.ts[skew ? r : e] = e;
      if (e == 0) s.alt = skew;
    }
    __syncthreads();
  }
  const int ntm = (g.M + BM - 1) / BM;
  return E * ntm * ntn;
}

template <int BM, int BNT, bool SORT = false>
__device__ __forceinline__ Tile sched_decode(const GemmArgs& g, const Sched& s, int L) {
  const int ntn = (g.N + BNT - 1) / BNT;
  Tile t;
  if (g.ragged == RAG_M) {
    const int E = ngroups(g);
    int mt = L / ntn, nt = L - mt * ntn;
    int lo = 0, hi = E;  // largest e in [0,E) with ts[e] <= mt
    while (hi - lo > 1) {
      int mid = (lo + hi) >> 1;
      if (s.ts[mid] <= mt) lo = mid; else hi = mid;
    }
    t.e = lo;
    // Order of an expert's tiles (g.m_fast): the index with fewer tiles runs
    // fastest.  Consecutive tiles run together on one XCD, so an expert split
    // across two such runs has its shared panels read by both: with N-tiles
    // fastest each run reads every weight panel the expert's M-tiles need
    // (about twice the weight bytes when an expert has 2-5 M-tiles), with
    // M-tiles fastest each run reads at most all of the expert's activation
    // rows and only its own weight panels.  A weight panel and an activation
    // block of a tile both hold 256 x K values, so the cheaper split is the
    // one that can duplicate fewer of them.  Set for the forward GEMMs and
    // the MXFP8 ones; the bf16 input-gradient GEMMs measured 1-2% slower with
    // it at 128 experts and keep N-tiles fastest.
    const int ntm_e = s.ts[lo + 1] - s.ts[lo];
    if (g.m_fast && ntm_e < ntn) {
      const int local = L - s.ts[lo] * ntn;
      nt = local / ntm_e;
      mt = s.ts[lo] + (local - nt * ntm_e);
    }
    t.m0 = (mt - s.ts[lo]) * BM;
    int ne = s.off[lo + 1] - s.off[lo];
    t.mlim = min(BM, ne - t.m0);
    t.row0 = s.off[lo] + t.m0;
    t.n0 = nt * BNT;
    t.klen = g.K;
  } else {
    const int ntm = (g.M + BM - 1) / BM;
    int per = ntm * ntn;
    const int q = L / per;
    t.e = SORT ? s.ts[q] : q;
    int r = L - q * per;
    int mt = r / ntn, nt = r - mt * ntn;
    t.m0 = mt * BM;
    t.mlim = min(BM, g.M - t.m0);
    t.n0 = nt * BNT;
    t.row0 = s.off[t.e];
    t.klen = s.off[t.e + 1] - s.off[t.e];
  }
  return t;
}

// Logical tile for iteration `it` of workgroup blockIdx.x: with G = 8*P
// workgroups, workgroup b sits on XCD b % 8, and the P workgroups of one XCD
// take P consecutive logical tiles.  With `alt` (skewed groups taken longest
// first, Sched::alt) every other round runs through the workgroups in
// reverse, so that a workgroup that took one of the longest tiles of a round
// takes one of the shortest of the next; an XCD still takes P consecutive
// tiles.
__device__ __forceinline__ int logical_tile(int it, bool alt = false) {
  const int G = gridDim.x, b = blockIdx.x;
  int slot = (G % 8) ? b : (b & 7) * (G >> 3) + (b >> 3);
  if (alt && (it & 1)) slot = G - 1 - slot;
  return it * G + slot;
}

// ---------------------------------------------------------------------------
// epilogue: four consecutive columns of one output row
// ---------------------------------------------------------------------------
template <typename TS>
__device__ __forceinline__ void store4(TS* p, const float (&v)[4], bool acc) {
  if constexpr (sizeof(TS) == 2) {
    uint2 u;
    if (acc) {
      uint2 o = *reinterpret_cast<const uint2*>(p);
      u.x = pack_bf16x2(v[0] + __uint_as_float(o.x << 16), v[1] + __uint_as_float(o.x & 0xffff0000u));
      u.y = pack_bf16x2(v[2] + __uint_as_float(o.y << 16), v[3] + __uint_as_float(o.y & 0xffff0000u));
    } else {
      u.x = pack_bf16x2(v[0], v[1]);
      u.y = pack_bf16x2(v[2], v[3]);
    }
    *reinterpret_cast<uint2*>(p) = u;
  } else {
    float4 o = acc ? *reinterpret_cast<const float4*>(p) : make_float4(0.f, 0.f, 0.f, 0.f);
    *reinterpret_cast<float4*>(p) = make_float4(v[0] + o.x, v[1] + o.y, v[2] + o.z, v[3] + o.w);
  }
}

template <typename TS>
__device__ __forceinline__ void load4(const TS* p, float (&v)[4]) {
  if constexpr (sizeof(TS) == 2) {
    uint2 u = *reinterpret_cast<const uint2*>(p);
    v[0] = __uint_as_float(u.x << 16); v[1] = __uint_as_float(u.x & 0xffff0000u);
    v[2] = __uint_as_float(u.y << 16); v[3] = __uint_as_float(u.y & 0xffff0000u);
  } else {
    float4 u = *reinterpret_cast<const float4*>(p);
    v[0] = u.x; v[1] = u.y; v[2] = u.z; v[3] = u.w;
  }
}

// Scalar store of the first nv of four values (router shapes whose width is
// not a multiple of 4).
template <typename TS>
__device__ __forceinline__ void store_part(TS* p, const float (&v)[4], int nv, bool acc) {
  for (int q = 0; q < nv; ++q) {
    float o = acc ? St<TS>::load(p + q) : 0.0f;
    St<TS>::store(p + q, v[q] + o);
  }
}

// m: row inside the tile (< t.mlim); n: output column (f column for the
// SwiGLU kinds), n < N.  u: the up-projection values for EPI_SWIGLU_FWD.
// The SwiGLU and weight-gradient kinds always have n + 3 < N and 4-aligned
// rows; the plain stores may end in a partial quad.
// PARTIAL: the engine may hand over quads that end past N or rows whose width
// is not a multiple of 4 (SIMT engine on router shapes); the MFMA engine only
// takes widths that are multiples of 8 and never does.
template <int EPI, typename TS, bool PARTIAL = true>
__device__ __forceinline__ void epilogue4(const GemmArgs& g, const Tile& t, int m, int n,
                                          const float (&v)[4], const float (&u)[4]) {
  if constexpr (EPI == EPI_STORE_F32) {
    long row = (g.ragged == RAG_M) ? (long)t.row0 + m : (long)t.m0 + m;
    float* p = static_cast<float*>(g.c0) + (g.ragged == RAG_M ? 0 : (long)t.e * g.c_es) + row * g.ldc + n;
    if (!PARTIAL || (n + 4 <= g.N && (g.ldc & 3) == 0))
      *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    else
      store_part(p, v, min(4, g.N - n), false);
  } else if constexpr (EPI == EPI_STORE) {
    long row = (g.ragged == RAG_M) ? (long)t.row0 + m : (long)t.m0 + m;
    TS* p = static_cast<TS*>(g.c0) + (g.ragged == RAG_M ? 0 : (long)t.e * g.c_es) + row * g.ldc + n;
    if (!PARTIAL || (n + 4 <= g.N && (g.ldc & 3) == 0))
      store4(p, v, g.accumulate != 0);
    else
      store_part(p, v, min(4, g.N - n), g.accumulate != 0);
  } else if constexpr (EPI == EPI_WGRAD_SPLIT) {
    long row = (long)t.m0 + m;
    TS* p;
    if (n < g.c_split)
      p = static_cast<TS*>(g.c0) + (long)t.e * g.c_es + row * g.ldc + n;
    else
      p = static_cast<TS*>(g.c1) + (long)t.e * g.c_es + row * g.ldc + (n - g.c_split);
    store4(p, v, g.accumulate != 0);
  } else if constexpr (EPI == EPI_WGRAD_SPLIT_F32) {
    long row = (long)t.m0 + m;
    float* p;
    if (n < g.c_split)
      p = static_cast<float*>(g.c0) + (long)t.e * g.c_es + row * g.ldc + n;
    else
      p = static_cast<float*>(g.c1) + (long)t.e * g.c_es + row * g.ldc + (n - g.c_split);
    store4(p, v, g.accumulate != 0);
  } else if constexpr (EPI == EPI_SWIGLU_FWD) {
    long off = ((long)t.row0 + m) * g.ldc + n;
    float a[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) a[q] = silu_f(v[q]) * u[q];
    store4(static_cast<TS*>(g.c0) + off, v, false);
    store4(static_cast<TS*>(g.c1) + off, u, false);
    store4(static_cast<TS*>(g.c2) + off, a, false);
  } else if constexpr (EPI == EPI_SWIGLU_BWD) {
    long row = (long)t.row0 + m;
    float hg[4], hu[4], dg[4], du[4];
    load4(static_cast<const TS*>(g.h0) + row * g.ldh + n, hg);
    load4(static_cast<const TS*>(g.h1) + row * g.ldh + n, hu);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float s = sigmoid_f(hg[q]);
      du[q] = v[q] * hg[q] * s;
      dg[q] = v[q] * hu[q] * s * (1.0f + hg[q] * (1.0f - s));
    }
    TS* p = static_cast<TS*>(g.c0) + row * g.ldc + n;
    store4(p, dg, false);
    store4(p + g.c_split, du, false);
  }
}

// ---------------------------------------------------------------------------
// MFMA engines (bf16 and MXFP8): shared stage ring
// ---------------------------------------------------------------------------
namespace mf {

// Tiles of 256x256 outputs; each stage holds 128 bytes of K for every tile
// row of both operands (64 bf16 or 128 e4m3 values): K-contiguous rows are
// fetched as whole 128-byte lines, which the buffer->LDS path moves about
// twice as fast as half lines.  Two stages (128 KiB) double-buffer the ring.
constexpr int BM = 256, BN = 256, NST = 2, NTHR = 256;
constexpr int ROWB = 128;             // bytes of K per tile row per stage
constexpr int BK = ROWB / 2;          // bf16 elements of K per stage
constexpr int OPB = BM * ROWB;        // bytes of one operand in one stage (32 KiB)
constexpr int STAGE = 2 * OPB;        // A then B
constexpr int DMA_PER_OP = 8;         // buffer->LDS loads per wave per operand per stage

typedef __attribute__((ext_vector_type(4))) int i32x4_t;
typedef __attribute__((ext_vector_type(4))) short i16x4_t;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

// Raw buffer resource over [base, base + bytes): loads beyond it return 0
// (and write 0 into LDS for the LDS-targeted form).
__device__ __forceinline__ i32x4_t make_rsrc(const void* base, long long bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint32_t n = bytes <= 0 ? 0u : (bytes >= 0xffffffffLL ? 0xffffffffu : (uint32_t)bytes);
  i32x4_t r;
  r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  r.y = __builtin_amdgcn_readfirstlane((int)((b >> 32) & 0xffffu));
  r.z = __builtin_amdgcn_readfirstlane((int)n);
  r.w = 0x00020000;
  return r;
}

// 16 bytes per lane from the buffer straight into LDS at lds_addr + 16*lane.
// Issued as inline asm so that the compiler's LDS-DMA tracking does not turn
// the ring's waits into full ones; completion is awaited explicitly with
// vmcnt before the barrier of the stage that reads the data.
__device__ __forceinline__ void dma16(i32x4_t rsrc, uint32_t lds_addr, uint32_t voff, uint32_t soff) {
  i32x4_t r;
  r.x = __builtin_amdgcn_readfirstlane(rsrc.x);
  r.y = __builtin_amdgcn_readfirstlane(rsrc.y);
  r.z = __builtin_amdgcn_readfirstlane(rsrc.z);
  r.w = __builtin_amdgcn_readfirstlane(rsrc.w);
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr);
  const uint32_t so = __builtin_amdgcn_readfirstlane(soff);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :: "s"(m0), "v"(voff), "s"(r), "s"(so) : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

__device__ __forceinline__ uint32_t lds_u32(const void* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char*)p);
}

// LDS layouts of one operand stage (32 KiB), in 16-byte chunks.
//  K-major ("KM": rows are M or N, 128 bytes of K per row = 8 chunks):
//    byte = row*128 + ((chunk ^ km_swz(row)) << 4)
//  MN-major ("MN": rows are k (64 of them), two panels of 128 columns):
//    byte = panel*16384 + k*256 + (((col/8) ^ mn_swz(k)) << 4) + 2*(col & 7)
// Both swizzles were chosen by measuring the LDS bank-conflict counter on
// gfx950 for the fragment reads below (32 rows x one chunk per half-wave
// with ds_read_b128; 4 k-rows x 4 column quads per 16 lanes with
// ds_read_b64_tr_b16): both read conflict-free.
__device__ __forceinline__ int km_swz(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int mn_swz(int k) { return (4 * (k & 3)) ^ (2 * ((k >> 1) & 1)); }
__device__ __forceinline__ int km_off(int row, int chunk) {
  return row * ROWB + ((chunk ^ km_swz(row)) << 4);
}
__device__ __forceinline__ int mn_off(int k, int col) {
  const int panel = col >> 7, cc = col & 127;
  return panel * 16384 + k * 256 + (((cc >> 3) ^ mn_swz(k)) << 4) + 2 * (cc & 7);
}

// Per-wave DMA plan of one operand for one tile.  Block i of the wave reads
// at per-lane offset (i odd ? v1 : v0) plus the uniform offset i*bstep plus
// the stage's K offset; both uniform parts travel in the instruction's
// scalar offset, which the buffer range check includes.
struct Plan {
  i32x4_t rs0, rs1;   // resources (rs1: second source: SPLIT_K, or MN panel of waves 2-3)
  uint32_t v0, v1;    // per-lane byte offsets of the wave's even / odd blocks
  uint32_t bstep;     // bytes between consecutive blocks of the wave
  uint32_t kstep;     // bytes the source advances per stage
  int split_stage;    // SPLIT_K: first stage read from rs1 (else a large value)
};
// LDS offset of the wave's i-th block inside the operand stage (DPO blocks
// per wave).
template <int DPO = DMA_PER_OP>
__device__ __forceinline__ uint32_t plan_lds(int wave, int i) { return (uint32_t)(wave * DPO + i) * 1024u; }

// K-major operand: row r of the tile is a row of `ldb` bytes at base + r*ldb;
// `bytes` are readable from base.  Block blk = wave*DPO + i holds rows
// 8*blk .. 8*blk+7, 128 bytes each; the swizzle of a row depends only on the
// parity of its block and on the lane.
template <int DPO = DMA_PER_OP>
__device__ __forceinline__ void plan_km(Plan& P, const void* base, long long bytes, const void* base1,
                                        long long bytes1, int split_stage, long ldb, int wave,
                                        int lane) {
  P.rs0 = make_rsrc(base, bytes);
  P.rs1 = make_rsrc(base1 ? base1 : base, base1 ? bytes1 : bytes);
  const int row0 = wave * DPO * 8 + (lane >> 3);
  P.v0 = (uint32_t)(row0 * ldb + (((lane & 7) ^ km_swz(row0)) * 16));
  P.v1 = (uint32_t)(row0 * ldb + (((lane & 7) ^ km_swz(row0 + 8)) * 16));
  P.bstep = (uint32_t)(8 * ldb);
  P.kstep = ROWB;
  P.split_stage = split_stage;
}

// MN-major operand (bf16): k-rows of a matrix with ld elements; panel p of
// the tile starts at base_p (its column 0 at k = 0); bytes_p readable from
// base_p.  Blocks 0-15 fill panel 0 (the first NWV/2 waves), 16-31 panel 1;
// block blk holds k-rows 4*(blk%16) .. +3, 256 bytes each.
template <int DPO = DMA_PER_OP, int NWV = 4>
__device__ __forceinline__ void plan_mn(Plan& P, const void* base0, long long bytes0,
                                        const void* base1, long long bytes1, long ld, int wave,
                                        int lane) {
  P.rs0 = make_rsrc(base0, bytes0);
  P.rs1 = make_rsrc(base1, bytes1);
  const int k0 = (wave % (NWV / 2)) * DPO * 4 + (lane >> 4);
  P.v0 = P.v1 = (uint32_t)(k0 * ld * 2 + (((lane & 15) ^ mn_swz(k0)) * 16));
  P.bstep = (uint32_t)(4 * ld * 2);
  P.kstep = (uint32_t)(BK * ld * 2);
  P.split_stage = 1 << 30;
}

// Issue the wave's DMA blocks of one operand for stage kt into the LDS
// operand region at lds_base.
template <bool MN, int DPO = DMA_PER_OP, int NWV = 4>
__device__ __forceinline__ void issue(const Plan& P, int kt, uint32_t lds_base, int wave) {
  i32x4_t rs;
  uint32_t soff;
  if constexpr (MN) {
    rs = (wave >= NWV / 2) ? P.rs1 : P.rs0;
    soff = (uint32_t)kt * P.kstep;
  } else {
    const bool second = kt >= P.split_stage;
    rs = second ? P.rs1 : P.rs0;
    soff = (uint32_t)(second ? kt - P.split_stage : kt) * P.kstep;
  }
#pragma unroll
  for (int i = 0; i < DPO; ++i)
    dma16(rs, lds_base + plan_lds<DPO>(wave, i), (i & 1) ? P.v1 : P.v0, soff + (uint32_t)i * P.bstep);
}

// Block i (0..DPO-1) of the wave's DMA of one operand for stage kt.
template <bool MN, int DPO = DMA_PER_OP, int NWV = 4>
__device__ __forceinline__ void issue_one(const Plan& P, int kt, uint32_t lds_base, int wave, int i) {
  i32x4_t rs;
  uint32_t soff;
  if constexpr (MN) {
    rs = (wave >= NWV / 2) ? P.rs1 : P.rs0;
    soff = (uint32_t)kt * P.kstep;
  } else {
    const bool second = kt >= P.split_stage;
    rs = second ? P.rs1 : P.rs0;
    soff = (uint32_t)(second ? kt - P.split_stage : kt) * P.kstep;
  }
  dma16(rs, lds_base + plan_lds<DPO>(wave, i), (i & 1) ? P.v1 : P.v0, soff + (uint32_t)i * P.bstep);
}

// L2 prefetch: one 4-byte buffer->LDS load per 128-byte line of a future
// stage pulls the line into L2 (the bytes land in a scratch word that is
// never read), so that the stage's own DMA, issued two stages later, hits in
// L2 instead of waiting on HBM.  The prefetch is shared out among the tiles
// that read the same lines at about the same time: the N-tiles of an M-block
// share its A rows, the M-tiles of an expert its K-contiguous weight rows,
// and consecutive tiles run together on one XCD.  A tile prefetches one
// quarter of each K-contiguous operand's 256 rows (quarter = its N-tile
// index for A, its M-tile index within the expert for B, modulo 4) with one
// load per wave (wave 0: A, wave 2: B).  Measured against every tile
// prefetching all of its rows (four loads per stage): 1-4% faster GEMMs,
// the bigger gains on the input gradients, where both operands are
// prefetched; the L2 request rate is what bounds these loops.
__device__ __forceinline__ void pf4(i32x4_t rsrc, uint32_t lds_addr, uint32_t voff, uint32_t soff) {
  i32x4_t r;
  r.x = __builtin_amdgcn_readfirstlane(rsrc.x);
  r.y = __builtin_amdgcn_readfirstlane(rsrc.y);
  r.z = __builtin_amdgcn_readfirstlane(rsrc.z);
  r.w = __builtin_amdgcn_readfirstlane(rsrc.w);
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr);
  const uint32_t so = __builtin_amdgcn_readfirstlane(soff);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, %3 offen lds"
               :: "s"(m0), "v"(voff), "s"(r), "s"(so) : "memory");
}
constexpr int PF_PER_STAGE = 1;   // prefetch loads per prefetching wave per stage
constexpr int PF_AHEAD = 2;       // stages between a line's prefetch and its DMA

// Per-lane offset of the prefetch of one quarter (q mod 4) of a K-contiguous
// operand's 256 tile rows, ld_bytes apart.
__device__ __forceinline__ uint32_t pf_quarter(int q, int lane, long ld_bytes) {
  return (uint32_t)((64 * (q & 3) + lane) * ld_bytes);
}
// The prefetch load of stage kt of a K-contiguous operand plan.
__device__ __forceinline__ void issue_pf(const Plan& P, uint32_t voff, int kt, uint32_t sink) {
  const bool second = kt >= P.split_stage;
  pf4(second ? P.rs1 : P.rs0, sink, voff, (uint32_t)(second ? kt - P.split_stage : kt) * P.kstep);
}

// MFMA fragment (8 consecutive k of one row/column) from an operand stage.
// row: M or N index inside the tile; s: k16 step inside the stage (0-3).
template <bool MN>
__device__ __forceinline__ bf16x8_t frag(const char* op, int rowblk, int s, int lane) {
  if constexpr (!MN) {
    const int row = rowblk + (lane & 31);
    return *reinterpret_cast<const bf16x8_t*>(op + km_off(row, 2 * s + (lane >> 5)));
  } else {
    // ds_read_b64_tr_b16: within each 16-lane group the lanes' 8-byte reads
    // (4 k-rows x 4 column quads) come back transposed, so lane i of the
    // group receives column i at 4 consecutive k.
    const int g = lane >> 4, r = lane & 15;
    const int k = 16 * s + 8 * (g >> 1) + (r >> 2);
    const int col = rowblk + 16 * (g & 1) + 4 * (r & 3);
    const char* p = op + mn_off(k, col);
    i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p));
    i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p + 4 * 256));
    typedef __attribute__((ext_vector_type(8))) short i16x8_t;
    i16x8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8_t, v);
  }
}

// Fragments of one k16 step of stage kt: 4 A fragments (rows wm*128 + 32i)
// and 4 B fragments (columns of wave column wn; gate/up pairs when DUAL).
template <bool AMN, bool BMN, bool DUAL>
__device__ __forceinline__ void load_frags(const char* smem, int kt, int s, int wm, int wn,
                                           int lane, bf16x8_t (&fa)[4], bf16x8_t (&fb)[4]) {
  const char* As = smem + (kt & (NST - 1)) * STAGE;
  const char* Bs = As + OPB;
#pragma unroll
  for (int i = 0; i < 4; ++i) fa[i] = frag<AMN>(As, wm * 128 + i * 32, s, lane);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int col = DUAL ? ((j >> 1) * 128 + wn * 64 + (j & 1) * 32) : (wn * 128 + j * 32);
    fb[j] = frag<BMN>(Bs, col, s, lane);
  }
}

// MFMAs 2q and 2q+1 of a k16 step (row block q/2, column blocks 2(q%2), +1).
__device__ __forceinline__ void mfma_pair(f32x16_t (&acc)[4][4], const bf16x8_t (&fa)[4],
                                          const bf16x8_t (&fb)[4], int q) {
  const int i = q >> 1, j = 2 * (q & 1);
  acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[j], fa[i], acc[i][j], 0, 0, 0);
  acc[i][j + 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[j + 1], fa[i], acc[i][j + 1], 0, 0, 0);
}

// One fragment of a k16 step: p = 0-3 the B fragments (columns of wave
// column wn; gate/up pairs when DUAL), p = 4-7 the A fragments (rows
// wm*128 + 32(p-4)).  The B fragments come first: the MFMAs of row block 0
// need all four of them and only the first A fragment.
template <bool AMN, bool BMN, bool DUAL>
__device__ __forceinline__ void load_frag(const char* smem, int kt, int s, int wm, int wn, int lane,
                                          bf16x8_t (&fa)[4], bf16x8_t (&fb)[4], int p) {
  const char* As = smem + (kt & (NST - 1)) * STAGE;
  const char* Bs = As + OPB;
  if (p < 4) {
    const int col = DUAL ? ((p >> 1) * 128 + wn * 64 + (p & 1) * 32) : (wn * 128 + p * 32);
    fb[p] = frag<BMN>(Bs, col, s, lane);
  } else {
    fa[p - 4] = frag<AMN>(As, wm * 128 + (p - 4) * 32, s, lane);
  }
}

// MFMA m (0-15) of a k16 step: row block m/4, column block m%4; FIRST: the
// tile's first step, from a zero accumulator.
template <bool FIRST>
__device__ __forceinline__ void mfma_one(f32x16_t (&acc)[4][4], const bf16x8_t (&fa)[4],
                                         const bf16x8_t (&fb)[4], int m) {
  const int i = m >> 2, j = m & 3;
  acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[j], fa[i], FIRST ? f32x16_t{} : acc[i][j],
                                                      0, 0, 0);
}

// s_waitcnt with lgkmcnt(0) and the other counters left alone (gfx9 encoding).
constexpr int kLgkm0 = 0xC07F;

// A k16 step without DMA: the 16 MFMAs of fragment set (ca, cb), and the
// reads of the next step's set into (na, nb) at (kt, s).  Row block 0 goes
// first (it needs the first reads of the current set); then one wait for the
// rest of the current set, after which the next set's reads go out two
// between each of the next MFMAs, so that the last of them has about ten
// MFMAs to land before the next step's wait.
template <bool AMN, bool BMN, bool DUAL, bool FIRST>
__device__ __forceinline__ void kstep(f32x16_t (&acc)[4][4], const bf16x8_t (&ca)[4],
                                      const bf16x8_t (&cb)[4], bf16x8_t (&na)[4], bf16x8_t (&nb)[4],
                                      const char* smem, int kt, int s, int wm, int wn, int lane) {
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int m = 0; m < 4; ++m) mfma_one<FIRST>(acc, ca, cb, m);
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(kLgkm0);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int p = 0; p < 8; ++p) load_frag<AMN, BMN, DUAL>(smem, kt, s, wm, wn, lane, na, nb, p);
#pragma unroll
  for (int m = 4; m < 16; ++m) mfma_one<FIRST>(acc, ca, cb, m);
#pragma unroll
  for (int i = 0; i < 6; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // DS reads
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 6, 0);
  __builtin_amdgcn_sched_barrier(0);
}


// Operand plans of one tile for each bf16 GEMM kind (NWV waves, DPO DMA
// blocks per wave and operand).
template <int KIND, int DPO = DMA_PER_OP, int NWV = 4>
__device__ __forceinline__ void plan_tile(const GemmArgs& g, const Tile& t, int wave, int lane,
                                          Plan& pa, Plan& pb) {
  const bf16_t* A = static_cast<const bf16_t*>(g.a);
  const bf16_t* B0 = static_cast<const bf16_t*>(g.b0);
  const bf16_t* B1 = static_cast<const bf16_t*>(g.b1);
  constexpr int BSP = KT<KIND>::BSP;
  // ---- A ----
  if constexpr (KT<KIND>::AK) {
    // rows t.row0 .. t.row0 + mlim of A (global rows), K contiguous: the
    // range ends at the tile's last row that exists, so the DMA lanes of the
    // rows past it (a ragged tail) read zeros without a memory request
    const bf16_t* base = A + (long)t.row0 * g.lda;
    const long long bytes = (long long)t.mlim * g.lda * 2;
    plan_km<DPO>(pa, base, bytes, nullptr, 0, 1 << 30, g.lda * 2, wave, lane);
  } else {
    // k-rows t.row0 .. t.row0 + klen of A, M contiguous; columns t.m0 + 128 p
    const bf16_t* b0 = A + (long)t.row0 * g.lda + t.m0;
    const long long avail = (long long)t.klen * g.lda * 2;
    plan_mn<DPO, NWV>(pa, b0, avail - 2LL * t.m0, b0 + 128, avail - 2LL * (t.m0 + 128), g.lda, wave, lane);
  }
  // ---- B ----
  if constexpr (KT<KIND>::BK_) {
    // B[n][k] per group, rows t.n0..
    const long e_off = (long)t.e * g.b_es + (long)t.n0 * g.ldb;
    const long long bytes = ((long long)g.N - t.n0) * g.ldb * 2;
    if constexpr (BSP == BS_SPLIT_K)
      plan_km<DPO>(pb, B0 + e_off, bytes, B1 + e_off, bytes, g.b_split / BK, g.ldb * 2, wave, lane);
    else
      plan_km<DPO>(pb, B0 + e_off, bytes, nullptr, 0, 1 << 30, g.ldb * 2, wave, lane);
  } else if (g.ragged == RAG_M) {
    // B[k][n] per group (weights), N contiguous
    const bf16_t* w0 = B0 + (long)t.e * g.b_es;
    const long long total = (long long)g.K * g.ldb * 2;
    if constexpr (BSP == BS_DUAL_N) {
      const bf16_t* w1 = B1 + (long)t.e * g.b_es;
      plan_mn<DPO, NWV>(pb, w0 + t.n0, total - 2LL * t.n0, w1 + t.n0, total - 2LL * t.n0, g.ldb, wave, lane);
    } else {
      plan_mn<DPO, NWV>(pb, w0 + t.n0, total - 2LL * t.n0, w0 + t.n0 + 128, total - 2LL * (t.n0 + 128),
              g.ldb, wave, lane);
    }
  } else {
    // B[krow][n] with global k-rows t.row0 .. t.row0 + klen
    const bf16_t* b0 = B0 + (long)t.row0 * g.ldb + t.n0;
    const long long avail = (long long)t.klen * g.ldb * 2;
    plan_mn<DPO, NWV>(pb, b0, avail - 2LL * t.n0, b0 + 128, avail - 2LL * (t.n0 + 128), g.ldb, wave, lane);
  }
}

// Float32 staging slice of one wave: 32 rows x 128 columns (16 KiB), 16-byte
// chunks XOR-swizzled by row so that both the accumulator writes (32 rows,
// one chunk) and the row reads (one row, 16 chunks) avoid bank conflicts.
constexpr int EPI_SLICE = 16384;
__device__ __forceinline__ int stage_off(int r, int chunk) { return r * 512 + ((chunk ^ (r & 31)) << 4); }
// bf16 staging of the same block: 32 rows x 128 columns, 256 bytes a row,
// 16-byte chunk c of row r at chunk c ^ (r & 15).
__device__ __forceinline__ int stage_bf_off(int r, int chunk) { return r * 256 + ((chunk ^ (r & 15)) << 4); }

// Epilogue of one 8-column piece: v = tile values (gate for the SwiGLU
// forward), u = up values (SwiGLU forward only).  grow: global row (RAG_M)
// or row inside the group's C (RAG_K); n: output column.
template <int EPI>
__device__ __forceinline__ void epi8(const GemmArgs& g, const Tile& t, long row, int n,
                                     const float (&v)[8], const float (&u)[8]) {
  if constexpr (EPI == EPI_STORE_F32) {
    float* p = static_cast<float*>(g.c0) + (g.ragged == RAG_M ? 0 : (long)t.e * g.c_es) + row * g.ldc + n;
    store8_nt(p, v);
  } else if constexpr (EPI == EPI_STORE || EPI == EPI_WGRAD_SPLIT) {
    bf16_t* p;
    if constexpr (EPI == EPI_WGRAD_SPLIT) {
      if (n < g.c_split)
        p = static_cast<bf16_t*>(g.c0) + (long)t.e * g.c_es + row * g.ldc + n;
      else
        p = static_cast<bf16_t*>(g.c1) + (long)t.e * g.c_es + row * g.ldc + (n - g.c_split);
    } else {
      p = static_cast<bf16_t*>(g.c0) + (g.ragged == RAG_M ? 0 : (long)t.e * g.c_es) + row * g.ldc + n;
    }
    if (g.accumulate) {
      float o[8], w[8];
      load8(p, o);
#pragma unroll
      for (int q = 0; q < 8; ++q) w[q] = v[q] + o[q];
      store8_nt(p, w);
    } else {
      store8_nt(p, v);
    }
  } else if constexpr (EPI == EPI_WGRAD_SPLIT_F32) {
    float* p;
    if (n < g.c_split)
      p = static_cast<float*>(g.c0) + (long)t.e * g.c_es + row * g.ldc + n;
    else
      p = static_cast<float*>(g.c1) + (long)t.e * g.c_es + row * g.ldc + (n - g.c_split);
    if (g.accumulate) {
      const float4 o0 = *reinterpret_cast<const float4*>(p);
      const float4 o1 = *reinterpret_cast<const float4*>(p + 4);
      const float w[8] = {v[0] + o0.x, v[1] + o0.y, v[2] + o0.z, v[3] + o0.w,
                          v[4] + o1.x, v[5] + o1.y, v[6] + o1.z, v[7] + o1.w};
      store8_nt(p, w);
    } else {
      store8_nt(p, v);
    }
  } else if constexpr (EPI == EPI_SWIGLU_FWD) {
    const long off = row * g.ldc + n;
    float a[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) a[q] = silu_f(v[q]) * u[q];
    store8_nt(static_cast<bf16_t*>(g.c0) + off, v);
    store8_nt(static_cast<bf16_t*>(g.c1) + off, u);
    store8_nt(static_cast<bf16_t*>(g.c2) + off, a);
  } else if constexpr (EPI == EPI_SWIGLU_BWD) {
    float hg[8], hu[8], dg[8], du[8];
    load8(static_cast<const bf16_t*>(g.h0) + row * g.ldh + n, hg);
    load8(static_cast<const bf16_t*>(g.h1) + row * g.ldh + n, hu);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float sg = sigmoid_f(hg[q]);
      du[q] = v[q] * hg[q] * sg;
      dg[q] = v[q] * hu[q] * sg * (1.0f + hg[q] * (1.0f - sg));
    }
    bf16_t* p = static_cast<bf16_t*>(g.c0) + row * g.ldc + n;
    store8_nt(p, dg);
    store8_nt(p + g.c_split, du);
  }
}

// Output element (row, n) of a plain bf16 store or of a split weight-gradient
// store (bf16 or float).
template <int EPI>
__device__ __forceinline__ auto epi_ptr(const GemmArgs& g, const Tile& t, long row, int n) {
  using T = std::conditional_t<EPI == EPI_WGRAD_SPLIT_F32, float, bf16_t>;
  if constexpr (EPI == EPI_WGRAD_SPLIT || EPI == EPI_WGRAD_SPLIT_F32) {
    if (n < g.c_split) return static_cast<T*>(g.c0) + (long)t.e * g.c_es + row * g.ldc + n;
    return static_cast<T*>(g.c1) + (long)t.e * g.c_es + row * g.ldc + (n - g.c_split);
  } else {
    return static_cast<T*>(g.c0) + (g.ragged == RAG_M ? 0 : (long)t.e * g.c_es) + row * g.ldc + n;
  }
}

// One 32-row block (I) of a wave's epilogue; a separate instantiation per
// block keeps every accumulator index static, so the accumulators stay in
// registers however large the block's code gets.
template <int KIND, int I>
__device__ __forceinline__ void epilogue_block(const GemmArgs& g, const Tile& t, char* slice,
                                               f32x16_t (&acc)[4][4], int wm, int wn, int lane) {
  constexpr int EPI = KT<KIND>::EPI;
  constexpr bool DUAL = KT<KIND>::BSP == BS_DUAL_N;
  {
    // keep each block's loads inside its own pass (registers)
    __builtin_amdgcn_sched_barrier(0);
    uint4 hg[8], hu[8];
    // Stores that add to the output (router dx, accumulated gradients): the
    // old values of the block's rows are loaded here, so that their latency
    // overlaps the staging instead of serialising the store loop (bf16: hg,
    // float: hg then hu).
    constexpr bool PRE_ACC =
        EPI == EPI_STORE || EPI == EPI_WGRAD_SPLIT || EPI == EPI_WGRAD_SPLIT_F32;
    const bool pre_acc = PRE_ACC && g.accumulate;
    if constexpr (PRE_ACC) {
      if (pre_acc) {
#pragma unroll
        for (int it = 0; it < 8; ++it) {
          const int m = wm * 128 + I * 32 + it * 4 + (lane >> 4);
          const int n = t.n0 + wn * 128 + (lane & 15) * 8;
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
      for (int it = 0; it < 8; ++it) {
        const int m = wm * 128 + I * 32 + it * 4 + (lane >> 4);
        const int n = t.n0 + wn * 128 + (lane & 15) * 8;
        hg[it] = hu[it] = make_uint4(0, 0, 0, 0);
        if (m < t.mlim && n < g.N) {
          const long off = ((long)t.row0 + m) * g.ldh + n;
          hg[it] = *reinterpret_cast<const uint4*>(static_cast<const bf16_t*>(g.h0) + off);
          hu[it] = *reinterpret_cast<const uint4*>(static_cast<const bf16_t*>(g.h1) + off);
        }
      }
    }
    // Plain bf16 stores that do not accumulate: the accumulators are rounded
    // to bf16 in registers and staged as bf16 (half the LDS traffic of the
    // float32 staging below; the same rounding, so the same bytes).  Not in
    // the MXFP8 engine, whose registers this second store path overflows.
    constexpr bool MX_KIND = (KIND >= GK_MX_GATEUP && KIND <= GK_MX_DGRAD_GATEUP) ||
                             KIND == GK_MX_WGRAD || KIND == GK_MX_WGRAD_F32;
    constexpr bool BF_STAGE = !MX_KIND && (EPI == EPI_STORE || EPI == EPI_WGRAD_SPLIT);
    if constexpr (BF_STAGE) {
      if (!g.accumulate) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int grp = 0; grp < 4; ++grp) {
            const int r = lane & 31;
            const uint2 w = make_uint2(pack_bf16x2(acc[I][j][4 * grp], acc[I][j][4 * grp + 1]),
                                       pack_bf16x2(acc[I][j][4 * grp + 2], acc[I][j][4 * grp + 3]));
            *reinterpret_cast<uint2*>(slice + stage_bf_off(r, 4 * j + grp) + 8 * (lane >> 5)) = w;
          }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll 2
        for (int it = 0; it < 8; ++it) {
          const int r = it * 4 + (lane >> 4);
          const int c = (lane & 15) * 8;
          const int m = wm * 128 + I * 32 + r;
          const u32x4_t v = *reinterpret_cast<const u32x4_t*>(slice + stage_bf_off(r, lane & 15));
          const int n = t.n0 + wn * 128 + c;
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
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        const int r = lane & 31;
        const int chunk = j * 8 + 2 * grp + (lane >> 5);
        f32x4_t v = {acc[I][j][4 * grp], acc[I][j][4 * grp + 1], acc[I][j][4 * grp + 2],
                     acc[I][j][4 * grp + 3]};
        *reinterpret_cast<f32x4_t*>(slice + stage_off(r, chunk)) = v;
      }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    // rows of this block: tile rows wm*128 + i*32 + r
    if constexpr (DUAL) {
      // slice columns 0..63: gate, 64..127: up, for f columns n0 + wn*64 + c
#pragma unroll 2
      for (int it = 0; it < 4; ++it) {
        const int r = it * 8 + (lane >> 3);
        const int c = (lane & 7) * 8;
        const int m = wm * 128 + I * 32 + r;
        float v[8], u[8];
        const f32x4_t a0 = *reinterpret_cast<const f32x4_t*>(slice + stage_off(r, c >> 2));
        const f32x4_t a1 = *reinterpret_cast<const f32x4_t*>(slice + stage_off(r, (c >> 2) + 1));
        const f32x4_t b0 = *reinterpret_cast<const f32x4_t*>(slice + stage_off(r, (c >> 2) + 16));
        const f32x4_t b1 = *reinterpret_cast<const f32x4_t*>(slice + stage_off(r, (c >> 2) + 17));
#pragma unroll
        for (int q = 0; q < 4; ++q) { v[q] = a0[q]; v[q + 4] = a1[q]; u[q] = b0[q]; u[q + 4] = b1[q]; }
        const int n = t.n0 + wn * 64 + c;
        const bool ok = m < t.mlim && n < g.N;  // uniform over each 4-lane block
        static_assert(EPI == EPI_SWIGLU_FWD, "paired gate/up columns feed the SwiGLU forward");
        if (ok) {
          float a[8];
#pragma unroll
          for (int q = 0; q < 8; ++q) a[q] = silu_f(v[q]) * u[q];
          const long row = (long)t.row0 + m;
          const long off = row * g.ldc + n;
          store8_nt(static_cast<bf16_t*>(g.c0) + off, v);
          store8_nt(static_cast<bf16_t*>(g.c1) + off, u);
          store8_nt(static_cast<bf16_t*>(g.c2) + off, a);
          if constexpr (qout_of<KIND>()) {
            float ar[8];
            round_bf16_8(a, ar);
            quant8_store(ar, g.q0 + off, g.qs + mx_scale_at(row, n, g.qs_pitch), lane);
          }
        }
      }
    } else if constexpr (EPI == EPI_SWIGLU_BWD) {
      // Hg, Hu of the block's rows were loaded before the accumulators went
      // to the slice (hg / hu below), so their latency overlaps the staging.
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int r = it * 4 + (lane >> 4);
        const int c = (lane & 15) * 8;
        const int m = wm * 128 + I * 32 + r;
        const int n = t.n0 + wn * 128 + c;
        if (m < t.mlim && n < g.N) {
          const f32x4_t a0 = *reinterpret_cast<const f32x4_t*>(slice + stage_off(r, c >> 2));
          const f32x4_t a1 = *reinterpret_cast<const f32x4_t*>(slice + stage_off(r, (c >> 2) + 1));
          float v[8], h0[8], h1[8], dg[8], du[8];
#pragma unroll
          for (int q = 0; q < 4; ++q) { v[q] = a0[q]; v[q + 4] = a1[q]; }
          unpack8(hg[it], h0);
          unpack8(hu[it], h1);
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const float sg = sigmoid_f(h0[q]);
            du[q] = v[q] * h0[q] * sg;
            dg[q] = v[q] * h1[q] * sg * (1.0f + h0[q] * (1.0f - sg));
          }
          const long row = (long)t.row0 + m;
          bf16_t* p = static_cast<bf16_t*>(g.c0) + row * g.ldc + n;
          store8_nt(p, dg);
          store8_nt(p + g.c_split, du);
          if constexpr (qout_of<KIND>()) {
            float r[8];
            round_bf16_8(dg, r);
            quant8_store(r, g.q0 + row * g.ldc + n, g.qs + mx_scale_at(row, n, g.qs_pitch), lane);
            round_bf16_8(du, r);
            quant8_store(r, g.q0 + row * g.ldc + g.c_split + n,
                         g.qs + mx_scale_at(row, (int)g.c_split + n, g.qs_pitch), lane);
          }
        }
      }
    } else if (pre_acc) {
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int r = it * 4 + (lane >> 4);
        const int c = (lane & 15) * 8;
        const int m = wm * 128 + I * 32 + r;
        const f32x4_t a0 = *reinterpret_cast<const f32x4_t*>(slice + stage_off(r, c >> 2));
        const f32x4_t a1 = *reinterpret_cast<const f32x4_t*>(slice + stage_off(r, (c >> 2) + 1));
        const int n = t.n0 + wn * 128 + c;
        if (m < t.mlim && n < g.N) {
          float o[8], v[8];
          if constexpr (EPI == EPI_WGRAD_SPLIT_F32) {
            const uint32_t* a = reinterpret_cast<const uint32_t*>(&hg[it]);
            const uint32_t* b = reinterpret_cast<const uint32_t*>(&hu[it]);
#pragma unroll
            for (int q = 0; q < 4; ++q) { o[q] = __uint_as_float(a[q]); o[q + 4] = __uint_as_float(b[q]); }
          } else {
            unpack8(hg[it], o);
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) { v[q] = a0[q] + o[q]; v[q + 4] = a1[q] + o[q + 4]; }
          const long row = (g.ragged == RAG_M) ? (long)t.row0 + m : (long)t.m0 + m;
          store8_nt(epi_ptr<EPI>(g, t, row, n), v);
        }
      }
    } else {
#pragma unroll 2
      for (int it = 0; it < 8; ++it) {
        const int r = it * 4 + (lane >> 4);
        const int c = (lane & 15) * 8;
        const int m = wm * 128 + I * 32 + r;
        float v[8];
        const f32x4_t a0 = *reinterpret_cast<const f32x4_t*>(slice + stage_off(r, c >> 2));
        const f32x4_t a1 = *reinterpret_cast<const f32x4_t*>(slice + stage_off(r, (c >> 2) + 1));
#pragma unroll
        for (int q = 0; q < 4; ++q) { v[q] = a0[q]; v[q + 4] = a1[q]; }
        const int n = t.n0 + wn * 128 + c;
        const long row = (g.ragged == RAG_M) ? (long)t.row0 + m : (long)t.m0 + m;
        if (m < t.mlim && n < g.N) epi8<EPI>(g, t, row, n, v, v);
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}
}

// Epilogue of a wave's 128x128 accumulator sub-tile through its private
// 16 KiB slice, one 32-row block at a time: the accumulators go to the slice
// straight from the accumulator registers, then each lane reads back 8
// consecutive columns of a row and applies the epilogue with 16-byte global
// accesses.
template <int KIND>
__device__ __forceinline__ void epilogue_lds(const GemmArgs& g, const Tile& tile, char* slice,
                                             f32x16_t (&acc)[4][4], int wm, int wn, int lane_in) {
  // The tile's coordinates and the lane pass through an empty asm statement so that the
  // compiler cannot hoist the epilogue's address arithmetic above the K loop
  // (where it would hold those registers, or spill them, for the whole loop).
  Tile t = tile;
  int lane = lane_in;
  asm volatile("" : "+v"(t.row0), "+v"(t.n0), "+v"(t.m0), "+v"(t.e), "+v"(t.mlim), "+v"(lane));
  // 32-row blocks past the tile's last row (a ragged tail) store nothing
  const int rows = t.mlim - wm * 128;
  if (rows > 0) epilogue_block<KIND, 0>(g, t, slice, acc, wm, wn, lane);
  if (rows > 32) epilogue_block<KIND, 1>(g, t, slice, acc, wm, wn, lane);
  if (rows > 64) epilogue_block<KIND, 2>(g, t, slice, acc, wm, wn, lane);
  if (rows > 96) epilogue_block<KIND, 3>(g, t, slice, acc, wm, wn, lane);
}

}  // namespace mf
}  // namespace moe
