// Grouped GEMM engine of the MoE expert layer (gfx950).
//
// One launch runs every expert's GEMM ("merge the many small per-expert
// matmuls into one kernel", olmoforge README, grouped-GEMM module).  The
// groups are read on the device from the routing offsets, so the host never
// waits for routing metadata (GPU-resident routing table, same README).
//
// bf16 engine: persistent workgroups of 256 threads (4 waves, one per SIMD)
// walk a tile list over the ragged expert segments.  Tiles are 256x256
// outputs with a K step of 64, staged through LDS in two buffers (128 KiB);
// each wave owns a 128x128 sub-tile as 4x4 MFMA 32x32x16 bf16 blocks with
// float32 accumulators.  LDS holds both operands K-contiguous (rows of 64
// bf16 = 128 bytes, 16-byte chunks XOR-swizzled by row), so every MFMA
// fragment is a single ds_read_b128.  Operands that are contiguous along M or
// N in HBM (the weights in the forward GEMMs, both operands of the weight
// gradient) are transposed in registers on their way into LDS (8x8 blocks of
// bf16 through v_perm_b32).  Consecutive logical tiles go to workgroups of the
// same XCD, so tiles that share an activation panel or a weight panel meet in
// the same L2.
//
// float32 engine (the fp32 layer and odd router shapes): a plain LDS-tiled
// SIMT kernel with the same tile schedule and the same epilogues.
#include "gemm.h"
#include "hook.h"
#include "moe_common.h"

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
  int ts[257];  // RAG_M: exclusive prefix of M tiles per group
};

// Fill the schedule; returns the number of tiles.  All threads must call it.
template <int BM, int BNT>
__device__ int sched_setup(const GemmArgs& g, Sched& s) {
  const int tid = threadIdx.x;
  const int E = g.offsets ? g.E : 1;
  if (g.offsets) {
    for (int e = tid; e <= E; e += blockDim.x) s.off[e] = g.offsets[e];
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
  const int ntm = (g.M + BM - 1) / BM;
  return E * ntm * ntn;
}

template <int BM, int BNT>
__device__ __forceinline__ Tile sched_decode(const GemmArgs& g, const Sched& s, int L) {
  const int ntn = (g.N + BNT - 1) / BNT;
  Tile t;
  if (g.ragged == RAG_M) {
    const int E = g.offsets ? g.E : 1;
    int mt = L / ntn, nt = L - mt * ntn;
    int lo = 0, hi = E;  // largest e in [0,E) with ts[e] <= mt
    while (hi - lo > 1) {
      int mid = (lo + hi) >> 1;
      if (s.ts[mid] <= mt) lo = mid; else hi = mid;
    }
    t.e = lo;
    t.m0 = (mt - s.ts[lo]) * BM;
    int ne = s.off[lo + 1] - s.off[lo];
    t.mlim = min(BM, ne - t.m0);
    t.row0 = s.off[lo] + t.m0;
    t.n0 = nt * BNT;
    t.klen = g.K;
  } else {
    const int ntm = (g.M + BM - 1) / BM;
    int per = ntm * ntn;
    t.e = L / per;
    int r = L - t.e * per;
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
// take P consecutive logical tiles.
__device__ __forceinline__ int logical_tile(int it) {
  const int G = gridDim.x, b = blockIdx.x;
  if (G % 8) return it * G + b;
  return it * G + (b & 7) * (G >> 3) + (b >> 3);
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
template <int EPI, typename TS>
__device__ __forceinline__ void epilogue4(const GemmArgs& g, const Tile& t, int m, int n,
                                          const float (&v)[4], const float (&u)[4]) {
  if constexpr (EPI == EPI_STORE_F32) {
    long row = (long)t.row0 + m;
    float* p = static_cast<float*>(g.c0) + row * g.ldc + n;
    if (n + 4 <= g.N && (g.ldc & 3) == 0)
      *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    else
      store_part(p, v, min(4, g.N - n), false);
  } else if constexpr (EPI == EPI_STORE) {
    long row = (g.ragged == RAG_M) ? (long)t.row0 + m : (long)t.m0 + m;
    TS* p = static_cast<TS*>(g.c0) + (g.ragged == RAG_M ? 0 : (long)t.e * g.c_es) + row * g.ldc + n;
    if (n + 4 <= g.N && (g.ldc & 3) == 0)
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
      float s = 1.0f / (1.0f + __expf(-hg[q]));
      du[q] = v[q] * hg[q] * s;
      dg[q] = v[q] * hu[q] * s * (1.0f + hg[q] * (1.0f - s));
    }
    TS* p = static_cast<TS*>(g.c0) + row * g.ldc + n;
    store4(p, dg, false);
    store4(p + g.c_split, du, false);
  }
}

// ---------------------------------------------------------------------------
// bf16 MFMA engine
// ---------------------------------------------------------------------------
namespace mf {

constexpr int BM = 256, BN = 256, BK = 64, NTHR = 256;
constexpr int ROWB = BK * 2;                       // bytes per LDS row
constexpr int STAGE = (BM + BN) * ROWB;            // bytes per LDS stage

__device__ __forceinline__ int lds_off(int row, int chunk) {
  return row * ROWB + ((chunk ^ ((row ^ (row >> 3)) & 7)) << 4);
}

// 8x8 bf16 transpose: in[r] holds row r (8 elements); out[i] holds column i.
__device__ __forceinline__ void transpose8x8(const uint4 (&in)[8], uint4 (&out)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t sel = (i & 1) ? 0x07060302u : 0x05040100u;
    uint32_t w[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint4& lo = in[2 * p];
      const uint4& hi = in[2 * p + 1];
      uint32_t l = (i >> 1) == 0 ? lo.x : (i >> 1) == 1 ? lo.y : (i >> 1) == 2 ? lo.z : lo.w;
      uint32_t h = (i >> 1) == 0 ? hi.x : (i >> 1) == 1 ? hi.y : (i >> 1) == 2 ? hi.z : hi.w;
      w[p] = __builtin_amdgcn_perm(h, l, sel);
    }
    out[i] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// Per-thread register image of one operand's stage.
struct Regs {
  uint4 v[8];
};

// ---- operand A ----
// K-contiguous A (RAG_M): rows are global rows t.row0 + r (clamped into the group).
template <int KIND>
__device__ __forceinline__ void load_a(const GemmArgs& g, const Tile& t, int k0, Regs& R) {
  const int tid = threadIdx.x;
  const bf16_t* A = static_cast<const bf16_t*>(g.a);
  if constexpr (KT<KIND>::AK) {
    const int c = tid & 7;
    const int k = k0 + c * 8;
    const bool kv = k < t.klen;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int r = (tid >> 3) + 32 * i;
      r = min(r, t.mlim - 1);
      const bf16_t* p = A + ((long)t.row0 + r) * g.lda + k;
      R.v[i] = kv ? *reinterpret_cast<const uint4*>(p) : make_uint4(0, 0, 0, 0);
    }
  } else {
    // A[krow][m], M contiguous: 8 k-rows x 8 m per thread
    const int kb = tid >> 5, mb = tid & 31;
    const int m = t.m0 + mb * 8;
    const bool mv = m < g.M;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      int k = k0 + kb * 8 + r;
      bool v = mv && k < t.klen;
      long row = (long)t.row0 + k;
      if (v && g.a_gather) row = g.a_gather[row];
      const bf16_t* p = A + row * g.lda + m;
      R.v[r] = v ? *reinterpret_cast<const uint4*>(p) : make_uint4(0, 0, 0, 0);
    }
  }
}

template <int KIND>
__device__ __forceinline__ void store_a(char* lds, const Regs& R) {
  const int tid = threadIdx.x;
  if constexpr (KT<KIND>::AK) {
    const int c = tid & 7;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int r = (tid >> 3) + 32 * i;
      *reinterpret_cast<uint4*>(lds + lds_off(r, c)) = R.v[i];
    }
  } else {
    const int kb = tid >> 5, mb = tid & 31;
    uint4 col[8];
    transpose8x8(R.v, col);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      *reinterpret_cast<uint4*>(lds + lds_off(mb * 8 + i, kb)) = col[i];
  }
}

// ---- operand B ----
template <int KIND>
__device__ __forceinline__ void load_b(const GemmArgs& g, const Tile& t, int k0, Regs& R) {
  const int tid = threadIdx.x;
  constexpr int BSP = KT<KIND>::BSP;
  if constexpr (KT<KIND>::BK_) {
    // B[n][k] (K contiguous), per-group matrix
    const int c = tid & 7;
    int kk = k0;
    const bf16_t* base;
    if constexpr (BSP == BS_SPLIT_K) {
      bool second = k0 >= g.b_split;
      base = static_cast<const bf16_t*>(second ? g.b1 : g.b0);
      kk = second ? k0 - g.b_split : k0;
    } else {
      base = static_cast<const bf16_t*>(g.b0);
    }
    base += (long)t.e * g.b_es;
    const int k = kk + c * 8;
    const bool kv = (k0 + c * 8) < t.klen;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int n = min(t.n0 + (tid >> 3) + 32 * i, g.N - 1);
      const bf16_t* p = base + (long)n * g.ldb + k;
      R.v[i] = kv ? *reinterpret_cast<const uint4*>(p) : make_uint4(0, 0, 0, 0);
    }
  } else {
    // B[k][n] (N contiguous): 8 k-rows x 8 n per thread
    const int kb = tid >> 5, nb = tid & 31;
    const bf16_t* base;
    int n;
    if constexpr (BSP == BS_DUAL_N) {
      const int c = nb * 8, blk = c >> 6;
      base = static_cast<const bf16_t*>((blk & 1) ? g.b1 : g.b0);
      n = t.n0 + (blk >> 1) * 64 + (c & 63);
    } else {
      base = static_cast<const bf16_t*>(g.b0);
      n = t.n0 + nb * 8;
    }
    const bool nv = n < g.N;
    if (g.ragged == RAG_M) base += (long)t.e * g.b_es;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      int k = k0 + kb * 8 + r;
      bool v = nv && k < t.klen;
      long row = (g.ragged == RAG_M) ? (long)k : (long)t.row0 + k;
      const bf16_t* p = base + row * g.ldb + n;
      R.v[r] = v ? *reinterpret_cast<const uint4*>(p) : make_uint4(0, 0, 0, 0);
    }
  }
}

template <int KIND>
__device__ __forceinline__ void store_b(char* lds, const Regs& R) {
  const int tid = threadIdx.x;
  if constexpr (KT<KIND>::BK_) {
    const int c = tid & 7;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int r = (tid >> 3) + 32 * i;
      *reinterpret_cast<uint4*>(lds + lds_off(r, c)) = R.v[i];
    }
  } else {
    const int kb = tid >> 5, nb = tid & 31;
    uint4 col[8];
    transpose8x8(R.v, col);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      *reinterpret_cast<uint4*>(lds + lds_off(nb * 8 + i, kb)) = col[i];
  }
}

template <int KIND>
__global__ __launch_bounds__(NTHR, 1) void gemm_bf16_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];
  __shared__ Sched sch;
  constexpr int BNT = (KT<KIND>::BSP == BS_DUAL_N) ? BN / 2 : BN;
  const int ntiles = sched_setup<BM, BNT>(g, sch);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  for (int it = 0;; ++it) {
    const int L = logical_tile(it);
    if (L >= ntiles) break;
    const Tile t = sched_decode<BM, BNT>(g, sch, L);

    f32x16_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    const int nk = (t.klen + BK - 1) / BK;
    Regs ra, rb;
    if (nk > 0) {
      load_a<KIND>(g, t, 0, ra);
      load_b<KIND>(g, t, 0, rb);
      store_a<KIND>(smem, ra);
      store_b<KIND>(smem + BM * ROWB, rb);
    }
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      char* cur = smem + (kt & 1) * STAGE;
      char* nxt = smem + ((kt + 1) & 1) * STAGE;
      const bool more = kt + 1 < nk;
      if (more) {
        load_a<KIND>(g, t, (kt + 1) * BK, ra);
        load_b<KIND>(g, t, (kt + 1) * BK, rb);
      }
      const char* As = cur;
      const char* Bs = cur + BM * ROWB;
#pragma unroll
      for (int s = 0; s < BK / 16; ++s) {
        const int chunk = 2 * s + (lane >> 5);
        bf16x8_t af[4], bfr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          af[i] = *reinterpret_cast<const bf16x8_t*>(As + lds_off(wm * 128 + i * 32 + (lane & 31), chunk));
#pragma unroll
        for (int j = 0; j < 4; ++j)
          bfr[j] = *reinterpret_cast<const bf16x8_t*>(Bs + lds_off(wn * 128 + j * 32 + (lane & 31), chunk));
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
      }
      if (more) {
        store_a<KIND>(nxt, ra);
        store_b<KIND>(nxt + BM * ROWB, rb);
      }
      __syncthreads();
    }

    // Epilogue.  Lane holds C[m][n..n+3] with m = wm*128 + i*32 + lane%32 and
    // n = wn*128 + j*32 + 8*grp + 4*(lane/32) for register group grp.
    constexpr int EPI = KT<KIND>::EPI;
    const int nq = 4 * (lane >> 5);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = wm * 128 + i * 32 + (lane & 31);
      if (m >= t.mlim) continue;
      if constexpr (EPI == EPI_SWIGLU_FWD) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int grp = 0; grp < 4; ++grp) {
            const int n = t.n0 + wn * 64 + j * 32 + 8 * grp + nq;
            if (n >= g.N) continue;
            float v[4], u[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              v[q] = acc[i][j][4 * grp + q];
              u[q] = acc[i][j + 2][4 * grp + q];
            }
            epilogue4<EPI, bf16_t>(g, t, m, n, v, u);
          }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int grp = 0; grp < 4; ++grp) {
            const int n = t.n0 + wn * 128 + j * 32 + 8 * grp + nq;
            if (n >= g.N) continue;
            float v[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) v[q] = acc[i][j][4 * grp + q];
            epilogue4<EPI, bf16_t>(g, t, m, n, v, v);
          }
      }
    }
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
