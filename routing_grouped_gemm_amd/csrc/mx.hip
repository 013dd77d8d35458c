// MXFP8 path of the expert layer (gfx950).
//
// MXFP8 block quantisation (olmoforge README, MXFP8 snippet and module
// table: blocks of 32 values share one scale; e4m3 elements up to 448).
// Reading of the snippet: the block scale is 2^E with E the least integer such
// that 448 * 2^E >= max|block| (0 for an all-zero block, clamped to the E8M0
// range [-127, 127]); each element is rounded to the nearest OCP e4m3 value,
// ties to even, saturating at 448.  Scales are stored as E8M0 bytes, E + 127.
//
// Every MX GEMM operand is quantised along that GEMM's contraction axis and
// laid out K-contiguous, so one grouped GEMM kernel (both operands K-major)
// serves all four MX GEMMs:
//   forward gate/up  Xq[R,d]   x WguT[e][rows, d]  (Wg, Wu along d, transposed;
//                    256-row panels of 128 gate rows then the 128 up rows of
//                    the same f columns, so the gate/up epilogue applies)
//   forward down     Aq[R,f]   x WdT[e][d, f]      (Wd along f, transposed)
//   down dgrad       dYsq[R,d] x Wd[e][f, d]       (Wd along d, as stored)
//   gate/up dgrad    dHq[R,2f] x Wgu[e][d, 2f]     (Wg | Wu along f, as stored)
// Scales are block-major ([block][row]) with the activation row pitch rounded
// up to 16, so each stage's scales arrive by the same buffer->LDS DMA as the
// codes.  The MFMA is v_mfma_scale_f32_32x32x64_f8f6f4 (e4m3 x e4m3, float32
// accumulate): within a lane's 32 code bytes, bytes 0-15 belong to the first
// 32-element K block (scale from lanes 0-31) and bytes 16-31 to the second
// (scale from lanes 32-63); lane half h holds k = 16h + 0..15 and 32 + 16h +
// 0..15.
#include "gemm.h"
#include "gemm_dev.h"
#include "hook.h"
#include "moe_common.h"
#include "mx.h"
#include "mx_codec.h"

namespace moe {

// ---------------------------------------------------------------------------
// quantisation kernels
// ---------------------------------------------------------------------------
// Dispatch row copy with quantisation: Xs[r] = x[src[r]] in bf16 (for the
// weight gradients) and Xq[r] / scales along d.  One wave per row.
__global__ __launch_bounds__(256) void mx_dispatch_kernel(const bf16_t* __restrict__ x,
                                                          const int32_t* __restrict__ src_token,
                                                          int R, int T, int d, bf16_t* __restrict__ Xs,
                                                          uint8_t* __restrict__ Xq,
                                                          uint8_t* __restrict__ scale, long pitch) {
  const int lane = threadIdx.x & 63;
  const long r = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= R) return;
  const int t = min(max(src_token[r], 0), T - 1);
  const bf16_t* src = x + (long)t * d;
  for (int c = lane * 8; c < d; c += 512) {
    const uint4 raw = *reinterpret_cast<const uint4*>(src + c);
    *reinterpret_cast<uint4*>(Xs + r * d + c) = raw;
    float v[8];
    load8(src + c, v);
    uint32_t codes[2];
    const int E = quant8(v, codes);
    *reinterpret_cast<uint2*>(Xq + r * d + c) = make_uint2(codes[0], codes[1]);
    if ((lane & 3) == 0) scale[(long)(c >> 5) * pitch + r] = (uint8_t)(E + 127);
  }
}

// Rows of a bf16 matrix quantised along their length K.  Row r belongs to
// group r / grows (index i = r % grows); codes go to dst + r*dst_ld + col0,
// the scale of block b to scale[g*sg_stride + (block0 + b)*pitch + i].
__global__ __launch_bounds__(256) void mx_quant_rows_kernel(
    const bf16_t* __restrict__ src, long nrows, int K, long src_ld, uint8_t* __restrict__ dst,
    long dst_ld, long col0, uint8_t* __restrict__ scale, long grows, long sg_stride, long pitch,
    int block0) {
  const int lane = threadIdx.x & 63;
  const long r = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= nrows) return;
  const long g = r / grows, i = r - g * grows;
  // up to 8 chunks of 8 values per lane are loaded before any is quantised
  for (int c0 = lane * 8; c0 < K; c0 += 8 * 512) {
    uint4 raw[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int c = c0 + u * 512;
      raw[u] = c < K ? *reinterpret_cast<const uint4*>(src + r * src_ld + c) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int c = c0 + u * 512;
      if (c < K) {  // whole 4-lane blocks together (K is a multiple of 32)
        float v[8];
        unpack8(raw[u], v);
        quant8_store(v, dst + r * dst_ld + col0 + c,
                     scale + g * sg_stride + (long)(block0 + (c >> 5)) * pitch + i, lane);
      }
    }
  }
}

// Columns of W[e][K][N] quantised along K and written transposed: column n
// becomes row rowmap(n) of dst[e] (rows of K codes); the scale of block b to
// scale[e*s_es + b*pitch + rowmap(n)].  half >= 0 selects the gate/up panel
// map rowmap(n) = 256*(n/128) + 128*half + n%128; half < 0 keeps rowmap(n) = n.
// A workgroup stages a 64 (k) x 64 (n) tile in LDS with coalesced 16-byte
// loads; thread t then takes column t/4 and rows 16*(t%4) .. +15, half of a
// 32-row block whose other half sits in the neighbouring lane, and writes 16
// codes (4 lanes write 64 contiguous bytes of the transposed row).
__global__ __launch_bounds__(256) void mx_quant_cols_kernel(
    const bf16_t* __restrict__ W, int K, int N, uint8_t* __restrict__ dst, long dst_es,
    int half, uint8_t* __restrict__ scale, long s_es, long pitch) {
  __shared__ __attribute__((aligned(16))) bf16_t tile[64][72];
  const int e = blockIdx.z, k0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  const int t = threadIdx.x, lane = t & 63;
  {
    const int r = t >> 2, c = (t & 3) * 16;
    uint4 a = make_uint4(0, 0, 0, 0), b = a;
    if (k0 + r < K && n0 + c < N) {
      const bf16_t* src = W + (long)e * K * N + (long)(k0 + r) * N + n0 + c;
      a = *reinterpret_cast<const uint4*>(src);
      b = *reinterpret_cast<const uint4*>(src + 8);
    }
    *reinterpret_cast<uint4*>(&tile[r][c]) = a;
    *reinterpret_cast<uint4*>(&tile[r][c + 8]) = b;
  }
  __syncthreads();
  const int n = t >> 2, q = t & 3;
  if (n0 + n >= N) return;  // whole 4-lane groups leave together
  float v[16];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    v[i] = bf16_to_f32(tile[16 * q + i][n]);
    amax = fmaxf(amax, fabsf(v[i]));
  }
  amax = fmaxf(amax, dpp_f<kDppQuad1032>(amax, amax));   // the partner lane (lane ^ 1)
  const int E = mx_block_exponent(amax);
  float sv[8];
  uint32_t w[4];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int i = 0; i < 8; ++i) sv[i] = ldexpf(v[8 * h + i], -E);
    uint32_t c2[2];
    e4m3_codes8(sv, c2);
    w[2 * h] = c2[0];
    w[2 * h + 1] = c2[1];
  }
  const int col = n0 + n;
  const long row = half >= 0 ? (long)((col >> 7) << 8) + 128 * half + (col & 127) : (long)col;
  if (k0 + 16 * q < K) {
    *reinterpret_cast<uint4*>(dst + (long)e * dst_es + row * K + k0 + 16 * q) =
        make_uint4(w[0], w[1], w[2], w[3]);
    if ((q & 1) == 0)
      scale[(long)e * s_es + (long)((k0 >> 5) + (q >> 1)) * pitch + row] = (uint8_t)(E + 127);
  }
  (void)lane;
}

// Weight-gradient operands, quantised along the tokens of each expert.
// poff[e] = sum over earlier experts of their row counts rounded up to 128:
// each expert's token segment starts a 128-aligned column range of the
// transposed codes (one GEMM stage holds 128 codes of a row).
__global__ __launch_bounds__(64) void mx_pad_offsets_kernel(const int32_t* __restrict__ offsets,
                                                            int E, int32_t* __restrict__ poff) {
  const int lane = threadIdx.x;
  int c[4], sum = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = lane * 4 + q;
    c[q] = (e < E) ? (offsets[e + 1] - offsets[e] + 127) / 128 * 128 : 0;
    sum += c[q];
  }
  int incl = sum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
  int run = incl - sum;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = lane * 4 + q;
    if (e <= E) poff[e] = run;
    run += c[q];
  }
  if (lane == 63 && E == 256) poff[256] = incl;
}

// src[R][C] (bf16, rows grouped by expert) quantised along its rows in
// blocks of 32 starting at each expert's first row and written transposed:
// padded token p of expert e (p - poff[e] < its row count, else zero) is
// column p of dst[C][dst_ld]; block p/32 of column c has its scale at
// scale[(p/32) * C + c].  A workgroup stages 64 padded tokens x 64 columns
// in LDS (a 64-token tile never straddles two experts' 128-aligned
// segments); thread t then takes column t/4 and tokens 16*(t%4) .. +15, half
// a 32-token block whose other half is in the neighbouring lane.
__global__ __launch_bounds__(256) void mx_quant_tokens_kernel(
    const bf16_t* __restrict__ src, int C, long src_ld, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ poff, int E, uint8_t* __restrict__ dst, long dst_ld,
    uint8_t* __restrict__ scale) {
  __shared__ __attribute__((aligned(16))) bf16_t tile[64][72];
  __shared__ int po[257];
  const int p0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const int t = threadIdx.x;
  for (int e = t; e <= E; e += 256) po[e] = poff[e];
  __syncthreads();
  if (p0 >= po[E]) return;                 // past the last segment (uniform)
  int lo = 0, hi = E;                      // the expert e with po[e] <= p0 < po[e+1]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (po[mid] <= p0) lo = mid; else hi = mid;
  }
  const int e = lo;
  const int row0 = offsets[e], n = offsets[e + 1] - row0;
  {
    const int r = t >> 2, c = (t & 3) * 16;
    const int pr = p0 + r - po[e];         // token inside the expert
    uint4 a = make_uint4(0, 0, 0, 0), b = a;
    if (pr < n) {
      const bf16_t* sp = src + (long)(row0 + pr) * src_ld + c0 + c;
      a = *reinterpret_cast<const uint4*>(sp);
      b = *reinterpret_cast<const uint4*>(sp + 8);
    }
    *reinterpret_cast<uint4*>(&tile[r][c]) = a;
    *reinterpret_cast<uint4*>(&tile[r][c + 8]) = b;
  }
  __syncthreads();
  const int col = t >> 2, q = t & 3;
  float v[16];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    v[i] = bf16_to_f32(tile[16 * q + i][col]);
    amax = fmaxf(amax, fabsf(v[i]));
  }
  amax = fmaxf(amax, dpp_f<kDppQuad1032>(amax, amax));   // the partner lane (lane ^ 1)
  const int E8 = mx_block_exponent(amax);
  float sv[8];
  uint32_t w[4];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int i = 0; i < 8; ++i) sv[i] = ldexpf(v[8 * h + i], -E8);
    uint32_t c2[2];
    e4m3_codes8(sv, c2);
    w[2 * h] = c2[0];
    w[2 * h + 1] = c2[1];
  }
  *reinterpret_cast<uint4*>(dst + (long)(c0 + col) * dst_ld + p0 + 16 * q) =
      make_uint4(w[0], w[1], w[2], w[3]);
  if ((q & 1) == 0) scale[(long)((p0 >> 5) + (q >> 1)) * C + c0 + col] = (uint8_t)(E8 + 127);
}

// ---------------------------------------------------------------------------
// MX grouped GEMM
// ---------------------------------------------------------------------------
namespace mf {

// A stage holds 128 code bytes (four 32-element scale blocks) of every tile
// row of both operands, plus those rows' scales: block b of the A rows at
// STAGE + b*1024, of the B rows at STAGE + 4096 + b*1024.  One MFMA k-step
// takes 64 codes (two blocks), so a stage is two k-steps.
constexpr int MX_KSTEP = 64;
constexpr int SCALE_BYTES = 8192;
constexpr int MSTAGE = STAGE + SCALE_BYTES;
constexpr int MX_DMA_PER_STAGE = 2 * DMA_PER_OP + 2;   // codes of A and B, two scale blocks

typedef __attribute__((ext_vector_type(8))) int i32x8_t;

struct MxPlan {
  Plan a, b;
  i32x4_t srs;       // this wave's scale resource (waves 0-1: A, 2-3: B)
  uint32_t svoff;    // per-lane offset of the scale DMA
  uint32_t spitch;   // bytes between consecutive K blocks of the scales
  int sblk;          // first of the two K blocks of a stage this wave loads (0 or 2)
  int amis;          // A rows: tile row 0 sits amis bytes into an A scale block
};

// Codes of one row for k-step j of a stage: lane half h takes 16-byte chunks
// 4j + h (its bytes 0-15, first scale block) and 4j + 2 + h (bytes 16-31,
// second scale block).
__device__ __forceinline__ i32x8_t fragq(const char* op, int rowblk, int j, int lane) {
  const int row = rowblk + (lane & 31), h = lane >> 5;
  const uint4 lo = *reinterpret_cast<const uint4*>(op + km_off(row, 4 * j + h));
  const uint4 hi = *reinterpret_cast<const uint4*>(op + km_off(row, 4 * j + 2 + h));
  i32x8_t r = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  return r;
}

struct MxFrags {
  i32x8_t a[4], b[4];
  int sa[4], sb[4];
};

// Fragments and scales of k-step j of stage kt.  Lanes 0-31 supply the
// scale of the first block of the k-step, lanes 32-63 of the second.
template <bool DUAL>
__device__ __forceinline__ void load_mx_frags(const char* smem, int kt, int j, int wm, int wn,
                                              int lane, int amis, MxFrags& F) {
  const char* st = smem + (kt & (NST - 1)) * MSTAGE;
  const char* As = st;
  const char* Bs = st + OPB;
  const uint8_t* Ss = reinterpret_cast<const uint8_t*>(st + STAGE);
  const int blk = 2 * j + (lane >> 5);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = wm * 128 + i * 32;
    F.a[i] = fragq(As, row, j, lane);
    F.sa[i] = Ss[blk * 1024 + amis + row + (lane & 31)];
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int col = DUAL ? ((q >> 1) * 128 + wn * 64 + (q & 1) * 32) : (wn * 128 + q * 32);
    F.b[q] = fragq(Bs, col, j, lane);
    F.sb[q] = Ss[4096 + blk * 1024 + col + (lane & 31)];
  }
}

__device__ __forceinline__ void mx_mfma16(f32x16_t (&acc)[4][4], const MxFrags& F) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(F.b[j], F.a[i], acc[i][j], 0, 0,
                                                                  0, F.sb[j], 0, F.sa[i]);
}

__device__ __forceinline__ void mx_issue(const MxPlan& P, int kt, uint32_t st_base, int wave) {
  issue<false>(P.a, kt, st_base, wave);
  issue<false>(P.b, kt, st_base + OPB, wave);
  // the block offset goes into the per-lane offset, which the range check covers
  const uint32_t dst = st_base + STAGE + (wave >> 1) * 4096 + P.sblk * 1024;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const uint32_t voff = P.svoff + (uint32_t)(4 * kt + P.sblk + b) * P.spitch;
    dma16(P.srs, dst + b * 1024, voff, 0u);
  }
}

// Ask the scheduler to alternate MFMAs and LDS reads in the current region.
__device__ __forceinline__ void interleave_mx() {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  }
}

template <int KIND>
__global__ __launch_bounds__(NTHR, 1) void gemm_mx_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(1024))) char smem[NST * MSTAGE];
  __shared__ Sched sch;
  constexpr bool DUAL = KT<KIND>::BSP == BS_DUAL_N;
  constexpr int BNT = DUAL ? BN / 2 : BN;
  const int ntiles = sched_setup<BM, BNT>(g, sch);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const uint32_t lds0 = lds_u32(smem);
  const uint8_t* A = static_cast<const uint8_t*>(g.a);
  const uint8_t* B = static_cast<const uint8_t*>(g.b0);

  // RK (weight gradients): the K axis is the tokens; tile rows are M rows
  // (features) of the transposed codes A[M][lda], columns N rows of B[N][ldb],
  // and the expert's K segment starts at byte t.row0 of every row (scale
  // block t.row0 / 32).  g.K is the padded token count.
  constexpr bool RK = KIND == GK_MX_WGRAD || KIND == GK_MX_WGRAD_F32;
  auto plan = [&](const Tile& t, MxPlan& P) {
    P.sblk = 2 * (wave & 1);
    if constexpr (RK) {
      const long long abytes = (long long)g.M * g.lda, bbytes = (long long)g.N * g.ldb;
      const long aoff = (long)t.m0 * g.lda + t.row0, boff = (long)t.n0 * g.ldb + t.row0;
      plan_km(P.a, A + aoff, abytes - aoff, nullptr, 0, 1 << 30, g.lda, wave, lane);
      plan_km(P.b, B + boff, bbytes - boff, nullptr, 0, 1 << 30, g.ldb, wave, lane);
      P.amis = 0;
      const int kb = t.row0 >> 5;
      if (wave < 2) {
        P.srs = make_rsrc(g.sa, (long long)(g.K / 32) * g.sa_pitch);
        P.svoff = (uint32_t)((long)kb * g.sa_pitch + t.m0 + lane * 16);
        P.spitch = (uint32_t)g.sa_pitch;
      } else {
        P.srs = make_rsrc(g.sb, (long long)(g.K / 32) * g.sb_pitch);
        P.svoff = (uint32_t)((long)kb * g.sb_pitch + t.n0 + lane * 16);
        P.spitch = (uint32_t)g.sb_pitch;
      }
    } else {
      // rows of B for this tile: gate/up panels hold 256 rows per 128 f columns
      const long brow0 = DUAL ? 2L * t.n0 : (long)t.n0;
      const long brows = DUAL ? 2L * ((g.N + 127) / 128) * 128 : (long)g.N;
      plan_km(P.a, A + (long)t.row0 * g.lda, ((long long)g.rows_total - t.row0) * g.lda, nullptr,
              0, 1 << 30, g.lda, wave, lane);
      plan_km(P.b, B + (long)t.e * g.b_es + brow0 * g.ldb, (brows - brow0) * g.ldb, nullptr, 0,
              1 << 30, g.ldb, wave, lane);
      const int row_al = t.row0 & ~15;
      P.amis = t.row0 - row_al;
      if (wave < 2) {
        P.srs = make_rsrc(g.sa, (long long)(g.K / 32) * g.sa_pitch);
        P.svoff = (uint32_t)(row_al + lane * 16);
        P.spitch = (uint32_t)g.sa_pitch;
      } else {
        P.srs = make_rsrc(g.sb + (long)t.e * g.sb_es, (long long)(g.K / 32) * g.sb_pitch);
        P.svoff = (uint32_t)(brow0 + lane * 16);
        P.spitch = (uint32_t)g.sb_pitch;
      }
    }
  };
  auto stage_base = [&](int s) { return lds0 + (s & 1) * MSTAGE; };

  int it = 0;
  int L = logical_tile(it);
  if (L >= ntiles) return;
  Tile t = sched_decode<BM, BNT>(g, sch, L);
  MxPlan P;
  plan(t, P);
  // K is a multiple of 64: a last stage may hold a single k-step
  int ns = t.klen / MX_KSTEP, nk = (ns + 1) / 2;
  if (nk > 0) mx_issue(P, 0, stage_base(0), wave);
  if (nk > 1) mx_issue(P, 1, stage_base(1), wave);

  for (;;) {
    f32x16_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x16_t{};

    // k-steps q = 0 .. ns-1; step q reads stage q/2, half q%2.  After the
    // reads of a stage's second step, one barrier publishes the next stage
    // and frees this one for the stage after next.
    MxFrags F0, F1;
    auto step = [&](int q, MxFrags& cur, MxFrags& nxt) {
      __builtin_amdgcn_s_waitcnt(kLgkm0);
      const int kt = q >> 1;
      if ((q & 1) == 0) {
        if (q + 1 < ns) load_mx_frags<DUAL>(smem, kt, 1, wm, wn, lane, P.amis, nxt);
      } else {
        const bool more = q + 1 < ns;
        if (more) wait_vmcnt<0>();
        barrier();
        if (kt + 2 < nk) mx_issue(P, kt + 2, stage_base(kt), wave);
        if (more) load_mx_frags<DUAL>(smem, kt + 1, 0, wm, wn, lane, P.amis, nxt);
      }
      mx_mfma16(acc, cur);
      interleave_mx();
      __builtin_amdgcn_sched_barrier(0);
    };
    if (nk > 0) {
      if (nk > 1) wait_vmcnt<MX_DMA_PER_STAGE>(); else wait_vmcnt<0>();
      barrier();
      load_mx_frags<DUAL>(smem, 0, 0, wm, wn, lane, P.amis, F0);
    }
    int q = 0;
    for (; q + 1 < ns; q += 2) {
      step(q, F0, F1);
      step(q + 1, F1, F0);
    }
    if (q < ns) step(q, F0, F1);
    __builtin_amdgcn_s_waitcnt(kLgkm0);
    barrier();

    // next tile's stage 0 loads into buffer 0 during this epilogue, which
    // stages through buffer 1; its stage 1 follows the epilogue
    L = logical_tile(++it);
    const bool has_next = L < ntiles;
    Tile tn = t;
    MxPlan Pn = P;
    int nsn = 0, nkn = 0;
    if (has_next) {
      tn = sched_decode<BM, BNT>(g, sch, L);
      plan(tn, Pn);
      nsn = tn.klen / MX_KSTEP;
      nkn = (nsn + 1) / 2;
      if (nkn > 0) mx_issue(Pn, 0, stage_base(0), wave);
    }
    epilogue_lds<KIND>(g, t, smem + MSTAGE + wave * EPI_SLICE, acc, wm, wn, lane);
    barrier();
    if (!has_next) break;
    if (nkn > 1) mx_issue(Pn, 1, stage_base(1), wave);
    t = tn; P = Pn; ns = nsn; nk = nkn;
  }
}

}  // namespace mf

namespace {
const char* mx_name(int kind) {
  switch (kind) {
    case GK_MX_GATEUP: return "gemm_mx_fwd_gateup_swiglu";
    case GK_MX_DOWN: return "gemm_mx_fwd_down";
    case GK_MX_DGRAD_DOWN: return "gemm_mx_dgrad_down_swiglu_bwd";
    case GK_MX_DGRAD_GATEUP: return "gemm_mx_dgrad_gateup";
  }
  return "gemm_mx";
}
const char* mx_name(int kind, const GemmArgs& g) {
  if (kind == GK_MX_WGRAD || kind == GK_MX_WGRAD_F32)
    return g.c1 ? "gemm_mx_wgrad_gateup" : "gemm_mx_wgrad_down";
  return mx_name(kind);
}

template <int KIND>
hipError_t launch_mx_kind(const GemmArgs& g, int num_cu, hipStream_t s) {
  constexpr int BNT = (KT<KIND>::BSP == BS_DUAL_N) ? mf::BN / 2 : mf::BN;
  const long ntn = (g.N + BNT - 1) / BNT;
  const long ub = g.ragged == RAG_K ? (long)ngroups(g) * ((g.M + mf::BM - 1) / mf::BM) * ntn
                                    : ((long)g.rows_total / mf::BM + ngroups(g)) * ntn;
  const int grid = (int)(ub < num_cu ? ub : (long)num_cu);
  if (grid <= 0) return hipSuccess;
  note_prelaunch(mx_name(KIND, g), s);
  hipLaunchKernelGGL(mf::gemm_mx_kernel<KIND>, dim3(grid), dim3(mf::NTHR), 0, s, g);
  note_launch(mx_name(KIND, g), s);
  return hipGetLastError();
}

constexpr size_t kAl = 256;
inline size_t al(size_t v) { return (v + kAl - 1) & ~(kAl - 1); }

// Bump allocator over the caller's workspace.
struct Carve {
  char* base;
  size_t used = 0;
  template <typename T> T* take(size_t bytes) {
    T* p = reinterpret_cast<T*>(base ? base + used : nullptr);
    used += al(bytes);
    return p;
  }
};

#define MX_TRY(expr)                        \
  do {                                      \
    hipError_t e_ = (expr);                 \
    if (e_ != hipSuccess) return e_;        \
  } while (0)

hipError_t quant_rows(const void* src, long nrows, int K, long src_ld, uint8_t* dst, long dst_ld,
                      long col0, uint8_t* scale, long grows, long sg_stride, long pitch, int block0,
                      hipStream_t s) {
  if (nrows <= 0) return hipSuccess;
  note_prelaunch("mx_quant_rows", s);
  hipLaunchKernelGGL(mx_quant_rows_kernel, dim3((unsigned)((nrows + 3) / 4)), dim3(256), 0, s,
                     static_cast<const bf16_t*>(src), nrows, K, src_ld, dst, dst_ld, col0, scale,
                     grows, sg_stride, pitch, block0);
  note_launch("mx_quant_rows", s);
  return hipGetLastError();
}

hipError_t quant_cols(const void* W, int E, int K, int N, uint8_t* dst, long dst_es, int half,
                      uint8_t* scale, long s_es, long pitch, hipStream_t s) {
  note_prelaunch("mx_quant_cols", s);
  hipLaunchKernelGGL(mx_quant_cols_kernel, dim3((N + 63) / 64, (K + 63) / 64, E), dim3(256), 0, s,
                     static_cast<const bf16_t*>(W), K, N, dst, dst_es, half, scale, s_es, pitch);
  note_launch("mx_quant_cols", s);
  return hipGetLastError();
}

inline long pitch_rows(long R) { return (R + 15) / 16 * 16; }
inline long fpanel(int f) { return (f + 127) / 128 * 128; }

// Forward workspace pieces, in carving order.
struct FwdWs {
  uint8_t *wgu, *wgu_s, *wd, *wd_s, *aq, *aq_s;
};
FwdWs carve_fwd(void* ws, long long R, int d, int f, int E, size_t* total) {
  Carve c{static_cast<char*>(ws)};
  FwdWs w;
  const long fp = fpanel(f), Rp = pitch_rows(R);
  w.wgu = c.take<uint8_t>((size_t)E * 2 * fp * d);
  w.wgu_s = c.take<uint8_t>((size_t)E * (d / 32) * 2 * fp);
  w.wd = c.take<uint8_t>((size_t)E * d * f);
  w.wd_s = c.take<uint8_t>((size_t)E * (f / 32) * d);
  w.aq = c.take<uint8_t>((size_t)R * f);
  w.aq_s = c.take<uint8_t>((size_t)(f / 32) * Rp);
  if (total) *total = c.used;
  return w;
}

// Padded token count bound: every expert's segment rounded up to 128.
inline long wgrad_kp(long long R, int E) { return (R + 127L * E + 127) / 128 * 128; }

// Token-quantised weight-gradient operands (after the dgrad workspace):
// padded offsets, the M-side codes [max(d,f)][Kp] and scales, the N-side codes
// [max(2f,d)][Kp] and scales; reused by the gate/up and the down gradient.
struct WgradWs {
  int32_t* poff;
  uint8_t *a, *a_s, *b, *b_s;
};
WgradWs carve_wgrad(void* ws, size_t skip, long long R, int d, int f, int E, size_t* total) {
  Carve c{static_cast<char*>(ws)};
  c.used = skip;
  WgradWs w;
  const long Kp = wgrad_kp(R, E);
  const long Mx = d > f ? d : f, Nx = 2 * f > d ? 2 * f : d;
  w.poff = c.take<int32_t>((size_t)(E + 1) * 4);
  w.a = c.take<uint8_t>((size_t)Mx * Kp);
  w.a_s = c.take<uint8_t>((size_t)(Kp / 32) * Mx);
  w.b = c.take<uint8_t>((size_t)Nx * Kp);
  w.b_s = c.take<uint8_t>((size_t)(Kp / 32) * Nx);
  if (total) *total = c.used;
  return w;
}

struct BwdWs {
  uint8_t *wd, *wd_s, *dhq, *dhq_s, *wgu, *wgu_s;
};
BwdWs carve_bwd(void* ws, long long R, int d, int f, int E, size_t* total) {
  Carve c{static_cast<char*>(ws)};
  BwdWs w;
  const long Rp = pitch_rows(R);
  w.wd = c.take<uint8_t>((size_t)E * f * d);
  w.wd_s = c.take<uint8_t>((size_t)E * (d / 32) * f);
  w.dhq = c.take<uint8_t>((size_t)R * 2 * f);
  w.dhq_s = c.take<uint8_t>((size_t)(2 * f / 32) * Rp);
  w.wgu = c.take<uint8_t>((size_t)E * d * 2 * f);
  w.wgu_s = c.take<uint8_t>((size_t)E * (2 * f / 32) * d);
  if (total) *total = c.used;
  return w;
}
}  // namespace

hipError_t launch_grouped_gemm_mx(GemmKind kind, const GemmArgs& g, int num_cu, hipStream_t s) {
  switch (kind) {
    case GK_MX_GATEUP: return launch_mx_kind<GK_MX_GATEUP>(g, num_cu, s);
    case GK_MX_DOWN: return launch_mx_kind<GK_MX_DOWN>(g, num_cu, s);
    case GK_MX_DGRAD_DOWN: return launch_mx_kind<GK_MX_DGRAD_DOWN>(g, num_cu, s);
    case GK_MX_DGRAD_GATEUP: return launch_mx_kind<GK_MX_DGRAD_GATEUP>(g, num_cu, s);
    case GK_MX_WGRAD: return launch_mx_kind<GK_MX_WGRAD>(g, num_cu, s);
    case GK_MX_WGRAD_F32: return launch_mx_kind<GK_MX_WGRAD_F32>(g, num_cu, s);
    default: break;
  }
  return hipErrorInvalidValue;
}

long mx_scale_pitch(long long R) { return pitch_rows(R); }

size_t mx_fwd_workspace(long long R, int d, int f, int E) {
  size_t t = 0;
  carve_fwd(nullptr, R, d, f, E, &t);
  return t;
}

size_t mx_bwd_workspace(long long R, int d, int f, int E) {
  size_t t = 0;
  carve_bwd(nullptr, R, d, f, E, &t);
  return t;
}

size_t mx_wgrad_workspace(long long R, int d, int f, int E) {
  size_t t = 0;
  carve_wgrad(nullptr, mx_bwd_workspace(R, d, f, E), R, d, f, E, &t);
  return t;
}

hipError_t launch_mx_dispatch_copy(const void* x, const int32_t* src_token, int R, int T, int d,
                                   void* Xs, void* Xq, uint8_t* Xq_scale, hipStream_t s) {
  if (R == 0) return hipSuccess;
  note_prelaunch("mx_dispatch_quant", s);
  hipLaunchKernelGGL(mx_dispatch_kernel, dim3((R + 3) / 4), dim3(256), 0, s,
                     static_cast<const bf16_t*>(x), src_token, R, T, d, static_cast<bf16_t*>(Xs),
                     static_cast<uint8_t*>(Xq), Xq_scale, pitch_rows(R));
  note_launch("mx_dispatch_quant", s);
  return hipGetLastError();
}

hipError_t mx_ffn_fwd(const void* Xq, const uint8_t* Xscale, const int32_t* offsets, int R, int d,
                      int f, int E, const void* Wg, const void* Wu, const void* Wd, void* Hg,
                      void* Hu, void* A, void* Ys, void* ws, int num_cu, hipStream_t s) {
  const FwdWs w = carve_fwd(ws, R, d, f, E, nullptr);
  const long fp = fpanel(f), Rp = pitch_rows(R);
  // weights: Wg, Wu along d into the gate/up panels; Wd along f, transposed
  MX_TRY(quant_cols(Wg, E, d, f, w.wgu, 2 * fp * d, 0, w.wgu_s, (d / 32) * 2 * fp, 2 * fp, s));
  MX_TRY(quant_cols(Wu, E, d, f, w.wgu, 2 * fp * d, 1, w.wgu_s, (d / 32) * 2 * fp, 2 * fp, s));
  MX_TRY(quant_cols(Wd, E, f, d, w.wd, (long)d * f, -1, w.wd_s, (long)(f / 32) * d, d, s));
  GemmArgs g{};
  g.E = E; g.offsets = offsets; g.rows_total = R; g.ragged = RAG_M;
  g.N = f; g.K = d;
  g.a = Xq; g.lda = d; g.sa = Xscale; g.sa_pitch = Rp;
  g.b0 = w.wgu; g.ldb = d; g.b_es = 2 * fp * d;
  g.sb = w.wgu_s; g.sb_es = (d / 32) * 2 * fp; g.sb_pitch = 2 * fp;
  g.c0 = Hg; g.c1 = Hu; g.c2 = A; g.ldc = f;
  g.q0 = w.aq; g.qs = w.aq_s; g.qs_pitch = Rp;   // A quantised along f in the epilogue
  MX_TRY(launch_grouped_gemm_mx(GK_MX_GATEUP, g, num_cu, s));
  GemmArgs h{};
  h.E = E; h.offsets = offsets; h.rows_total = R; h.ragged = RAG_M;
  h.N = d; h.K = f;
  h.a = w.aq; h.lda = f; h.sa = w.aq_s; h.sa_pitch = Rp;
  h.b0 = w.wd; h.ldb = f; h.b_es = (long)d * f;
  h.sb = w.wd_s; h.sb_es = (long)(f / 32) * d; h.sb_pitch = d;
  h.c0 = Ys; h.ldc = d;
  return launch_grouped_gemm_mx(GK_MX_DOWN, h, num_cu, s);
}

hipError_t mx_ffn_dgrad(const void* dYsq, const uint8_t* dYsq_scale, const void* Hg,
                        const void* Hu, const int32_t* offsets, int R, int d, int f, int E,
                        const void* Wg, const void* Wu, const void* Wd, void* dH, void* dXs,
                        void* ws, int num_cu, hipStream_t s) {
  const BwdWs w = carve_bwd(ws, R, d, f, E, nullptr);
  const long Rp = pitch_rows(R);
  // down dgrad: dYs (quantised along d by the combine backward) and Wd along d
  MX_TRY(quant_rows(Wd, (long)E * f, d, d, w.wd, d, 0, w.wd_s, f, (long)(d / 32) * f, f, 0, s));
  GemmArgs g{};
  g.E = E; g.offsets = offsets; g.rows_total = R; g.ragged = RAG_M;
  g.N = f; g.K = d;
  g.a = dYsq; g.lda = d; g.sa = dYsq_scale; g.sa_pitch = Rp;
  g.b0 = w.wd; g.ldb = d; g.b_es = (long)f * d;
  g.sb = w.wd_s; g.sb_es = (long)(d / 32) * f; g.sb_pitch = f;
  g.c0 = dH; g.ldc = 2L * f; g.c_split = f;
  g.h0 = Hg; g.h1 = Hu; g.ldh = f;
  g.q0 = w.dhq; g.qs = w.dhq_s; g.qs_pitch = Rp;   // dH quantised along 2f in the epilogue
  MX_TRY(launch_grouped_gemm_mx(GK_MX_DGRAD_DOWN, g, num_cu, s));
  // gate/up dgrad: Wg | Wu along f into one [d][2f] matrix per expert
  MX_TRY(quant_rows(Wg, (long)E * d, f, f, w.wgu, 2L * f, 0, w.wgu_s, d, (long)(2 * f / 32) * d, d,
                    0, s));
  MX_TRY(quant_rows(Wu, (long)E * d, f, f, w.wgu, 2L * f, f, w.wgu_s, d, (long)(2 * f / 32) * d, d,
                    f / 32, s));
  GemmArgs h{};
  h.E = E; h.offsets = offsets; h.rows_total = R; h.ragged = RAG_M;
  h.N = d; h.K = 2 * f;
  h.a = w.dhq; h.lda = 2L * f; h.sa = w.dhq_s; h.sa_pitch = Rp;
  h.b0 = w.wgu; h.ldb = 2L * f; h.b_es = (long)d * 2 * f;
  h.sb = w.wgu_s; h.sb_es = (long)(2 * f / 32) * d; h.sb_pitch = d;
  h.c0 = dXs; h.ldc = d;
  return launch_grouped_gemm_mx(GK_MX_DGRAD_GATEUP, h, num_cu, s);
}

namespace {
hipError_t quant_tokens(const void* src, int C, long src_ld, const int32_t* offsets,
                        const int32_t* poff, int E, long Kp, uint8_t* dst, uint8_t* scale,
                        hipStream_t s) {
  note_prelaunch("mx_quant_tokens", s);
  hipLaunchKernelGGL(mx_quant_tokens_kernel, dim3(C / 64, (unsigned)(Kp / 64)), dim3(256), 0, s,
                     static_cast<const bf16_t*>(src), C, src_ld, offsets, poff, E, dst, Kp, scale);
  note_launch("mx_quant_tokens", s);
  return hipGetLastError();
}
}  // namespace

hipError_t mx_ffn_wgrad(const void* Xs, const void* dH, const void* A, const void* dYs,
                        const int32_t* offsets, int R, int d, int f, int E, int f32_out,
                        int accumulate, void* dWg, void* dWu, void* dWd, void* ws, int num_cu,
                        hipStream_t s) {
  const WgradWs w = carve_wgrad(ws, mx_bwd_workspace(R, d, f, E), R, d, f, E, nullptr);
  const long Kp = wgrad_kp(R, E);
  note_prelaunch("mx_pad_offsets", s);
  hipLaunchKernelGGL(mx_pad_offsets_kernel, dim3(1), dim3(64), 0, s, offsets, E, w.poff);
  note_launch("mx_pad_offsets", s);
  MX_TRY(hipGetLastError());
  const GemmKind kind = f32_out ? GK_MX_WGRAD_F32 : GK_MX_WGRAD;
  // dWg | dWu = Xs^T . dH: Xs along its tokens -> a [d][Kp], dH -> b [2f][Kp]
  MX_TRY(quant_tokens(Xs, d, d, offsets, w.poff, E, Kp, w.a, w.a_s, s));
  MX_TRY(quant_tokens(dH, 2 * f, 2L * f, offsets, w.poff, E, Kp, w.b, w.b_s, s));
  GemmArgs g{};
  g.E = E; g.offsets = w.poff; g.rows_total = (int)Kp; g.ragged = RAG_K;
  g.M = d; g.N = 2 * f; g.K = (int)Kp;
  g.a = w.a; g.lda = Kp; g.sa = w.a_s; g.sa_pitch = d;
  g.b0 = w.b; g.ldb = Kp; g.sb = w.b_s; g.sb_pitch = 2 * f;
  g.c0 = dWg; g.c1 = dWu; g.ldc = f; g.c_es = (long)d * f; g.c_split = f;
  g.accumulate = accumulate;
  MX_TRY(launch_grouped_gemm_mx(kind, g, num_cu, s));
  // dWd = A^T . dYs: A -> a [f][Kp], dYs -> b [d][Kp]
  MX_TRY(quant_tokens(A, f, f, offsets, w.poff, E, Kp, w.a, w.a_s, s));
  MX_TRY(quant_tokens(dYs, d, d, offsets, w.poff, E, Kp, w.b, w.b_s, s));
  GemmArgs h{};
  h.E = E; h.offsets = w.poff; h.rows_total = (int)Kp; h.ragged = RAG_K;
  h.M = f; h.N = d; h.K = (int)Kp;
  h.a = w.a; h.lda = Kp; h.sa = w.a_s; h.sa_pitch = f;
  h.b0 = w.b; h.ldb = Kp; h.sb = w.b_s; h.sb_pitch = d;
  h.c0 = dWd; h.ldc = d; h.c_es = (long)f * d; h.c_split = d;
  h.accumulate = accumulate;
  return launch_grouped_gemm_mx(kind, h, num_cu, s);
}

}  // namespace moe
