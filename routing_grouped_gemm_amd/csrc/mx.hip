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
// Weight scales are block-major ([block][row]); activation scales come in
// groups of four blocks, [K/128][row][4] with the row pitch rounded up to 16
// (mx_scale_at), so a stage's scales of a tile's 256 rows are one contiguous
// kilobyte.  Either way they arrive by the same buffer->LDS DMA as the
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
// Dispatch row copy with quantisation, token-major: each token row of x is
// read once (non-temporal: read once), quantised along d once, and written to
// every one of its k rows r = dest_row[t, j] as Xs[r] (bf16, for the weight
// gradients), Xq[r] (e4m3 codes) and the block scales of row r.  One wave per
// token; a lane holds four 8-value chunks 512 columns apart (a 32-value
// block spans the 4 lanes 4g..4g+3).  A slot whose row lies outside [0, R)
// writes nothing.
__global__ __launch_bounds__(256) void mx_dispatch_kernel(const bf16_t* __restrict__ x,
                                                          const int32_t* __restrict__ dest_row,
                                                          int T, int d, int k,
                                                          bf16_t* __restrict__ Xs,
                                                          uint8_t* __restrict__ Xq,
                                                          uint8_t* __restrict__ scale, long pitch) {
  const int lane = threadIdx.x & 63;
  const long t = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int R = T * k;
  for (int c0 = lane * 8; c0 < d; c0 += 2048) {
    uint4 raw[4];
    uint2 q[4];
    int E[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = min(c0 + 512 * u, d - 8);
      const u32x4_t w = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(x + t * d + c));
      raw[u] = uint4{w[0], w[1], w[2], w[3]};
      float v[8];
      unpack8(raw[u], v);
      uint32_t codes[2];
      E[u] = quant8(v, codes);
      q[u] = make_uint2(codes[0], codes[1]);
    }
    for (int j = 0; j < k; ++j) {
      const int r = dest_row[t * k + j];
      if (r < 0 || r >= R) continue;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int c = c0 + 512 * u;
        if (c < d) {
          const u32x4_t w = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
          __builtin_nontemporal_store(w, reinterpret_cast<u32x4_t*>(Xs + (long)r * d + c));
          *reinterpret_cast<uint2*>(Xq + (long)r * d + c) = q[u];
          if ((lane & 3) == 0) scale[mx_scale_at(r, c, pitch)] = (uint8_t)(E[u] + 127);
        }
      }
    }
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

// One pass over W[e][K][N] for both directions of the MXFP8 layer: a tile of
// 128 (k) x 128 (n) is read from HBM once (16 lanes a 256-byte row), staged
// in LDS, and quantised
//  * along N, written as stored exactly as mx_quant_rows_kernel writes it:
//    codes at dstR + (e*K + k)*dstR_ld + col0 + n, the scale of block b of row
//    k at sR[e*sR_es + (block0 + b)*pitchR + k] (the input-gradient GEMM's
//    operand); 16 lanes quantise one row, 8 values each, and write its 128
//    code bytes as one line;
//  * along K, written transposed exactly as mx_quant_cols_kernel writes it
//    (the forward GEMM's operand); a thread takes two adjacent columns (one
//    4-byte LDS read gives both) and one whole 32-value block of each; the
//    codes and scales are staged in LDS and written back as whole lines.
// K and N are multiples of 64 (every width the layer accepts); a tile's
// halves past them are skipped.  The grid is persistent (about as many
// workgroups as the chip holds at once): a workgroup takes tiles blockIdx.x,
// + gridDim.x, ..., and loads its next tile into registers before it
// quantises the current one, so the loads stream under the arithmetic.
__global__ __launch_bounds__(256) void mx_quant_both_kernel(
    const bf16_t* __restrict__ W, int E, int K, int N, uint8_t* __restrict__ dstC, long dstC_es,
    int half, uint8_t* __restrict__ sC, long sC_es, long pitchC, uint8_t* __restrict__ dstR,
    long dstR_ld, long col0, uint8_t* __restrict__ sR, long sR_es, long pitchR, int block0) {
  constexpr int TP = 136;  // LDS row pitch (bf16): 128 + 8
  __shared__ __attribute__((aligned(16))) bf16_t tile[128 * TP];
  const int t = threadIdx.x, lane = t & 63;
  const int nN = (N + 127) / 128, nK = (K + 127) / 128, ntiles = nN * nK * E;
  // tile L: n tiles fastest, then k tiles, then experts
  auto corner = [&](int L, int& e, int& k0, int& n0) {
    const int q = L / nN;
    n0 = (L - q * nN) * 128;
    e = q / nK;
    k0 = (q - e * nK) * 128;
  };
  // this thread's eight 16-byte pieces of tile L: rows t/16 + 16i, columns 8*(t%16) .. +7
  auto fetch = [&](int L, uint4 (&a)[8]) {
    int e, k0, n0;
    corner(L, e, k0, n0);
    const bf16_t* We = W + (long)e * K * N;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = (t >> 4) + 16 * i, c = (t & 15) * 8;
      a[i] = make_uint4(0, 0, 0, 0);
      if (k0 + r < K && n0 + c < N)
        a[i] = *reinterpret_cast<const uint4*>(We + (long)(k0 + r) * N + n0 + c);
    }
  };
  int L = blockIdx.x;
  if (L >= ntiles) return;
  uint4 nx[8];
  fetch(L, nx);
  for (; L < ntiles; L += gridDim.x) {
    int e, k0, n0;
    corner(L, e, k0, n0);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = (t >> 4) + 16 * i, c = (t & 15) * 8;
      *reinterpret_cast<uint4*>(&tile[r * TP + c]) = nx[i];
    }
    __syncthreads();
    // the next tile's loads are in flight while this one is quantised and written
    if (L + (int)gridDim.x < ntiles) fetch(L + gridDim.x, nx);
    // along N: rows 16p + t/16, columns 8*(t%16) .. +7
#pragma unroll 2
    for (int p = 0; p < 8; ++p) {
      const int r = 16 * p + (t >> 4), c = (t & 15) * 8;
      float v[8];
      unpack8(*reinterpret_cast<const uint4*>(&tile[r * TP + c]), v);
      const long k = k0 + r;
      // K and N are multiples of 64: the 4 lanes of a block leave together
      if (k < K && n0 + c < N)
        quant8_store(v, dstR + ((long)e * K + k) * dstR_ld + col0 + n0 + c,
                     sR + (long)e * sR_es + (long)(block0 + ((n0 + c) >> 5)) * pitchR + k, lane);
    }
    // along K: columns n0 + 2*(t%64) and +1, k = k0 + 32*(t/64) .. +31 (one
    // whole 32-value block of each of the two columns, read 4 bytes at a time)
    const int n = 2 * (t & 63), b = t >> 6;
    const int kb = k0 + 32 * b;
    const bool cval = n0 + n < N && kb < K;
    uint32_t wc[2][8];
    int ec[2] = {0, 0};
    if (cval) {
      float v0[32], v1[32];
      float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const uint32_t w2 = *reinterpret_cast<const uint32_t*>(&tile[(32 * b + i) * TP + n]);
        v0[i] = __uint_as_float(w2 << 16);
        v1[i] = __uint_as_float(w2 & 0xffff0000u);
        a0 = fmaxf(a0, fabsf(v0[i]));
        a1 = fmaxf(a1, fabsf(v1[i]));
      }
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const float(&v)[32] = c ? v1 : v0;
        const int ex = mx_block_exponent(c ? a1 : a0);
        ec[c] = ex;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float sv[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) sv[i] = ldexpf(v[8 * g + i], -ex);
          uint32_t c2[2];
          e4m3_codes8(sv, c2);
          wc[c][2 * g] = c2[0];
          wc[c][2 * g + 1] = c2[1];
        }
      }
    }
    // The transposed codes go out as whole 128-byte lines: staged in the tile's
    // LDS (free once every thread has read it) as 128 code rows, one per
    // column, of the tile's 128 k (16-byte chunks XOR-swizzled by the row),
    // plus the four blocks' scales of the 128 columns, then written back a
    // row's eight chunks by eight consecutive threads.  (Each thread writing
    // its own 32 bytes to four lines shared with three other waves took 60%
    // longer than the row half of the pass.)
    __syncthreads();
    uint8_t* cs = reinterpret_cast<uint8_t*>(tile);   // 16 KiB of codes, then 512 B of scales
    auto cswz = [](int r) { return (r >> 1) & 7; };
    if (cval) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int r = n + c;
        *reinterpret_cast<uint4*>(cs + r * 128 + (((2 * b) ^ cswz(r)) << 4)) =
            make_uint4(wc[c][0], wc[c][1], wc[c][2], wc[c][3]);
        *reinterpret_cast<uint4*>(cs + r * 128 + (((2 * b + 1) ^ cswz(r)) << 4)) =
            make_uint4(wc[c][4], wc[c][5], wc[c][6], wc[c][7]);
        cs[16384 + b * 128 + r] = (uint8_t)(ec[c] + 127);
      }
    }
    __syncthreads();
    const int kvalid = min(128, K - k0), nvalid = min(128, N - n0);
    // code row of column col (the gate/up panels interleave 128 gate and 128 up rows)
    auto rowof = [&](int col) -> long {
      return half >= 0 ? (long)((col >> 7) << 8) + 128 * half + (col & 127) : (long)col;
    };
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = t + 256 * i, r = q >> 3, ch = q & 7;
      if (r < nvalid && ch * 16 < kvalid) {
        const uint4 w = *reinterpret_cast<const uint4*>(cs + r * 128 + ((ch ^ cswz(r)) << 4));
        *reinterpret_cast<uint4*>(dstC + (long)e * dstC_es + rowof(n0 + r) * K + k0 + ch * 16) = w;
      }
    }
    // scales: block bb of the 128 columns is 128 consecutive bytes (their code
    // rows are consecutive), written as eight 16-byte pieces
    if (t < 32) {
      const int bb = t >> 3, piece = t & 7;
      if (bb * 32 < kvalid && piece * 16 < nvalid)
        *reinterpret_cast<uint4*>(sC + (long)e * sC_es + (long)((k0 >> 5) + bb) * pitchC + rowof(n0) +
                                  piece * 16) =
            *reinterpret_cast<const uint4*>(cs + 16384 + bb * 128 + piece * 16);
    }
    // every thread is done with the staged codes before the next tile is staged
    __syncthreads();
  }
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
// row of both operands, plus those rows' scales: block b of the B rows at
// STAGE + 4096 + b*1024; of the A rows of a weight gradient at STAGE +
// b*1024, of other A rows (grouped activation scales) the 4-byte word of
// tile row i at STAGE + (amis + i)*4, amis the tile's first row modulo 4.  One MFMA k-step
// takes 64 codes (two blocks), so a stage is two k-steps.
constexpr int MX_KSTEP = 64;
constexpr int SCALE_BYTES = 8192;
constexpr int MSTAGE = STAGE + SCALE_BYTES;
constexpr int MX_DMA_PER_STAGE = 2 * DMA_PER_OP + 2;   // codes of A and B, two scale blocks

typedef __attribute__((ext_vector_type(8))) int i32x8_t;

struct MxPlan {
  Plan a, b;
  i32x4_t srs;       // this wave's scale resource (waves 0-1: A, 2-3: B)
  uint32_t svoff;    // per-lane offset of the first scale DMA of stage 0 (kOutside: none)
  uint32_t sdelta;   // offset of the second scale DMA from the first
  uint32_t sstage;   // bytes between the scales of consecutive stages
  uint32_t sdst[2];  // LDS offsets of the two scale DMAs in the wave pair's 4 KiB
  int amis;          // A rows of grouped scales: the tile's first row modulo 4
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
template <bool DUAL, bool RK>
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
    F.sa[i] = RK ? Ss[blk * 1024 + row + (lane & 31)] : Ss[(amis + row + (lane & 31)) * 4 + blk];
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int col = DUAL ? ((q >> 1) * 128 + wn * 64 + (q & 1) * 32) : (wn * 128 + q * 32);
    F.b[q] = fragq(Bs, col, j, lane);
    F.sb[q] = Ss[4096 + blk * 1024 + col + (lane & 31)];
  }
}

// The first k-step of a tile: accumulators from a zero operand.
__device__ __forceinline__ void mx_mfma16_first(f32x16_t (&acc)[4][4], const MxFrags& F) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(F.b[j], F.a[i], f32x16_t{}, 0, 0,
                                                                  0, F.sb[j], 0, F.sa[i]);
}

__device__ __forceinline__ void mx_mfma16(f32x16_t (&acc)[4][4], const MxFrags& F) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(F.b[j], F.a[i], acc[i][j], 0, 0,
                                                                  0, F.sb[j], 0, F.sa[i]);
}

// Per-lane scale offset of the lanes past a tile's rows: outside every scale
// buffer (the host keeps each below 2^30 bytes), also after the stage and
// second-load offsets (each below 2^30) are added, so the lane makes no
// memory request and writes zeros to LDS bytes never read.
constexpr uint32_t kOutside = 0x80000000u;

// DMA of stage kt (codes of both operands, then this wave's two scale
// blocks), then the L2 prefetch of stage kt + PF_AHEAD: one 4-byte load per
// 128-byte line of a quarter of the tile's rows at per-lane offset pfv
// (wave 0: A, wave 2: B; waves 1 and 3 issue theirs against an empty range
// so that every wave counts the same).  Every call adds MX_DMA_PER_STAGE +
// PF_PER_STAGE loads to vmcnt, the prefetch last.  live == false (a stage
// past the tile's K) issues the same loads with an empty buffer range: no
// memory request, zeros into the stage buffer (free at that point; the K
// loop waits for these loads before the buffer is used again), and the
// vmcnt accounting of every other stage, without a branch.
__device__ __forceinline__ i32x4_t live_rsrc(i32x4_t r, bool live) {
  r.z = live ? r.z : 0;
  return r;
}
__device__ __forceinline__ void mx_issue(const MxPlan& P, uint32_t pfv, int kt, bool live,
                                         uint32_t st_base, uint32_t sink, int wave) {
  const i32x4_t ra = live_rsrc(P.a.rs0, live), rb = live_rsrc(P.b.rs0, live);
  const uint32_t soa = (uint32_t)kt * P.a.kstep, sob = (uint32_t)kt * P.b.kstep;
#pragma unroll
  for (int i = 0; i < DMA_PER_OP; ++i)
    dma16(ra, st_base + plan_lds(wave, i), (i & 1) ? P.a.v1 : P.a.v0, soa + (uint32_t)i * P.a.bstep);
#pragma unroll
  for (int i = 0; i < DMA_PER_OP; ++i)
    dma16(rb, st_base + OPB + plan_lds(wave, i), (i & 1) ? P.b.v1 : P.b.v0, sob + (uint32_t)i * P.b.bstep);
  // the stage offset goes into the per-lane offset, which the range check covers
  const i32x4_t rsc = live_rsrc(P.srs, live);
  const uint32_t dst = st_base + STAGE + (wave >> 1) * 4096;
#pragma unroll
  for (int b = 0; b < 2; ++b)
    dma16(rsc, dst + P.sdst[b], P.svoff + (uint32_t)b * P.sdelta + (uint32_t)kt * P.sstage, 0u);
  const i32x4_t rpf = live_rsrc(wave < 2 ? P.a.rs0 : P.b.rs0, live && (wave & 1) == 0);
  pf4(rpf, sink, pfv, (uint32_t)(kt + PF_AHEAD) * ROWB);
}

// The same loads as mx_issue in pieces: piece q < 16 is code block q of the
// wave (A's eight, then B's), piece 16 the scales and the prefetch.
__device__ __forceinline__ void mx_issue_piece(const MxPlan& P, uint32_t pfv, int kt, bool live,
                                               uint32_t st_base, uint32_t sink, int wave, int q) {
  if (q < DMA_PER_OP) {
    const i32x4_t ra = live_rsrc(P.a.rs0, live);
    dma16(ra, st_base + plan_lds(wave, q), (q & 1) ? P.a.v1 : P.a.v0,
          (uint32_t)kt * P.a.kstep + (uint32_t)q * P.a.bstep);
  } else if (q < 2 * DMA_PER_OP) {
    const int i = q - DMA_PER_OP;
    const i32x4_t rb = live_rsrc(P.b.rs0, live);
    dma16(rb, st_base + OPB + plan_lds(wave, i), (i & 1) ? P.b.v1 : P.b.v0,
          (uint32_t)kt * P.b.kstep + (uint32_t)i * P.b.bstep);
  } else {
    const i32x4_t rsc = live_rsrc(P.srs, live);
    const uint32_t dst = st_base + STAGE + (wave >> 1) * 4096;
#pragma unroll
    for (int b = 0; b < 2; ++b)
      dma16(rsc, dst + P.sdst[b], P.svoff + (uint32_t)b * P.sdelta + (uint32_t)kt * P.sstage, 0u);
    const i32x4_t rpf = live_rsrc(wave < 2 ? P.a.rs0 : P.b.rs0, live && (wave & 1) == 0);
    pf4(rpf, sink, pfv, (uint32_t)(kt + PF_AHEAD) * ROWB);
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
  __shared__ __attribute__((aligned(256))) uint32_t pf_sink[64];
  constexpr bool DUAL = KT<KIND>::BSP == BS_DUAL_N;
  constexpr int BNT = DUAL ? BN / 2 : BN;
  const int ntiles = sched_setup<BM, BNT, wgrad_kind(KIND)>(g, sch);
  const bool alt = wgrad_kind(KIND) && sch.alt;  // alternating rounds (logical_tile)
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const uint32_t lds0 = lds_u32(smem), sink = lds_u32(pf_sink);
  const uint8_t* A = static_cast<const uint8_t*>(g.a);
  const uint8_t* B = static_cast<const uint8_t*>(g.b0);

  // RK (weight gradients): the K axis is the tokens; tile rows are M rows
  // (features) of the transposed codes A[M][lda], columns N rows of B[N][ldb],
  // and the expert's K segment starts at byte t.row0 of every row (scale
  // block t.row0 / 32).  g.K is the padded token count.
  constexpr bool RK = KIND == GK_MX_WGRAD || KIND == GK_MX_WGRAD_F32;
  // Block-major scales (weights; both operands of a weight gradient): the
  // wave loads blocks sblk and sblk + 1 of every stage, 16 lanes x 16 bytes
  // each; base is the lane's offset of stage 0's block 0.
  auto plan_blockmajor = [&](MxPlan& P, long base, long pitch, bool lane_live) {
    const int sblk = 2 * (wave & 1);
    P.svoff = lane_live ? (uint32_t)(base + sblk * pitch) : kOutside;
    P.sdelta = (uint32_t)pitch;
    P.sstage = (uint32_t)(4 * pitch);
    P.sdst[0] = (uint32_t)sblk * 1024;
    P.sdst[1] = P.sdst[0] + 1024;
  };
  auto plan = [&](const Tile& t, MxPlan& P) {
    if constexpr (RK) {
      const long long abytes = (long long)g.M * g.lda, bbytes = (long long)g.N * g.ldb;
      const long aoff = (long)t.m0 * g.lda + t.row0, boff = (long)t.n0 * g.ldb + t.row0;
      plan_km(P.a, A + aoff, abytes - aoff, nullptr, 0, 1 << 30, g.lda, wave, lane);
      plan_km(P.b, B + boff, bbytes - boff, nullptr, 0, 1 << 30, g.ldb, wave, lane);
      P.amis = 0;
      const int kb = t.row0 >> 5;
      if (wave < 2) {
        P.srs = make_rsrc(g.sa, (long long)(g.K / 32) * g.sa_pitch);
        plan_blockmajor(P, (long)kb * g.sa_pitch + t.m0 + lane * 16, g.sa_pitch, lane < BM / 16);
      } else {
        P.srs = make_rsrc(g.sb, (long long)(g.K / 32) * g.sb_pitch);
        plan_blockmajor(P, (long)kb * g.sb_pitch + t.n0 + lane * 16, g.sb_pitch, lane < BM / 16);
      }
    } else {
      // rows of B for this tile: gate/up panels hold 256 rows per 128 f columns
      const long brow0 = DUAL ? 2L * t.n0 : (long)t.n0;
      const long brows = DUAL ? 2L * ((g.N + 127) / 128) * 128 : (long)g.N;
      // A's range ends at the tile's last row that exists: the DMA lanes of
      // the rows past it (a ragged tail) read zeros without a memory request
      plan_km(P.a, A + (long)t.row0 * g.lda, (long long)t.mlim * g.lda, nullptr, 0, 1 << 30,
              g.lda, wave, lane);
      plan_km(P.b, B + (long)t.e * g.b_es + brow0 * g.ldb, (brows - brow0) * g.ldb, nullptr, 0,
              1 << 30, g.ldb, wave, lane);
      // every wave reads A fragments, so every wave needs amis
      const int row_al = t.row0 & ~3;
      P.amis = t.row0 - row_al;
      if (wave < 2) {
        // Grouped activation scales: stage kt's scales of rows row_al .. are
        // the run of (amis + 256) 4-byte words at (kt * pitch + row_al) * 4;
        // wave 0 loads its first kilobyte, wave 1 the rest (at most 12
        // bytes).  The second DMA of each wave is an empty one (offset past
        // the range, zeros into LDS bytes never read) so that every wave
        // counts the same loads.
        const int o = (wave & 1) * 1024 + lane * 16;
        P.srs = make_rsrc(g.sa, (long long)((g.K + 127) / 128) * 4 * g.sa_pitch);
        P.svoff = o < (P.amis + BM) * 4 ? (uint32_t)(row_al * 4 + o) : kOutside;
        P.sdelta = 1u << 30;
        P.sstage = (uint32_t)(4 * g.sa_pitch);
        P.sdst[0] = (uint32_t)(wave & 1) * 1024;
        P.sdst[1] = 2048 + P.sdst[0];
      } else {
        P.srs = make_rsrc(g.sb + (long)t.e * g.sb_es, (long long)(g.K / 32) * g.sb_pitch);
        plan_blockmajor(P, brow0 + lane * 16, g.sb_pitch, lane < BM / 16);
      }
    }
  };
  auto stage_base = [&](int s) { return lds0 + (s & 1) * MSTAGE; };
  // the lane's L2 prefetch offset for tile t: a quarter of its A rows
  // (shared with the other N-tiles of the M-block) or of its B rows (shared
  // with the other M-tiles of the expert)
  auto pf_plan = [&](const Tile& t) -> uint32_t {
    return wave < 2 ? pf_quarter(t.n0 / BNT, lane, g.lda) : pf_quarter(t.m0 / BM, lane, g.ldb);
  };

  int it = 0;
  int L = logical_tile(it, alt);
  if (L >= ntiles) return;
  Tile t = sched_decode<BM, BNT, wgrad_kind(KIND)>(g, sch, L);
  MxPlan P;
  plan(t, P);
  uint32_t pfv = pf_plan(t);
  // K is a multiple of 64: a last stage may hold a single k-step
  int ns = t.klen / MX_KSTEP, nk = (ns + 1) / 2;
  mx_issue(P, pfv, 0, nk > 0, stage_base(0), sink, wave);
  mx_issue(P, pfv, 1, nk > 1, stage_base(1), sink, wave);

  for (;;) {
    // Stages 0 and 1 of tile t are in flight (as far as they exist).  A
    // stage is two k-steps; K an odd multiple of 64 ends with a half stage.
    // The first k-step writes the accumulators from a zero operand, so they
    // are cleared only for a tile without a full stage.
    const int nfull = ns >> 1;
    f32x16_t acc[4][4];
    if (nfull == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x16_t{};
    }

    // Per stage: the fragments of step 1 are read while the MFMAs of step 0
    // run; after them one barrier publishes stage kt+1 (each wave waited for
    // its own DMA) and frees stage kt's buffer for stage kt+2, whose DMA
    // then runs under the MFMAs of step 1 and of all of stage kt+1; the
    // fragments of stage kt+1's step 0 are read under step 1's MFMAs.  The
    // fragment sets keep their roles from stage to stage (straight-line
    // code, no register copies).
    MxFrags F0, F1;
    if (nk > 0) {
      // stage 1 and both prefetches may still be in flight
      wait_vmcnt<MX_DMA_PER_STAGE + 2 * PF_PER_STAGE>();
      barrier();
      load_mx_frags<DUAL, RK>(smem, 0, 0, wm, wn, lane, P.amis, F0);
    }
    // One full stage (FIRST: the tile's first, accumulators from a zero
    // operand).  The loop body is one basic block: with a branch between
    // the two k-steps the compiler sank the first step's MFMAs below the
    // barrier and the DMA issue.
    auto stage = [&](int kt, auto FIRST) {
      __builtin_amdgcn_s_waitcnt(kLgkm0);
      load_mx_frags<DUAL, RK>(smem, kt, 1, wm, wn, lane, P.amis, F1);
      if constexpr (decltype(FIRST)::value) mx_mfma16_first(acc, F0); else mx_mfma16(acc, F0);
      interleave_mx();
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(kLgkm0);
      // stage kt+1 (possibly an empty one past K) has landed once only its
      // prefetch loads may be pending
      wait_vmcnt<PF_PER_STAGE>();
      barrier();
      // read even past the last stage (stale bytes, never used), so that
      // the fragment registers have one definition
      load_mx_frags<DUAL, RK>(smem, kt + 1, 0, wm, wn, lane, P.amis, F0);
      __builtin_amdgcn_sched_barrier(0);
      // Stage kt+2's loads (an empty stage's past K) go out one after each
      // MFMA of step 1: a wave stalls while the load path takes a load, and
      // the MFMA issued just before it keeps the matrix core busy meanwhile
      // (one burst after the barrier left it idle for the whole issue).
      {
        const bool live = kt + 2 < nk;
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int i = q >> 2, j = q & 3;
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(F1.b[j], F1.a[i], acc[i][j], 0,
                                                                      0, 0, F1.sb[j], 0, F1.sa[i]);
          mx_issue_piece(P, pfv, kt + 2, live, stage_base(kt), sink, wave, q);
          __builtin_amdgcn_sched_barrier(0);
        }
        mx_issue_piece(P, pfv, kt + 2, live, stage_base(kt), sink, wave, 16);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    if (nfull > 0) {
      stage(0, std::true_type{});
      for (int kt = 1; kt < nfull; ++kt) stage(kt, std::false_type{});
    }
    if (ns & 1) {
      // the half stage: its step 0 was read into F0
      __builtin_amdgcn_s_waitcnt(kLgkm0);
      mx_mfma16(acc, F0);
      __builtin_amdgcn_sched_barrier(0);
    }
    // the loads of the last stages (empty ones, which write zeros into the
    // stage buffers) are done before the epilogue stages through buffer 1
    // and the next tile's stage 0 loads into buffer 0
    wait_vmcnt<0>();
    __builtin_amdgcn_s_waitcnt(kLgkm0);
    barrier();

    // next tile's stage 0 loads into buffer 0 during this epilogue, which
    // stages through buffer 1; its stage 1 follows the epilogue
    L = logical_tile(++it, alt);
    const bool has_next = L < ntiles;
    Tile tn = t;
    MxPlan Pn = P;
    int nsn = 0, nkn = 0;
    if (has_next) {
      tn = sched_decode<BM, BNT, wgrad_kind(KIND)>(g, sch, L);
      plan(tn, Pn);
      pfv = pf_plan(tn);
      nsn = tn.klen / MX_KSTEP;
      nkn = (nsn + 1) / 2;
      mx_issue(Pn, pfv, 0, nkn > 0, stage_base(0), sink, wave);
    }
    epilogue_lds<KIND>(g, t, smem + MSTAGE + wave * EPI_SLICE, acc, wm, wn, lane);
    barrier();
    if (!has_next) break;
    mx_issue(Pn, pfv, 1, nkn > 1, stage_base(1), sink, wave);
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

// W[E][K][N] quantised along K into the forward's transposed layout (as
// quant_cols) and along N into the input gradient's layout (as quant_rows
// with groups of K rows), from one read of W.
hipError_t quant_both(const void* W, int E, int K, int N, uint8_t* dstC, long dstC_es, int half,
                      uint8_t* sC, long sC_es, long pitchC, uint8_t* dstR, long dstR_ld, long col0,
                      uint8_t* sR, long sR_es, long pitchR, int block0, int num_cu,
                      hipStream_t s) {
  const long ntiles = (long)((N + 127) / 128) * ((K + 127) / 128) * E;
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, mx_quant_both_kernel, 256, 0) !=
          hipSuccess ||
      per_cu < 1)
    per_cu = 1;
  const long cap = (long)num_cu * per_cu;
  const int grid = (int)(ntiles < cap ? ntiles : cap);
  note_prelaunch("mx_quant_weights", s);
  hipLaunchKernelGGL(mx_quant_both_kernel, dim3(grid), dim3(256), 0, s,
                     static_cast<const bf16_t*>(W), E, K, N, dstC, dstC_es, half, sC, sC_es,
                     pitchC, dstR, dstR_ld, col0, sR, sR_es, pitchR, block0);
  note_launch("mx_quant_weights", s);
  return hipGetLastError();
}

inline long pitch_rows(long R) { return (R + 15) / 16 * 16; }
// bytes of the grouped activation scales of R rows of K elements
inline size_t act_scale_bytes(long R, long K) { return (size_t)((K + 127) / 128) * 4 * pitch_rows(R); }
inline long fpanel(int f) { return (f + 127) / 128 * 128; }

// Forward workspace pieces, in carving order.
// keep: the backward's weight codes follow (moe_grouped_ffn_fwd with
// MOE_MX_KEEP_WEIGHTS writes them, moe_grouped_ffn_bwd with the flag reads
// them): Wd along d [E][f][d], and Wg | Wu along f [E][d][2f], with scales.
struct FwdWs {
  uint8_t *wgu, *wgu_s, *wd, *wd_s, *aq, *aq_s;
  uint8_t *bwd_wd, *bwd_wd_s, *bwd_wgu, *bwd_wgu_s;
};
FwdWs carve_fwd(void* ws, long long R, int d, int f, int E, bool keep, size_t* total) {
  Carve c{static_cast<char*>(ws)};
  FwdWs w;
  const long fp = fpanel(f);
  w.wgu = c.take<uint8_t>((size_t)E * 2 * fp * d);
  w.wgu_s = c.take<uint8_t>((size_t)E * (d / 32) * 2 * fp);
  w.wd = c.take<uint8_t>((size_t)E * d * f);
  w.wd_s = c.take<uint8_t>((size_t)E * (f / 32) * d);
  w.aq = c.take<uint8_t>((size_t)R * f);
  w.aq_s = c.take<uint8_t>(act_scale_bytes(R, f));
  w.bwd_wd = w.bwd_wd_s = w.bwd_wgu = w.bwd_wgu_s = nullptr;
  if (keep) {
    w.bwd_wd = c.take<uint8_t>((size_t)E * f * d);
    w.bwd_wd_s = c.take<uint8_t>((size_t)E * (d / 32) * f);
    w.bwd_wgu = c.take<uint8_t>((size_t)E * d * 2 * f);
    w.bwd_wgu_s = c.take<uint8_t>((size_t)E * (2 * f / 32) * d);
  }
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
  w.wd = c.take<uint8_t>((size_t)E * f * d);
  w.wd_s = c.take<uint8_t>((size_t)E * (d / 32) * f);
  w.dhq = c.take<uint8_t>((size_t)R * 2 * f);
  w.dhq_s = c.take<uint8_t>(act_scale_bytes(R, 2L * f));
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

size_t mx_fwd_workspace(long long R, int d, int f, int E, bool keep) {
  size_t t = 0;
  carve_fwd(nullptr, R, d, f, E, keep, &t);
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

hipError_t launch_mx_dispatch_copy(const void* x, const int32_t* dest_row, int T, int d, int k,
                                   void* Xs, void* Xq, uint8_t* Xq_scale, hipStream_t s) {
  if (T == 0) return hipSuccess;
  note_prelaunch("mx_dispatch_quant", s);
  hipLaunchKernelGGL(mx_dispatch_kernel, dim3((T + 3) / 4), dim3(256), 0, s,
                     static_cast<const bf16_t*>(x), dest_row, T, d, k, static_cast<bf16_t*>(Xs),
                     static_cast<uint8_t*>(Xq), Xq_scale, pitch_rows((long)T * k));
  note_launch("mx_dispatch_quant", s);
  return hipGetLastError();
}

hipError_t mx_ffn_fwd(const void* Xq, const uint8_t* Xscale, const int32_t* offsets, int R, int d,
                      int f, int E, const void* Wg, const void* Wu, const void* Wd, void* Hg,
                      void* Hu, void* A, void* Ys, void* ws, bool keep, int num_cu,
                      hipStream_t s) {
  const FwdWs w = carve_fwd(ws, R, d, f, E, keep, nullptr);
  const long fp = fpanel(f), Rp = pitch_rows(R);
  // weights: Wg, Wu along d into the gate/up panels; Wd along f, transposed;
  // keep: in the same pass, Wd along d and Wg | Wu along f for the backward
  if (keep) {
    MX_TRY(quant_both(Wg, E, d, f, w.wgu, 2 * fp * d, 0, w.wgu_s, (d / 32) * 2 * fp, 2 * fp,
                      w.bwd_wgu, 2L * f, 0, w.bwd_wgu_s, (long)(2 * f / 32) * d, d, 0, num_cu, s));
    MX_TRY(quant_both(Wu, E, d, f, w.wgu, 2 * fp * d, 1, w.wgu_s, (d / 32) * 2 * fp, 2 * fp,
                      w.bwd_wgu, 2L * f, f, w.bwd_wgu_s, (long)(2 * f / 32) * d, d, f / 32, num_cu, s));
    MX_TRY(quant_both(Wd, E, f, d, w.wd, (long)d * f, -1, w.wd_s, (long)(f / 32) * d, d,
                      w.bwd_wd, d, 0, w.bwd_wd_s, (long)(d / 32) * f, f, 0, num_cu, s));
  } else {
    MX_TRY(quant_cols(Wg, E, d, f, w.wgu, 2 * fp * d, 0, w.wgu_s, (d / 32) * 2 * fp, 2 * fp, s));
    MX_TRY(quant_cols(Wu, E, d, f, w.wgu, 2 * fp * d, 1, w.wgu_s, (d / 32) * 2 * fp, 2 * fp, s));
    MX_TRY(quant_cols(Wd, E, f, d, w.wd, (long)d * f, -1, w.wd_s, (long)(f / 32) * d, d, s));
  }
  GemmArgs g{};
  g.E = E; g.offsets = offsets; g.rows_total = R; g.ragged = RAG_M;
  g.N = f; g.K = d;
  g.a = Xq; g.lda = d; g.sa = Xscale; g.sa_pitch = Rp;
  g.b0 = w.wgu; g.ldb = d; g.b_es = 2 * fp * d;
  g.sb = w.wgu_s; g.sb_es = (d / 32) * 2 * fp; g.sb_pitch = 2 * fp;
  g.c0 = Hg; g.c1 = Hu; g.c2 = A; g.ldc = f;
  g.q0 = w.aq; g.qs = w.aq_s; g.qs_pitch = Rp;   // A quantised along f in the epilogue
  g.m_fast = 1;
  MX_TRY(launch_grouped_gemm_mx(GK_MX_GATEUP, g, num_cu, s));
  GemmArgs h{};
  h.E = E; h.offsets = offsets; h.rows_total = R; h.ragged = RAG_M;
  h.N = d; h.K = f;
  h.a = w.aq; h.lda = f; h.sa = w.aq_s; h.sa_pitch = Rp;
  h.b0 = w.wd; h.ldb = f; h.b_es = (long)d * f;
  h.sb = w.wd_s; h.sb_es = (long)(f / 32) * d; h.sb_pitch = d;
  h.c0 = Ys; h.ldc = d;
  h.m_fast = 1;
  return launch_grouped_gemm_mx(GK_MX_DOWN, h, num_cu, s);
}

hipError_t mx_ffn_dgrad(const void* dYsq, const uint8_t* dYsq_scale, const void* Hg,
                        const void* Hu, const int32_t* offsets, int R, int d, int f, int E,
                        const void* Wg, const void* Wu, const void* Wd, void* dH, void* dXs,
                        void* ws, const void* kept, int num_cu, hipStream_t s) {
  BwdWs w = carve_bwd(ws, R, d, f, E, nullptr);
  const long Rp = pitch_rows(R);
  if (kept) {
    // the forward's workspace holds Wd along d and Wg | Wu along f already
    const FwdWs k = carve_fwd(const_cast<void*>(kept), R, d, f, E, true, nullptr);
    w.wd = k.bwd_wd; w.wd_s = k.bwd_wd_s; w.wgu = k.bwd_wgu; w.wgu_s = k.bwd_wgu_s;
  } else {
    // down dgrad: dYs (quantised along d by the combine backward) and Wd along d
    MX_TRY(quant_rows(Wd, (long)E * f, d, d, w.wd, d, 0, w.wd_s, f, (long)(d / 32) * f, f, 0, s));
  }
  GemmArgs g{};
  g.E = E; g.offsets = offsets; g.rows_total = R; g.ragged = RAG_M;
  g.N = f; g.K = d;
  g.a = dYsq; g.lda = d; g.sa = dYsq_scale; g.sa_pitch = Rp;
  g.b0 = w.wd; g.ldb = d; g.b_es = (long)f * d;
  g.sb = w.wd_s; g.sb_es = (long)(d / 32) * f; g.sb_pitch = f;
  g.c0 = dH; g.ldc = 2L * f; g.c_split = f;
  g.h0 = Hg; g.h1 = Hu; g.ldh = f;
  g.q0 = w.dhq; g.qs = w.dhq_s; g.qs_pitch = Rp;   // dH quantised along 2f in the epilogue
  g.m_fast = 1;
  MX_TRY(launch_grouped_gemm_mx(GK_MX_DGRAD_DOWN, g, num_cu, s));
  // gate/up dgrad: Wg | Wu along f into one [d][2f] matrix per expert
  if (!kept) {
    MX_TRY(quant_rows(Wg, (long)E * d, f, f, w.wgu, 2L * f, 0, w.wgu_s, d, (long)(2 * f / 32) * d,
                      d, 0, s));
    MX_TRY(quant_rows(Wu, (long)E * d, f, f, w.wgu, 2L * f, f, w.wgu_s, d, (long)(2 * f / 32) * d,
                      d, f / 32, s));
  }
  GemmArgs h{};
  h.E = E; h.offsets = offsets; h.rows_total = R; h.ragged = RAG_M;
  h.N = d; h.K = 2 * f;
  h.a = w.dhq; h.lda = 2L * f; h.sa = w.dhq_s; h.sa_pitch = Rp;
  h.b0 = w.wgu; h.ldb = 2L * f; h.b_es = (long)d * 2 * f;
  h.sb = w.wgu_s; h.sb_es = (long)(2 * f / 32) * d; h.sb_pitch = d;
  h.c0 = dXs; h.ldc = d;
  h.m_fast = 1;
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
