// Router logits of a bf16 batch: logits[t][e] = sum_k x[t][k] Wr[k][e] with
// float32 accumulation (HF OLMoE walkthrough, section 2: the router is one
// linear map from a token's hidden state to a logit per expert).
//
// The product is thin (at most 256 expert columns), so the general grouped
// GEMM's 256x256 tiles would use a few dozen workgroups and waste most of
// their MFMA work on absent columns.  Here a workgroup takes 32 tokens and
// every expert over the whole contraction: the router weights
// pass through LDS in chunks of KC k-rows, transposed on the way in so that
// each expert's k run is contiguous, and each wave multiplies them with its
// tokens' rows, read straight from HBM into registers, on 16x16x32 bf16
// MFMAs.  Later chunks of both operands are loaded while the current one is
// multiplied.  No workspace, one kernel; softmax and top-k follow in their
// own kernel.
#include <type_traits>

#include "gemm_dev.h"
#include "hook.h"
#include "moe_common.h"
#include "route.h"

namespace moe {

constexpr int kRlTokens = 32;    // tokens per workgroup

typedef __attribute__((ext_vector_type(4))) short i16x4_t;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

// NB blocks of 16 experts (1, 2, 4, 8 or 16): chunk length KC (a multiple
// of 64 in [64, 256], chunk within 32 KiB) and bytes per chunk row (one k).
__host__ __device__ constexpr int rl_kc(int nb) {
  return (16384 / (16 * nb)) / 64 * 64 < 64    ? 64
         : (16384 / (16 * nb)) / 64 * 64 > 256 ? 256
                                                : (16384 / (16 * nb)) / 64 * 64;
}
__host__ __device__ constexpr int rl_rowb(int nb) { return 32 * nb; }
__host__ __device__ constexpr int rl_lds(int nb) { return 2 * rl_kc(nb) * rl_rowb(nb); }

// A chunk sits in LDS as Wr's own rows (k-major, 16-byte chunks of 8
// experts), each row's chunks XOR-permuted in pairs by a function of k.
// Weight fragments are read with ds_read_b64_tr_b16: a 16-lane group reads
// 4 k-rows x 16 experts and each lane receives one expert at 4 consecutive
// k.  One fragment read of a wave touches k-rows kb + 8G + j (G = lane/16,
// j = 0..3) and one 32-byte pair per row; the permutation puts those 16 rows
// on distinct 32-byte bank positions two by two (the least a 512-byte read
// needs), given where each row starts in the 256-byte bank window.
template <int NB>
__device__ __forceinline__ int rl_swz(int k) {
  const int j = k & 3, G = (k >> 3) & 3;
  if constexpr (NB >= 8) return j | ((G & 1) << 2);
  else if constexpr (NB == 4) return ((j >> 1) ^ G) & 3;
  else if constexpr (NB == 2) return G & 1;
  else return 0;
}
template <int NB>
__device__ __forceinline__ int rl_off(int k, int chunk) {
  return k * rl_rowb(NB) + ((chunk ^ (2 * rl_swz<NB>(k))) << 4);
}

// Waves 0-1 take tokens 0-15 and 16-31 of the workgroup for k 0-31 of every
// 64-row piece, waves 2-3 the same tokens for k 32-63; the two halves are
// added at the end.  Each wave's rows of x arrive three chunks ahead of
// their use and the weight chunks two ahead (in registers), so several HBM
// and L2 round trips are in flight at once.  Every global load is issued
// unconditionally (addresses past the end are clamped to loaded data that is
// then not used), which keeps the compiler's wait counts exact.
template <int NB>
__global__ __launch_bounds__(256, 1) void router_logits_kernel(const uint16_t* __restrict__ x,
                                                               const uint16_t* __restrict__ Wr,
                                                               int T, int d, int E,
                                                               float* __restrict__ logits) {
  constexpr int KC = rl_kc(NB), NP = KC / 64, RB = rl_rowb(NB);
  constexpr int NCH = 2 * NB;               // 16-byte chunks per row
  constexpr int UPT = KC * NCH / 256;       // fill units (one chunk of one row) per thread
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  char* const buf0 = lds;
  char* const buf1 = lds + KC * RB;
  const int tg = wave & 1, h = wave >> 1;
  const int t0 = blockIdx.x * kRlTokens + tg * 16;
  const int tl = lane & 15, G = lane >> 4;
  const long trow = min(t0 + tl, T - 1);
  // lane (token tl, k-group G) of half h supplies k = 64p + 32h + 8G + (0..7)
  // of piece p; the weight fragments use the same k assignment
  const uint16_t* xp = x + trow * d + 32 * h + 8 * G;
  const int oct = E >> 3;                  // chunks of a row that hold experts
  const int units = KC * oct;              // fill units per chunk
  const int nch = (d + KC - 1) / KC;
  const int np_last = (d - (nch - 1) * KC) >> 6;  // pieces of the last chunk

  // chunks oct.. of every row of both buffers hold the zero padding experts
  if (oct < NCH) {
    const int per = KC * (NCH - oct);
    for (int i = tid; i < 2 * per; i += 256) {
      const int b = i / per, r = i - b * per;
      const int k = r / (NCH - oct), c = oct + r % (NCH - oct);
      *reinterpret_cast<u32x4_t*>((b ? buf1 : buf0) + rl_off<NB>(k, c)) = u32x4_t{0, 0, 0, 0};
    }
  }

  // this thread's fill units: row uk and 8-expert group uo (clamped into
  // range for the loads; units past the end are not stored)
  int uk[UPT], uo[UPT];
#pragma unroll
  for (int i = 0; i < UPT; ++i) {
    const int u = min(tid + 256 * i, units - 1);
    uk[i] = u / oct;
    uo[i] = u - uk[i] * oct;
  }
  auto load_w = [&](int c, u32x4_t (&wr)[UPT]) __attribute__((always_inline)) {
    const int k0 = c * KC, klast = min(KC, d - k0) - 1;
    const uint16_t* const base = Wr + (long)k0 * E;
#pragma unroll
    for (int i = 0; i < UPT; ++i)
      wr[i] = *reinterpret_cast<const u32x4_t*>(base + min(uk[i], klast) * E + 8 * uo[i]);
  };
  auto store_w = [&](int c, const u32x4_t (&wr)[UPT]) __attribute__((always_inline)) {
    char* const B = (c & 1) ? buf1 : buf0;
#pragma unroll
    for (int i = 0; i < UPT; ++i)
      if (tid + 256 * i < units) *reinterpret_cast<u32x4_t*>(B + rl_off<NB>(uk[i], uo[i])) = wr[i];
  };
  auto load_x = [&](int c, u32x4_t (&xv)[NP]) __attribute__((always_inline)) {
    const int k0 = c * KC, pl = (min(KC, d - k0) >> 6) - 1;
#pragma unroll
    for (int p = 0; p < NP; ++p)
      xv[p] = *reinterpret_cast<const u32x4_t*>(xp + k0 + 64 * min(p, pl));
  };
  // weight fragment of expert block nb, piece p: experts 16nb + tl at
  // k = 64p + 32h + 8G + (0..7), from two transposing reads of 4 k-rows
  auto wfrag = [&](const char* B, int nb, int p) __attribute__((always_inline)) {
    const int r = tl;
    const int k = 64 * p + 32 * h + 8 * G + (r >> 2);
    const int chunk = 2 * nb + ((r & 3) >> 1);
    const char* q = B + rl_off<NB>(k, chunk) + 8 * (r & 1);
    const char* q4 = B + rl_off<NB>(k + 4, chunk) + 8 * (r & 1);
    const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(q));
    const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(q4));
    typedef __attribute__((ext_vector_type(8))) short i16x8_t;
    const i16x8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8_t, v);
  };

  f32x4_t acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // D[expert][token]: this lane gets experts 16nb + 4G + (0..3) of token tl
  auto mma = [&](int c, const u32x4_t (&xv)[NP]) __attribute__((always_inline)) {
    const char* const B = (c & 1) ? buf1 : buf0;
    const int np = (c < nch - 1) ? NP : np_last;
#pragma unroll
    for (int p = 0; p < NP; ++p)
      if (p < np) {
        const bf16x8_t xf = __builtin_bit_cast(bf16x8_t, xv[p]);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wfrag(B, nb, p), xf, acc[nb], 0, 0, 0);
      }
  };

  u32x4_t xr[4][NP];    // x pieces of chunks c .. c+3 (slot c & 3)
  u32x4_t wr[2][UPT];   // weight units of chunks c+1, c+2 (slot c & 1)
  load_w(0, wr[0]);
#pragma unroll
  for (int i = 0; i < 3; ++i) load_x(min(i, nch - 1), xr[i]);
  store_w(0, wr[0]);
  load_w(min(1, nch - 1), wr[1]);
  load_w(min(2, nch - 1), wr[0]);
  __syncthreads();
  // chunk c: x and weights of chunk c+3 are requested, chunk c is
  // multiplied, chunk c+1's weights go to the other buffer (which every wave
  // left at the barrier closing chunk c-1); past the last chunk the loads
  // repeat it and the rest is skipped
  auto step = [&](auto slot, int c) __attribute__((always_inline)) {
    constexpr int X = decltype(slot)::value;
    load_x(min(c + 3, nch - 1), xr[(X + 3) & 3]);
    if (c < nch) mma(c, xr[X]);
    if (c + 1 < nch) store_w(c + 1, wr[(X + 1) & 1]);
    load_w(min(c + 3, nch - 1), wr[(X + 1) & 1]);
    __syncthreads();
  };
  for (int c = 0; c < nch; c += 4) {
    step(std::integral_constant<int, 0>{}, c);
    step(std::integral_constant<int, 1>{}, c + 1);
    step(std::integral_constant<int, 2>{}, c + 2);
    step(std::integral_constant<int, 3>{}, c + 3);
  }

  // k halves: waves 2-3 leave their sums in LDS, waves 0-1 add them (in that
  // order) and store
  float* const red = reinterpret_cast<float*>(lds);  // [2 token groups][NB][64 lanes][4]
  if (h == 1) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      *reinterpret_cast<f32x4_t*>(red + ((tg * NB + nb) * 64 + lane) * 4) = acc[nb];
  }
  __syncthreads();
  const int t = t0 + tl;
  if (h == 0 && t < T) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int e = 16 * nb + 4 * G;
      if (e < E) {
        const f32x4_t o = *reinterpret_cast<const f32x4_t*>(red + ((tg * NB + nb) * 64 + lane) * 4);
        *reinterpret_cast<f32x4_t*>(logits + (long)t * E + e) = acc[nb] + o;
      }
    }
  }
}

bool router_logits_applies(int d, int E) { return E % 8 == 0 && E <= 256 && d % 64 == 0; }

hipError_t launch_router_logits(const uint16_t* x, const uint16_t* Wr, int T, int d, int E,
                                float* logits, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const dim3 grid((T + kRlTokens - 1) / kRlTokens);
  const int nb = (E + 15) / 16;
  // expert blocks rounded up to a power of two (the padding experts are zero)
  note_prelaunch("router_logits", s);
  if (nb <= 1)
    hipLaunchKernelGGL(router_logits_kernel<1>, grid, dim3(256), rl_lds(1), s, x, Wr, T, d, E, logits);
  else if (nb <= 2)
    hipLaunchKernelGGL(router_logits_kernel<2>, grid, dim3(256), rl_lds(2), s, x, Wr, T, d, E, logits);
  else if (nb <= 4)
    hipLaunchKernelGGL(router_logits_kernel<4>, grid, dim3(256), rl_lds(4), s, x, Wr, T, d, E, logits);
  else if (nb <= 8)
    hipLaunchKernelGGL(router_logits_kernel<8>, grid, dim3(256), rl_lds(8), s, x, Wr, T, d, E, logits);
  else
    hipLaunchKernelGGL(router_logits_kernel<16>, grid, dim3(256), rl_lds(16), s, x, Wr, T, d, E,
                       logits);
  note_launch("router_logits", s);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// router backward, input gradient: dx[t][c] += sum_e dl[t][e] Wr[c][e]
// ---------------------------------------------------------------------------
// dl16 [T][ld] bf16 (zero past E, ld = 64 * ceil(E / 64)) and Wr [d][E] both
// run along e in memory, so both MFMA operands come straight from global
// memory (Wr from L2).  A workgroup takes 64 tokens (32 when ld > 128) and
// each of its waves one of P column parts, 64 columns at a time as four
// 16x16 blocks per 16-token quarter (D[column][token] on 16x16x32 bf16
// MFMAs over K = ld); each weight fragment read from L2 feeds the MFMAs of
// every quarter, so Wr is read once per 64 tokens (with 16 tokens a wave it
// was read four times as often: 156 -> 104 us at 16384 tokens x 4096 x 128
// experts going from 16 to 32 tokens).  The block sums pass through a private LDS slice so that dx is
// read and written in 16-byte pieces along its rows (8 tokens x 128 bytes
// per instruction); each element gets one bf16 rounding of old + sum.  The
// old dx of the next 64 columns is loaded while the current ones are
// computed; loads are unconditional (clamped to the last group, whose
// duplicate is not stored).
// NK = ld / 32 K-steps; H 16-token halves per wave (2 or 4: 32 or 64 tokens,
// each weight fragment feeding H MFMAs).
constexpr int kRdxPitch = 68;  // floats per token row of a wave's LDS slice (64 + skew)

template <int NK, int H>
__global__ __launch_bounds__(256) void router_dx_kernel(const uint16_t* __restrict__ dl16, int ld,
                                                        const uint16_t* __restrict__ Wr, int T,
                                                        int d, int E, uint16_t* __restrict__ dx) {
  constexpr int TW = 16 * H;   // tokens of the workgroup
  constexpr int NQ = TW / 8;   // dx row groups of a lane
  __shared__ __attribute__((aligned(16))) float slice_all[4][TW * kRdxPitch];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // the workgroup's TW tokens, each wave a column part of them
  const int part = blockIdx.y * 4 + wave, P = gridDim.y * 4;
  const int tl = lane & 15, G = lane >> 4;
  const int tbase = blockIdx.x * TW;
  float* const slice = slice_all[wave];
  // MFMA side: token set h (tokens 16h + tl), lane k-group G supplies
  // k = 32s + 8G + (0..7); each weight fragment serves every set
  bf16x8_t bfr[H][NK];
#pragma unroll
  for (int h = 0; h < H; ++h) {
    const long trow = min(tbase + 16 * h + tl, T - 1);
#pragma unroll
    for (int s = 0; s < NK; ++s)
      bfr[h][s] = __builtin_bit_cast(
          bf16x8_t, *reinterpret_cast<const u32x4_t*>(dl16 + trow * ld + 32 * s + 8 * G));
  }
  bool eok[NK];
  int eoff[NK];
#pragma unroll
  for (int s = 0; s < NK; ++s) {
    const int e = 32 * s + 8 * G;
    eok[s] = e < E;
    eoff[s] = min(e, E - 8);
  }
  // dx side: lane (rows r + 8q, q = 0..NQ-1; 8 columns at 8cq)
  const int r = lane >> 3, cq = lane & 7;
  int trw[NQ];
  uint16_t* xr[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    trw[q] = tbase + r + 8 * q;
    xr[q] = dx + (long)min(trw[q], T - 1) * d + 8 * cq;
  }

  const int ngrp = d / 64;
  const int per = (ngrp + P - 1) / P;  // 64-column groups of each part
  const int g0 = part * per;
  const int ng = min(per, ngrp - g0);
  if (ng <= 0) return;

  auto load_old = [&](int gi, u32x4_t (&o)[NQ]) __attribute__((always_inline)) {
    const int c0 = 64 * (g0 + min(gi, ng - 1));
#pragma unroll
    for (int q = 0; q < NQ; ++q) o[q] = *reinterpret_cast<const u32x4_t*>(xr[q] + c0);
  };
  auto compute = [&](int gi, const u32x4_t (&o)[NQ]) __attribute__((always_inline)) {
    const int c0 = 64 * (g0 + gi);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint16_t* const wr = Wr + (long)(c0 + 16 * j + tl) * E;
      u32x4_t w[NK];
#pragma unroll
      for (int s = 0; s < NK; ++s) w[s] = *reinterpret_cast<const u32x4_t*>(wr + eoff[s]);
      f32x4_t acc[H];
#pragma unroll
      for (int h = 0; h < H; ++h) acc[h] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NK; ++s) {
        const bf16x8_t a = __builtin_bit_cast(bf16x8_t, eok[s] ? w[s] : u32x4_t{0, 0, 0, 0});
#pragma unroll
        for (int h = 0; h < H; ++h)
          acc[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bfr[h][s], acc[h], 0, 0, 0);
      }
      // columns 16j + 4G + (0..3) of tokens 16h + tl
#pragma unroll
      for (int h = 0; h < H; ++h)
        *reinterpret_cast<f32x4_t*>(slice + (16 * h + tl) * kRdxPitch + 16 * j + 4 * G) = acc[h];
    }
    // the slice is private to the wave and LDS accesses of a wave complete in order
    __builtin_amdgcn_wave_barrier();
    f32x4_t v0[NQ], v1[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const f32x4_t* pv = reinterpret_cast<const f32x4_t*>(slice + (r + 8 * q) * kRdxPitch + 8 * cq);
      v0[q] = pv[0];
      v1[q] = pv[1];
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      float o8[8], v[8];
      unpack8(uint4{o[q][0], o[q][1], o[q][2], o[q][3]}, o8);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        v[u] = v0[q][u] + o8[u];
        v[u + 4] = v1[q][u] + o8[u + 4];
      }
      if (trw[q] < T) store8(xr[q] + c0, v);
    }
  };

  u32x4_t oa[NQ], ob[NQ];
  load_old(0, oa);
  for (int gi = 0; gi < ng; gi += 2) {
    load_old(gi + 1, ob);
    compute(gi, oa);
    load_old(gi + 2, oa);
    if (gi + 1 < ng) compute(gi + 1, ob);
  }
}

bool router_dx_applies(int d, int E) { return E % 8 == 0 && E <= 256 && d % 64 == 0; }

hipError_t launch_router_dx(const uint16_t* dl16, int ld, const uint16_t* Wr, int T, int d, int E,
                            uint16_t* dx, hipStream_t s) {
  if (T == 0) return hipSuccess;
  // Up to 128 experts (ld <= 128) a wave takes 64 tokens, so that each weight
  // fragment read from L2 feeds four MFMAs (the weights are read once per
  // 64 tokens instead of per 32); wider rows keep 32 tokens a wave (the
  // token operands' registers).  Column parts: about W waves in all (2048
  // for 64 tokens, 4096 for 32), 4 to d/64 parts (four a workgroup).
  const int nk = ld / 32;
  const int tw = nk <= 4 ? 64 : 32;
  const int tiles = (T + tw - 1) / tw;
  const long W = tw == 64 ? 2048 : 4096;
  int P = 4;
  while (2 * P <= d / 64 && (long)tiles * P < W) P *= 2;
  const dim3 grid(tiles, P / 4);
  note_prelaunch("router_dx", s);
  switch (nk) {
    case 2:
      hipLaunchKernelGGL((router_dx_kernel<2, 4>), grid, dim3(256), 0, s, dl16, ld, Wr, T, d, E, dx);
      break;
    case 4:
      hipLaunchKernelGGL((router_dx_kernel<4, 4>), grid, dim3(256), 0, s, dl16, ld, Wr, T, d, E, dx);
      break;
    case 6:
      hipLaunchKernelGGL((router_dx_kernel<6, 2>), grid, dim3(256), 0, s, dl16, ld, Wr, T, d, E, dx);
      break;
    case 8:
      hipLaunchKernelGGL((router_dx_kernel<8, 2>), grid, dim3(256), 0, s, dl16, ld, Wr, T, d, E, dx);
      break;
    default:
      return hipErrorInvalidValue;
  }
  note_launch("router_dx", s);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// router backward, weight gradient: part[s][c][e] = sum over the tokens of
// slice s of x[t][c] dl[t][e]  (the slices' partials are then added in order)
// ---------------------------------------------------------------------------
// Both operands run along the tokens (the contraction), so a workgroup (64
// x-columns x 64 experts, one token slice) stages 64-token chunks of both as
// token rows in LDS, in the engine's M/N-major layout (rows of 256 bytes with
// XOR-permuted 16-byte chunks), and reads the MFMA fragments with
// ds_read_b64_tr_b16; each wave owns a 32x32 block (32x32x16 bf16 MFMAs).
// The next chunk is loaded into registers while the current one multiplies.
constexpr int kRdwChunk = 64;

__global__ __launch_bounds__(256) void router_dwr_kernel(const uint16_t* __restrict__ x,
                                                         const uint16_t* __restrict__ dl16, int ld,
                                                         int T, int d, int E, int ts,
                                                         float* __restrict__ part) {
  __shared__ __attribute__((aligned(1024))) char smem[2][2][16384];  // [buffer][x | dl]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c0 = blockIdx.x * 64, e0 = blockIdx.z * 64, sl = blockIdx.y;
  const int t0 = sl * ts, t1 = min(T, t0 + ts);
  const int nch = t1 > t0 ? (t1 - t0 + kRdwChunk - 1) / kRdwChunk : 0;
  // fill units: operand o (x, dl), token row r of the chunk, 8-column group q
  int uo[4], ur[4], uq[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int u = tid + 256 * i;
    uo[i] = u >> 9;
    ur[i] = (u >> 3) & 63;
    uq[i] = u & 7;
  }
  u32x4_t v[4];
  auto load = [&](int ch) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + ch * kRdwChunk + ur[i];
      const long tc = min(t, T - 1);
      const u32x4_t a = uo[i] == 0
                            ? *reinterpret_cast<const u32x4_t*>(x + tc * d + c0 + 8 * uq[i])
                            : *reinterpret_cast<const u32x4_t*>(dl16 + tc * ld + e0 + 8 * uq[i]);
      v[i] = t < t1 ? a : u32x4_t{0, 0, 0, 0};
    }
  };
  auto store = [&](int b) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<u32x4_t*>(smem[b][uo[i]] + mf::mn_off(ur[i], 8 * uq[i])) = v[i];
  };
  const int cb = (wave >> 1) * 32, eb = (wave & 1) * 32;
  f32x16_t acc = {};
  if (nch > 0) {
    load(0);
    store(0);
    __syncthreads();
  }
  for (int ch = 0; ch < nch; ++ch) {
    const bool more = ch + 1 < nch;
    if (more) load(ch + 1);
    const char* const xs = smem[ch & 1][0];
    const char* const ds = smem[ch & 1][1];
#pragma unroll
    for (int s16 = 0; s16 < kRdwChunk / 16; ++s16) {
      const bf16x8_t fc = mf::frag<true>(xs, cb, s16, lane);
      const bf16x8_t fe = mf::frag<true>(ds, eb, s16, lane);
      // D[c][e]: this lane gets column c = cb + lane%32, experts eb + 8grp + 4(lane/32) + q
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fe, fc, acc, 0, 0, 0);
    }
    if (more) store((ch + 1) & 1);
    __syncthreads();
  }
  const int c = c0 + cb + (lane & 31);
  if (c < d) {
    float* const out = part + ((long)sl * d + c) * E;
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) {
      const int e = e0 + eb + 8 * grp + 4 * (lane >> 5);
      if (e < E)
        *reinterpret_cast<f32x4_t*>(out + e) =
            f32x4_t{acc[4 * grp], acc[4 * grp + 1], acc[4 * grp + 2], acc[4 * grp + 3]};
    }
  }
}

bool router_dwr_applies(int d, int E) { return E % 8 == 0 && E <= 256 && d % 64 == 0; }

int router_dwr_launch_slices(int T, int d, int E, int max_slices) {
  const int blocks = (d / 64) * ((E + 63) / 64);
  int S = (1024 + blocks - 1) / blocks;
  if (S > max_slices) S = max_slices;
  if (S > (T + kRdwChunk - 1) / kRdwChunk) S = (T + kRdwChunk - 1) / kRdwChunk;
  return S < 1 ? 1 : S;
}

hipError_t launch_router_dwr(const uint16_t* x, const uint16_t* dl16, int ld, int T, int d, int E,
                             int S, float* part, hipStream_t s) {
  const int ts = ((T + S - 1) / S + kRdwChunk - 1) / kRdwChunk * kRdwChunk;
  const dim3 grid(d / 64, S, (E + 63) / 64);
  note_prelaunch("router_dwr", s);
  hipLaunchKernelGGL(router_dwr_kernel, grid, dim3(256), 0, s, x, dl16, ld, T, d, E, ts, part);
  note_launch("router_dwr", s);
  return hipGetLastError();
}

}  // namespace moe
