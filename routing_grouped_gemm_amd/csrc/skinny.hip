// Expert GEMMs of the forward pass for small batches (a few rows per expert,
// as in token-by-token generation).
//
// With a handful of rows per expert the forward GEMMs stream the weights of
// the experts that received rows and do almost no arithmetic per weight
// byte, so the 256x256-tile engine (one workgroup per 256 output columns of
// an expert, 256 rows of which are mostly empty) leaves most CUs idle.  Here
// a workgroup owns one block of output columns of one expert and one slice of
// the contraction: 64 gate plus the same 64 up columns (gate/up GEMM), or 128
// output columns (down GEMM).  Its weight panels stream through a three-deep
// LDS ring by buffer->LDS DMA, 64 k-rows per stage, with the expert's rows
// (32 at a time) beside them; each of the four waves computes one 32x32
// block with MFMA 32x32x16 bf16, the weight fragments read transposed from
// the k-row-major panels by ds_read_b64_tr_b16.  Slices of the contraction
// (when the experts and column blocks alone would leave CUs idle) write
// float32 partial sums that a second kernel adds in slice order before the
// SwiGLU / bf16 store, so results do not depend on timing.
#include "gemm.h"
#include "gemm_dev.h"
#include "hook.h"
#include "moe_common.h"
#include "skinny.h"

namespace moe {
namespace sk {

using mf::barrier;
using mf::dma16;
using mf::i32x4_t;
using mf::km_off;
using mf::km_swz;
using mf::lds_u32;
using mf::make_rsrc;

constexpr int NTHR = 256;
constexpr int KB = 64;                  // k per stage
constexpr int ROWB = 128;               // bytes per LDS row (64 bf16)
constexpr int XT = 32 * ROWB;           // 32 activation rows (4 KiB)
constexpr int PB = KB * ROWB;           // one weight panel: 64 k-rows x 64 columns (8 KiB)
constexpr int SSTAGE = XT + 2 * PB;     // 20 KiB
constexpr int NBUF = 3;                 // LDS ring depth (60 KiB: two workgroups per CU)
constexpr int PRE = NBUF - 1;           // stages in flight ahead of the one consumed
constexpr int DMA_PER_STAGE = 5;        // per wave: 4 weight blocks + 1 activation block

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}
// Wait until at most n stages' loads (issued after the awaited one) remain.
__device__ __forceinline__ void wait_stages(int n) {
  switch (n) {
    case 0: wait_vm<0>(); break;
    case 1: wait_vm<DMA_PER_STAGE>(); break;
    case 2: wait_vm<2 * DMA_PER_STAGE>(); break;
    case 3: wait_vm<3 * DMA_PER_STAGE>(); break;
    default: wait_vm<4 * DMA_PER_STAGE>(); break;
  }
}
static_assert(PRE - 1 <= 4, "wait_stages covers up to four stages in flight");

// Weight fragment of MFMA B: 8 consecutive k (k16 step s, half lane>>5) of
// panel column colblk + (lane & 31), from a panel stored as 64 k-rows of 128
// bytes with 16-byte chunks at (chunk ^ km_swz(k)).  ds_read_b64_tr_b16
// transposes 4 k-rows x 16 columns within each 16-lane group.
__device__ __forceinline__ bf16x8_t wfrag(const char* panel, int colblk, int s, int lane) {
  typedef __attribute__((ext_vector_type(4))) short i16x4_t;
  typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
  typedef __attribute__((ext_vector_type(8))) short i16x8_t;
  const int g = lane >> 4, r = lane & 15;
  const int k = 16 * s + 8 * (g >> 1) + (r >> 2);
  const int col = colblk + 16 * (g & 1) + 4 * (r & 3);
  const char* p0 = panel + k * ROWB + (((col >> 3) ^ km_swz(k)) << 4) + 2 * (col & 7);
  const char* p1 = panel + (k + 4) * ROWB + (((col >> 3) ^ km_swz(k + 4)) << 4) + 2 * (col & 7);
  i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p0));
  i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p1));
  i16x8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8_t, v);
}

// Activation fragment of MFMA A: row lane & 31, 8 consecutive k.
__device__ __forceinline__ bf16x8_t xfrag(const char* xt, int s, int lane) {
  return *reinterpret_cast<const bf16x8_t*>(xt + km_off(lane & 31, 2 * s + (lane >> 5)));
}

// KIND 0: gate/up (panels: Wg and Wu columns n0..n0+63, outputs Hg, Hu, A or
// partials of [gate | up]); KIND 1: down (panels: Wd columns n0..n0+63 and
// n0+64..n0+127, output Ys or its partials).
template <int KIND>
__global__ __launch_bounds__(NTHR) void skinny_kernel(SkArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[NBUF * SSTAGE];
  const int cb = blockIdx.x, split = blockIdx.y, e = blockIdx.z;
  const int lo = a.offsets[e];
  const int ne = a.offsets[e + 1] - lo;
  if (ne <= 0) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const long n0 = (KIND == 0) ? 64L * cb : 128L * cb;
  const long long wbytes = (long long)a.K * a.ldw * 2;   // one expert's weight matrix
  const bf16_t* p0 = a.w0 + (long)e * a.w_es + n0;
  const bf16_t* p1 = (KIND == 0) ? a.w1 + (long)e * a.w_es + n0 : p0 + 64;
  const i32x4_t rw0 = make_rsrc(p0, wbytes - 2LL * n0);
  const i32x4_t rw1 = make_rsrc(p1, wbytes - 2LL * (KIND == 0 ? n0 : n0 + 64));
  const i32x4_t rx = make_rsrc(a.x, (long long)a.rows_total * a.ldx * 2);
  const uint32_t lds0 = lds_u32(smem);
  const int k0 = split * a.kc;
  const int nst = a.kc / KB;

  // this wave's weight DMA: panel wave>>1, k-rows 32*(wave&1) + 8i + lane/8
  const i32x4_t rwp = (wave >> 1) ? rw1 : rw0;
  uint32_t wv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 32 * (wave & 1) + 8 * i + (lane >> 3);
    wv[i] = (uint32_t)(row * a.ldw * 2 + (((lane & 7) ^ km_swz(row)) << 4));
  }
  const uint32_t w_lds = (uint32_t)(XT + (wave >> 1) * PB + 32 * (wave & 1) * ROWB);
  const int xrow = 8 * wave + (lane >> 3);  // activation row of this lane's DMA (0..31)

  for (int c0 = 0; c0 < ne; c0 += 32) {
    if (c0 > 0) wait_vm<0>();   // the previous chunk's stores, before the ring's counts
    const uint32_t xv = (uint32_t)(((long)lo + c0 + xrow) * a.ldx * 2 +
                                   (((lane & 7) ^ km_swz(xrow)) << 4));
    auto issue = [&](int t) {
      const uint32_t buf = lds0 + (t % NBUF) * SSTAGE;
      const uint32_t kw = (uint32_t)((long)(k0 + t * KB) * a.ldw * 2);
#pragma unroll
      for (int i = 0; i < 4; ++i) dma16(rwp, buf + w_lds + i * 8 * ROWB, wv[i], kw);
      dma16(rx, buf + 8 * wave * ROWB, xv, (uint32_t)((k0 + t * KB) * 2));
    };
    f32x16_t acc = f32x16_t{};
    for (int t = 0; t < PRE && t < nst; ++t) issue(t);
    for (int t = 0; t < nst; ++t) {
      // stages t+1 .. min(t+PRE-1, nst-1) may still be in flight
      wait_stages(min(PRE - 1, nst - 1 - t));
      barrier();
      if (t + PRE < nst) issue(t + PRE);   // into the buffer of stage t-1
      const char* buf = smem + (t % NBUF) * SSTAGE;
      const char* panel = buf + XT + (wave >> 1) * PB;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const bf16x8_t fb = wfrag(panel, 32 * (wave & 1), s, lane);
        const bf16x8_t fa = xfrag(buf, s, lane);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb, fa, acc, 0, 0, 0);
      }
    }
    // every wave is done with the ring: stage the 32 x 128 float results
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    barrier();
    float* st = reinterpret_cast<float*>(smem);   // [32][128]
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) {
      const int col = 32 * wave + 8 * grp + 4 * (lane >> 5);
      *reinterpret_cast<f32x4_t*>(st + (lane & 31) * 128 + col) =
          f32x4_t{acc[4 * grp], acc[4 * grp + 1], acc[4 * grp + 2], acc[4 * grp + 3]};
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    barrier();
    const int r = tid >> 3;            // row of the chunk
    const long grow = (long)lo + c0 + r;
    if (c0 + r < ne) {
      if constexpr (KIND == 0) {
        const int c = (tid & 7) * 8;   // gate/up column inside the block
        float g[8], u[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) { g[q] = st[r * 128 + c + q]; u[q] = st[r * 128 + 64 + c + q]; }
        const long n = n0 + c;
        if (a.S == 1) {
          float v[8];
#pragma unroll
          for (int q = 0; q < 8; ++q) v[q] = silu_f(g[q]) * u[q];
          store8(a.c0 + grow * a.ldc + n, g);
          store8(a.c1 + grow * a.ldc + n, u);
          store8(a.c2 + grow * a.ldc + n, v);
        } else {
          float* pp = a.part + ((long)split * a.rows_total + grow) * a.part_ld;
          store8(pp + n, g);
          store8(pp + a.N + n, u);
        }
      } else {
        const int c = (tid & 7) * 16;  // 16 output columns
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const long n = n0 + c + 8 * h;
          if (n < a.N) {
            float v[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) v[q] = st[r * 128 + c + 8 * h + q];
            if (a.S == 1)
              store8(a.c0 + grow * a.ldc + n, v);
            else
              store8(a.part + ((long)split * a.rows_total + grow) * a.part_ld + n, v);
          }
        }
      }
    }
    barrier();   // the staging area is the next chunk's ring
  }
}

// Sum of the S partials in slice order, then the gate/up epilogue (Hg, Hu,
// A = silu(Hg)*Hu from the float sums) or the down store (Ys).
template <int KIND>
__global__ __launch_bounds__(256) void skinny_reduce_kernel(SkArgs a) {
  const long cols8 = a.N / 8;
  const long total = (long)a.rows_total * cols8;
  for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (long)gridDim.x * blockDim.x) {
    const long r = i / cols8, n = (i - r * cols8) * 8;
    float g[8] = {}, u[8] = {};
#pragma unroll 8
    for (int s = 0; s < a.S; ++s) {
      const float* pp = a.part + ((long)s * a.rows_total + r) * a.part_ld;
      const float4 g0 = *reinterpret_cast<const float4*>(pp + n);
      const float4 g1 = *reinterpret_cast<const float4*>(pp + n + 4);
      g[0] += g0.x; g[1] += g0.y; g[2] += g0.z; g[3] += g0.w;
      g[4] += g1.x; g[5] += g1.y; g[6] += g1.z; g[7] += g1.w;
      if constexpr (KIND == 0) {
        const float4 u0 = *reinterpret_cast<const float4*>(pp + a.N + n);
        const float4 u1 = *reinterpret_cast<const float4*>(pp + a.N + n + 4);
        u[0] += u0.x; u[1] += u0.y; u[2] += u0.z; u[3] += u0.w;
        u[4] += u1.x; u[5] += u1.y; u[6] += u1.z; u[7] += u1.w;
      }
    }
    if constexpr (KIND == 0) {
      float v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] = silu_f(g[q]) * u[q];
      store8(a.c0 + r * a.ldc + n, g);
      store8(a.c1 + r * a.ldc + n, u);
      store8(a.c2 + r * a.ldc + n, v);
    } else {
      store8(a.c0 + r * a.ldc + n, g);
    }
  }
}

}  // namespace sk

int skinny_splits(int E, int R, int K, int ncb) {
  const long units = (long)(E < R ? E : R) * ncb;
  int S = 1;
  while (S < 8 && units * S < kSkinnyMinUnits && (K / sk::KB) % (2 * S) == 0) S *= 2;
  return S;
}

bool skinny_applies(int R, int E, int d, int f) {
  return R <= kSkinnyMaxRows && R <= 32 * E && (long long)R * (d > 2 * f ? d : 2 * f) * 2 < (1LL << 31) &&
         (long long)d * f * 2 < (1LL << 31);
}

size_t skinny_workspace(int R, int E, int d, int f) {
  if (!skinny_applies(R, E, d, f)) return 0;
  const int sg = skinny_splits(E, R, d, f / 64);
  const int sd = skinny_splits(E, R, f, (d + 127) / 128);
  const size_t g = sg > 1 ? (size_t)sg * R * 2 * f * sizeof(float) : 0;
  const size_t dn = sd > 1 ? (size_t)sd * R * d * sizeof(float) : 0;
  return g > dn ? g : dn;
}

hipError_t launch_skinny_ffn_fwd(const int* offsets, int E, int R, int d, int f,
                                 const bf16_t* Xs, const bf16_t* Wg, const bf16_t* Wu,
                                 const bf16_t* Wd, bf16_t* Hg, bf16_t* Hu, bf16_t* A, bf16_t* Ys,
                                 float* ws, hipStream_t st) {
  // gate/up: Xs[R,d] . [Wg|Wu][e][d,f]
  sk::SkArgs g{};
  g.offsets = offsets; g.E = E; g.x = Xs; g.ldx = d; g.rows_total = R;
  g.w0 = Wg; g.w1 = Wu; g.ldw = f; g.w_es = (long)d * f; g.K = d; g.N = f;
  g.S = skinny_splits(E, R, d, f / 64); g.kc = d / g.S;
  g.c0 = Hg; g.c1 = Hu; g.c2 = A; g.ldc = f;
  g.part = ws; g.part_ld = 2L * f;
  note_prelaunch("skinny_fwd_gateup", st);
  hipLaunchKernelGGL(sk::skinny_kernel<0>, dim3(f / 64, g.S, E), dim3(sk::NTHR), 0, st, g);
  note_launch("skinny_fwd_gateup", st);
  if (hipError_t err = hipGetLastError(); err != hipSuccess) return err;
  if (g.S > 1) {
    const long n = (long)R * (f / 8);
    const int blocks = (int)((n + 255) / 256 < 2048 ? (n + 255) / 256 : 2048);
    note_prelaunch("skinny_reduce_gateup", st);
    hipLaunchKernelGGL(sk::skinny_reduce_kernel<0>, dim3(blocks), dim3(256), 0, st, g);
    note_launch("skinny_reduce_gateup", st);
    if (hipError_t err = hipGetLastError(); err != hipSuccess) return err;
  }
  // down: A[R,f] . Wd[e][f,d]
  sk::SkArgs h{};
  h.offsets = offsets; h.E = E; h.x = A; h.ldx = f; h.rows_total = R;
  h.w0 = Wd; h.w1 = Wd; h.ldw = d; h.w_es = (long)f * d; h.K = f; h.N = d;
  h.S = skinny_splits(E, R, f, (d + 127) / 128); h.kc = f / h.S;
  h.c0 = Ys; h.ldc = d;
  h.part = ws; h.part_ld = d;
  note_prelaunch("skinny_fwd_down", st);
  hipLaunchKernelGGL(sk::skinny_kernel<1>, dim3((d + 127) / 128, h.S, E), dim3(sk::NTHR), 0, st,
                     h);
  note_launch("skinny_fwd_down", st);
  if (hipError_t err = hipGetLastError(); err != hipSuccess) return err;
  if (h.S > 1) {
    const long n = (long)R * (d / 8);
    const int blocks = (int)((n + 255) / 256 < 2048 ? (n + 255) / 256 : 2048);
    note_prelaunch("skinny_reduce_down", st);
    hipLaunchKernelGGL(sk::skinny_reduce_kernel<1>, dim3(blocks), dim3(256), 0, st, h);
    note_launch("skinny_reduce_down", st);
  }
  return hipGetLastError();
}

}  // namespace moe
