// Device-side helpers shared by the HIP kernels of the MoE expert layer
// (gfx950, wave64).  Storage types: float, or bf16 held as raw uint16_t.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef uint16_t bf16_t;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(8))) int i32x8_t;

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

// float32 -> bf16, round to nearest, ties to even (gfx950's v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16_t f32_to_bf16(float v) {
  return __builtin_bit_cast(bf16_t, static_cast<__bf16>(v));
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

// Storage-type adaptors.
template <typename T> struct St;
template <> struct St<float> {
  __device__ __forceinline__ static float load(const float* p) { return *p; }
  __device__ __forceinline__ static void store(float* p, float v) { *p = v; }
  __device__ __forceinline__ static float to_f(float v) { return v; }
  __device__ __forceinline__ static float from_f(float v) { return v; }
};
template <> struct St<bf16_t> {
  __device__ __forceinline__ static float load(const bf16_t* p) { return bf16_to_f32(*p); }
  __device__ __forceinline__ static void store(bf16_t* p, float v) { *p = f32_to_bf16(v); }
  __device__ __forceinline__ static float to_f(bf16_t v) { return bf16_to_f32(v); }
  __device__ __forceinline__ static bf16_t from_f(float v) { return f32_to_bf16(v); }
};

// 8 consecutive elements as floats from a 16-byte (bf16) or 2x16-byte (fp32) load.
__device__ __forceinline__ void load8(const bf16_t* p, float (&v)[8]) {
  uint4 u = *reinterpret_cast<const uint4*>(p);
  uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void unpack8(const uint4 u, float (&v)[8]) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void load8(const float* p, float (&v)[8]) {
  float4 a = *reinterpret_cast<const float4*>(p);
  float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void store8(bf16_t* p, const float (&v)[8]) {
  uint4 u;
  u.x = pack_bf16x2(v[0], v[1]);
  u.y = pack_bf16x2(v[2], v[3]);
  u.z = pack_bf16x2(v[4], v[5]);
  u.w = pack_bf16x2(v[6], v[7]);
  *reinterpret_cast<uint4*>(p) = u;
}
// Streaming (non-temporal) 16-byte stores of 8 values, for the GEMM
// epilogues: measured ~1% faster there than plain stores.
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;
__device__ __forceinline__ void store8_nt(bf16_t* p, const float (&v)[8]) {
  const u32x4_t w = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                     pack_bf16x2(v[6], v[7])};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x4_t*>(p));
}
__device__ __forceinline__ void store8_nt(float* p, const float (&v)[8]) {
  const f32x4_t a = {v[0], v[1], v[2], v[3]}, b = {v[4], v[5], v[6], v[7]};
  __builtin_nontemporal_store(a, reinterpret_cast<f32x4_t*>(p));
  __builtin_nontemporal_store(b, reinterpret_cast<f32x4_t*>(p + 4));
}
__device__ __forceinline__ void store8(float* p, const float (&v)[8]) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}

// Logistic sigmoid and SiLU with the hardware reciprocal (1 ulp) in place of
// an IEEE division: the results are rounded to bf16 or feed bf16 GEMMs.
__device__ __forceinline__ float sigmoid_f(float z) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}
__device__ __forceinline__ float silu_f(float z) { return z * sigmoid_f(z); }

// Cross-lane moves by DPP (gfx9 controls).  A lane that the row mask leaves
// unwritten receives `old`.  Shuffles by ds_bpermute go through LDS and cost
// an LDS round trip each; these stay in the VALU.
constexpr int kDppQuad1032 = 0xB1;     // quad_perm [1,0,3,2]: lane ^ 1
constexpr int kDppQuad2301 = 0x4E;     // quad_perm [2,3,0,1]: lane ^ 2
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;
constexpr int kDppRowBcast15 = 0x142;  // lane 15 of a row to the next row
constexpr int kDppRowBcast31 = 0x143;  // lane 31 to rows 2 and 3

template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ float dpp_f(float old, float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old),
                                                               __builtin_bit_cast(int, v), CTRL,
                                                               ROWS, 0xF, false));
}
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ int dpp_i(int old, int v) {
  return __builtin_amdgcn_update_dpp(old, v, CTRL, ROWS, 0xF, false);
}
__device__ __forceinline__ float lane63_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// Sum over the wave, returned to every lane: pairs, quads, half-rows, rows,
// then rows 0+1 and 0+1+2+3 (fixed order).
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<kDppQuad1032>(0.0f, v);
  v += dpp_f<kDppQuad2301>(0.0f, v);
  v += dpp_f<kDppRowHalfMirror>(0.0f, v);
  v += dpp_f<kDppRowMirror>(0.0f, v);
  v += dpp_f<kDppRowBcast15, 0xA>(0.0f, v);
  v += dpp_f<kDppRowBcast31, 0xC>(0.0f, v);
  return lane63_f(v);
}

// Maximum over the wave, returned to every lane.
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<kDppQuad1032>(v, v));
  v = fmaxf(v, dpp_f<kDppQuad2301>(v, v));
  v = fmaxf(v, dpp_f<kDppRowHalfMirror>(v, v));
  v = fmaxf(v, dpp_f<kDppRowMirror>(v, v));
  v = fmaxf(v, dpp_f<kDppRowBcast15, 0xA>(v, v));
  v = fmaxf(v, dpp_f<kDppRowBcast31, 0xC>(v, v));
  return lane63_f(v);
}

// Maximum over the 4 lanes of each quad (lane ^ 1, lane ^ 2).
__device__ __forceinline__ float quad_max(float v) {
  v = fmaxf(v, dpp_f<kDppQuad1032>(v, v));
  return fmaxf(v, dpp_f<kDppQuad2301>(v, v));
}

}  // namespace moe
