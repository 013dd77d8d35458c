// MXFP8 element codec shared by the quantising kernels (dispatch, combine
// backward, GEMM epilogues, weight quantizers).
//
// MXFP8 block quantisation (olmoforge README, MXFP8 snippet and module
// table: blocks of 32 values share one scale; e4m3 elements up to 448).
// Reading of the snippet: the block scale is 2^E with E the least integer such
// that 448 * 2^E >= max|block| (0 for an all-zero block, clamped to the E8M0
// range [-127, 127]); each element is rounded to the nearest OCP e4m3 value,
// ties to even, saturating at 448.  Scales are stored as E8M0 bytes, E + 127.
#pragma once

#include "moe_common.h"

namespace moe {

__device__ __forceinline__ int mx_block_exponent(float amax) {
  if (!(amax > 0.0f)) return 0;
  int ex;
  const float m = frexpf(amax, &ex);  // amax = m * 2^ex, m in [0.5, 1)
  const int top = ex - 1;             // amax in [2^top, 2^(top+1))
  // 448 * 2^(top-8) = 1.75 * 2^top >= amax iff 2m <= 1.75; else top-7 suffices
  const int E = (2.0f * m <= 1.75f) ? top - 8 : top - 7;
  return min(max(E, -127), 127);
}

// e4m3 codes of 8 values already divided by their block scale (|v| <= 448):
// v_cvt_pk_fp8_f32 rounds to the nearest OCP e4m3 value, ties to even, with
// e4m3 subnormals.  Checked on gfx950 against a plain encoder of the rule
// (sign | biased exponent | 3 mantissa bits, subnormal step 2^-9) for every
// finite bf16 value at block exponents -127 .. 127: identical bytes.
__device__ __forceinline__ void e4m3_codes8(const float (&v)[8], uint32_t (&codes)[2]) {
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    int lo = __builtin_amdgcn_cvt_pk_fp8_f32(v[4 * w], v[4 * w + 1], 0, false);
    codes[w] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v[4 * w + 2], v[4 * w + 3], lo, true);
  }
}

// 8 values of one lane; the 32-element block spans the 4 lanes 4g..4g+3.
// Returns the block exponent; codes[0..1] receive the 8 bytes.
__device__ __forceinline__ int quant8(const float (&v)[8], uint32_t (&codes)[2]) {
  float amax = 0.0f;
#pragma unroll
  for (int q = 0; q < 8; ++q) amax = fmaxf(amax, fabsf(v[q]));
  amax = quad_max(amax);
  const int E = mx_block_exponent(amax);
  float s[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) s[q] = ldexpf(v[q], -E);
  e4m3_codes8(s, codes);
  return E;
}

// Byte offset of the scale of column col's 32-element block in row row of an
// activation scale array: groups of four consecutive blocks, each group
// [rows][4] with pitch rows (the row count rounded up to 16).  A row's four
// scales of one 128-column group are one 4-byte word, a 128-column stage of
// 256 consecutive rows one contiguous kilobyte, and the four lanes that
// write a row's scales of one group hit the same word.
__device__ __forceinline__ long mx_scale_at(long row, int col, long pitch) {
  return (((long)(col >> 7) * pitch + row) << 2) + ((col >> 5) & 3);
}

// Block-quantise 8 values of each lane (already rounded to their stored
// precision) in 32-element blocks held by 4 consecutive lanes, and write the
// codes to q (8 bytes) and, from the first lane of the block, the biased
// exponent to *scale.  All 4 lanes of a block must be active together.
__device__ __forceinline__ void quant8_store(const float (&v)[8], uint8_t* q, uint8_t* scale,
                                             int lane) {
  uint32_t codes[2];
  const int E = quant8(v, codes);
  *reinterpret_cast<uint2*>(q) = make_uint2(codes[0], codes[1]);
  if ((lane & 3) == 0) *scale = (uint8_t)(E + 127);
}

// Values of 8 floats after rounding to bf16 (what a bf16 store keeps).
__device__ __forceinline__ void round_bf16_8(const float (&v)[8], float (&r)[8]) {
#pragma unroll
  for (int q = 0; q < 8; ++q) r[q] = bf16_to_f32(f32_to_bf16(v[q]));
}

}  // namespace moe
