// MXFP8 path of the expert layer: e4m3 elements with one E8M0 scale per 32
// elements along each GEMM's contraction axis.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

size_t mx_fwd_workspace(long long R, int d, int f, int E);
size_t mx_bwd_workspace(long long R, int d, int f, int E);
// Backward workspace when the weight gradients are MXFP8 too (the dgrad
// workspace, then the token-quantised operands).
size_t mx_wgrad_workspace(long long R, int d, int f, int E);
// Row pitch of block-major activation scales: R rounded up to 16.
long mx_scale_pitch(long long R);

// Xs[r] = x[src_token[r]] (bf16); Xq[r] = its e4m3 codes along d and
// Xq_scale[b * pitch + r] = E_b + 127 for each 32-element block b.
hipError_t launch_mx_dispatch_copy(const void* x, const int32_t* src_token, int R, int T, int d,
                                   void* Xs, void* Xq, uint8_t* Xq_scale, hipStream_t s);
hipError_t mx_ffn_fwd(const void* Xq, const uint8_t* Xscale, const int32_t* offsets, int R, int d,
                      int f, int E, const void* Wg, const void* Wu, const void* Wd, void* Hg,
                      void* Hu, void* A, void* Ys, void* ws, int num_cu, hipStream_t s);
// dYsq / dYsq_scale: dYs quantised along d (as the combine backward writes it).
hipError_t mx_ffn_dgrad(const void* dYsq, const uint8_t* dYsq_scale, const void* Hg,
                        const void* Hu, const int32_t* offsets, int R, int d, int f, int E,
                        const void* Wg, const void* Wu, const void* Wd, void* dH, void* dXs,
                        void* ws, int num_cu, hipStream_t s);

// Weight gradients in MXFP8: Xs, dH, A, dYs (bf16) quantised along each
// expert's tokens; dW stored as bf16, or float32 with f32_out.
hipError_t mx_ffn_wgrad(const void* Xs, const void* dH, const void* A, const void* dYs,
                        const int32_t* offsets, int R, int d, int f, int E, int f32_out,
                        int accumulate, void* dWg, void* dWu, void* dWd, void* ws, int num_cu,
                        hipStream_t s);

}  // namespace moe
