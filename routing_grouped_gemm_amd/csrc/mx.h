// MXFP8 path of the expert layer: e4m3 elements with one E8M0 scale per 32
// elements along each GEMM's contraction axis.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// keep: room for the backward's weight codes after the forward's pieces.
size_t mx_fwd_workspace(long long R, int d, int f, int E, bool keep = false);
size_t mx_bwd_workspace(long long R, int d, int f, int E);
// Backward workspace when the weight gradients are MXFP8 too (the dgrad
// workspace, then the token-quantised operands).
size_t mx_wgrad_workspace(long long R, int d, int f, int E);
// Row pitch of the activation scales: R rounded up to 16.  Block b of row r
// sits at ((b / 4) * pitch + r) * 4 + b % 4, ceil(K / 128) * 4 * pitch bytes
// for rows of K elements.
long mx_scale_pitch(long long R);

// For every slot (t, j) with row r = dest_row[t, j] in [0, T*k): Xs[r] = x[t]
// (bf16); Xq[r] = its e4m3 codes along d and the scale of each 32-element
// block b, E_b + 127, at Xq_scale[((b / 4) * pitch + r) * 4 + b % 4] (pitch:
// T*k rounded up to 16).
hipError_t launch_mx_dispatch_copy(const void* x, const int32_t* dest_row, int T, int d, int k,
                                   void* Xs, void* Xq, uint8_t* Xq_scale, hipStream_t s);
// keep: every weight matrix is quantised in one pass for both directions, and
// the backward's codes stay in ws (mx_fwd_workspace(..., true) bytes).
hipError_t mx_ffn_fwd(const void* Xq, const uint8_t* Xscale, const int32_t* offsets, int R, int d,
                      int f, int E, const void* Wg, const void* Wu, const void* Wd, void* Hg,
                      void* Hu, void* A, void* Ys, void* ws, bool keep, int num_cu,
                      hipStream_t s);
// dYsq / dYsq_scale: dYs quantised along d (as the combine backward writes it).
// kept: the forward's workspace written with keep (its backward weight codes
// are read instead of quantising the weights again), or nullptr.
hipError_t mx_ffn_dgrad(const void* dYsq, const uint8_t* dYsq_scale, const void* Hg,
                        const void* Hu, const int32_t* offsets, int R, int d, int f, int E,
                        const void* Wg, const void* Wu, const void* Wd, void* dH, void* dXs,
                        void* ws, const void* kept, int num_cu, hipStream_t s);

// Weight gradients in MXFP8: Xs, dH, A, dYs (bf16) quantised along each
// expert's tokens; dW stored as bf16, or float32 with f32_out.
hipError_t mx_ffn_wgrad(const void* Xs, const void* dH, const void* A, const void* dYs,
                        const int32_t* offsets, int R, int d, int f, int E, int f32_out,
                        int accumulate, void* dWg, void* dWu, void* dWd, void* ws, int num_cu,
                        hipStream_t s);

}  // namespace moe
