// MXFP8 path of the expert layer: e4m3 elements with one E8M0 scale per 32
// elements along each GEMM's contraction axis.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

size_t mx_fwd_workspace(long long R, int d, int f, int E);
size_t mx_bwd_workspace(long long R, int d, int f, int E);

// Xs[r] = e4m3(x[src_token[r]] / 2^E_b), Xs_scale[r][b] = E_b + 127 per 32-block b along d.
hipError_t launch_mx_dispatch_copy(const void* x, const int32_t* src_token, int R, int T, int d,
                                   void* Xs, uint8_t* Xs_scale, hipStream_t s);
hipError_t mx_ffn_fwd(const void* Xq, const uint8_t* Xscale, const int32_t* offsets, int R, int d,
                      int f, int E, const void* Wg, const void* Wu, const void* Wd, void* Hg,
                      void* Hu, void* A, void* Ys, void* ws, int num_cu, hipStream_t s);
hipError_t mx_ffn_dgrad(const void* dYs, const void* Hg, const void* Hu, const int32_t* offsets,
                        int R, int d, int f, int E, const void* Wg, const void* Wu, const void* Wd,
                        void* dH, void* dXs, void* ws, int num_cu, hipStream_t s);

}  // namespace moe
