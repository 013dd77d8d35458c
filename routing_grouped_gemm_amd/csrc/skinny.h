// Forward expert GEMMs for small batches (few rows per expert): host side.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe_common.h"

namespace moe {

// The small-batch engine takes a bf16 forward with at most this many routed
// rows and on average at most 32 rows per expert.
constexpr int kSkinnyMaxRows = 2048;
// The contraction is sliced (float partials, one more kernel) only while the
// experts that can hold rows times the column blocks stay below this many
// workgroups.
constexpr int kSkinnyMinUnits = 512;

namespace sk {
struct SkArgs {
  const int* offsets;      // [E+1] row offsets of the experts
  int E;
  const bf16_t* x;         // rows [rows_total][ldx], K contiguous (Xs or A)
  long ldx;
  long rows_total;         // R
  const bf16_t* w0;        // weight panels: gate/up: Wg, Wu; down: Wd (both)
  const bf16_t* w1;
  long ldw;                // elements per k-row of a weight matrix (its N)
  long w_es;               // elements between experts
  int K, N;                // contraction length, output columns (f or d)
  int S, kc;               // contraction slices and k per slice (multiple of 64)
  bf16_t* c0;              // gate/up: Hg, Hu, A; down: Ys (c0)
  bf16_t* c1;
  bf16_t* c2;
  long ldc;
  float* part;             // S > 1: float partials [S][rows_total][part_ld]
  long part_ld;
};
}  // namespace sk

bool skinny_applies(int R, int E, int d, int f);
int skinny_splits(int E, int R, int K, int ncb);
size_t skinny_workspace(int R, int E, int d, int f);
hipError_t launch_skinny_ffn_fwd(const int* offsets, int E, int R, int d, int f,
                                 const bf16_t* Xs, const bf16_t* Wg, const bf16_t* Wu,
                                 const bf16_t* Wd, bf16_t* Hg, bf16_t* Hu, bf16_t* A, bf16_t* Ys,
                                 float* ws, hipStream_t st);

}  // namespace moe
