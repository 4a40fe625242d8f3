// Launchers of the grouped FP8 GEMM and the combine (gemm.hip): the problem
// description every GEMM launch takes.  Kept apart from the other launchers
// so that the GEMM's sources are gemm.hip, common.h and this file alone.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsmoe {

enum class Epilogue : int {
  kStore = 0,      // c[r][n] = acc (bf16 or f32)
  kGateStore = 1,  // c[r][n] = acc * row_gate[r]
  kSwiGLUQuant = 2,// h = [gate | up] -> a = silu(gate) * up -> 1x128 FP8 codes + scales
};

struct GemmProblem {
  const uint8_t* a;          // [*][K] codes
  const float* a_scale;      // [*][K/128]
  const int32_t* a_rows;     // [M_total] or null
  const int32_t* offsets;    // [G+1] device
  int32_t G;
  int64_t M_total;           // upper bound on the rows the groups hold (grid sizing)
  const uint8_t* w;          // [G][N][K] codes (or G-1 matrices + w_last)
  const float* w_scale;      // [G][N/128][K/128]
  const uint8_t* w_last;     // when non-null: group G-1 uses these
  const float* w_scale_last;
  int64_t N, K;              // N = columns of W (for SwiGLU: 2I)
  void* c;                   // output
  bool c_f32;
  // epilogue extras
  Epilogue epi;
  const float* row_gate;     // kGateStore
  float* c_scale;            // kSwiGLUQuant: [M_total][N/2/128]
  int64_t row_limit;         // rows >= row_limit are never read or written
  int64_t rows_hint;         // typical rows per group (selects the kernel shape)
  int64_t a_rows_total;      // rows of A when known (every a_rows entry is below it), else 0
};

hipError_t launch_grouped_gemm(const GemmProblem& p, hipStream_t s);
// y[t] = o[shared0 + t] (if shared0 >= 0) + sum over k ascending of
// o[inv[t][k]]; o and y bf16 or f32 (f32), rows of H columns, H % 8 == 0.
hipError_t launch_combine(const void* o, const int32_t* inv, int64_t T, int32_t K, int64_t H,
                          int64_t shared0, void* y, bool f32, hipStream_t s);

}  // namespace dsmoe
