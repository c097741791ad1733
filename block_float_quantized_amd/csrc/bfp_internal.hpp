// Internal interface between the C ABI (api.cpp) and the kernel launchers (*.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace bfp {

// Encode fp32 [n][k] (row stride ldw) into exponent and code planes; `flag` is a device int
// set to 1 when a non-finite value is met (the caller clears it before and reads it after).
hipError_t quantize_launch(int fmt, const float* w, int64_t n, int64_t k, int64_t ldw, uint8_t* exp,
                           uint8_t* code, int* flag, hipStream_t s);

// Decode a whole matrix to fp32 or bf16 [n][k].
hipError_t dequant_launch(int fmt, const uint8_t* exp, const uint8_t* code, int64_t n, int64_t k,
                          int out_bf16, void* out, hipStream_t s);

struct GemvParams {
  int fmt;
  const uint8_t* w_exp;
  const uint8_t* w_code;
  const uint8_t* u_exp;        // SwiGLU up-projection, or null
  const uint8_t* u_code;
  int64_t n, k;
  const void* x;
  int64_t ldx;
  int x_bf16;
  int64_t m;
  void* y;
  int64_t ldy;
  int y_bf16;
  void* ws;                    // workspace of gemv_workspace_bytes bytes (or null when that is 0),
                               // gemv_argmax_workspace_bytes in argmax mode
  int32_t* am_idx;             // argmax mode (one matrix, bf16 x): per row of x, the column of the
  float* am_val;               // largest output and its value; y is not written. Else null.
  int invariant;               // one summation order for every m (the matrix-core kernel at m = 1 too)
};

// Workspace bytes gemv_launch needs for these shapes (0: none).
size_t gemv_workspace_bytes(int fmt, bool swiglu, int64_t n, int64_t k, int64_t m, bool invariant);

// Workspace bytes of argmax mode.
size_t gemv_argmax_workspace_bytes(int fmt, int64_t n, int64_t k, int64_t m, bool invariant);

// The vector kernel's workgroups own at least this many weight rows each (bounds the argmax
// candidates per row of x).
constexpr int kVectorMinRowsPerWg = 8;

hipError_t gemv_launch(const GemvParams& g, hipStream_t s);

}  // namespace bfp
