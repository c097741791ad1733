// Internal interface of the MoE prefill path (expert-grouped bf16 matrix-core GEMMs).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/libbfp.h"

namespace bfp {

struct PrefillArgs {
  const bfp_moe_layer* L;
  const uint16_t* x;          // bf16 [m][hidden]
  int m;
  float* y;                   // [m][hidden]
  const float* w;             // [m][top_k] routing weights
  const float* g;             // [m] shared gate, or null without a shared expert
  const int32_t* inv;         // [m*top_k] position of each pair in perm
  const int32_t* perm;        // [m*top_k] pairs sorted by (expert, token)
  const int32_t* offsets;     // [E+1]
  const int32_t* counts;      // [E]
  const int32_t* active;      // [E]
  const int32_t* n_active;    // [1]
  uint16_t* h;                // bf16 [m*top_k + m][inter]
  float* o;                   // fp32 [m*top_k + m][hidden]
  int32_t* extra;             // the region sized by prefill_workspace_extra_bytes: first the
                              // per-group row-tile starts the dispatch kernel writes (tile_m
                              // rows), then scratch of the prefill kernels
};

// Bytes of the region after the pair buffers: the dispatch kernel's row-tile starts, the row
// tiles sorted by size, and x permuted to the weight unpack's pair order; and the row-tile
// height the dispatch kernel must use.
size_t prefill_workspace_extra_bytes(int m, int n_exp, int top_k, int hidden);
int prefill_tile_rows();
// Whether the prefill kernels take this layer and token count (tile divisibility, 32-bit byte
// offsets); checked on the host before anything is launched.
bool prefill_supported(const bfp_moe_layer* L, int64_t m);
hipError_t prefill_launch(const PrefillArgs& p, hipStream_t s);

}  // namespace bfp
