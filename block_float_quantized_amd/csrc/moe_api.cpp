// C ABI of the MoE entry points (placeholder until the MoE kernels land).
#include <hip/hip_runtime.h>

#include "../../include/libbfp.h"

extern "C" {

int32_t bfp_moe_route(const bfp_moe_layer*, const uint16_t*, int64_t, int32_t*, float*, float*, void*) {
  return BFP_E_UNSUPPORTED;
}

int32_t bfp_moe_dispatch(const int32_t*, int64_t, int32_t, int32_t, int32_t*, int32_t*, int32_t*, void*) {
  return BFP_E_UNSUPPORTED;
}

size_t bfp_moe_workspace_bytes(const bfp_moe_layer*, int64_t) { return 0; }

int32_t bfp_moe_forward(const bfp_moe_layer*, const uint16_t*, int64_t, float*, int32_t*, float*, void*,
                        size_t, void*) {
  return BFP_E_UNSUPPORTED;
}

}  // extern "C"
