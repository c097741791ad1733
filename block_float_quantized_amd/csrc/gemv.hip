// Skinny BFP4/BFP8 matmul dispatch: picks the instantiation for the format and activation
// type (the kernels themselves are in gemv_impl.hpp, compiled in four translation units).
#include "bfp_internal.hpp"

namespace bfp {

hipError_t gemv_launch_b4_bf16x(const GemvParams& g, hipStream_t s);
hipError_t gemv_launch_b4_f32x(const GemvParams& g, hipStream_t s);
hipError_t gemv_launch_b8_bf16x(const GemvParams& g, hipStream_t s);
hipError_t gemv_launch_b8_f32x(const GemvParams& g, hipStream_t s);

hipError_t gemv_launch(const GemvParams& g, hipStream_t s) {
  if (g.fmt == 4) return g.x_bf16 ? gemv_launch_b4_bf16x(g, s) : gemv_launch_b4_f32x(g, s);
  return g.x_bf16 ? gemv_launch_b8_bf16x(g, s) : gemv_launch_b8_f32x(g, s);
}

}  // namespace bfp
