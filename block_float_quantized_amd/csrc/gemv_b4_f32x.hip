// Instantiates the skinny BFP4 matmul kernels for fp32 activations.
#include "gemv_impl.hpp"

namespace bfp {

hipError_t gemv_launch_b4_f32x(const GemvParams& g, hipStream_t s) {
  gemv_detail::GemvArgs a{};
  a.exp0 = g.w_exp; a.code0 = g.w_code;
  a.exp1 = g.u_exp; a.code1 = g.u_code;
  a.x = g.x; a.ldx = g.ldx; a.y = g.y; a.ldy = g.ldy;
  a.n = (int)g.n; a.k = (int)g.k; a.m = (int)g.m;
  a.y_bf16 = g.y_bf16;
  a.kc = 0;
  if (g.u_code != nullptr) return gemv_detail::launch_gemv<4, 2, false>(a, s);
  return gemv_detail::launch_gemv<4, 1, false>(a, s);
}

}  // namespace bfp
