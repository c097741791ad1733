// Instantiates the skinny BFP4 matmul kernels for bf16 activations.
#include "gemv_impl.hpp"

namespace bfp {

hipError_t gemv_launch_b4_bf16x(const GemvParams& g, hipStream_t s) {
  gemv_detail::GemvArgs a{};
  a.exp0 = g.w_exp; a.code0 = g.w_code;
  a.exp1 = g.u_exp; a.code1 = g.u_code;
  a.x = g.x; a.ldx = g.ldx; a.y = g.y; a.ldy = g.ldy;
  a.n = (int)g.n; a.k = (int)g.k; a.m = (int)g.m;
  a.y_bf16 = g.y_bf16;
  a.kc = 0;
  if (g.am_idx != nullptr) {
    a.cand = static_cast<uint64_t*>(g.ws);
    a.am_idx = g.am_idx;
    a.am_val = g.am_val;
  }
  if (g.u_code != nullptr) return gemv_detail::launch_gemv<4, 2, true>(a, s);
  return gemv_detail::launch_gemv<4, 1, true>(a, s);
}

}  // namespace bfp
