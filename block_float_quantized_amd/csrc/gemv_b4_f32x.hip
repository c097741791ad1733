// Instantiates the skinny BFP4 matmul kernels for fp32 activations.
#include "gemv_impl.hpp"
#include "gemv_row.hpp"

namespace bfp {

hipError_t gemv_launch_b4_f32x(const GemvParams& g, hipStream_t s) {
  const bool am = g.am_idx != nullptr;
  if (g.m == 1 && rowk::supported((int)g.n, (int)g.k, false, g.u_code != nullptr ? 2 : 1)) {
    // one activation row: the wave-per-row kernel
    rowk::RowArgs r{};
    r.exp[0] = g.w_exp; r.code[0] = g.w_code;
    r.exp[1] = g.u_exp; r.code[1] = g.u_code;
    r.x = g.x; r.y = g.y; r.y_bf16 = g.y_bf16;
    r.n = (int)g.n; r.k = (int)g.k;
    r.cand = am ? static_cast<uint64_t*>(g.ws) : nullptr;
    int grid = 0;
    const hipError_t e = rowk::launch<4, false>(r, g.u_code != nullptr ? 2 : 1, &grid, s);
    if (e != hipSuccess || !am) return e;
    return am::launch_rows<false>(r.cand, nullptr, 0, grid, 1, g.am_idx, g.am_val, s);
  }
  gemv_detail::GemvArgs a{};
  a.exp0 = g.w_exp; a.code0 = g.w_code;
  a.exp1 = g.u_exp; a.code1 = g.u_code;
  a.x = g.x; a.ldx = g.ldx; a.y = g.y; a.ldy = g.ldy;
  a.n = (int)g.n; a.k = (int)g.k; a.m = (int)g.m;
  a.y_bf16 = g.y_bf16;
  a.kc = 0;
  if (am) {
    a.cand = static_cast<uint64_t*>(g.ws);
    a.am_idx = g.am_idx;
    a.am_val = g.am_val;
  }
  if (g.u_code != nullptr) return gemv_detail::launch_gemv<4, 2, false>(a, s);
  return gemv_detail::launch_gemv<4, 1, false>(a, s);
}

}  // namespace bfp
