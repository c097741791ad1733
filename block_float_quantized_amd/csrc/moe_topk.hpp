#pragma once
// Top-k routing of one token on one wave (gfx950), shared by the routing kernels and the
// one-token decode kernels.
//
// "Qwen3.6-35B-A3B — TT-native mixed BFP4/BFP8 (GPTQ experts)", sections "Precision as served"
// (BF16 router) and "Fused decode kernels" (device top-k routing): the experts are ranked by
// (logit descending, expert index ascending) and the first top_k taken, in that order.
#include "bfp_device.hpp"

namespace bfp {
namespace tk {

// Cross-lane moves without LDS: DPP inside each 16-lane row (partners l^1, l^2, the mirror
// inside the 8-lane half, l^8), then the four row results read back with v_readlane. Every
// lane ends with the same value, combined in a fixed order.
template <int CTRL>
__device__ __forceinline__ int dpp_i32(int v) { return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, true); }
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const long long b = __double_as_longlong(v);
  const int lo = dpp_i32<CTRL>((int)(b & 0xffffffffll)), hi = dpp_i32<CTRL>((int)(b >> 32));
  return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}
__device__ __forceinline__ double readlane_f64(double v, int l) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane((int)(b & 0xffffffffll), l), hi = __builtin_amdgcn_readlane((int)(b >> 32), l);
  return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}

// wave-wide maximum (fp64 max is exact, so the combination order does not matter)
__device__ __forceinline__ double wave_max_f64(double v) {
  v = fmax(v, dpp_f64<kDppQuadXor1>(v));
  v = fmax(v, dpp_f64<kDppQuadXor2>(v));
  v = fmax(v, dpp_f64<kDppHalfMirror>(v));
  v = fmax(v, dpp_f64<kDppRowRor8>(v));
  return fmax(fmax(readlane_f64(v, 0), readlane_f64(v, 16)), fmax(readlane_f64(v, 32), readlane_f64(v, 48)));
}

__device__ __forceinline__ double wave_sum_f64(double v) {
  v += dpp_f64<kDppQuadXor1>(v);
  v += dpp_f64<kDppQuadXor2>(v);
  v += dpp_f64<kDppHalfMirror>(v);
  v += dpp_f64<kDppRowRor8>(v);
  return (readlane_f64(v, 0) + readlane_f64(v, 16)) + (readlane_f64(v, 32) + readlane_f64(v, 48));
}

// The top_k experts of one token (logits l[0..n_exp), fp64) by (logit descending, expert
// ascending), computed by one wave: sel_e / sel_l in rank order, the same in every lane.
// n_exp <= 256, top_k <= 8.
__device__ __forceinline__ void topk_select(const double* l, int n_exp, int top_k, int lane, double (&sel_l)[8],
                                            int (&sel_e)[8]) {
  constexpr int kPer = 4;                                   // n_exp <= 256
  double v[kPer];
  int ix[kPer];
  bool live[kPer];                                          // not selected yet
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    ix[q] = lane + 64 * q;
    live[q] = ix[q] < n_exp;
    const double lv = live[q] ? l[ix[q]] : -__builtin_huge_val();
    v[q] = lv != lv ? -__builtin_huge_val() : lv;         // a NaN logit ranks below every number
  }
  for (int j = 0; j < top_k; ++j) {
    // the largest remaining logit M (a max-reduction: exact, order-free), then the smallest
    // unselected expert index holding it: expert 64 q + lane, so the first q with a match, then
    // its lowest lane (equality ballots, no divergent branch). M is never NaN and at least
    // n_exp - j >= 1 experts are live, so a match always exists: the ids are distinct and in
    // range whatever the logits hold.
    const double M = wave_max_f64(fmax(fmax(v[0], v[1]), fmax(v[2], v[3])));
    int bi = -1;
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const uint64_t b = __ballot(live[q] && v[q] == M);
      if (bi < 0 && b != 0) bi = 64 * q + __builtin_ctzll(b);
    }
    sel_l[j] = M;
    sel_e[j] = bi;
#pragma unroll
    for (int q = 0; q < kPer; ++q)
      if (ix[q] == bi) { v[q] = -__builtin_huge_val(); live[q] = false; }
  }
}

// The outputs of one token's routing, from its selection: lanes j < top_k write ids[j] (and
// eid[j] when given) and the weight w[j] = exp(l_j - l_0) / z, z the sum of the numerators in
// rank order (a softmax over the selection, fp64, then rounded to fp32); when g is given, lane
// 63 writes the shared-expert gate sigmoid(l[n_exp]) (1 without a gate row).
__device__ __forceinline__ void topk_store(const double* l, int n_exp, int top_k, bool gate_row, int lane,
                                           const double (&sel_l)[8], const int (&sel_e)[8], int32_t* ids,
                                           float* w, float* g, uint8_t* eid) {
  double ex = 0.0;
  double lj = sel_l[0];
  int ej = sel_e[0];
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (j == lane && j < top_k) { lj = sel_l[j]; ej = sel_e[j]; }
  if (lane < top_k) ex = exp(lj - sel_l[0]);
  double z = 0.0;
  for (int j = 0; j < top_k; ++j) z += __shfl(ex, j);
  if (lane < top_k) {
    ids[lane] = ej;
    w[lane] = (float)(ex / z);
    if (eid) eid[lane] = (uint8_t)ej;
  }
  if (g && lane == 63) {
    float gv = 1.0f;
    if (gate_row) gv = (float)(1.0 / (1.0 + exp(-l[n_exp])));
    *g = gv;
  }
}

}  // namespace tk
}  // namespace bfp
