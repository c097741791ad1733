#pragma once
// Top-k routing of one token on one wave (gfx950), shared by the routing kernels and the
// per-token decode kernels.
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

// Wave-wide maximum of an unsigned 32-bit value, in every lane: DPP inside each 16-lane row,
// then v_permlane16_swap and v_permlane32_swap across rows (no scalar round trip).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)dpp_i32<kDppQuadXor1>((int)v));
  v = max(v, (uint32_t)dpp_i32<kDppQuadXor2>((int)v));
  v = max(v, (uint32_t)dpp_i32<kDppHalfMirror>((int)v));
  v = max(v, (uint32_t)dpp_i32<kDppRowRor8>((int)v));
  const auto r16 = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = max((uint32_t)r16[0], (uint32_t)r16[1]);
  const auto r32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return max((uint32_t)r32[0], (uint32_t)r32[1]);
}

// A 64-bit key whose unsigned order is the numeric order of fp64 logits: NaN is taken as -inf
// (it ranks below every number) and -0 as +0 (equal values tie). Every logit's key is at least
// key(-inf) > 0, so 0 marks an empty slot.
__device__ __forceinline__ uint64_t order_key(double v) {
  if (v != v) v = -__builtin_huge_val();
  if (v == 0.0) v = 0.0;
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  return (b >> 63) ? ~b : (b | (1ull << 63));
}
__device__ __forceinline__ double key_value(uint64_t k) {
  return __longlong_as_double((long long)((k >> 63) ? (k & ~(1ull << 63)) : ~k));
}

// The top_k experts of one token (logits l[0..n_exp), fp64) by (logit descending, expert
// ascending), computed by one wave: sel_e / sel_l in rank order, the same in every lane.
// n_exp <= 256, top_k <= 8.
//
// Lane p holds experts 4p .. 4p+3 as keys, sorted (key descending, expert ascending); each
// round takes the largest head key over the wave (high words, then the low words of the lanes
// that tie on them) and the lowest lane holding it, which holds the lowest such expert, and
// that lane drops its head. The keys are distinct per (value, expert) order, so the result is
// the plain sort's; at least n_exp - j >= 1 live keys remain in round j, so the ids are
// distinct and in range whatever the logits hold.
__device__ __forceinline__ void topk_select(const double* l, int n_exp, int top_k, int lane, double (&sel_l)[8],
                                            int (&sel_e)[8]) {
  uint64_t k[4];
  int ix[4];
  double lv[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {                      // every load issued before any use
    ix[q] = 4 * lane + q;
    lv[q] = l[min(ix[q], n_exp - 1)];
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) k[q] = order_key(lv[q]) & (ix[q] < n_exp ? ~0ull : 0ull);
  // sorting network on (key descending, expert ascending)
  auto cx = [&](int a, int b) {
    const bool swap = k[b] > k[a] || (k[b] == k[a] && ix[b] < ix[a]);
    const uint64_t ka = k[a];
    const int ia = ix[a];
    k[a] = swap ? k[b] : k[a];
    ix[a] = swap ? ix[b] : ix[a];
    k[b] = swap ? ka : k[b];
    ix[b] = swap ? ia : ix[b];
  };
  cx(0, 1); cx(2, 3); cx(0, 2); cx(1, 3); cx(1, 2);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j >= top_k) break;
    const uint32_t hh = (uint32_t)(k[0] >> 32), hl = (uint32_t)k[0];
    const uint32_t mh = wave_max_u32(hh);
    uint64_t b = __ballot(hh == mh);
    uint32_t ml;
    if (__popcll(b) > 1) {
      ml = wave_max_u32(hh == mh ? hl : 0u);
      b = __ballot(hh == mh && hl == ml);
    } else {
      ml = (uint32_t)__builtin_amdgcn_readlane((int)hl, __builtin_ctzll(b));
    }
    const int wl = __builtin_ctzll(b);
    sel_l[j] = key_value(((uint64_t)mh << 32) | ml);
    sel_e[j] = __builtin_amdgcn_readlane(ix[0], wl);
    if (lane == wl) {
      k[0] = k[1]; ix[0] = ix[1];
      k[1] = k[2]; ix[1] = ix[2];
      k[2] = k[3]; ix[2] = ix[3];
      k[3] = 0ull;
    }
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
