#pragma once
// Greedy argmax over the output columns of a skinny matmul, without storing the outputs
// ("Qwen3.6-35B-A3B — TT-native mixed BFP4/BFP8", section "Fused decode kernels": the greedy
// token is picked from tiled LM-head logits, up to 16 rows, with no vocabulary-wide copy of them).
//
// A (value, column) pair is packed into one 64-bit key whose unsigned order is the order the
// argmax needs: larger value first, then smaller column. NaN sorts above every number (as in
// numpy's and torch's argmax, which return the first NaN) and -0 equals +0. Because the key
// order is total, the maximum over any grouping of the columns is the same key: the matmul
// workgroups each reduce their own columns to one candidate key per activation row, and
// argmax_rows_kernel reduces the candidates of a row.
#include "bfp_device.hpp"

namespace bfp {
namespace am {

__device__ __forceinline__ uint64_t key_of(float v, int col) {
  uint32_t u = __float_as_uint(v);
  if (v == 0.f) u = 0;                                 // -0 -> +0
  uint32_t k = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  if (v != v) k = 0xffffffffu;                         // NaN above +inf
  return ((uint64_t)k << 32) | (uint32_t)~(uint32_t)col;
}

// Key 0 is below every key_of: it fills slots without a column.
constexpr uint64_t kNone = 0;

// The value of a key; every NaN comes back as the quiet NaN 0x7fc00000.
__device__ __forceinline__ float value_of(uint64_t key) {
  const uint32_t k = (uint32_t)(key >> 32);
  if (k == 0xffffffffu) return __uint_as_float(0x7fc00000u);
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

__device__ __forceinline__ int column_of(uint64_t key) { return (int)~(uint32_t)key; }

__device__ __forceinline__ uint64_t kmax(uint64_t a, uint64_t b) { return a > b ? a : b; }

// Maximum over lanes with the same lane / W (W a power of two, W <= 64).
template <int W>
__device__ __forceinline__ uint64_t lane_max(uint64_t k) {
#pragma unroll
  for (int o = 1; o < W; o <<= 1) k = kmax(k, __shfl_xor(k, o, 64));
  return k;
}

constexpr int kRowThreads = 1024;
constexpr int kRowLoads = 8;          // independent loads in flight per thread

// One workgroup per activation row: idx[i], val[i] from the row's `count` keys
// (keys[i * count + j]), or, with FROM_VALUES, from the row's `count` fp32 values
// (values[i * ld + j], the column being j). Each thread issues kRowLoads clamped loads before
// it compares any of them.
template <bool FROM_VALUES>
__global__ __launch_bounds__(kRowThreads) void argmax_rows_kernel(const uint64_t* keys, const float* values,
                                                                  int64_t ld, int count, int32_t* idx,
                                                                  float* val) {
  __shared__ uint64_t part[kRowThreads / kWave];
  const int i = blockIdx.x;
  uint64_t best = kNone;
  for (int j0 = threadIdx.x; j0 < count; j0 += kRowThreads * kRowLoads) {
    uint64_t k[kRowLoads];
    float v[kRowLoads];
#pragma unroll
    for (int u = 0; u < kRowLoads; ++u) {
      const int j = min(j0 + u * kRowThreads, count - 1);
      if constexpr (FROM_VALUES) v[u] = values[(int64_t)i * ld + j];
      else k[u] = keys[(int64_t)i * count + j];
    }
#pragma unroll
    for (int u = 0; u < kRowLoads; ++u) {
      const int j = j0 + u * kRowThreads;
      const uint64_t kk = FROM_VALUES ? key_of(v[u], j) : k[u];
      best = kmax(best, j < count ? kk : kNone);
    }
  }
  best = lane_max<kWave>(best);
  if ((threadIdx.x & (kWave - 1)) == 0) part[threadIdx.x / kWave] = best;
  __syncthreads();
  if (threadIdx.x != 0) return;
#pragma unroll
  for (int w = 1; w < kRowThreads / kWave; ++w) best = kmax(best, part[w]);
  if (best == kNone) {                                 // no columns
    idx[i] = -1;
    val[i] = 0.f;
    return;
  }
  idx[i] = column_of(best);
  val[i] = value_of(best);
}

template <bool FROM_VALUES>
inline hipError_t launch_rows(const uint64_t* keys, const float* values, int64_t ld, int count, int m,
                              int32_t* idx, float* val, hipStream_t s) {
  if (m <= 0) return hipSuccess;
  hipLaunchKernelGGL((argmax_rows_kernel<FROM_VALUES>), dim3(m), dim3(kRowThreads), 0, s, keys, values, ld, count,
                     idx, val);
  return hipGetLastError();
}

}  // namespace am
}  // namespace bfp
