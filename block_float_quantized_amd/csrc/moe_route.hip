// MoE routing and dispatch for gfx950: router logits, top-k selection, counting sort.
//
// The layer ("qwen3.6-a3b-blackhole" bundle page, introduction; "Qwen3.6-35B-A3B — TT-native
// mixed BFP4/BFP8", sections "Precision as served" and "Fused decode kernels"): a BF16 router
// over 256 experts, device top-8 routing, a shared expert.
//
//  * Logits l_e = sum_k x_k * Wr[e][k] (+ b_e): bf16 x bf16 products are exact in fp64 and
//    summed in fp64, so the selection is decided on (almost) exact values. The shared-expert
//    gate x . g_s is computed as one more logit row.
//  * Selection: the top-k experts by (logit descending, expert ascending), in that order;
//    weights = softmax over the selection (identical to a softmax over all experts followed
//    by renormalisation over the selection); g = sigmoid(x . g_s).
//  * Dispatch: counts, exclusive offsets and the (token, slot) pairs sorted by (expert,
//    token): a stable counting sort whose within-expert ranks come from per-expert token
//    bitmaps and popcounts, so every integer result is deterministic.
#include "bfp_device.hpp"
#include "bfp_moe.hpp"

namespace bfp {

namespace {

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// One wave per (token, 4 experts). Expert index n_exp is the shared-expert gate row.
__global__ __launch_bounds__(256) void router_logits_kernel(RouteArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int t = blockIdx.y;
  const int e0 = (blockIdx.x * 4 + wave) * 4;
  const int rows = a.n_exp + (a.sh_gate_w ? 1 : 0);
  if (e0 >= rows) return;
  const uint16_t* xr = a.x + (int64_t)t * a.hidden;
  double acc[4] = {0.0, 0.0, 0.0, 0.0};
  const int chunks = a.hidden / 8;
  for (int c = lane; c < chunks; c += 64) {
    const uint4 xv = *reinterpret_cast<const uint4*>(xr + c * 8);
    const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = e0 + q;
      if (e >= rows) break;
      const uint16_t* wr = (e < a.n_exp) ? a.router_w + (int64_t)e * a.hidden : a.sh_gate_w;
      const uint4 wv = *reinterpret_cast<const uint4*>(wr + c * 8);
      const uint32_t ww[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[q] = __builtin_fma((double)bf16_lo(xw[i]), (double)bf16_lo(ww[i]), acc[q]);
        acc[q] = __builtin_fma((double)bf16_hi(xw[i]), (double)bf16_hi(ww[i]), acc[q]);
      }
    }
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = e0 + q;
    const double s = wave_sum_f64(acc[q]);
    if (lane == 0 && e < rows) {
      const double b = (e < a.n_exp && a.bias) ? (double)a.bias[e] : 0.0;
      a.logits[(int64_t)t * a.ld_logits + e] = s + b;
    }
  }
}

// One wave per token: top-k by (logit desc, expert asc), softmax weights, shared gate.
__global__ __launch_bounds__(256) void topk_kernel(RouteArgs a) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.m) return;
  const double* l = a.logits + (int64_t)t * a.ld_logits;
  constexpr int kPer = 4;                                   // n_exp <= 256
  double v[kPer];
  int ix[kPer];
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    ix[q] = lane + 64 * q;
    v[q] = ix[q] < a.n_exp ? l[ix[q]] : -__builtin_huge_val();
  }
  double sel_l[8];
  int sel_e[8];
  for (int j = 0; j < a.top_k; ++j) {
    // best candidate of this lane
    double bv = -__builtin_huge_val();
    int bi = 0x7fffffff;
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      if (ix[q] < a.n_exp && (v[q] > bv || (v[q] == bv && ix[q] < bi))) { bv = v[q]; bi = ix[q]; }
    }
    // wave argmax with the same order
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const double ov = __shfl_xor(bv, o);
      const int oi = __shfl_xor(bi, o);
      if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
    }
    sel_l[j] = bv;
    sel_e[j] = bi;
#pragma unroll
    for (int q = 0; q < kPer; ++q)
      if (ix[q] == bi) { v[q] = -__builtin_huge_val(); ix[q] = 0x7fffffff; }
  }
  if (lane == 0) {
    double z = 0.0;
    double ex[8];
    for (int j = 0; j < a.top_k; ++j) { ex[j] = exp(sel_l[j] - sel_l[0]); z += ex[j]; }
    for (int j = 0; j < a.top_k; ++j) {
      a.ids[(int64_t)t * a.top_k + j] = sel_e[j];
      a.w[(int64_t)t * a.top_k + j] = (float)(ex[j] / z);
    }
    if (a.g) {
      float gv = 1.0f;
      if (a.sh_gate_w) gv = (float)(1.0 / (1.0 + exp(-l[a.n_exp])));
      a.g[t] = gv;
    }
  }
}

// Counting sort of the (token, slot) pairs by expert; one workgroup of 1024 threads.
// Tokens are processed in chunks of 1024 with a per-expert token bitmap in LDS: the rank of
// a pair inside its expert is the number of earlier tokens in the bitmap row (prefix of
// popcounts) plus the pairs of earlier chunks.
constexpr int kDispThreads = 1024;
__global__ __launch_bounds__(kDispThreads) void dispatch_kernel(DispatchArgs a) {
  __shared__ uint32_t bitmap[256][33];                      // 32 words + pad per expert
  __shared__ int cnt[256];
  __shared__ int off[257];
  __shared__ int base[256];
  __shared__ int wpre[256][33];
  const int tid = threadIdx.x;
  const int E = a.n_exp, K = a.top_k;
  if (tid < 256) { cnt[tid] = 0; base[tid] = 0; }
  __syncthreads();
  const int np = a.m * K;
  for (int p = tid; p < np; p += kDispThreads) atomicAdd(&cnt[a.ids[p]], 1);
  __syncthreads();
  if (tid == 0) {
    int s = 0, na = 0;
    for (int e = 0; e < E; ++e) {
      off[e] = s;
      s += cnt[e];
      if (cnt[e] > 0 && a.active) a.active[na++] = e;
    }
    off[E] = s;
    if (a.n_active) *a.n_active = na;
    if (a.tile_m > 0) {
      // groups: the active experts in ascending order, then (optionally) the shared group
      int ts = 0, g = 0;
      for (int e = 0; e < E; ++e)
        if (cnt[e] > 0) { a.tile_start[g++] = ts; ts += (cnt[e] + a.tile_m - 1) / a.tile_m; }
      if (a.with_shared) { a.tile_start[g++] = ts; ts += (a.m + a.tile_m - 1) / a.tile_m; }
      a.tile_start[g] = ts;
    }
  }
  __syncthreads();
  if (tid < E) a.counts[tid] = cnt[tid];
  if (tid <= E) a.offsets[tid] = off[tid];
  for (int c0 = 0; c0 < a.m; c0 += kDispThreads) {
    for (int i = tid; i < 256 * 32; i += kDispThreads) bitmap[i / 32][i % 32] = 0;
    __syncthreads();
    const int t = c0 + tid;
    if (t < a.m)
      for (int j = 0; j < K; ++j) {
        const int e = a.ids[(int64_t)t * K + j];
        atomicOr(&bitmap[e][tid / 32], 1u << (tid % 32));
      }
    __syncthreads();
    if (tid < E) {
      int s = 0;
      for (int w = 0; w < 32; ++w) { wpre[tid][w] = s; s += __popc(bitmap[tid][w]); }
      wpre[tid][32] = s;
    }
    __syncthreads();
    if (t < a.m)
      for (int j = 0; j < K; ++j) {
        const int e = a.ids[(int64_t)t * K + j];
        const int w = tid / 32, b = tid % 32;
        const int rank = base[e] + wpre[e][w] + __popc(bitmap[e][w] & ((1u << b) - 1u));
        const int pos = off[e] + rank;
        a.perm[pos] = t * K + j;
        if (a.inv) a.inv[t * K + j] = pos;
      }
    __syncthreads();
    if (tid < E) base[tid] += wpre[tid][32];
    __syncthreads();
  }
}

}  // namespace

hipError_t router_launch(const RouteArgs& a, hipStream_t s) {
  const int rows = a.n_exp + (a.sh_gate_w ? 1 : 0);
  dim3 grid((rows + 15) / 16, a.m);
  hipLaunchKernelGGL(router_logits_kernel, grid, dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(topk_kernel, dim3((a.m + 3) / 4), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t dispatch_launch(const DispatchArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(dispatch_kernel, dim3(1), dim3(kDispThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace bfp
