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

// Many-token routing (prefill) is certified rather than computed in fp64 for every expert:
//  1. approximate logits L~ = x . w_e on the bf16 matrix cores, fp32 accumulation. Every
//     product of two bf16 values is exact in fp32, so |L~ - L| <= gamma * sum_k |x_k w_k| with
//     gamma = n u / (1 - n u), n = hidden, u = 2^-23 (any summation order, any rounding that is
//     at least truncation), plus 2^-126 (|x|_1 + |w|_1) for products flushed as subnormals;
//     sum_k |x_k w_k| <= |x|_2 |w|_2 (Cauchy-Schwarz). This gives an interval per logit.
//  2. per token, L_k = the k-th largest lower end. An expert whose upper end is below L_k is
//     beaten by k experts and cannot be selected, so the top-k is among the candidates
//     {e : upper_e >= L_k}. Their logits are recomputed exactly (fp64 sums of exact
//     products) and the top-k, its order and its weights come from those exact values, as in
//     the decode path.

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
  // lane j < top_k: exp(l_j - l_0) in fp64; the sum is taken in rank order (a fixed order)
  double ex = 0.0;
  double lj = sel_l[0];
  int ej = sel_e[0];
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (j == lane && j < a.top_k) { lj = sel_l[j]; ej = sel_e[j]; }
  if (lane < a.top_k) ex = exp(lj - sel_l[0]);
  double z = 0.0;
  for (int j = 0; j < a.top_k; ++j) z += __shfl(ex, j);
  if (lane < a.top_k) {
    a.ids[(int64_t)t * a.top_k + lane] = ej;
    a.w[(int64_t)t * a.top_k + lane] = (float)(ex / z);
  }
  if (a.g && lane == 63) {
    float gv = 1.0f;
    if (a.sh_gate_w) gv = (float)(1.0 / (1.0 + exp(-l[a.n_exp])));
    a.g[t] = gv;
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
  __shared__ int wtot[4][3];
  const int tid = threadIdx.x;
  const int E = a.n_exp, K = a.top_k;
  if (tid < 256) { cnt[tid] = 0; base[tid] = 0; }
  __syncthreads();
  const int np = a.m * K;
  for (int p = tid; p < np; p += kDispThreads) atomicAdd(&cnt[a.ids[p]], 1);
  __syncthreads();
  // exclusive scans over the experts (threads 0..255, one value each): pair offsets, the
  // rank of each active expert, and the first row tile of each active expert's group
  {
    const int c = (tid < E) ? cnt[tid] : 0;
    const int act = c > 0 ? 1 : 0;
    const int tl = (a.tile_m > 0 && c > 0) ? (c + a.tile_m - 1) / a.tile_m : 0;
    int3 v = make_int3(c, act, tl);
    int3 inc = v;
    if (tid < 256) {
      const int lane = tid & 63;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int x0 = __shfl_up(inc.x, o), x1 = __shfl_up(inc.y, o), x2 = __shfl_up(inc.z, o);
        if (lane >= o) { inc.x += x0; inc.y += x1; inc.z += x2; }
      }
      if (lane == 63) { wtot[tid >> 6][0] = inc.x; wtot[tid >> 6][1] = inc.y; wtot[tid >> 6][2] = inc.z; }
    }
    __syncthreads();
    if (tid < 256) {
      int3 base3 = make_int3(0, 0, 0);
      for (int w = 0; w < (tid >> 6); ++w) { base3.x += wtot[w][0]; base3.y += wtot[w][1]; base3.z += wtot[w][2]; }
      const int ex_off = base3.x + inc.x - v.x;
      const int ex_act = base3.y + inc.y - v.y;
      const int ex_til = base3.z + inc.z - v.z;
      if (tid < E) {
        off[tid] = ex_off;
        if (act && a.active) a.active[ex_act] = tid;
        if (act && a.tile_m > 0) a.tile_start[ex_act] = ex_til;
      }
      if (tid == 255) {
        const int tot_pairs = base3.x + inc.x, na = base3.y + inc.y, tiles = base3.z + inc.z;
        off[E] = tot_pairs;
        if (a.n_active) *a.n_active = na;
        if (a.tile_m > 0) {
          int ts = tiles, g = na;
          if (a.with_shared) { a.tile_start[g++] = ts; ts += (a.m + a.tile_m - 1) / a.tile_m; }
          a.tile_start[g] = ts;
        }
      }
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
    {
      // 4 threads per expert, 8 bitmap words each; prefix over the 4 quarters by shuffles
      const int e = tid >> 2, q = tid & 3;
      int pc[8], sq = 0;
#pragma unroll
      for (int w = 0; w < 8; ++w) { pc[w] = (e < E) ? __popc(bitmap[e][q * 8 + w]) : 0; sq += pc[w]; }
      int incl = sq;
      const int u1 = __shfl_up(incl, 1, 4);
      if (q >= 1) incl += u1;
      const int u2 = __shfl_up(incl, 2, 4);
      if (q >= 2) incl += u2;
      int run = incl - sq;
      if (e < E) {
#pragma unroll
        for (int w = 0; w < 8; ++w) { wpre[e][q * 8 + w] = run; run += pc[w]; }
        if (q == 3) wpre[e][32] = run;
      }
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


// ---- many-token routing --------------------------------------------------------------------

constexpr int kRT = 64;           // tokens per router tile
constexpr int kRE = 64;           // logit rows (experts) per router tile
constexpr int kRK = 64;           // K per step
constexpr int kRLDK = kRK + 8;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

struct CertArgs {
  RouteArgs r;
  float* approx;      // [m][ld_approx]
  int ld_approx;
  double* norm_x;     // [m]
  double* norm_w;     // [n_exp + 1]
};

__device__ __forceinline__ const uint16_t* logit_row(const RouteArgs& a, int e) {
  if (e < a.n_exp) return a.router_w + (int64_t)e * a.hidden;
  if (e == a.n_exp) return a.sh_gate_w;       // may be null
  return nullptr;
}

// Row norms in fp64: rows [0, m) are tokens, [m, m + n_exp + 1) are logit rows.
__global__ __launch_bounds__(256) void row_norms_kernel(CertArgs c) {
  const RouteArgs& a = c.r;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.m + a.n_exp + 1) return;
  const uint16_t* p = row < a.m ? a.x + (int64_t)row * a.hidden : logit_row(a, row - a.m);
  double s = 0.0;
  if (p)
    for (int cidx = lane; cidx < a.hidden / 8; cidx += 64) {
      const uint4 v = *reinterpret_cast<const uint4*>(p + cidx * 8);
      const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const double lo = bf16_lo(w4[i]), hi = bf16_hi(w4[i]);
        s = __builtin_fma(lo, lo, s);
        s = __builtin_fma(hi, hi, s);
      }
    }
  s = wave_sum_f64(s);
  if (lane == 0) {
    // a slightly enlarged norm keeps the bound an upper bound despite fp64 rounding
    const double nrm = sqrt(s) * (1.0 + 1e-12);
    if (row < a.m) c.norm_x[row] = nrm; else c.norm_w[row - a.m] = nrm;
  }
}

// Approximate logits on the bf16 matrix cores: a 64-token x 64-row tile per workgroup.
__global__ __launch_bounds__(256) void router_mfma_kernel(CertArgs c) {
  const RouteArgs& a = c.r;
  __shared__ __align__(16) uint16_t As[kRT][kRLDK];
  __shared__ __align__(16) uint16_t Bs[kRE][kRLDK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * kRT, e0 = blockIdx.y * kRE;
  const int r = tid / 4, q = tid % 4;            // 64 rows x 4 quarters of 16 values
  const int tok = t0 + r;
  const uint16_t* arow = tok < a.m ? a.x + (int64_t)tok * a.hidden : nullptr;
  const uint16_t* brow = logit_row(a, e0 + r);
  f32x4 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  uint4 ra[2], rb[2];
  auto load = [&](int k0) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      ra[h] = arow ? *reinterpret_cast<const uint4*>(arow + k0 + q * 16 + h * 8) : make_uint4(0, 0, 0, 0);
      rb[h] = brow ? *reinterpret_cast<const uint4*>(brow + k0 + q * 16 + h * 8) : make_uint4(0, 0, 0, 0);
    }
  };
  load(0);
  for (int k0 = 0; k0 < a.hidden; k0 += kRK) {
    __syncthreads();
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      *reinterpret_cast<uint4*>(&As[r][q * 16 + h * 8]) = ra[h];
      *reinterpret_cast<uint4*>(&Bs[r][q * 16 + h * 8]) = rb[h];
    }
    __syncthreads();
    if (k0 + kRK < a.hidden) load(k0 + kRK);
#pragma unroll
    for (int ks = 0; ks < kRK / 32; ++ks) {
      const int kk = ks * 32 + 8 * (lane / 16);
      const bf16x8_t af = *reinterpret_cast<const bf16x8_t*>(&As[wave * 16 + (lane % 16)][kk]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bf16x8_t bf = *reinterpret_cast<const bf16x8_t*>(&Bs[j * 16 + (lane % 16)][kk]);
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf, acc[j], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int tt = t0 + wave * 16 + 4 * (lane / 16) + i;
    if (tt >= a.m) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = e0 + j * 16 + (lane % 16);
      if (e <= a.n_exp) c.approx[(int64_t)tt * c.ld_approx + e] = acc[j][i];
    }
  }
}

// exact fp64 logit of one row (wave-wide)
__device__ __forceinline__ double exact_logit(const uint16_t* x, const uint16_t* w, int hidden, int lane) {
  double s = 0.0;
  for (int cidx = lane; cidx < hidden / 8; cidx += 64) {
    const uint4 xv = *reinterpret_cast<const uint4*>(x + cidx * 8);
    const uint4 wv = *reinterpret_cast<const uint4*>(w + cidx * 8);
    const uint32_t xa[4] = {xv.x, xv.y, xv.z, xv.w}, wa[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s = __builtin_fma((double)bf16_lo(xa[i]), (double)bf16_lo(wa[i]), s);
      s = __builtin_fma((double)bf16_hi(xa[i]), (double)bf16_hi(wa[i]), s);
    }
  }
  return wave_sum_f64(s);
}

// One wave per token: certify the candidate set, recompute its logits exactly, select.
__global__ __launch_bounds__(256) void certify_topk_kernel(CertArgs c) {
  const RouteArgs& a = c.r;
  __shared__ int cand[4][256];
  __shared__ double cval[4][256];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wv;
  if (t >= a.m) return;
  const uint16_t* xr = a.x + (int64_t)t * a.hidden;
  const double n = (double)a.hidden;
  const double u = 1.0 / 8388608.0;                       // 2^-23
  const double gamma = n * u / (1.0 - n * u);
  const double tiny = 1.1754943508222875e-38;             // 2^-126
  const double nx = c.norm_x[t];
  double lo[4], hi[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = lane + 64 * q;
    if (e < a.n_exp) {
      const double nw = c.norm_w[e];
      const double d = gamma * nx * nw + tiny * sqrt(n) * (nx + nw) * 1.01;
      const double b = a.bias ? (double)a.bias[e] : 0.0;
      const double v = (double)c.approx[(int64_t)t * c.ld_approx + e] + b;
      lo[q] = v - d;
      hi[q] = v + d;
    } else {
      lo[q] = -__builtin_huge_val();
      hi[q] = -__builtin_huge_val();
    }
  }
  // k-th largest lower end
  double lk = __builtin_huge_val();
  {
    double v[4] = {lo[0], lo[1], lo[2], lo[3]};
    for (int j = 0; j < a.top_k; ++j) {
      double bv = -__builtin_huge_val();
      int bq = -1;
#pragma unroll
      for (int q = 0; q < 4; ++q) if (v[q] > bv) { bv = v[q]; bq = q; }
      double mv = bv;
      int ml = lane;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const double ov = __shfl_xor(mv, o);
        const int ol = __shfl_xor(ml, o);
        if (ov > mv || (ov == mv && ol < ml)) { mv = ov; ml = ol; }
      }
      lk = mv;
      if (lane == ml && bq >= 0) v[bq] = -__builtin_huge_val();
    }
  }
  // candidates, in expert order
  int nc = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const bool isc = (lane + 64 * q) < a.n_exp && hi[q] >= lk;
    const uint64_t bal = __ballot(isc);
    if (isc) {
      const int rank = nc + __popcll(bal & ((1ull << lane) - 1ull));
      cand[wv][rank] = lane + 64 * q;
    }
    nc += __popcll(bal);
  }
  __builtin_amdgcn_wave_barrier();
  // exact logits of the candidates
  for (int i = 0; i < nc; ++i) {
    const int e = cand[wv][i];
    const double s = exact_logit(xr, a.router_w + (int64_t)e * a.hidden, a.hidden, lane);
    if (lane == 0) cval[wv][i] = s + (a.bias ? (double)a.bias[e] : 0.0);
  }
  double glog = 0.0;
  if (a.sh_gate_w) glog = exact_logit(xr, a.sh_gate_w, a.hidden, lane);
  __builtin_amdgcn_wave_barrier();
  // top-k among the candidates by (exact logit desc, expert asc)
  double v[4];
  int ix[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int i = lane + 64 * q;
    ix[q] = i < nc ? cand[wv][i] : 0x7fffffff;
    v[q] = i < nc ? cval[wv][i] : -__builtin_huge_val();
  }
  double sel_l[8];
  int sel_e[8];
  for (int j = 0; j < a.top_k; ++j) {
    double bv = -__builtin_huge_val();
    int bi = 0x7fffffff;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (ix[q] != 0x7fffffff && (v[q] > bv || (v[q] == bv && ix[q] < bi))) { bv = v[q]; bi = ix[q]; }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const double ov = __shfl_xor(bv, o);
      const int oi = __shfl_xor(bi, o);
      if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
    }
    sel_l[j] = bv;
    sel_e[j] = bi;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (ix[q] == bi) { v[q] = -__builtin_huge_val(); ix[q] = 0x7fffffff; }
  }
  double ex = 0.0, lj = sel_l[0];
  int ej = sel_e[0];
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (j == lane && j < a.top_k) { lj = sel_l[j]; ej = sel_e[j]; }
  if (lane < a.top_k) ex = exp(lj - sel_l[0]);
  double z = 0.0;
  for (int j = 0; j < a.top_k; ++j) z += __shfl(ex, j);
  if (lane < a.top_k) {
    a.ids[(int64_t)t * a.top_k + lane] = ej;
    a.w[(int64_t)t * a.top_k + lane] = (float)(ex / z);
  }
  if (a.g && lane == 0) a.g[t] = a.sh_gate_w ? (float)(1.0 / (1.0 + exp(-glog))) : 1.0f;
}

}  // namespace

size_t route_workspace_bytes(int m, int n_exp) {
  const size_t fp64 = (size_t)m * (n_exp + 1) * sizeof(double);
  const int ld = (n_exp + 1 + kRE - 1) / kRE * kRE;
  const size_t cert = (size_t)m * ld * sizeof(float) + (size_t)m * sizeof(double) + (size_t)(n_exp + 1) * sizeof(double) + 64;
  return fp64 > cert ? fp64 : cert;
}

hipError_t router_launch(const RouteArgs& a, hipStream_t s) {
  if (a.m > 32) {
    // certified many-token routing; the logits region holds approx, then the two norm arrays
    CertArgs c;
    c.r = a;
    c.ld_approx = (a.n_exp + 1 + kRE - 1) / kRE * kRE;
    c.approx = reinterpret_cast<float*>(a.logits);
    char* base = reinterpret_cast<char*>(a.logits) + (size_t)a.m * c.ld_approx * sizeof(float);
    c.norm_x = reinterpret_cast<double*>(base);
    c.norm_w = c.norm_x + a.m;
    hipLaunchKernelGGL(row_norms_kernel, dim3((a.m + a.n_exp + 1 + 3) / 4), dim3(256), 0, s, c);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(router_mfma_kernel, dim3((a.m + kRT - 1) / kRT, (a.n_exp + 1 + kRE - 1) / kRE), dim3(256), 0,
                       s, c);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(certify_topk_kernel, dim3((a.m + 3) / 4), dim3(256), 0, s, c);
    return hipGetLastError();
  }
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
