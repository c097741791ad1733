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
#include "moe_topk.hpp"

// Many-token routing (prefill) is certified rather than computed in fp64 for every expert:
//  1. approximate logits L~ = x . w_e on the bf16 matrix cores, fp32 accumulation over up
//     to four K slices whose partial sums are added in fp64 (a summation order like any other
//     for the bound below, plus the rounding of that fp64 addition). Every
//     product of two bf16 values is exact in fp32, so |L~ - L| <= gamma * sum_k |x_k w_k| with
//     gamma = n u / (1 - n u), n = hidden, u = 2^-23 (any summation order, any rounding that is
//     at least truncation), plus 2^-126 (|x|_1 + |w|_1) for subnormal bf16 inputs flushed to
//     zero and n 2^-126 for products of normal inputs that underflow and are flushed;
//     sum_k |x_k w_k| <= |x|_2 |w|_2 (Cauchy-Schwarz). This gives an interval per logit.
//  2. per token, L_k = the k-th largest lower end. An expert whose upper end is below L_k is
//     beaten by k experts and cannot be selected, so the top-k is among the candidates
//     {e : upper_e >= L_k}. Their logits are recomputed exactly (fp64 sums of exact
//     products) and the top-k, its order and its weights come from those exact values, as in
//     the decode path.

namespace bfp {

namespace {

using tk::readlane_f64;
using tk::wave_max_f64;
using tk::wave_sum_f64;

// One wave per (token, R experts). Expert index n_exp is the shared-expert gate row. Each
// logit is the same sum (chunk order, then the wave reduction) whatever R is.
template <int R>
__global__ __launch_bounds__(256) void router_logits_kernel(RouteArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int t = blockIdx.y;
  const int e0 = (blockIdx.x * 4 + wave) * R;
  const int rows = a.n_exp + (a.sh_gate_w ? 1 : 0);
  if (e0 >= rows) return;
  const uint16_t* xr = a.x + (int64_t)t * a.hidden;
  double acc[R];
#pragma unroll
  for (int q = 0; q < R; ++q) acc[q] = 0.0;
  const int chunks = a.hidden / 8;
  const uint16_t* wr[R];
#pragma unroll
  for (int q = 0; q < R; ++q) {
    const int e = min(e0 + q, rows - 1);       // rows past the end re-read the last one, unused
    wr[q] = (e < a.n_exp) ? a.router_w + (int64_t)e * a.hidden : a.sh_gate_w;
  }
  // kU chunks per lane in flight: every load of a batch is issued (clamped to the row, no
  // branch) before any product; the sums keep the chunk order
  constexpr int kU = 4;
  for (int c0 = lane; c0 < chunks; c0 += 64 * kU) {
    uint4 xv[kU], wv[kU][R];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int c = min(c0 + 64 * u, chunks - 1);
      xv[u] = *reinterpret_cast<const uint4*>(xr + c * 8);
#pragma unroll
      for (int q = 0; q < R; ++q) wv[u][q] = *reinterpret_cast<const uint4*>(wr[q] + c * 8);
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (c0 + 64 * u >= chunks) break;
      const uint32_t xw[4] = {xv[u].x, xv[u].y, xv[u].z, xv[u].w};
#pragma unroll
      for (int q = 0; q < R; ++q) {
        const uint32_t ww[4] = {wv[u][q].x, wv[u][q].y, wv[u][q].z, wv[u][q].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[q] = __builtin_fma((double)bf16_lo(xw[i]), (double)bf16_lo(ww[i]), acc[q]);
          acc[q] = __builtin_fma((double)bf16_hi(xw[i]), (double)bf16_hi(ww[i]), acc[q]);
        }
      }
    }
  }
#pragma unroll
  for (int q = 0; q < R; ++q) {
    const int e = e0 + q;
    const double s = wave_sum_f64(acc[q]);
    if (lane == 0 && e < rows) {
      const double b = (e < a.n_exp && a.bias) ? (double)a.bias[e] : 0.0;
      a.logits[(int64_t)t * a.ld_logits + e] = s + b;
    }
  }
}

// One wave, token t: top-k by (logit desc, expert asc), softmax weights, shared gate. With
// eid, the selected experts also go to eid[t * top_k + j] (LDS bytes).
__device__ __forceinline__ void topk_token(const RouteArgs& a, int t, int lane, uint8_t* eid) {
  const double* l = a.logits + (int64_t)t * a.ld_logits;
  double sel_l[8];
  int sel_e[8];
  tk::topk_select(l, a.n_exp, a.top_k, lane, sel_l, sel_e);
  tk::topk_store(l, a.n_exp, a.top_k, a.sh_gate_w != nullptr, lane, sel_l, sel_e, a.ids + (int64_t)t * a.top_k,
                 a.w + (int64_t)t * a.top_k, a.g ? a.g + t : nullptr, eid ? eid + t * a.top_k : nullptr);
}

// One wave per token.
__global__ __launch_bounds__(256) void topk_kernel(RouteArgs a) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.m) return;
  topk_token(a, t, threadIdx.x & 63, nullptr);
}

// Counting sort of the (token, slot) pairs by expert; one workgroup of 1024 threads. The
// expert ids are read from global memory once (16-byte loads, several in flight per thread)
// into LDS as bytes; counts, scans, ranks and the stores then work from LDS. Tokens are ranked
// in chunks of 1024 with a per-expert token bitmap: the rank of a pair inside its expert is
// the number of earlier tokens in the bitmap row (prefix of popcounts) plus the pairs of
// earlier chunks.
constexpr int kDispThreads = 1024;
constexpr int kDispMaxPairs = 8192 * 8;          // most tokens x top_k the kernel takes

// Exclusive scans over the experts of a workgroup's counts cnt[0..n_exp) (threads 0..255 one
// value each; every thread of the workgroup calls it): pair offsets into off[0..n_exp], and,
// with lists, the active-expert list, its length and the first row tile of each active
// expert's group (plus the shared group's and the total) to global memory.
__device__ __forceinline__ void expert_scan(const DispatchArgs& a, const int* cnt, int* off, int (*wtot)[3],
                                            bool lists) {
  const int tid = threadIdx.x;
  const int E = a.n_exp;
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
        if (act && lists && a.active) a.active[ex_act] = tid;
        if (act && lists && a.tile_m > 0) a.tile_start[ex_act] = ex_til;
      }
      if (tid == 255) {
        const int tot_pairs = base3.x + inc.x, na = base3.y + inc.y, tiles = base3.z + inc.z;
        off[E] = tot_pairs;
        if (lists && a.n_active) *a.n_active = na;
        if (lists && a.tile_m > 0) {
          int ts = tiles, g = na;
          if (a.with_shared) { a.tile_start[g++] = ts; ts += (a.m + a.tile_m - 1) / a.tile_m; }
          a.tile_start[g] = ts;
        }
      }
    }
  }
  __syncthreads();
}

template <int MAXP>
struct DispLds {
  uint8_t eid[MAXP];                              // expert of each pair
  uint32_t bitmap[256][33];                       // 32 words + pad per expert
  int cnt[256];
  int off[257];
  int base[256];
  int wpre[256][33];
  int wtot[4][3];
};

// The counting sort on one workgroup of kDispThreads threads. With ids_in_lds the pairs'
// experts are already in sh.eid (and sh.cnt is not counted yet); else they are read from a.ids.
template <int MAXP>
__device__ __forceinline__ void dispatch_block(const DispatchArgs& a, DispLds<MAXP>& sh, bool ids_in_lds) {
  uint8_t* eid = sh.eid;
  auto& bitmap = sh.bitmap;
  int* cnt = sh.cnt;
  int* off = sh.off;
  int* base = sh.base;
  auto& wpre = sh.wpre;
  auto& wtot = sh.wtot;
  const int tid = threadIdx.x;
  const int E = a.n_exp, K = a.top_k;
  if (tid < 256) { cnt[tid] = 0; base[tid] = 0; }
  __syncthreads();
  const int np = a.m * K;
  if (ids_in_lds) {
    for (int p = tid; p < np; p += kDispThreads) atomicAdd(&cnt[eid[p]], 1);
  } else {
  // ids -> LDS bytes and counts; four 16-byte loads issued before their use
  const bool vec = (reinterpret_cast<uintptr_t>(a.ids) & 15) == 0;
  const int nq = vec ? np / 4 : 0;
  for (int q0 = tid; q0 < nq; q0 += 4 * kDispThreads) {
    int4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int q = q0 + u * kDispThreads;
      v[u] = q < nq ? reinterpret_cast<const int4*>(a.ids)[q] : make_int4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int q = q0 + u * kDispThreads;
      if (q >= nq) continue;
      const int e4[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        eid[4 * q + i] = (uint8_t)e4[i];
        atomicAdd(&cnt[e4[i]], 1);
      }
    }
  }
  for (int p = 4 * nq + tid; p < np; p += kDispThreads) {
    const int e = a.ids[p];
    eid[p] = (uint8_t)e;
    atomicAdd(&cnt[e], 1);
  }
  }
  __syncthreads();
  expert_scan(a, cnt, off, wtot, true);
  if (tid < E) a.counts[tid] = cnt[tid];
  if (tid <= E) a.offsets[tid] = off[tid];
  if (a.m <= 32) {
    // at most 32 tokens: one bitmap word per expert, a token's rank among the expert's tokens
    // is the popcount of the lower bits (the general path below with a single word)
    if (tid < 256) bitmap[tid][0] = 0;
    __syncthreads();
    if (tid < a.m)
      for (int j = 0; j < K; ++j) atomicOr(&bitmap[eid[tid * K + j]][0], 1u << tid);
    __syncthreads();
    if (tid < a.m)
      for (int j = 0; j < K; ++j) {
        const int e = eid[tid * K + j];
        const int pos = off[e] + __popc(bitmap[e][0] & ((1u << tid) - 1u));
        a.perm[pos] = tid * K + j;
        if (a.inv) a.inv[tid * K + j] = pos;
      }
    return;
  }
  for (int c0 = 0; c0 < a.m; c0 += kDispThreads) {
    for (int i = tid; i < 256 * 32; i += kDispThreads) bitmap[i / 32][i % 32] = 0;
    __syncthreads();
    const int t = c0 + tid;
    if (t < a.m)
      for (int j = 0; j < K; ++j) atomicOr(&bitmap[eid[t * K + j]][tid / 32], 1u << (tid % 32));
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
        const int e = eid[t * K + j];
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

__global__ __launch_bounds__(kDispThreads) void dispatch_kernel(DispatchArgs a) {
  __shared__ DispLds<kDispMaxPairs> sh;
  dispatch_block(a, sh, false);
}

// Decode (m <= 32 tokens): top-k of every token (one wave per token) and the counting sort in
// one workgroup; the selected experts pass from the first part to the second through LDS.
constexpr int kDecodeMaxPairs = 32 * 8;
__global__ __launch_bounds__(kDispThreads) void topk_dispatch_kernel(RouteArgs r, DispatchArgs a) {
  __shared__ DispLds<kDecodeMaxPairs> sh;
  const int lane = threadIdx.x & 63;
  for (int t = threadIdx.x >> 6; t < r.m; t += kDispThreads / 64) topk_token(r, t, lane, sh.eid);
  __syncthreads();
  dispatch_block(a, sh, true);
}

// Many tokens: the same counting sort over several workgroups, with the same result. Chunk g
// holds tokens [g C, (g + 1) C). dispatch_count_kernel: workgroup g counts the experts of its
// chunk into chunk_counts[g][0..256). dispatch_scatter_kernel: workgroup g adds, per expert,
// the counts of the chunks before its own and of all chunks, ranks its own pairs by token
// inside each expert (LDS bitmap of the chunk's tokens) and writes their perm and inv entries;
// workgroup 0 also writes counts, offsets and the lists.
constexpr int kChunkTokens = 128;                 // kChunkTokens x top_k <= kDispThreads
__global__ __launch_bounds__(kDispThreads) void dispatch_count_kernel(DispatchArgs a, int32_t* chunk_counts) {
  __shared__ int cnt[256];
  const int tid = threadIdx.x, g = blockIdx.x;
  const int t0 = g * kChunkTokens;
  const int np = min(kChunkTokens, a.m - t0) * a.top_k;
  if (tid < 256) cnt[tid] = 0;
  __syncthreads();
  if (tid < np) atomicAdd(&cnt[a.ids[(int64_t)t0 * a.top_k + tid]], 1);
  __syncthreads();
  if (tid < 256) chunk_counts[(int64_t)g * 256 + tid] = cnt[tid];
}

__global__ __launch_bounds__(kDispThreads) void dispatch_scatter_kernel(DispatchArgs a, const int32_t* chunk_counts,
                                                                        int nchunks) {
  __shared__ int before[4][256], all[4][256];
  __shared__ int tot[256], pre[256], off[257];
  __shared__ int wtot[4][3];
  __shared__ uint32_t bitmap[256][kChunkTokens / 32];
  __shared__ uint8_t eid[kChunkTokens * 8];
  const int tid = threadIdx.x, g = blockIdx.x;
  const int K = a.top_k;
  {
    // four threads per expert, each over a quarter of the chunks
    const int e = tid & 255, q = tid >> 8;
    int sb = 0, sa = 0;
    for (int c = q; c < nchunks; c += 4) {
      const int v = chunk_counts[(int64_t)c * 256 + e];
      sa += v;
      if (c < g) sb += v;
    }
    before[q][e] = sb;
    all[q][e] = sa;
  }
  __syncthreads();
  if (tid < 256) {
    pre[tid] = before[0][tid] + before[1][tid] + before[2][tid] + before[3][tid];
    tot[tid] = all[0][tid] + all[1][tid] + all[2][tid] + all[3][tid];
  }
  if (tid < 256 * (kChunkTokens / 32)) bitmap[tid / (kChunkTokens / 32)][tid % (kChunkTokens / 32)] = 0;
  __syncthreads();
  expert_scan(a, tot, off, wtot, g == 0);
  if (g == 0) {
    if (tid < a.n_exp) a.counts[tid] = tot[tid];
    if (tid <= a.n_exp) a.offsets[tid] = off[tid];
  }
  const int t0 = g * kChunkTokens;
  const int np = min(kChunkTokens, a.m - t0) * K;
  const int tl = tid / K;
  if (tid < np) {
    const int e = a.ids[(int64_t)t0 * K + tid];
    eid[tid] = (uint8_t)e;
    atomicOr(&bitmap[e][tl / 32], 1u << (tl % 32));
  }
  __syncthreads();
  if (tid < np) {
    const int e = eid[tid];
    int rank = __popc(bitmap[e][tl / 32] & ((1u << (tl % 32)) - 1u));
    for (int w = 0; w < tl / 32; ++w) rank += __popc(bitmap[e][w]);
    const int pos = off[e] + pre[e] + rank;
    a.perm[pos] = t0 * K + tid;
    if (a.inv) a.inv[t0 * K + tid] = pos;
  }
}


// ---- many-token routing --------------------------------------------------------------------

constexpr int kRT = 64;           // tokens per router tile
constexpr int kRE = 64;           // logit rows (experts) per router tile
constexpr int kRK = 64;           // K per step
constexpr int kRLDK = kRK + 8;
constexpr int kRKS = 4;           // K slices of the many-token router (when hidden % 256 == 0)

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

struct CertArgs {
  RouteArgs r;
  float* approx;      // [ks][m][ld_approx] partial logits, one plane per K slice
  int ld_approx;
  int ks;             // K slices
  double* norm2_w;    // [ks][n_exp + 1] partial squared norms of the logit rows
};

__device__ __forceinline__ const uint16_t* logit_row(const RouteArgs& a, int e) {
  if (e < a.n_exp) return a.router_w + (int64_t)e * a.hidden;
  if (e == a.n_exp) return a.sh_gate_w;       // may be null
  return nullptr;
}

// Approximate logits on the bf16 matrix cores: a 64-token x 64-row tile over one K slice per
// workgroup (grid z = slice). Workgroups of the first token tile also accumulate the squared
// norms of their 64 logit rows over the slice, in fp64.
__global__ __launch_bounds__(256) void router_mfma_kernel(CertArgs c) {
  const RouteArgs& a = c.r;
  __shared__ __align__(16) uint16_t As[kRT][kRLDK];
  __shared__ __align__(16) uint16_t Bs[kRE][kRLDK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * kRT, e0 = blockIdx.y * kRE;
  const int kslice = a.hidden / c.ks, kbeg = blockIdx.z * kslice;
  const int r = tid / 4, q = tid % 4;            // 64 rows x 4 quarters of 16 values
  const int tok = t0 + r;
  const uint16_t* arow = tok < a.m ? a.x + (int64_t)tok * a.hidden : nullptr;
  const uint16_t* brow = logit_row(a, e0 + r);
  const bool norms = blockIdx.x == 0;
  double nw2 = 0.0;
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
  load(kbeg);
  for (int k0 = kbeg; k0 < kbeg + kslice; k0 += kRK) {
    __syncthreads();
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      *reinterpret_cast<uint4*>(&As[r][q * 16 + h * 8]) = ra[h];
      *reinterpret_cast<uint4*>(&Bs[r][q * 16 + h * 8]) = rb[h];
    }
    if (norms) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t w4[4] = {rb[h].x, rb[h].y, rb[h].z, rb[h].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const double lo = bf16_lo(w4[i]), hi = bf16_hi(w4[i]);
          nw2 = __builtin_fma(lo, lo, nw2);
          nw2 = __builtin_fma(hi, hi, nw2);
        }
      }
    }
    __syncthreads();
    if (k0 + kRK < kbeg + kslice) load(k0 + kRK);
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
  float* out = c.approx + (int64_t)blockIdx.z * a.m * c.ld_approx;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int tt = t0 + wave * 16 + 4 * (lane / 16) + i;
    if (tt >= a.m) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = e0 + j * 16 + (lane % 16);
      if (e <= a.n_exp) out[(int64_t)tt * c.ld_approx + e] = acc[j][i];
    }
  }
  if (norms) {
    // the 4 quarters of a row are adjacent lanes
    nw2 += __shfl_xor(nw2, 1);
    nw2 += __shfl_xor(nw2, 2);
    if (q == 0 && e0 + r <= a.n_exp) c.norm2_w[(int64_t)blockIdx.z * (a.n_exp + 1) + e0 + r] = nw2;
  }
}

// Exact fp64 logits of NR rows against one token row (wave-wide). Each pass covers up to four
// 8-value chunks per lane of x and of every row, all loaded before any arithmetic.
template <int NR>
__device__ __forceinline__ void exact_logits(const uint16_t* x, const uint16_t* const* w, int hidden, int lane,
                                             double* out) {
  double s[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i) s[i] = 0.0;
  const int chunks = hidden / 8;
  for (int c0 = 0; c0 < chunks; c0 += 4 * 64) {
    uint4 xv[4], wv[NR][4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = c0 + u * 64 + lane;
      const bool ok = c < chunks;
      xv[u] = ok ? *reinterpret_cast<const uint4*>(x + c * 8) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < NR; ++i) wv[i][u] = ok ? *reinterpret_cast<const uint4*>(w[i] + c * 8) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t xa[4] = {xv[u].x, xv[u].y, xv[u].z, xv[u].w};
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        const uint32_t wa[4] = {wv[i][u].x, wv[i][u].y, wv[i][u].z, wv[i][u].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          s[i] = __builtin_fma((double)bf16_lo(xa[j]), (double)bf16_lo(wa[j]), s[i]);
          s[i] = __builtin_fma((double)bf16_hi(xa[j]), (double)bf16_hi(wa[j]), s[i]);
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < NR; ++i) out[i] = wave_sum_f64(s[i]);
}

// One wave per token: certify the candidate set, recompute its logits exactly, select.
__global__ __launch_bounds__(256) void certify_topk_kernel(CertArgs c) {
  const RouteArgs& a = c.r;
  __shared__ int cand[4][256];
  __shared__ double cval[4][257];            // candidate logits, then the shared-expert logit
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wv;
  if (t >= a.m) return;
  const uint16_t* xr = a.x + (int64_t)t * a.hidden;
  const double n = (double)a.hidden;
  const double u = 1.0 / 8388608.0;                       // 2^-23
  const double gamma = n * u / (1.0 - n * u);
  const double tiny = 1.1754943508222875e-38;             // 2^-126
  // |x|_2 of this token (fp64, slightly enlarged so that the bound stays an upper bound)
  double sx = 0.0;
  for (int c0 = 0; c0 < a.hidden / 8; c0 += 4 * 64) {
    uint4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int cidx = c0 + u * 64 + lane;
      v[u] = cidx < a.hidden / 8 ? *reinterpret_cast<const uint4*>(xr + cidx * 8) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t w4[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const double l = bf16_lo(w4[i]), h = bf16_hi(w4[i]);
        sx = __builtin_fma(l, l, sx);
        sx = __builtin_fma(h, h, sx);
      }
    }
  }
  const double nx = sqrt(wave_sum_f64(sx)) * (1.0 + 1e-12);
  double lo[4], hi[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = lane + 64 * q;
    if (e < a.n_exp) {
      double nw2 = 0.0, v = 0.0, av = 0.0;
#pragma unroll 4
      for (int z = 0; z < c.ks; ++z) {
        nw2 += c.norm2_w[(int64_t)z * (a.n_exp + 1) + e];
        const double p = (double)c.approx[((int64_t)z * a.m + t) * c.ld_approx + e];
        v += p;
        av += __builtin_fabs(p);
      }
      const double nw = sqrt(nw2) * (1.0 + 1e-12);
      // fp32 sums inside the slices: gamma |x| |w| (any summation order); the slices are added
      // in fp64 (1e-15 of their magnitudes covers that rounding)
      // + n 2^-126: products of two normal bf16 values that fall below the fp32 normal range
      // (each off by less than 2^-126 if the matrix cores flush them)
      const double d = gamma * nx * nw + tiny * sqrt(n) * (nx + nw) * 1.01 + n * tiny + 1e-15 * av;
      const double b = a.bias ? (double)a.bias[e] : 0.0;
      // non-finite inputs: an unknown lower end is -inf and an unknown upper end +inf, so
      // such an expert stays a candidate and at least top_k candidates always exist
      const double l0 = v + b - d, h0 = v + b + d;
      lo[q] = l0 != l0 ? -__builtin_huge_val() : l0;
      hi[q] = h0 != h0 ? __builtin_huge_val() : h0;
    } else {
      lo[q] = -__builtin_huge_val();
      hi[q] = -__builtin_huge_val();
    }
  }
  // k-th largest lower end: the lower ends staged in this wave's row of cval (expert e at
  // position e), then the wave's top-k selection over them; the last value it takes
  double lk;
  {
#pragma unroll
    for (int q = 0; q < 4; ++q) cval[wv][lane + 64 * q] = lo[q];
    __builtin_amdgcn_wave_barrier();
    double sl[8];
    int sp[8];
    tk::topk_select(cval[wv], a.n_exp, a.top_k, lane, sl, sp);
    lk = sl[0];
#pragma unroll
    for (int j = 1; j < 8; ++j)
      if (j == a.top_k - 1) lk = sl[j];
    __builtin_amdgcn_wave_barrier();
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
  // exact logits of the candidates, four rows per pass
  for (int i0 = 0; i0 < nc; i0 += 4) {
    const uint16_t* rows[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) rows[i] = a.router_w + (int64_t)cand[wv][min(i0 + i, nc - 1)] * a.hidden;
    double ex4[4];
    exact_logits<4>(xr, rows, a.hidden, lane, ex4);
    if (lane == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (i0 + i < nc) {
          const int e = cand[wv][i0 + i];
          cval[wv][i0 + i] = ex4[i] + (a.bias ? (double)a.bias[e] : 0.0);
        }
    }
  }
  double glog = 0.0;
  if (a.sh_gate_w) {
    const uint16_t* rows[1] = {a.sh_gate_w};
    exact_logits<1>(xr, rows, a.hidden, lane, &glog);
  }
  // top-k among the candidates by (exact logit desc, expert asc): candidates are in expert
  // order, so the selection over their positions (a NaN ranks below every number) picks them
  // in that order; the shared-expert logit goes after them for the gate
  if (lane == 0) cval[wv][nc] = glog;
  __builtin_amdgcn_wave_barrier();
  double sel_l[8];
  int sel_p[8], sel_e[8];
  tk::topk_select(cval[wv], nc, a.top_k, lane, sel_l, sel_p);
#pragma unroll
  for (int j = 0; j < 8; ++j) sel_e[j] = j < a.top_k ? cand[wv][sel_p[j]] : 0;
  tk::topk_store(cval[wv], nc, a.top_k, a.sh_gate_w != nullptr, lane, sel_l, sel_e, a.ids + (int64_t)t * a.top_k,
                 a.w + (int64_t)t * a.top_k, a.g ? a.g + t : nullptr, nullptr);
}

}  // namespace

// Router rows per wave for m <= 32 (more waves in flight for these short calls).
constexpr int kDecodeRouterRows = 1;

size_t route_workspace_bytes(int m, int n_exp) {
  const size_t fp64 = (size_t)m * (n_exp + 1) * sizeof(double);
  const int ld = (n_exp + 1 + kRE - 1) / kRE * kRE;
  const size_t cert = (size_t)kRKS * m * ld * sizeof(float) + (size_t)kRKS * (n_exp + 1) * sizeof(double) + 64;
  return fp64 > cert ? fp64 : cert;
}

hipError_t router_launch(const RouteArgs& a, hipStream_t s) {
  if (a.m > 32) {
    // certified many-token routing; the logits region holds the partial logits, then the
    // partial squared norms of the logit rows
    CertArgs c;
    c.r = a;
    c.ks = a.hidden % (kRKS * kRK) == 0 ? kRKS : 1;
    c.ld_approx = (a.n_exp + 1 + kRE - 1) / kRE * kRE;
    c.approx = reinterpret_cast<float*>(a.logits);
    char* base = reinterpret_cast<char*>(a.logits) + (size_t)kRKS * a.m * c.ld_approx * sizeof(float);
    c.norm2_w = reinterpret_cast<double*>(base);
    hipLaunchKernelGGL(router_mfma_kernel, dim3((a.m + kRT - 1) / kRT, (a.n_exp + 1 + kRE - 1) / kRE, c.ks),
                       dim3(256), 0, s, c);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(certify_topk_kernel, dim3((a.m + 3) / 4), dim3(256), 0, s, c);
    return hipGetLastError();
  }
  const int rows = a.n_exp + (a.sh_gate_w ? 1 : 0);
  dim3 grid((rows + 4 * kDecodeRouterRows - 1) / (4 * kDecodeRouterRows), a.m);
  hipLaunchKernelGGL(router_logits_kernel<kDecodeRouterRows>, grid, dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(topk_kernel, dim3((a.m + 3) / 4), dim3(256), 0, s, a);
  return hipGetLastError();
}

size_t dispatch_scratch_bytes(int m) { return (size_t)((m + kChunkTokens - 1) / kChunkTokens) * 256 * sizeof(int32_t); }

hipError_t dispatch_launch(const DispatchArgs& a, hipStream_t s) {
  if (a.chunk_counts != nullptr && a.m > kChunkTokens) {
    const int nchunks = (a.m + kChunkTokens - 1) / kChunkTokens;
    hipLaunchKernelGGL(dispatch_count_kernel, dim3(nchunks), dim3(kDispThreads), 0, s, a, a.chunk_counts);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(dispatch_scatter_kernel, dim3(nchunks), dim3(kDispThreads), 0, s, a, a.chunk_counts, nchunks);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(dispatch_kernel, dim3(1), dim3(kDispThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t router_logits_launch(const RouteArgs& a, hipStream_t s) {
  if (a.m > 32) return hipErrorInvalidValue;
  const int rows = a.n_exp + (a.sh_gate_w ? 1 : 0);
  hipLaunchKernelGGL(router_logits_kernel<kDecodeRouterRows>, dim3((rows + 4 * kDecodeRouterRows - 1) / (4 * kDecodeRouterRows), a.m),
                     dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t route_dispatch_launch(const RouteArgs& r, const DispatchArgs& d, hipStream_t s) {
  if (r.m > 32 || r.m * r.top_k > kDecodeMaxPairs) return hipErrorInvalidValue;
  const int rows = r.n_exp + (r.sh_gate_w ? 1 : 0);
  hipLaunchKernelGGL(router_logits_kernel<kDecodeRouterRows>, dim3((rows + 4 * kDecodeRouterRows - 1) / (4 * kDecodeRouterRows), r.m),
                     dim3(256), 0, s, r);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(topk_dispatch_kernel, dim3(1), dim3(kDispThreads), 0, s, r, d);
  return hipGetLastError();
}

}  // namespace bfp
