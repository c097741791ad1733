// Expert-grouped skinny BFP4 matmuls and the weighted combine for MoE decode (gfx950).
//
// "Qwen3.6-35B-A3B — TT-native mixed BFP4/BFP8", section "Fused decode kernels": MoE decode
// runs through device top-k routing and batched expert streams, one gate/up and one down
// program for all rows; "Qwen3.8-27B ...", "Multi-user decode": every weight is read once per
// step for all rows. Here each selected expert's rows are streamed once by the same kernel
// tile as the dense GEMV, for all (token, slot) pairs routed to it; the shared expert is one
// more group with every token. The combine then forms y_t = sum_j w_tj o_tj (slots in rank
// order) + g_t * shared_t, a fixed order, so the result does not depend on scheduling.
//
// For a few tokens the same tiles run per (token, slot) instead (the per-token path below):
// every gate/up workgroup ranks its token's experts itself, and the down kernel combines each
// token's slots in the same order, so no dispatch, per-pair outputs or combine launch remain.
// Both paths give each token the same bits.
#include "bfp_moe.hpp"
#include "gemv_impl.hpp"
#include "moe_topk.hpp"

namespace bfp {

namespace {

using namespace gemv_detail;

constexpr int kMoeThreads = 256;

inline __host__ __device__ int mb_bucket(int n) {
  return n <= 1 ? 1 : n <= 2 ? 2 : n <= 4 ? 4 : n <= 8 ? 8 : n <= 16 ? 16 : 32;
}

// rows per lane group (one: these calls are short and latency-bound, so more workgroups win)
template <int NMAT> constexpr int moe_rt() { return 1; }

template <int NMAT, bool XB, int MB, int LPR>
__device__ __forceinline__ void run_tile(const GemvArgs& a, int row_base, const int* xrow, const int* yrow,
                                         uint32_t* xs) {
  // units in flight per lane group: two for one activation row; one for the grouped tiles
  // (fewer VGPRs: 89 instead of 105 for gate/up, a fifth workgroup resident per CU)
  constexpr int U = MB <= 1 ? 2 : 1;
  constexpr int RT = MB <= 8 ? moe_rt<NMAT>() : 1;
  gemv_tile<4, MB, RT, LPR, NMAT, U, 2, XB, kMoeThreads>(a, row_base, xrow, yrow, xs);
}

template <int NMAT, bool XB, int MBMAX, int LPR>
__global__ __launch_bounds__(kMoeThreads) void moe_gemv_kernel(MoeGemvArgs ma, int kc) {
  extern __shared__ uint32_t xs[];
  __shared__ int xrow[32], yrow[32];
  const int na = *ma.n_active;
  int d = blockIdx.y, r0 = 0;     // group, and its first pair in this workgroup's tile
  if (ma.tile_start) {
    const int ng = na + (ma.scode0 != nullptr ? 1 : 0);
    if ((int)blockIdx.y >= ma.tile_start[ng]) return;
    int lo = 0, hi = ng - 1;      // last group whose first tile is <= blockIdx.y
    while (lo < hi) {
      const int mid = (lo + hi + 1) / 2;
      if (ma.tile_start[mid] <= (int)blockIdx.y) lo = mid; else hi = mid - 1;
    }
    d = lo;
    r0 = ((int)blockIdx.y - ma.tile_start[lo]) * ma.tile_m;
  }
  const bool shared = d == na && ma.scode0 != nullptr;
  if (d > na || (d == na && !shared)) return;
  int e = -1, p0, n;
  if (!shared) {
    e = ma.active[d];
    p0 = ma.offsets[e];
    n = ma.offsets[e + 1] - p0;
  } else {
    p0 = ma.m * ma.top_k;
    n = ma.m;
  }
  p0 += r0;
  n -= r0;
  if (ma.tile_start && n > ma.tile_m) n = ma.tile_m;
  if ((int)threadIdx.x < n) {
    const int pos = p0 + threadIdx.x;
    const int tok = shared ? pos - ma.m * ma.top_k : ma.perm[pos] / ma.top_k;
    xrow[threadIdx.x] = ma.x_by_token ? tok : pos;
    yrow[threadIdx.x] = pos;
  }
  GemvArgs a;
  const int64_t nbk = ma.k / kBlock;
  const int64_t rows0 = shared ? 0 : (int64_t)e * ma.rows_per_expert;
  a.exp0 = (shared ? ma.sexp0 : ma.exp0) + rows0 * nbk;
  a.code0 = (shared ? ma.scode0 : ma.code0) + rows0 * (ma.k / 2);
  a.exp1 = NMAT == 2 ? (shared ? ma.sexp1 : ma.exp1) + rows0 * nbk : nullptr;
  a.code1 = NMAT == 2 ? (shared ? ma.scode1 : ma.code1) + rows0 * (ma.k / 2) : nullptr;
  a.x = ma.x; a.ldx = ma.ldx;
  a.y = ma.y; a.ldy = ma.ldy; a.y_bf16 = ma.y_bf16;
  a.n = ma.rows_per_expert; a.k = ma.k; a.m = n; a.kc = kc;
  const int rpw = (kMoeThreads / kWave) * (kWave / LPR) * (mb_bucket(n) <= 8 ? moe_rt<NMAT>() : 1);
  const int row_base = blockIdx.x * rpw;
  if (row_base >= ma.rows_per_expert) return;
  // xrow/yrow are read after the first barrier inside the tile
  switch (mb_bucket(n)) {
    case 1: run_tile<NMAT, XB, 1, LPR>(a, row_base, xrow, yrow, xs); break;
    case 2: if constexpr (MBMAX >= 2) run_tile<NMAT, XB, 2, LPR>(a, row_base, xrow, yrow, xs); break;
    case 4: if constexpr (MBMAX >= 4) run_tile<NMAT, XB, 4, LPR>(a, row_base, xrow, yrow, xs); break;
    case 8: if constexpr (MBMAX >= 8) run_tile<NMAT, XB, 8, LPR>(a, row_base, xrow, yrow, xs); break;
    case 16: if constexpr (MBMAX >= 16) run_tile<NMAT, XB, 16, LPR>(a, row_base, xrow, yrow, xs); break;
    default: if constexpr (MBMAX >= 32) run_tile<NMAT, XB, 32, LPR>(a, row_base, xrow, yrow, xs); break;
  }
}

template <int NMAT, bool XB, int MBMAX, int LPR>
hipError_t launch_lpr(const MoeGemvArgs& ma, hipStream_t s) {
  using L = XLayout<XB, 32>;
  const int kc = pick_kc(ma.k, MBMAX, 32, LPR, L::kBytesPerValue);
  const size_t lds = (size_t)MBMAX * (kc / 32) * L::kStrideDw * sizeof(uint32_t);
  // enough row tiles for the smallest rows-per-workgroup a group can pick (RT = 1 when
  // more than 8 pairs share an expert); workgroups past the end of a group exit
  constexpr int RPW = (kMoeThreads / kWave) * (kWave / LPR);
  const int pairs = ma.m * ma.top_k;
  int groups = (pairs < 256 ? pairs : 256) + (ma.scode0 ? 1 : 0);
  if (ma.tile_start)   // at most one partial tile per group beyond pairs / tile_m full ones
    groups += pairs / ma.tile_m + (ma.scode0 ? ma.m / ma.tile_m : 0);
  dim3 grid((ma.rows_per_expert + RPW - 1) / RPW, groups);
  hipLaunchKernelGGL((moe_gemv_kernel<NMAT, XB, MBMAX, LPR>), grid, dim3(kMoeThreads), lds, s, ma, kc);
  return hipGetLastError();
}

// Lanes per row from K alone: about four 32-value units per lane (4 to 16 lanes), so that
// short rows (the down projection) still give every lane several loads and a workgroup many
// rows.
template <int NMAT, bool XB, int MBMAX>
hipError_t launch_mbmax(const MoeGemvArgs& ma, hipStream_t s) {
  const int units = ma.k / 32;
  if (units <= 16) return launch_lpr<NMAT, XB, MBMAX, 4>(ma, s);
  if (units <= 32) return launch_lpr<NMAT, XB, MBMAX, 8>(ma, s);
  return launch_lpr<NMAT, XB, MBMAX, 16>(ma, s);
}

template <int NMAT, bool XB>
hipError_t launch_x(const MoeGemvArgs& ma, hipStream_t s) {
  if (ma.tile_start) {
    if (ma.tile_m != kDecodeTileRows) return hipErrorInvalidValue;
    return launch_mbmax<NMAT, XB, kDecodeTileRows>(ma, s);
  }
  switch (mb_bucket(ma.m)) {
    case 1: return launch_mbmax<NMAT, XB, 1>(ma, s);
    case 2: return launch_mbmax<NMAT, XB, 2>(ma, s);
    case 4: return launch_mbmax<NMAT, XB, 4>(ma, s);
    case 8: return launch_mbmax<NMAT, XB, 8>(ma, s);
    case 16: return launch_mbmax<NMAT, XB, 16>(ma, s);
    default: return launch_mbmax<NMAT, XB, 32>(ma, s);
  }
}

// y[t][n] = sum_j w[t][j] * o[inv[t*K+j]][n] + g[t] * o[m*K + t][n]; four outputs per thread.
// The weights and positions of all slots (top_k <= 8) are loaded first, then all their rows,
// with the shared expert's, then the products are added in rank order: two memory round trips
// per token, not two per slot.
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  const int t = blockIdx.y;
  const int n4 = blockIdx.x * 256 + threadIdx.x;
  if (n4 * 4 >= a.hidden) return;
  float wj[8];
  int pos[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int jj = min(j, a.top_k - 1);
    wj[j] = a.w[(int64_t)t * a.top_k + jj];
    pos[j] = a.inv[(int64_t)t * a.top_k + jj];
  }
  f32x4 o[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) o[j] = *reinterpret_cast<const f32x4*>(a.o + (int64_t)pos[j] * a.hidden + n4 * 4);
  float gt = 0.f;                                     // the shared expert's gate and row
  f32x4 os = f32x4{0.f, 0.f, 0.f, 0.f};
  if (a.g) {
    gt = a.g[t];
    os = *reinterpret_cast<const f32x4*>(a.o + ((int64_t)a.m * a.top_k + t) * a.hidden + n4 * 4);
  }
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j >= a.top_k) break;
    acc.x = __builtin_fmaf(wj[j], o[j].x, acc.x);
    acc.y = __builtin_fmaf(wj[j], o[j].y, acc.y);
    acc.z = __builtin_fmaf(wj[j], o[j].z, acc.z);
    acc.w = __builtin_fmaf(wj[j], o[j].w, acc.w);
  }
  if (a.g) {
    acc.x = __builtin_fmaf(gt, os.x, acc.x);
    acc.y = __builtin_fmaf(gt, os.y, acc.y);
    acc.z = __builtin_fmaf(gt, os.z, acc.z);
    acc.w = __builtin_fmaf(gt, os.w, acc.w);
  }
  *reinterpret_cast<f32x4*>(a.y + (int64_t)t * a.hidden + n4 * 4) = acc;
}

// ---- per-token path ------------------------------------------------------------------------

// Gate/up + SwiGLU of token t and slot d (blockIdx.y = t * ns + d, ns = top_k + 1 with a
// shared expert, d == top_k: the shared expert), rows [blockIdx.x * RPW, +RPW) of it: the tile
// of the grouped kernel with one activation row. h row t * ns + d.
template <int LPR>
__global__ __launch_bounds__(kMoeThreads) void tok_gateup_kernel(MoeTokArgs ma, int kc) {
  extern __shared__ uint32_t xs[];
  __shared__ int xrow[1], yrow[1], sel[1];
  const int ns = ma.top_k + (ma.sg_code ? 1 : 0);
  const int t = blockIdx.y / ns, d = blockIdx.y % ns;
  const bool shared = d == ma.top_k;
  const double* l = ma.logits + (int64_t)t * ma.ld_logits;
  if (threadIdx.x < kWave && !shared) {
    const int lane = threadIdx.x;
    double sel_l[8];
    int sel_e[8];
    tk::topk_select(l, ma.n_exp, ma.top_k, lane, sel_l, sel_e);
    int e = sel_e[0];
#pragma unroll
    for (int j = 1; j < 8; ++j)
      if (j == d) e = sel_e[j];
    if (blockIdx.x == 0 && d == 0)
      tk::topk_store(l, ma.n_exp, ma.top_k, ma.gate_row != 0, lane, sel_l, sel_e, ma.ids + (int64_t)t * ma.top_k,
                     ma.w + (int64_t)t * ma.top_k, ma.sg_code ? ma.g + t : nullptr, nullptr);
    if (lane == 0) sel[0] = e;
  }
  if (threadIdx.x == 0) {
    xrow[0] = t;
    yrow[0] = blockIdx.y;
    if (shared) sel[0] = 0;
  }
  __syncthreads();
  const int64_t nbk = ma.hidden / kBlock;
  const int64_t rows0 = shared ? 0 : (int64_t)sel[0] * ma.inter;
  GemvArgs a;
  a.exp0 = (shared ? ma.sg_exp : ma.g_exp) + rows0 * nbk;
  a.code0 = (shared ? ma.sg_code : ma.g_code) + rows0 * (ma.hidden / 2);
  a.exp1 = (shared ? ma.su_exp : ma.u_exp) + rows0 * nbk;
  a.code1 = (shared ? ma.su_code : ma.u_code) + rows0 * (ma.hidden / 2);
  a.x = ma.x; a.ldx = ma.hidden;
  a.y = ma.h; a.ldy = ma.inter; a.y_bf16 = 0;
  a.n = ma.inter; a.k = ma.hidden; a.m = 1; a.kc = kc;
  constexpr int RPW = (kMoeThreads / kWave) * (kWave / LPR);
  run_tile<2, true, 1, LPR>(a, blockIdx.x * RPW, xrow, yrow, xs);
}

// Down projection + combine of token t = blockIdx.y for output columns [blockIdx.x * RPW,
// +RPW): wave d computes slot d's values (the grouped kernel's lane split, groups and
// reduction for one activation row), then y = sum_j w_j o_j in rank order + g o_shared, as
// the combine kernel does.
template <int LPR>
__global__ __launch_bounds__(kWave * 9) void tok_down_kernel(MoeTokArgs ma) {
  extern __shared__ uint32_t xs[];                 // every slot's h row, fp32 LDS layout
  constexpr int RPW = kWave / LPR;
  constexpr int BPU = 2;
  using L = XLayout<false, 32>;
  using GroupT = Group<4, BPU, 2, 1, 1>;
  __shared__ float os[9][RPW];
  const int ns = blockDim.x / kWave;               // slots: top_k (+ 1 shared)
  const int t = blockIdx.y;
  const int d = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = threadIdx.x % kWave;   // d wave-uniform
  const bool shared = d == ma.top_k;
  const int32_t* ids = ma.ids + (int64_t)t * ma.top_k;
  const float* wt = ma.w + (int64_t)t * ma.top_k;
  // the combine's factors, read now so that their latency overlaps the weights'
  float wf[9];
  if ((int)threadIdx.x < RPW) {
#pragma unroll
    for (int j = 0; j < 8; ++j) wf[j] = j < ma.top_k ? wt[j] : 0.f;
    wf[8] = ma.sd_code ? ma.g[t] : 0.f;
  }
  const int e = shared ? 0 : ids[d];
  const int nbk = ma.inter / kBlock;
  const int nuc = ma.inter / 32;
  const int64_t rows0 = shared ? 0 : (int64_t)e * ma.hidden;
  const uint8_t* expm[1] = {(shared ? ma.sd_exp : ma.d_exp) + rows0 * nbk};
  const uint8_t* codem[1] = {(shared ? ma.sd_code : ma.d_code) + rows0 * (ma.inter / 2)};
  const int grp = lane / LPR, p = lane % LPR;
  const int col = blockIdx.x * RPW + grp;
  bool rowok[1] = {col < ma.hidden};
  int64_t rowc[1] = {rowok[0] ? col : ma.hidden - 1};
  constexpr int STEP = 2 * LPR;
  const int ng = (nuc + STEP - 1) / STEP;          // 1 or 2 (inter <= 64 LPR values)
  GroupT ga, gb;
  load_group<4, BPU, 2, 1, 1, LPR>(ga, codem, expm, rowc, ma.inter, nbk, 0, 0, p, nuc);
  if (ng > 1) load_group<4, BPU, 2, 1, 1, LPR>(gb, codem, expm, rowc, ma.inter, nbk, 0, STEP, p, nuc);
  const int per_row = ma.inter / 4;
  auto hrow = [&](int dd) -> int64_t {
    if (!ma.inv) return (int64_t)t * ns + dd;
    return dd < ma.top_k ? ma.inv[(int64_t)t * ma.top_k + dd] : (int64_t)ma.m * ma.top_k + t;
  };
  for (int idx = threadIdx.x; idx < ns * per_row; idx += blockDim.x) {
    const int mi = idx / per_row, c4 = idx % per_row;
    const uint4 v = *reinterpret_cast<const uint4*>(ma.h + hrow(mi) * ma.inter + c4 * 4);
    const int kk = c4 * 4;
    *reinterpret_cast<uint4*>(xs + ((size_t)mi * nuc + kk / 32) * L::kStrideDw + (kk % 32)) = v;
  }
  __syncthreads();
  float acc[1][1][1] = {{{0.f}}};
  const uint32_t* xd = xs + (size_t)d * nuc * L::kStrideDw;
  compute_group<4, 1, BPU, 2, 1, 1, false>(acc, ga, rowok, xd, nuc);
  if (ng > 1) compute_group<4, 1, BPU, 2, 1, 1, false>(acc, gb, rowok, xd, nuc);
  float v[1] = {acc[0][0][0]};
  LaneReduce<1, 1, LPR>::run(v, lane);
  if (p == 0) os[d][grp] = v[0];
  __syncthreads();
  const int c = blockIdx.x * RPW + (int)threadIdx.x;
  if ((int)threadIdx.x < RPW && c < ma.hidden) {
    float y = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j < ma.top_k) y = __builtin_fmaf(wf[j], os[j][threadIdx.x], y);
    if (ma.sd_code) y = __builtin_fmaf(wf[8], os[ma.top_k][threadIdx.x], y);
    ma.y[(int64_t)t * ma.hidden + c] = y;
  }
}

// Lanes per row as the grouped kernels pick them from K (launch_mbmax).
inline int moe_lpr(int k) {
  const int units = k / 32;
  return units <= 16 ? 4 : units <= 32 ? 8 : 16;
}

template <int LPR>
hipError_t tok_gateup(const MoeTokArgs& a, hipStream_t s) {
  using L = XLayout<true, 32>;
  const int kc = pick_kc(a.hidden, 1, 32, LPR, L::kBytesPerValue);
  const size_t lds = (size_t)(kc / 32) * L::kStrideDw * sizeof(uint32_t);
  constexpr int RPW = (kMoeThreads / kWave) * (kWave / LPR);
  const dim3 grid((a.inter + RPW - 1) / RPW, a.m * (a.top_k + (a.sg_code ? 1 : 0)));
  hipLaunchKernelGGL(tok_gateup_kernel<LPR>, grid, dim3(kMoeThreads), lds, s, a, kc);
  return hipGetLastError();
}

template <int LPR>
hipError_t tok_down(const MoeTokArgs& a, hipStream_t s) {
  using L = XLayout<false, 32>;
  const int ns = a.top_k + (a.sd_code ? 1 : 0);
  const size_t lds = (size_t)ns * (a.inter / 32) * L::kStrideDw * sizeof(uint32_t);
  constexpr int RPW = kWave / LPR;
  hipLaunchKernelGGL(tok_down_kernel<LPR>, dim3((a.hidden + RPW - 1) / RPW, a.m), dim3(kWave * ns), lds, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t moe_tok_down_launch(const MoeTokArgs& a, hipStream_t s) {
  if (a.m < 1 || a.m > 32 || a.top_k < 1 || a.top_k > 8 || a.inter % 32 != 0 || a.inter > 2048)
    return hipErrorInvalidValue;
  switch (moe_lpr(a.inter)) {
    case 4: return tok_down<4>(a, s);
    case 8: return tok_down<8>(a, s);
    default: return tok_down<16>(a, s);
  }
}

bool moe_tok_supported(int m, int top_k, int inter) {
  // the down kernel's LDS: every slot's h row, 144 bytes per 32 values (at most 83 KB)
  return m >= 1 && m <= kTokPathMaxM && top_k >= 1 && top_k <= 8 && inter % 32 == 0 && inter <= 2048;
}

hipError_t moe_tok_launch(const MoeTokArgs& a, hipStream_t s) {
  if (!moe_tok_supported(a.m, a.top_k, a.inter)) return hipErrorInvalidValue;
  hipError_t e;
  switch (moe_lpr(a.hidden)) {
    case 4: e = tok_gateup<4>(a, s); break;
    case 8: e = tok_gateup<8>(a, s); break;
    default: e = tok_gateup<16>(a, s); break;
  }
  if (e != hipSuccess) return e;
  switch (moe_lpr(a.inter)) {
    case 4: return tok_down<4>(a, s);
    case 8: return tok_down<8>(a, s);
    default: return tok_down<16>(a, s);
  }
}

hipError_t moe_gemv_launch(const MoeGemvArgs& a, int nmat, hipStream_t s) {
  if (nmat == 2) return a.x_bf16 ? launch_x<2, true>(a, s) : launch_x<2, false>(a, s);
  return a.x_bf16 ? launch_x<1, true>(a, s) : launch_x<1, false>(a, s);
}

hipError_t combine_launch(const CombineArgs& a, hipStream_t s) {
  dim3 grid((a.hidden / 4 + 255) / 256, a.m);
  hipLaunchKernelGGL(combine_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace bfp
