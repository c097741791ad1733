#pragma once
// Skinny BFP4/BFP8 matmul (decode GEMV, 1..32 activation rows) for gfx950: kernel template.
//
// What it computes ("Qwen3.8-27B — TT-native mixed BFP4/BFP8 (GPTQ)", sections "What
// changed in this release (s27v6-20261024)" and "Multi-user decode": up to 32 rows share one
// pass over every weight): y[i][j] = sum_k x[i][k] * W[j][k], W stored as BFP blocks along K,
// optionally followed by SwiGLU with a second matrix (h = silu(x Wg^T) * (x Wu^T)).
//
// Design (bound by HBM at M = 1, by the VALU for larger M):
//  * A lane group of LPR lanes (32 or 16, chosen from K alone) owns RT weight rows. Lane p
//    owns the "units" p, p + LPR, ... of every row, a unit being 16 code bytes (two BFP4
//    blocks or one BFP8 block): a wave-wide load covers consecutive bytes of a row.
//  * All loads of a group of U units are issued before any arithmetic (indices are clamped
//    rather than branched on); the first group is in flight while the activations are
//    staged, and later groups are loaded one group ahead of the arithmetic.
//  * Activations are staged per workgroup in LDS, padded per unit so that lanes reading
//    consecutive units hit distinct banks. bf16 activations stay bf16, pre-permuted into the
//    pair order the weight unpack produces, and the products run on v_dot2_f32_bf16 (two
//    products per instruction); fp32 activations use fp32 FMAs.
//  * Weights are unpacked in registers exactly (see bfp_device.hpp); each block's partial
//    sum is scaled once by its power-of-two block scale (v_ldexp_f32, exact for every E).
//  * Partial sums are reduced across the lane group by recursive halving with DPP row moves
//    and v_permlane16_swap; one lane per value writes y (with the SwiGLU epilogue).
//  * Each lane's share of K and the order of its sums depend on K only, so row i of an
//    M-row call is bit-identical to the same row computed alone.
#include "argmax.hpp"
#include "bfp_device.hpp"
#include "bfp_internal.hpp"

namespace bfp {
namespace gemv_detail {


struct GemvArgs {
  const uint8_t* exp0;
  const uint8_t* code0;
  const uint8_t* exp1;                     // up-projection planes (SwiGLU) or null
  const uint8_t* code1;
  const void* x;
  int64_t ldx;
  void* y;
  int64_t ldy;
  int n, k, m;
  int y_bf16;
  int kc;                                  // K values staged per LDS chunk
  uint64_t* cand;                          // argmax mode: candidate keys [m][workgroups], else null
  int32_t* am_idx;                         // argmax mode: per activation row, the column
  float* am_val;                           //   and its value
};

// A unit: what one lane loads per row with one instruction.
template <int FMT, int BPU>
struct Unit {
  static constexpr int kBytes = FMT == 8 ? 16 * BPU : 8 * BPU;
  static constexpr int kDwords = kBytes / 4;
  static constexpr int kValues = 16 * BPU;
  static constexpr int kGroups = kValues / 8;           // 8-value groups
  static constexpr int kDwordsPerGroup = FMT == 8 ? 2 : 1;
};

// LDS layout of staged activations, per unit: fp32 values + 4 pad, or bf16 + 8 pad.
template <bool XB, int UVALS>
struct XLayout {
  static constexpr int kStrideDw = XB ? (UVALS / 2 + 4) : (UVALS + 4);   // dwords per unit
  static constexpr double kBytesPerValue = 4.0 * kStrideDw / UVALS;
};

template <int NDW> struct DwordVec;
template <> struct DwordVec<2> { using T = u32x2; };
template <> struct DwordVec<4> { using T = u32x4; };

template <int FMT, int BPU>
__device__ __forceinline__ typename DwordVec<Unit<FMT, BPU>::kDwords>::T
load_unit(const uint8_t* code, int64_t row, int k, int unit) {
  using T = typename DwordVec<Unit<FMT, BPU>::kDwords>::T;
  const int64_t row_bytes = (FMT == 8) ? (int64_t)k : (int64_t)k / 2;
  return __builtin_nontemporal_load(reinterpret_cast<const T*>(code + row * row_bytes) + unit);
}

// exponent bytes of the BPU blocks of a unit, packed into one integer
template <int BPU>
__device__ __forceinline__ uint32_t load_exps(const uint8_t* exp, int64_t row, int nbk, int unit) {
  const uint8_t* p = exp + row * nbk + (int64_t)unit * BPU;
  if constexpr (BPU == 2) return *reinterpret_cast<const uint16_t*>(p);
  else return *p;
}

// Stage x[:, kc0:kc0+kcn) into LDS (rows >= m are zero).
// Activation row of slot mi: xrow[mi] when a row list is given (gathered rows), else mi.
template <int FMT, int MB, bool XB, int UVALS, int kThreads>
__device__ __forceinline__ void stage_x(uint32_t* xs, const void* x, int64_t ldx, int m, int kc0, int kcn,
                                        const int* xrow) {
  using L = XLayout<XB, UVALS>;
  const int nuc = kcn / UVALS;
  if constexpr (XB) {
    // 8 bf16 per thread step, permuted into the unpack's pair order:
    // BFP4 8-groups (0,2)(4,6)(1,3)(5,7); BFP8 4-groups (0,2)(1,3)
    const int per_row = kcn / 8;
    for (int idx = threadIdx.x; idx < MB * per_row; idx += kThreads) {
      const int mi = idx / per_row, c8 = idx % per_row;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (mi < m)
        v = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + (int64_t)(xrow ? xrow[mi] : mi) * ldx +
                                            kc0 + c8 * 8);
      uint4 o;
      if constexpr (FMT == 4) {
        o.x = __builtin_amdgcn_perm(v.y, v.x, 0x05040100u);   // (x0, x2)
        o.y = __builtin_amdgcn_perm(v.w, v.z, 0x05040100u);   // (x4, x6)
        o.z = __builtin_amdgcn_perm(v.y, v.x, 0x07060302u);   // (x1, x3)
        o.w = __builtin_amdgcn_perm(v.w, v.z, 0x07060302u);   // (x5, x7)
      } else {
        o.x = __builtin_amdgcn_perm(v.y, v.x, 0x05040100u);   // (x0, x2)
        o.y = __builtin_amdgcn_perm(v.y, v.x, 0x07060302u);   // (x1, x3)
        o.z = __builtin_amdgcn_perm(v.w, v.z, 0x05040100u);   // (x4, x6)
        o.w = __builtin_amdgcn_perm(v.w, v.z, 0x07060302u);   // (x5, x7)
      }
      const int kk = c8 * 8;
      uint32_t* dst = xs + ((size_t)mi * nuc + kk / UVALS) * L::kStrideDw + (kk % UVALS) / 2;
      *reinterpret_cast<uint4*>(dst) = o;
    }
  } else {
    const int per_row = kcn / 4;
    for (int idx = threadIdx.x; idx < MB * per_row; idx += kThreads) {
      const int mi = idx / per_row, c4 = idx % per_row;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (mi < m)
        v = *reinterpret_cast<const uint4*>(static_cast<const float*>(x) + (int64_t)(xrow ? xrow[mi] : mi) * ldx +
                                            kc0 + c4 * 4);
      const int kk = c4 * 4;
      *reinterpret_cast<uint4*>(xs + ((size_t)mi * nuc + kk / UVALS) * L::kStrideDw + (kk % UVALS)) = v;
    }
  }
}

// Registers of one group of U units per lane: the codes and exponent bytes of U units of
// each of the lane group's NMAT x RT rows.
template <int FMT, int BPU, int U, int NMAT, int RT>
struct Group {
  using VecT = typename DwordVec<Unit<FMT, BPU>::kDwords>::T;
  VecT c[U][NMAT][RT];
  uint32_t e[U][NMAT][RT];
  int uc[U];
  bool uok[U];
};

// Issue every load of a group (units it + u*LPR + p, clamped into the chunk; a clamped unit
// is marked invalid and contributes nothing).
template <int FMT, int BPU, int U, int NMAT, int RT, int LPR>
__device__ __forceinline__ void load_group(Group<FMT, BPU, U, NMAT, RT>& g, const uint8_t* const* codem,
                                           const uint8_t* const* expm, const int64_t* rowc, int k, int nbk,
                                           int ub0, int it, int p, int nuc) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int uu = it + u * LPR + p;
    g.uok[u] = uu < nuc;
    g.uc[u] = g.uok[u] ? uu : nuc - 1;
#pragma unroll
    for (int t = 0; t < NMAT; ++t)
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        g.c[u][t][r] = load_unit<FMT, BPU>(codem[t], rowc[r], k, ub0 + g.uc[u]);
        g.e[u][t][r] = load_exps<BPU>(expm[t], rowc[r], nbk, ub0 + g.uc[u]);
      }
  }
}

// Unpack a loaded group and multiply it against the staged activations.
template <int FMT, int MB, int BPU, int U, int NMAT, int RT, bool XB>
__device__ __forceinline__ void compute_group(float (&acc)[NMAT][RT][MB], const Group<FMT, BPU, U, NMAT, RT>& g,
                                              const bool* rowok, const uint32_t* xs, int nuc) {
  using UT = Unit<FMT, BPU>;
  using L = XLayout<XB, UT::kValues>;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    float part[BPU][NMAT][RT][MB];
#pragma unroll
    for (int j = 0; j < BPU; ++j)
#pragma unroll
      for (int t = 0; t < NMAT; ++t)
#pragma unroll
        for (int r = 0; r < RT; ++r)
#pragma unroll
          for (int i = 0; i < MB; ++i) part[j][t][r][i] = 0.f;
    const uint32_t* xu = xs + (size_t)g.uc[u] * L::kStrideDw;
#pragma unroll
    for (int gg = 0; gg < UT::kGroups; ++gg) {
      constexpr int DPG = UT::kDwordsPerGroup;
      const int blk = gg / 2;
      if constexpr (XB) {
        uint32_t wp[NMAT][RT][4];
#pragma unroll
        for (int t = 0; t < NMAT; ++t)
#pragma unroll
          for (int r = 0; r < RT; ++r) {
            if constexpr (FMT == 4) {
              unpack8_bfp4_bf16(g.c[u][t][r][gg], wp[t][r]);
            } else {
              unpack4_bfp8_bf16(g.c[u][t][r][DPG * gg], wp[t][r]);
              unpack4_bfp8_bf16(g.c[u][t][r][DPG * gg + 1], wp[t][r] + 2);
            }
          }
#pragma unroll
        for (int i = 0; i < MB; ++i) {
          const u32x4 xp = *reinterpret_cast<const u32x4*>(xu + (size_t)i * nuc * L::kStrideDw + gg * 4);
#pragma unroll
          for (int t = 0; t < NMAT; ++t)
#pragma unroll
            for (int r = 0; r < RT; ++r) {
              float s = part[blk][t][r][i];
              s = dot2_bf16(wp[t][r][0], xp.x, s);
              s = dot2_bf16(wp[t][r][1], xp.y, s);
              s = dot2_bf16(wp[t][r][2], xp.z, s);
              s = dot2_bf16(wp[t][r][3], xp.w, s);
              part[blk][t][r][i] = s;
            }
        }
      } else {
        float w[NMAT][RT][8];
#pragma unroll
        for (int t = 0; t < NMAT; ++t)
#pragma unroll
          for (int r = 0; r < RT; ++r) {
            if constexpr (FMT == 4) {
              unpack8_bfp4(g.c[u][t][r][gg], w[t][r]);
            } else {
              unpack4_bfp8(g.c[u][t][r][DPG * gg], w[t][r]);
              unpack4_bfp8(g.c[u][t][r][DPG * gg + 1], w[t][r] + 4);
            }
          }
#pragma unroll
        for (int i = 0; i < MB; ++i) {
          const float* xr = reinterpret_cast<const float*>(xu + (size_t)i * nuc * L::kStrideDw) + gg * 8;
          const f32x4 xa = *reinterpret_cast<const f32x4*>(xr);
          const f32x4 xb = *reinterpret_cast<const f32x4*>(xr + 4);
          const float xv[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
#pragma unroll
          for (int t = 0; t < NMAT; ++t)
#pragma unroll
            for (int r = 0; r < RT; ++r) {
              float s = part[blk][t][r][i];
#pragma unroll
              for (int v = 0; v < 8; ++v) s = __builtin_fmaf(xv[v], w[t][r][v], s);
              part[blk][t][r][i] = s;
            }
        }
      }
    }
#pragma unroll
    for (int j = 0; j < BPU; ++j)
#pragma unroll
      for (int t = 0; t < NMAT; ++t)
#pragma unroll
        for (int r = 0; r < RT; ++r) {
          const int sh = (g.uok[u] && rowok[r]) ? block_shift<FMT>((g.e[u][t][r] >> (8 * j)) & 0xffu) : kShiftToZero;
#pragma unroll
          for (int i = 0; i < MB; ++i) acc[t][r][i] += apply_shift(part[j][t][r][i], sh);
        }
  }
}

// One kernel per (format, activation rows MB, rows per lane group RT, lanes per row LPR,
// matrices NMAT, units per group U, blocks per unit BPU, bf16 activations XB, threads per
// workgroup). When a chunk holds more than one group per lane, the next group's loads are
// issued before the current group's arithmetic (two register buffers).
//
// gemv_tile computes the rows [row_base, row_base + rows per workgroup) of one matrix view for
// a.m activation rows; xrow/yrow (in LDS, or null for the identity) map activation slot i to
// the row of x it reads and the row of y it writes. With AM (argmax mode, one matrix) nothing is
// written to y: the workgroup stores, per activation row, the key of its largest output
// (argmax.hpp) in a.cand[i][blockIdx.x].
template <int FMT, int MB, int RT, int LPR, int NMAT, int U, int BPU, bool XB, int kThreads, bool AM = false>
__device__ __forceinline__ void gemv_tile(const GemvArgs& a, int row_base, const int* xrow, const int* yrow,
                                          uint32_t* xs) {
  using UT = Unit<FMT, BPU>;
  using GroupT = Group<FMT, BPU, U, NMAT, RT>;
  constexpr int G = kWave / LPR;           // lane groups per wave
  constexpr int C = NMAT * RT * MB;        // partial sums per lane
  using Red = LaneReduce<C, NMAT, LPR>;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int grp = lane / LPR;
  const int p = lane % LPR;
  const int row0 = row_base + (wave * G + grp) * RT;

  const uint8_t* expm[2] = {a.exp0, a.exp1};
  const uint8_t* codem[2] = {a.code0, a.code1};
  const int nbk = a.k / kBlock;

  int64_t rowc[RT];
  bool rowok[RT];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    rowok[r] = row0 + r < a.n;
    rowc[r] = rowok[r] ? row0 + r : a.n - 1;
  }

  float acc[NMAT][RT][MB];
#pragma unroll
  for (int t = 0; t < NMAT; ++t)
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int i = 0; i < MB; ++i) acc[t][r][i] = 0.f;

  for (int kc0 = 0; kc0 < a.k; kc0 += a.kc) {
    const int kcn = min(a.kc, a.k - kc0);
    const int nuc = kcn / UT::kValues;     // units in this chunk
    const int ub0 = kc0 / UT::kValues;
    constexpr int STEP = U * LPR;
    const int ng = (nuc + STEP - 1) / STEP;
    GroupT ga;
    // the first weights are in flight while the activations are staged
    load_group<FMT, BPU, U, NMAT, RT, LPR>(ga, codem, expm, rowc, a.k, nbk, ub0, 0, p, nuc);
    __syncthreads();
    stage_x<FMT, MB, XB, UT::kValues, kThreads>(xs, a.x, a.ldx, a.m, kc0, kcn, xrow);
    __syncthreads();
    {
      GroupT gb;
      for (int gi = 0; gi < ng; gi += 2) {
        if (gi + 1 < ng)
          load_group<FMT, BPU, U, NMAT, RT, LPR>(gb, codem, expm, rowc, a.k, nbk, ub0, (gi + 1) * STEP, p, nuc);
        compute_group<FMT, MB, BPU, U, NMAT, RT, XB>(acc, ga, rowok, xs, nuc);
        if (gi + 1 < ng) {
          if (gi + 2 < ng)
            load_group<FMT, BPU, U, NMAT, RT, LPR>(ga, codem, expm, rowc, a.k, nbk, ub0, (gi + 2) * STEP, p, nuc);
          compute_group<FMT, MB, BPU, U, NMAT, RT, XB>(acc, gb, rowok, xs, nuc);
        }
      }
    }
  }

  // ---- reduce over the lane group; value index = ((r * MB) + i) * NMAT + t ----
  float v[C];
#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int t = 0; t < NMAT; ++t) v[(r * MB + i) * NMAT + t] = acc[t][r][i];
  Red::run(v, lane);
  if constexpr (AM) {
    static_assert(NMAT == 1, "argmax of one matrix");
    constexpr int RPW = (kThreads / kWave) * G * RT;    // weight rows per workgroup
    __shared__ uint64_t keys[MB][RPW];
    if (Red::writer(p)) {
      const int first = Red::first_index(p);
#pragma unroll
      for (int q = 0; q < Red::kCount; ++q) {
        const int r = (first + q) / MB, i = (first + q) % MB;
        const int row = row0 + r;
        keys[i][row - row_base] = (row < a.n && i < a.m) ? am::key_of(v[q], row) : am::kNone;
      }
    }
    __syncthreads();
    for (int i = wave; i < MB; i += kThreads / kWave) {
      uint64_t k = am::kNone;
      for (int j = lane; j < RPW; j += kWave) k = am::kmax(k, keys[i][j]);
      k = am::lane_max<kWave>(k);
      if (lane == 0 && i < a.m) a.cand[(int64_t)i * gridDim.x + blockIdx.x] = k;
    }
    return;
  }
  if (!Red::writer(p)) return;
  const int first = Red::first_index(p);
#pragma unroll
  for (int q = 0; q < Red::kCount; q += NMAT) {
    const int idx = (first + q) / NMAT;
    const int r = idx / MB, i = idx % MB;
    const int row = row0 + r;
    if (row >= a.n || i >= a.m) continue;
    float out = v[q];
    if constexpr (NMAT == 2) {
      const float g = v[q], u = v[q + 1];
      out = g / (1.0f + __expf(-g)) * u;
    }
    const int64_t yo = (int64_t)(yrow ? yrow[i] : i) * a.ldy + row;
    if (a.y_bf16)
      static_cast<uint16_t*>(a.y)[yo] = (uint16_t)f32_to_bf16_rne(out);
    else
      static_cast<float*>(a.y)[yo] = out;
  }
}

template <int FMT, int MB, int RT, int LPR, int NMAT, int U, int BPU, bool XB, int kThreads, bool AM = false>
__global__ __launch_bounds__(kThreads) void gemv_kernel(GemvArgs a) {
  extern __shared__ uint32_t xs[];
  constexpr int rows_per_wg = (kThreads / kWave) * (kWave / LPR) * RT;
  gemv_tile<FMT, MB, RT, LPR, NMAT, U, BPU, XB, kThreads, AM>(a, blockIdx.x * rows_per_wg, nullptr, nullptr, xs);
}

// ---- launch selection (host) --------------------------------------------------------------

// Lanes per row, from K alone: 32 when every lane then streams at least 8 units of a row
// (long rows), else 16.
inline int pick_lpr(int units) { return units >= 32 * 8 ? 32 : 16; }

constexpr int kLdsBudget = 80 * 1024;     // bytes of LDS for staged activations per workgroup

// K values per LDS chunk: all of K if MB rows fit the budget, else the largest multiple of one
// unit per lane that fits (at least one such step: at most 32 x 32 values x 4.5 B x 32 rows
// = 144 KB, inside the 160 KB of LDS a workgroup may use on gfx950). Chunks that are whole
// steps keep every lane on the same units of K whatever the chunk size.
inline int pick_kc(int k, int mb, int uvals, int lpr, double bytes_per_value) {
  const int kc = (int)(kLdsBudget / (bytes_per_value * mb));
  if (kc >= k) return k;
  const int step = uvals * lpr;
  return kc >= step ? kc / step * step : step;
}

// Threads per workgroup: 1024 when the staged activations take more than 40 KB of LDS (so
// two workgroups still give 32 waves per CU), else 256.
template <int FMT, int MB, int LPR, int NMAT, int BPU, bool XB, int T>
hipError_t launch_th(const GemvArgs& a, size_t lds, hipStream_t s) {
  constexpr int RT = 1;
  constexpr int U = MB <= 4 ? 2 : 1;
  constexpr int rows_per_wg = (T / kWave) * (kWave / LPR) * RT;
  static_assert(rows_per_wg >= kVectorMinRowsPerWg, "argmax workspace bound");
  const int grid = (a.n + rows_per_wg - 1) / rows_per_wg;
  if constexpr (NMAT == 1 && XB) {
    if (a.cand != nullptr) {
      hipLaunchKernelGGL((gemv_kernel<FMT, MB, RT, LPR, NMAT, U, BPU, XB, T, true>), dim3(grid), dim3(T), lds, s, a);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      return am::launch_rows<false>(a.cand, nullptr, 0, grid, a.m, a.am_idx, a.am_val, s);
    }
  }
  hipLaunchKernelGGL((gemv_kernel<FMT, MB, RT, LPR, NMAT, U, BPU, XB, T>), dim3(grid), dim3(T), lds, s, a);
  return hipGetLastError();
}

template <int FMT, int MB, int LPR, int NMAT, int BPU, bool XB>
hipError_t launch_t(GemvArgs a, hipStream_t s) {
  using UT = Unit<FMT, BPU>;
  using L = XLayout<XB, UT::kValues>;
  a.kc = pick_kc(a.k, MB, UT::kValues, LPR, L::kBytesPerValue);
  const size_t lds = (size_t)MB * (a.kc / UT::kValues) * L::kStrideDw * sizeof(uint32_t);
  if constexpr (LPR == 32) {
    if (lds > 40 * 1024) return launch_th<FMT, MB, LPR, NMAT, BPU, XB, 1024>(a, lds, s);
  }
  return launch_th<FMT, MB, LPR, NMAT, BPU, XB, 256>(a, lds, s);
}

template <int FMT, int MB, int NMAT, int BPU, bool XB>
hipError_t launch_lpr(const GemvArgs& a, hipStream_t s) {
  const int units = a.k / Unit<FMT, BPU>::kValues;
  if constexpr (BPU == 2 || FMT == 8) {
    if (pick_lpr(units) == 32) return launch_t<FMT, MB, 32, NMAT, BPU, XB>(a, s);
  }
  return launch_t<FMT, MB, 16, NMAT, BPU, XB>(a, s);
}

template <int FMT, int MB, int NMAT, bool XB>
hipError_t launch_bpu(const GemvArgs& a, hipStream_t s) {
  if constexpr (FMT == 4) {
    const bool pairs = (a.k % 32) == 0 &&
                       ((reinterpret_cast<uintptr_t>(a.exp0) | reinterpret_cast<uintptr_t>(a.exp1)) & 1) == 0;
    if (pairs) return launch_lpr<FMT, MB, NMAT, 2, XB>(a, s);
  }
  return launch_lpr<FMT, MB, NMAT, 1, XB>(a, s);
}

// Entry for one (format, matrices, activation type): picks the row bucket MB >= m.
template <int FMT, int NMAT, bool XB>
hipError_t launch_gemv(const GemvArgs& a, hipStream_t s) {
  if (a.m <= 1) return launch_bpu<FMT, 1, NMAT, XB>(a, s);
  if (a.m <= 2) return launch_bpu<FMT, 2, NMAT, XB>(a, s);
  if (a.m <= 4) return launch_bpu<FMT, 4, NMAT, XB>(a, s);
  if (a.m <= 8) return launch_bpu<FMT, 8, NMAT, XB>(a, s);
  if (a.m <= 16) return launch_bpu<FMT, 16, NMAT, XB>(a, s);
  return launch_bpu<FMT, 32, NMAT, XB>(a, s);
}

}  // namespace gemv_detail
}  // namespace bfp
