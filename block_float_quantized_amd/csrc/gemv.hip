// Skinny BFP4/BFP8 matmul (decode GEMV, 1..32 activation rows) for gfx950.
//
// What it computes ("Qwen3.8-27B — TT-native mixed BFP4/BFP8 (GPTQ)", sections "What
// changed in this release (s27v6-20261024)" and "Multi-user decode": up to 32 rows share one
// pass over every weight): y[i][j] = sum_k x[i][k] * W[j][k], W stored as BFP blocks along K,
// optionally followed by SwiGLU with a second matrix (h = silu(x Wg^T) * (x Wu^T)).
//
// Design (HBM-bound at M = 1, VALU-bound for larger M on this design):
//  * A lane group of LPR lanes (16 or 64) owns RT weight rows. Lane p of the group owns the
//    K-blocks p, p + LPR, p + 2*LPR, ...: a wave-wide load then covers LPR consecutive blocks
//    of a row, i.e. contiguous code bytes (8 B/lane for BFP4, 16 B/lane for BFP8).
//  * Activations are staged once per workgroup in LDS as fp32, padded to 20 floats per
//    16-value block so that lanes reading consecutive blocks hit distinct banks.
//  * Codes are unpacked in registers to exact fp32 integers (see bfp_device.hpp); each block's
//    partial dot product is scaled once by its power-of-two block scale.
//  * Partial sums are reduced across the lane group by recursive halving with DPP row moves
//    and v_permlane16/32_swap; one lane per value writes y (with the SwiGLU epilogue).
#include "bfp_device.hpp"
#include "bfp_internal.hpp"

namespace bfp {

namespace {

constexpr int kThreads = 256;
constexpr int kXPad = 20;                  // floats per 16-value block in LDS

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
  int x_bf16, y_bf16;
  int kc;                                  // K values staged per LDS chunk (multiple of 16)
};

template <int FMT>
struct CodeVec;
template <> struct CodeVec<4> { using T = u32x2; };
template <> struct CodeVec<8> { using T = u32x4; };

template <int FMT>
__device__ __forceinline__ typename CodeVec<FMT>::T load_codes(const uint8_t* code, int64_t row, int k, int b) {
  using T = typename CodeVec<FMT>::T;
  const int64_t row_bytes = (FMT == 8) ? (int64_t)k : (int64_t)k / 2;
  return __builtin_nontemporal_load(reinterpret_cast<const T*>(code + row * row_bytes) + b);
}

template <int FMT, int MB, int RT, int LPR, int NMAT>
__global__ __launch_bounds__(kThreads) void gemv_kernel(GemvArgs a) {
  extern __shared__ float xs[];            // [MB][kc/16][kXPad]
  constexpr int G = kWave / LPR;           // lane groups per wave
  constexpr int C = NMAT * RT * MB;        // partial sums per lane
  using Red = LaneReduce<C, NMAT, LPR>;
  using CodeT = typename CodeVec<FMT>::T;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int grp = lane / LPR;
  const int p = lane % LPR;
  const int rows_per_wg = (kThreads / kWave) * G * RT;
  const int row0 = blockIdx.x * rows_per_wg + (wave * G + grp) * RT;

  const uint8_t* expm[2] = {a.exp0, a.exp1};
  const uint8_t* codem[2] = {a.code0, a.code1};
  const int nbk = a.k / kBlock;            // blocks per row

  float acc[NMAT][RT][MB];
#pragma unroll
  for (int t = 0; t < NMAT; ++t)
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int i = 0; i < MB; ++i) acc[t][r][i] = 0.f;

  for (int kc0 = 0; kc0 < a.k; kc0 += a.kc) {
    const int kcn = min(a.kc, a.k - kc0);
    const int nbc = kcn / kBlock;
    __syncthreads();
    // ---- stage x[:, kc0:kc0+kcn) as fp32 into LDS (rows >= m are zero) ----
    if (a.x_bf16) {
      const int per_row = kcn / 8;                       // 8 bf16 (16 B) per thread step
      for (int idx = threadIdx.x; idx < MB * per_row; idx += kThreads) {
        const int mi = idx / per_row, c8 = idx % per_row;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (mi < a.m)
          v = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.x) + mi * a.ldx + kc0 + c8 * 8);
        const int kk = c8 * 8;
        float* dst = xs + ((size_t)mi * nbc + kk / kBlock) * kXPad + (kk % kBlock);
        *reinterpret_cast<f32x4*>(dst) = f32x4{bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y)};
        *reinterpret_cast<f32x4*>(dst + 4) = f32x4{bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w)};
      }
    } else {
      const int per_row = kcn / 4;
      for (int idx = threadIdx.x; idx < MB * per_row; idx += kThreads) {
        const int mi = idx / per_row, c4 = idx % per_row;
        f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
        if (mi < a.m)
          v = *reinterpret_cast<const f32x4*>(static_cast<const float*>(a.x) + mi * a.ldx + kc0 + c4 * 4);
        const int kk = c4 * 4;
        *reinterpret_cast<f32x4*>(xs + ((size_t)mi * nbc + kk / kBlock) * kXPad + (kk % kBlock)) = v;
      }
    }
    __syncthreads();

    // ---- stream this chunk's blocks of the lane group's rows ----
    const int b0 = kc0 / kBlock;
    for (int jb = p; jb < nbc; jb += LPR) {
      CodeT c[NMAT][RT];
      float sc[NMAT][RT];
#pragma unroll
      for (int t = 0; t < NMAT; ++t)
#pragma unroll
        for (int r = 0; r < RT; ++r) {
          const int row = row0 + r;
          if (row < a.n) {
            c[t][r] = load_codes<FMT>(codem[t], row, a.k, b0 + jb);
            sc[t][r] = block_scale<FMT>(expm[t][(int64_t)row * nbk + b0 + jb]);
          } else {
            c[t][r] = CodeT{};
            sc[t][r] = 0.f;
          }
        }
      float part[NMAT][RT][MB];
#pragma unroll
      for (int t = 0; t < NMAT; ++t)
#pragma unroll
        for (int r = 0; r < RT; ++r)
#pragma unroll
          for (int i = 0; i < MB; ++i) part[t][r][i] = 0.f;

      const float* xb = xs + (size_t)jb * kXPad;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        // 8 values of the block per half: unpack them for every (matrix, row)
        float w[NMAT][RT][8];
#pragma unroll
        for (int t = 0; t < NMAT; ++t)
#pragma unroll
          for (int r = 0; r < RT; ++r) {
            if constexpr (FMT == 4) {
              unpack8_bfp4(half == 0 ? c[t][r].x : c[t][r].y, w[t][r]);
            } else {
              unpack4_bfp8(half == 0 ? c[t][r].x : c[t][r].z, w[t][r]);
              unpack4_bfp8(half == 0 ? c[t][r].y : c[t][r].w, w[t][r] + 4);
            }
          }
#pragma unroll
        for (int i = 0; i < MB; ++i) {
          const float* xr = xb + (size_t)i * nbc * kXPad + half * 8;
          const f32x4 xa = *reinterpret_cast<const f32x4*>(xr);
          const f32x4 xc = *reinterpret_cast<const f32x4*>(xr + 4);
#pragma unroll
          for (int t = 0; t < NMAT; ++t)
#pragma unroll
            for (int r = 0; r < RT; ++r) {
              float s = part[t][r][i];
              s = __builtin_fmaf(xa.x, w[t][r][0], s);
              s = __builtin_fmaf(xa.y, w[t][r][1], s);
              s = __builtin_fmaf(xa.z, w[t][r][2], s);
              s = __builtin_fmaf(xa.w, w[t][r][3], s);
              s = __builtin_fmaf(xc.x, w[t][r][4], s);
              s = __builtin_fmaf(xc.y, w[t][r][5], s);
              s = __builtin_fmaf(xc.z, w[t][r][6], s);
              s = __builtin_fmaf(xc.w, w[t][r][7], s);
              part[t][r][i] = s;
            }
        }
      }
#pragma unroll
      for (int t = 0; t < NMAT; ++t)
#pragma unroll
        for (int r = 0; r < RT; ++r)
#pragma unroll
          for (int i = 0; i < MB; ++i) acc[t][r][i] = __builtin_fmaf(part[t][r][i], sc[t][r], acc[t][r][i]);
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
    if (a.y_bf16)
      static_cast<uint16_t*>(a.y)[(int64_t)i * a.ldy + row] = (uint16_t)f32_to_bf16_rne(out);
    else
      static_cast<float*>(a.y)[(int64_t)i * a.ldy + row] = out;
  }
}

template <int FMT, int MB, int LPR, int NMAT>
hipError_t launch_t(const GemvArgs& a, hipStream_t s) {
  constexpr int RT = MB <= 2 ? 2 : (MB <= 4 ? 2 : 1);
  constexpr int rows_per_wg = (kThreads / kWave) * (kWave / LPR) * RT;
  const int grid = (a.n + rows_per_wg - 1) / rows_per_wg;
  const size_t lds = (size_t)MB * (a.kc / kBlock) * kXPad * sizeof(float);
  hipLaunchKernelGGL((gemv_kernel<FMT, MB, RT, LPR, NMAT>), dim3(grid), dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

template <int FMT, int MB, int NMAT>
hipError_t launch_lpr(const GemvArgs& a, hipStream_t s) {
  if (a.k >= 64 * kBlock) return launch_t<FMT, MB, 64, NMAT>(a, s);
  return launch_t<FMT, MB, 16, NMAT>(a, s);
}

template <int FMT, int NMAT>
hipError_t launch_mb(const GemvArgs& a, hipStream_t s) {
  if (a.m <= 1) return launch_lpr<FMT, 1, NMAT>(a, s);
  if (a.m <= 2) return launch_lpr<FMT, 2, NMAT>(a, s);
  if (a.m <= 4) return launch_lpr<FMT, 4, NMAT>(a, s);
  if (a.m <= 8) return launch_lpr<FMT, 8, NMAT>(a, s);
  if (a.m <= 16) return launch_lpr<FMT, 16, NMAT>(a, s);
  return launch_lpr<FMT, 32, NMAT>(a, s);
}

// Largest K chunk (multiple of 1024, or all of K) whose fp32 copy of MB rows fits the budget.
int pick_kc(int k, int mb) {
  const int budget = 64 * 1024;            // bytes of LDS for staged activations
  const int per_value = mb * kXPad * 4 / kBlock;
  int kc = budget / per_value;
  if (kc >= k) return k;
  kc = (kc / 1024) * 1024;
  return kc < 1024 ? 1024 : kc;
}

}  // namespace

hipError_t gemv_launch(const GemvParams& g, hipStream_t s) {
  GemvArgs a;
  a.exp0 = g.w_exp; a.code0 = g.w_code;
  a.exp1 = g.u_exp; a.code1 = g.u_code;
  a.x = g.x; a.ldx = g.ldx; a.y = g.y; a.ldy = g.ldy;
  a.n = (int)g.n; a.k = (int)g.k; a.m = (int)g.m;
  a.x_bf16 = g.x_bf16; a.y_bf16 = g.y_bf16;
  const int mb = g.m <= 1 ? 1 : g.m <= 2 ? 2 : g.m <= 4 ? 4 : g.m <= 8 ? 8 : g.m <= 16 ? 16 : 32;
  a.kc = pick_kc(a.k, mb);
  const bool swiglu = g.u_code != nullptr;
  if (g.fmt == 4) return swiglu ? launch_mb<4, 2>(a, s) : launch_mb<4, 1>(a, s);
  return swiglu ? launch_mb<8, 2>(a, s) : launch_mb<8, 1>(a, s);
}

}  // namespace bfp
