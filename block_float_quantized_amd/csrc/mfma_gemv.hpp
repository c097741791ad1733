#pragma once
// Skinny BFP4/BFP8 matmul on the bf16 matrix cores (gfx950 v_mfma_f32_16x16x32_bf16), for 1 to
// 32 activation rows.
//
// What it computes ("Qwen3.8-27B — TT-native mixed BFP4/BFP8 (GPTQ)", sections "What changed
// in this release (s27v6-20261024)" and "Multi-user decode": up to 32 rows share one pass over
// every weight): y[i][j] = sum_k x[i][k] * W[j][k], W stored as BFP blocks along K, optionally
// followed by SwiGLU with a second matrix (h = silu(x Wg^T) * (x Wu^T)).
//
// Design:
//  * K is cut into steps of SK = 128 G values (G from the format alone) and the steps into
//    KS slices (KS from N and K alone). Workgroup (c, s) owns 128 output columns (16 per wave,
//    of each matrix) over slice s: its eight waves walk the same K positions in lockstep, so
//    the activations staged in LDS for them are one short window shared by all eight (wider
//    workgroups stage each activation row for more columns).
//  * In a step, lane l takes weight row l % 16 and the SK / 4 consecutive values starting at
//    (l / 16) SK / 4: G 16-byte loads (BFP4) or 2G (BFP8) plus one load of its 2G exponent
//    bytes. Every weight byte is loaded once, straight into registers, one step ahead of use.
//  * The values a lane holds feed 4G MFMAs (8 values each); the activation fragment of each
//    MFMA comes from LDS at the same K positions, staged per workgroup in the permuted bf16
//    pair order the weight unpack produces. fp32 activations are staged as two bf16 planes
//    hi + lo (hi = bf16(x), lo = bf16(x - hi)) and take two MFMAs, keeping about 16
//    significant bits of x; the products themselves are exact and sums are fp32.
//  * Dequantisation to bf16 is exact: BFP4 through the scaled FP8 conversion (a nibble is an
//    E4M3 subnormal, the block scale is the conversion's scale), BFP8 through integer
//    conversion and a power-of-two multiply. Steps whose block exponents fall outside the
//    scaled conversion's exact range take an fp32 path, decided once per wave and step.
//  * Rows >= m read a valid staged row: an MFMA output row depends only on its own input row,
//    so those rows are computed and dropped.
//  * With one slice the epilogue runs in registers; with several, each workgroup writes its
//    fp32 partial tile to the workspace and a second kernel adds the slices in slice order and
//    applies the epilogue. The slicing and every summation order depend on N and K only, so
//    row i of an m-row call is bit-identical to the same row computed alone.
#include "argmax.hpp"
#include "bfp_device.hpp"
#include "bfp_internal.hpp"

namespace bfp {
namespace mg {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
template <bool B> struct Flag { static constexpr bool value = B; };

constexpr int kWaves = 8;                   // waves per workgroup (columns: 16 per wave)
constexpr int kCols = 16 * kWaves;          // output columns per workgroup
constexpr int kLdsStage = 40 * 1024;        // LDS budget for staged activations

struct MgArgs {
  const uint8_t* exp[2];
  const uint8_t* code[2];
  const void* x;
  int64_t ldx;
  void* y;
  int64_t ldy;
  int n, k, m;
  int y_bf16;
  float* ws;         // slice partials [ks][nmat][m][n] (ks > 1)
  int ks;            // K slices
  int sps;           // steps per slice
  int kc;            // K values staged per chunk (a whole number of steps)
  int exp_vec;       // a lane's exponent bytes may be read with one aligned load
  int whole;         // every step whole, BFP4 rows 16-byte aligned and exp_vec: the loads of a
                     // step take one form, with no branches (see the kernel's steady loop)
  int code16;        // BFP4 rows start on 16-byte boundaries (K a multiple of 32)
  uint64_t* cand;    // argmax mode: workspace (argmax_workspace_bytes), else null
  int32_t* am_idx;   // argmax mode: per activation row, the column of the largest output
  float* am_val;     //   and its value
};

// One step of one matrix as loaded by a wave: 16 weight rows x SK values, read row-contiguously
// (RB code bytes and EB exponent bytes per row). Lane i holds code bytes [16 (i % CPR), +16) of
// row q (64 / CPR) + i / CPR for each load q, CPR = RB / 16 lanes per row, and exponent bytes
// [(i % 4) EB / 4, +EB / 4) of row i / 4.
template <int FMT, int G>
struct StepRegs {
  static constexpr int kRB = (FMT == 8 ? 128 : 64) * G;   // code bytes per row and step
  static constexpr int kEB = 8 * G;                        // exponent bytes per row and step
  static constexpr int kLoads = 16 * kRB / 1024;           // 16-byte loads per lane
  u32x4 c[kLoads];
  uint32_t e[(kEB / 4 + 3) / 4];                           // kEB / 4 bytes per lane
};

// ---- dequantisation to bf16 pairs (8 values -> 4 dwords) -----------------------------------

// BFP8, any exponent: |code| as fp32 times the block scale 2^(E-133) (exact: at most 7
// significant bits, a multiple of 2^-133), sign bit copied, top halves packed. Pair order
// (v0, v2) (v1, v3) (v4, v6) (v5, v7).
__device__ __forceinline__ u32x4 dq8_bfp8(uint32_t c0, uint32_t c1, float sc) {
  u32x4 o;
  const uint32_t cc[2] = {c0, c1};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t c = cc[h];
    const uint32_t a = c & 0x7f7f7f7fu;
    const uint32_t f0 = __float_as_uint((float)(a & 0xffu) * sc);
    const uint32_t f1 = __float_as_uint((float)((a >> 8) & 0xffu) * sc);
    const uint32_t f2 = __float_as_uint((float)((a >> 16) & 0xffu) * sc);
    const uint32_t f3 = __float_as_uint((float)(a >> 24) * sc);
    const uint32_t p02 = __builtin_amdgcn_perm(f2, f0, 0x07060302u) | ((c << 8) & 0x80008000u);
    const uint32_t p13 = __builtin_amdgcn_perm(f3, f1, 0x07060302u) | (c & 0x80008000u);
    if (h == 0) { o.x = p02; o.y = p13; } else { o.z = p02; o.w = p13; }
  }
  return o;
}

// ---- activation staging -----------------------------------------------------------------

__device__ __forceinline__ uint32_t pack_bf16_rne(float lo, float hi) {
  return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

// Stage x[0..m)[kb, kb + kcn) into LDS planes [XS][m][sk] (bf16, permuted pairs); positions at
// or beyond k are zero so that the tail of the last step multiplies zeros.
template <int FMT, int XS>
__device__ __forceinline__ void stage(uint16_t* xs, const MgArgs& a, int kb, int kcn, int sk) {
  const int per_row = kcn / 8;
  const size_t plane = (size_t)a.m * sk;
  for (int idx = threadIdx.x; idx < a.m * per_row; idx += kWaves * 64) {
    const int mi = idx / per_row, c8 = idx % per_row;
    const int kk = kb + c8 * 8;
    if constexpr (XS == 1) {
      uint4 r = make_uint4(0, 0, 0, 0);
      if (kk < a.k) r = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.x) + (int64_t)mi * a.ldx + kk);
      uint4 o;
      if constexpr (FMT == 4) {
        o.x = __builtin_amdgcn_perm(r.y, r.x, 0x05040100u);   // (x0, x2)
        o.y = __builtin_amdgcn_perm(r.w, r.z, 0x05040100u);   // (x4, x6)
        o.z = __builtin_amdgcn_perm(r.y, r.x, 0x07060302u);   // (x1, x3)
        o.w = __builtin_amdgcn_perm(r.w, r.z, 0x07060302u);   // (x5, x7)
      } else {
        o.x = __builtin_amdgcn_perm(r.y, r.x, 0x05040100u);   // (x0, x2)
        o.y = __builtin_amdgcn_perm(r.y, r.x, 0x07060302u);   // (x1, x3)
        o.z = __builtin_amdgcn_perm(r.w, r.z, 0x05040100u);   // (x4, x6)
        o.w = __builtin_amdgcn_perm(r.w, r.z, 0x07060302u);   // (x5, x7)
      }
      *reinterpret_cast<uint4*>(xs + (size_t)mi * sk + c8 * 8) = o;
    } else {
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = 0.f;
      if (kk < a.k) {
        const float* p = static_cast<const float*>(a.x) + (int64_t)mi * a.ldx + kk;
        const f32x4 q0 = *reinterpret_cast<const f32x4*>(p);
        const f32x4 q1 = *reinterpret_cast<const f32x4*>(p + 4);
        v[0] = q0.x; v[1] = q0.y; v[2] = q0.z; v[3] = q0.w;
        v[4] = q1.x; v[5] = q1.y; v[6] = q1.z; v[7] = q1.w;
      }
      float hi[8], lo[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        hi[i] = __uint_as_float(f32_to_bf16_rne(v[i]) << 16);
        const float d = v[i] - hi[i];
        lo[i] = (d == d && __builtin_fabsf(d) != __builtin_inff()) ? d : 0.f;   // non-finite x: all in hi
      }
      constexpr int P4[8] = {0, 2, 4, 6, 1, 3, 5, 7};
      constexpr int P8[8] = {0, 2, 1, 3, 4, 6, 5, 7};
      const int* P = FMT == 4 ? P4 : P8;
      uint4 oh, ol;
      oh.x = pack_bf16_rne(hi[P[0]], hi[P[1]]); ol.x = pack_bf16_rne(lo[P[0]], lo[P[1]]);
      oh.y = pack_bf16_rne(hi[P[2]], hi[P[3]]); ol.y = pack_bf16_rne(lo[P[2]], lo[P[3]]);
      oh.z = pack_bf16_rne(hi[P[4]], hi[P[5]]); ol.z = pack_bf16_rne(lo[P[4]], lo[P[5]]);
      oh.w = pack_bf16_rne(hi[P[6]], hi[P[7]]); ol.w = pack_bf16_rne(lo[P[6]], lo[P[7]]);
      *reinterpret_cast<uint4*>(xs + (size_t)mi * sk + c8 * 8) = oh;
      *reinterpret_cast<uint4*>(xs + plane + (size_t)mi * sk + c8 * 8) = ol;
    }
  }
}

// ---- weights ------------------------------------------------------------------------------

// Load step st (K values [st SK, (st + 1) SK)) of one matrix, rows row0 .. row0 + 15 (clamped
// to n - 1), in the row-contiguous lane order of StepRegs. K is a multiple of 16: in the last
// step a row holds a whole number of 16-value blocks, zeros after.
template <int FMT, int G, bool WHOLE = false>
__device__ __forceinline__ void load_step(StepRegs<FMT, G>& r, const uint8_t* code, const uint8_t* exp,
                                          int row0, const MgArgs& a, int st, int lane) {
  using R = StepRegs<FMT, G>;
  constexpr int SK = 128 * G;
  constexpr int CPR = R::kRB / 16;                 // lanes per row in a code load
  constexpr int RPL = 64 / CPR;                    // rows per code load
  constexpr int EPL = R::kEB / 4;                  // exponent bytes per lane
  const int nbk = a.k / kBlock;
  const int64_t row_bytes = FMT == 8 ? (int64_t)a.k : (int64_t)a.k / 2;
  const int kb0 = st * SK;                          // first K value of the step
  const bool full = WHOLE || kb0 + SK <= a.k;
  // codes
#pragma unroll
  for (int q = 0; q < R::kLoads; ++q) {
    const int rr = q * RPL + lane / CPR;
    const int64_t row = min(row0 + rr, a.n - 1);
    const int cb = (lane % CPR) * 16;              // byte offset inside the row's step
    const uint8_t* cp = code + row * row_bytes + (FMT == 8 ? kb0 : kb0 / 2) + cb;
    const int v0 = kb0 + (FMT == 8 ? cb : 2 * cb);  // first K value of these 16 bytes
    if (full) {
      if (FMT == 8 || WHOLE || a.code16) {
        r.c[q] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(cp));
      } else {
        // BFP4 rows of K/2 bytes with K an odd multiple of 16 are only 8-byte aligned
        const u32x2 lo = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(cp));
        const u32x2 hi = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(cp) + 1);
        r.c[q] = u32x4{lo.x, lo.y, hi.x, hi.y};
      }
    } else {
      // 16 bytes = one BFP8 block or two BFP4 blocks: load the blocks that exist
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      const uint32_t* p = reinterpret_cast<const uint32_t*>(cp);
      if (FMT == 8) {
        if (v0 < a.k) v = u32x4{p[0], p[1], p[2], p[3]};
      } else {
        if (v0 < a.k) { v.x = p[0]; v.y = p[1]; }
        if (v0 + 16 < a.k) { v.z = p[2]; v.w = p[3]; }
      }
      r.c[q] = v;
    }
  }
  // exponents: lane i takes bytes [(i % 4) EPL, +EPL) of row i / 4
  {
    const int64_t row = min(row0 + lane / 4, a.n - 1);
    const int b0 = (lane % 4) * EPL;               // block offset inside the step
    const uint8_t* ep = exp + row * nbk + kb0 / 16 + b0;
    if (WHOLE || (full && a.exp_vec)) {
      if constexpr (EPL == 2) r.e[0] = *reinterpret_cast<const uint16_t*>(ep);
      else if constexpr (EPL == 4) r.e[0] = *reinterpret_cast<const uint32_t*>(ep);
      else {
        const u32x2 v = *reinterpret_cast<const u32x2*>(ep);
        r.e[0] = v.x; r.e[1] = v.y;
      }
    } else {
#pragma unroll
      for (int i = 0; i < (EPL + 3) / 4; ++i) r.e[i] = 0;
#pragma unroll
      for (int b = 0; b < EPL; ++b)
        if (kb0 + 16 * (b0 + b) < a.k) r.e[b / 4] |= (uint32_t)ep[b] << (8 * (b % 4));
    }
  }
}

// ---- the kernel ---------------------------------------------------------------------------

// Codes of one lane in MFMA operand order: LV = SK / 4 consecutive values of one row.
template <int FMT, int G>
struct LaneCodes {
  static constexpr int kBytes = (FMT == 8 ? 32 : 16) * G;
  static constexpr int kDw = kBytes / 4;
};

// Bytes of the staged activations (XS bf16 planes of m rows, kc + 8 values per row).
__host__ __device__ inline size_t stage_bytes(int m, int xs, int kc) {
  return ((size_t)xs * m * (kc + 8) * sizeof(uint16_t) + 15) / 16 * 16;
}

// A wave's LDS area for one matrix and step: 16 rows of codes (stride RB + 16 bytes, which
// spreads the 16 rows of an operand read over all banks) and 16 rows of exponents.
template <int FMT, int G>
struct WaveLds {
  using R = StepRegs<FMT, G>;
  static constexpr int kRS = R::kRB + 16;
  static constexpr int kES = R::kEB + (G == 4 ? 8 : 4);
  static constexpr int kBytes = 16 * kRS + 16 * kES;
  // row-contiguous, as loaded
  static __device__ __forceinline__ void put(uint8_t* w, const R& r, int lane) {
    constexpr int CPR = R::kRB / 16, RPL = 64 / CPR, EPL = R::kEB / 4;
#pragma unroll
    for (int q = 0; q < R::kLoads; ++q)
      *reinterpret_cast<u32x4*>(w + (q * RPL + lane / CPR) * kRS + (lane % CPR) * 16) = r.c[q];
    uint8_t* e = w + 16 * kRS + (lane / 4) * kES + (lane % 4) * EPL;
    if constexpr (EPL == 2) *reinterpret_cast<uint16_t*>(e) = (uint16_t)r.e[0];
    else if constexpr (EPL == 4) *reinterpret_cast<uint32_t*>(e) = r.e[0];
    else *reinterpret_cast<u32x2*>(e) = u32x2{r.e[0], r.e[1]};
  }
  // MFMA operand order: row c, values [g LV, (g + 1) LV) and their 2G exponents
  static __device__ __forceinline__ void get(const uint8_t* w, uint32_t* cw, uint32_t* ew, int c, int g) {
    constexpr int LB = LaneCodes<FMT, G>::kBytes;
#pragma unroll
    for (int q = 0; q < LB / 16; ++q) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(w + c * kRS + g * LB + q * 16);
      cw[4 * q] = v.x; cw[4 * q + 1] = v.y; cw[4 * q + 2] = v.z; cw[4 * q + 3] = v.w;
    }
    const uint8_t* e = w + 16 * kRS + c * kES + g * 2 * G;
    if constexpr (G == 1) ew[0] = *reinterpret_cast<const uint16_t*>(e);
    else if constexpr (G == 2) ew[0] = *reinterpret_cast<const uint32_t*>(e);
    else {
      const u32x2 v = *reinterpret_cast<const u32x2*>(e);
      ew[0] = v.x; ew[1] = v.y;
    }
  }
};

// FMT: 4 or 8. NMAT: 1, or 2 for SwiGLU (same columns of gate and up). MT: 16-row activation
// tiles (1 for m <= 16, 2 for m <= 32). XS: bf16 planes per activation (1 bf16, 2 fp32).
// G: 128-value units per step. AM (argmax mode, one matrix, one slice): nothing is written to
// y; the workgroup stores, per activation row, the key of its largest output (argmax.hpp) in
// a.cand[i][blockIdx.x].
template <int FMT, int NMAT, int MT, int XS, int G, bool AM = false>
__global__ __launch_bounds__(kWaves * 64) void mfma_gemv_kernel(MgArgs a) {
  using R = StepRegs<FMT, G>;
  using W = WaveLds<FMT, G>;
  constexpr int SK = 128 * G, LV = SK / 4;
  extern __shared__ __align__(16) uint16_t lds[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform: scalar row arithmetic
  const int c = lane & 15, g = lane >> 4;
  const int col0 = blockIdx.x * kCols + wave * 16;

  const int nst = (a.k + SK - 1) / SK;            // steps of K
  const int st0 = blockIdx.y * a.sps;
  const int st1 = min(st0 + a.sps, nst);
  const int kbeg = st0 * SK;
  const int spc = a.kc / SK;                      // steps per staged chunk
  const int sk = a.kc + 8;                        // bf16 per staged row (padded)
  int arow[MT];                                   // rows >= m read row m - 1
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) arow[mt] = min(mt * 16 + c, a.m - 1);
  const size_t plane = (size_t)a.m * sk;
  // this wave's weight transposition area, after the staged activations
  uint8_t* wl = reinterpret_cast<uint8_t*>(lds) + stage_bytes(a.m, XS, a.kc) + (size_t)wave * NMAT * W::kBytes;

  f32x4 acc[NMAT][MT];
#pragma unroll
  for (int t = 0; t < NMAT; ++t)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[t][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  constexpr int D = NMAT == 1 ? 2 : 1;            // prefetch distance in steps
  R ra[NMAT], rb[NMAT], rc[NMAT];
  auto load = [&](R (&r)[NMAT], int st, auto whole) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < NMAT; ++t)
      load_step<FMT, G, decltype(whole)::value>(r[t], a.code[t], a.exp[t], col0, a, st, lane);
  };
  auto compute = [&](R (&r)[NMAT], int st, int kb) __attribute__((always_inline)) {
    // through this wave's LDS area: row-contiguous as loaded, read back as MFMA operands
    // (lane l: weight row l % 16, values [(l / 16) LV, +LV) of the step)
    uint32_t cw[NMAT][LaneCodes<FMT, G>::kDw];
    uint32_t ew[NMAT][(2 * G + 3) / 4];
#pragma unroll
    for (int t = 0; t < NMAT; ++t) W::put(wl + t * W::kBytes, r[t], lane);
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int t = 0; t < NMAT; ++t) W::get(wl + t * W::kBytes, cw[t], ew[t], c, g);
    auto exp_of = [&](int t, int b) __attribute__((always_inline)) {
      return (ew[t][b / 4] >> (8 * (b % 4))) & 0xffu;
    };
    // one decision per wave and step: every exponent inside the scaled conversion's range?
    bool fast = true;
    if constexpr (FMT == 4) {
      bool ok = true;
#pragma unroll
      for (int t = 0; t < NMAT; ++t)
#pragma unroll
        for (int b = 0; b < 2 * G; ++b) ok = ok && (exp_of(t, b) - 8u) <= 239u;
      fast = __builtin_amdgcn_ballot_w64(!ok) == 0;
    }
    const int off = st * SK - kb + g * LV;        // lane's first staged position
#pragma unroll
    for (int j = 0; j < 4 * G; ++j) {
      bf16x8 bfr[NMAT];
#pragma unroll
      for (int t = 0; t < NMAT; ++t) {
        const uint32_t e = exp_of(t, j / 2);
        u32x4 d;
        if constexpr (FMT == 4) {
          if (fast) d = dq8_bfp4_fast(cw[t][j], __uint_as_float((e + 7u) << 23));
          else d = dq8_bfp4_any(cw[t][j], e);
        } else {
          d = dq8_bfp8(cw[t][2 * j], cw[t][2 * j + 1], block_scale<8>(e));
        }
        bfr[t] = __builtin_bit_cast(bf16x8, d);
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int xs = 0; xs < XS; ++xs) {
          const bf16x8 af = *reinterpret_cast<const bf16x8*>(lds + xs * plane + (size_t)arow[mt] * sk + off + 8 * j);
#pragma unroll
          for (int t = 0; t < NMAT; ++t)
            acc[t][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bfr[t], acc[t][mt], 0, 0, 0);
        }
    }
  };
  // stage the chunk that step st starts, if it starts one; returns the chunk's first position
  auto chunk_at = [&](int st) __attribute__((always_inline)) {
    const int ci = (st - st0) / spc;
    const int kb = kbeg + ci * a.kc;
    if ((st - st0) % spc == 0) {
      if (st != st0) __syncthreads();
      stage<FMT, XS>(lds, a, kb, min(a.kc, st1 * SK - kb), sk);
      __syncthreads();
    }
    return kb;
  };

  // the first weights are in flight while the activations are staged; loads run D steps
  // ahead of the MFMAs (register sets used in rotation). The steady loop issues every load
  // unconditionally, in one form (whole steps): a load behind a branch, or a step whose loads
  // may take another form, leaves the compiler unable to count the loads in flight, and it
  // then waits for all of them (the prefetch included) before each step. The last steps take
  // the guarded form.
  auto body = [&](R (&cur)[NMAT], R (&nxt)[NMAT], int st, auto whole) __attribute__((always_inline)) {
    const int kb = chunk_at(st);
    if (st + D < st1) load(nxt, st + D, whole);
    compute(cur, st, kb);
  };
  auto body_steady = [&](R (&cur)[NMAT], R (&nxt)[NMAT], int st) __attribute__((always_inline)) {
    const int kb = chunk_at(st);
    load(nxt, st + D, Flag<true>{});
    compute(cur, st, kb);
  };
  auto run = [&](auto whole) __attribute__((always_inline)) {
    constexpr bool WH = decltype(whole)::value;
    int st = st0;
    load(ra, st0, whole);
    if constexpr (D == 1) {
      if constexpr (WH) {
        for (; st + 2 < st1; st += 2) {
          body_steady(ra, rb, st);
          body_steady(rb, ra, st + 1);
        }
      }
      for (; st < st1; st += 2) {
        body(ra, rb, st, whole);
        if (st + 1 < st1) body(rb, ra, st + 1, whole);
      }
    } else {
      if (WH && st0 + 4 < st1) {
        load(rb, st0 + 1, whole);   // unconditional: the loop starts with exactly two steps in flight
        for (; st + 4 < st1; st += 3) {
          body_steady(ra, rc, st);
          body_steady(rb, ra, st + 1);
          body_steady(rc, rb, st + 2);
        }
      } else if (st0 + 1 < st1) {
        load(rb, st0 + 1, whole);
      }
      for (; st < st1; st += 3) {
        body(ra, rc, st, whole);
        if (st + 1 < st1) body(rb, ra, st + 1, whole);
        if (st + 2 < st1) body(rc, rb, st + 2, whole);
      }
    }
  };
  // (slices too short for one pass of the steady loop keep the guarded form throughout: it was
  // faster there, 2-step slices of the QKV / O projections at m = 16)
  if (a.whole && st1 - st0 >= 2 * D + 1) run(Flag<true>{});
  else run(Flag<false>{});

  // element i of a 16x16 output tile: activation row 4 g + i, column c
  auto store = [&](int yr, int yc, const float* v) __attribute__((always_inline)) {
    float out = v[0];
    if constexpr (NMAT == 2) out = out / (1.0f + __expf(-out)) * v[1];
    const int64_t yo = (int64_t)yr * a.ldy + yc;
    if (a.y_bf16) static_cast<uint16_t*>(a.y)[yo] = (uint16_t)f32_to_bf16_rne(out);
    else static_cast<float*>(a.y)[yo] = out;
  };
  if constexpr (AM) {
    static_assert(NMAT == 1, "argmax of one matrix");
    // over the 16 columns of each wave (lanes with equal g), then over the four waves
    __shared__ uint64_t keys[kWaves][MT * 16];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int yc = col0 + c;
        uint64_t k = yc < a.n ? am::key_of(acc[0][mt][i], yc) : am::kNone;
        k = am::lane_max<16>(k);
        if (c == 0) keys[wave][mt * 16 + 4 * g + i] = k;
      }
    __syncthreads();
    if (wave == 0 && lane < MT * 16 && lane < a.m) {
      uint64_t k = keys[0][lane];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) k = am::kmax(k, keys[w][lane]);
      a.cand[(int64_t)lane * gridDim.x + blockIdx.x] = k;
    }
    return;
  }
  if (a.ks == 1) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int yr = mt * 16 + 4 * g + i, yc = col0 + c;
        if (yr >= a.m || yc >= a.n) continue;
        float v[NMAT];
#pragma unroll
        for (int t = 0; t < NMAT; ++t) v[t] = acc[t][mt][i];
        store(yr, yc, v);
      }
    return;
  }
  // several slices: this slice's fp32 tile goes to the workspace; slice_sum_kernel adds the
  // slices in slice order and applies the epilogue
  const int64_t mn = (int64_t)a.m * a.n;
#pragma unroll
  for (int t = 0; t < NMAT; ++t)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int yr = mt * 16 + 4 * g + i, yc = col0 + c;
        if (yr >= a.m || yc >= a.n) continue;
        a.ws[((int64_t)blockIdx.y * NMAT + t) * mn + (int64_t)yr * a.n + yc] = acc[t][mt][i];
      }
}

// y[i][j] = epilogue(sum over slices s = 0, 1, ... of the partials), in slice order. The loads
// of eight slices (of every matrix) are issued before their additions, so that a call costs one
// memory round trip per eight slices instead of one per slice.
template <int NMAT>
__global__ __launch_bounds__(256) void slice_sum_kernel(MgArgs a) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t mn = (int64_t)a.m * a.n;
  if (idx >= mn) return;
  float v[NMAT];
#pragma unroll
  for (int t = 0; t < NMAT; ++t) v[t] = 0.f;
  for (int s0 = 0; s0 < a.ks; s0 += 8) {
    float p[NMAT][8];
#pragma unroll
    for (int t = 0; t < NMAT; ++t)
#pragma unroll
      for (int u = 0; u < 8; ++u) p[t][u] = a.ws[((int64_t)min(s0 + u, a.ks - 1) * NMAT + t) * mn + idx];
#pragma unroll
    for (int t = 0; t < NMAT; ++t)
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (s0 + u < a.ks) v[t] += p[t][u];
  }
  float out = v[0];
  if constexpr (NMAT == 2) out = out / (1.0f + __expf(-out)) * v[1];
  const int64_t yo = idx / a.n * a.ldy + idx % a.n;
  if (a.y_bf16) static_cast<uint16_t*>(a.y)[yo] = (uint16_t)f32_to_bf16_rne(out);
  else static_cast<float*>(a.y)[yo] = out;
}

// ---- launch (host) --------------------------------------------------------------------------

// 128-value units per step, from the format alone.
template <int FMT, int NMAT> constexpr int kG = FMT == 4 ? 2 : 1;

// Slices of K: the count that minimises (rounds of resident workgroups) x (fixed start of a
// workgroup + its steps), plus the slice partials' cost (an eighth of a step per slice, and a
// step for the slice-sum launch itself). Two workgroups stay resident on each compute unit,
// 512 on the 256 of an MI355X (a constant, not the device's count: the slicing, hence every
// summation order, must depend on N and K alone); a workgroup's first operands take about two
// steps' time to arrive. A grid slightly larger than the resident slots costs a whole second
// round for its last few workgroups. Matrices with two rounds of column groups are not sliced.
constexpr int kResidentSlots = 512;
constexpr int kStartSteps = 2;
inline void pick_slices(int n, int k, int sk_values, int& ks, int& sps) {
  const int groups = (n + kCols - 1) / kCols;
  const int nst = (k + sk_values - 1) / sk_values;
  ks = 1;
  sps = nst;
  if (groups >= 2 * kResidentSlots) return;
  long best = -1;
  for (int p = nst; p >= 1; --p) {                 // steps per slice, fewest slices first
    const int s = (nst + p - 1) / p;
    if (s > 64) break;
    const long rounds = ((long)groups * s + kResidentSlots - 1) / kResidentSlots;
    const long cost = 8 * rounds * (kStartSteps + p) + s + (s > 1 ? 8 : 0);   // in eighths of a step
    if (best < 0 || cost < best) {
      best = cost;
      sps = p;
    }
  }
  ks = (nst + sps - 1) / sps;
}

// Workspace: the fp32 slice partials.
template <int FMT, int NMAT>
size_t workspace_bytes(int n, int k, int m) {
  int ks, sps;
  pick_slices(n, k, 128 * kG<FMT, NMAT>, ks, sps);
  return ks > 1 ? (size_t)ks * NMAT * m * n * sizeof(float) : 0;
}

// Argmax mode's workspace: with one slice, the candidate keys [m][workgroups]; with several,
// the fp32 outputs [m][n] (256-byte aligned size) and after them the slice partials.
inline size_t am_outputs_bytes(int n, int m) { return ((size_t)m * n * sizeof(float) + 255) / 256 * 256; }
template <int FMT>
size_t argmax_workspace_bytes(int n, int k, int m) {
  int ks, sps;
  pick_slices(n, k, 128 * kG<FMT, 1>, ks, sps);
  if (ks == 1) return (size_t)m * ((n + kCols - 1) / kCols) * sizeof(uint64_t);
  return am_outputs_bytes(n, m) + workspace_bytes<FMT, 1>(n, k, m);
}

template <int FMT, int NMAT, int MT, int XS>
hipError_t launch_mt(MgArgs a, hipStream_t s) {
  constexpr int G = kG<FMT, NMAT>;
  constexpr int SK = 128 * G;
  pick_slices(a.n, a.k, SK, a.ks, a.sps);
  // a lane's 2G exponent bytes start at a multiple of 2G within the row
  const int nbk = a.k / kBlock;
  const uintptr_t ep = reinterpret_cast<uintptr_t>(a.exp[0]) | reinterpret_cast<uintptr_t>(a.exp[1]);
  a.exp_vec = (nbk % (2 * G)) == 0 && (ep % (2 * G)) == 0;
  a.whole = a.k % SK == 0 && (FMT == 8 || a.code16) && a.exp_vec;
  // activations: the whole slice if it fits, else chunks of whole steps
  const size_t per_k = (size_t)XS * a.m * sizeof(uint16_t);
  const int slice_k = a.sps * SK;
  int steps = (int)((kLdsStage / per_k - 8) / SK);
  if (steps < 1) steps = 1;
  a.kc = steps * SK < slice_k ? steps * SK : slice_k;
  const size_t lds = stage_bytes(a.m, XS, a.kc) + (size_t)kWaves * NMAT * WaveLds<FMT, G>::kBytes;
  const dim3 grid((a.n + kCols - 1) / kCols, a.ks);
  const bool am_mode = a.cand != nullptr;
  if constexpr (NMAT == 1 && XS == 1) {
    if (am_mode && a.ks == 1) {
      hipLaunchKernelGGL((mfma_gemv_kernel<FMT, NMAT, MT, XS, G, true>), grid, dim3(kWaves * 64), lds, s, a);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      return am::launch_rows<false>(a.cand, nullptr, 0, (int)grid.x, a.m, a.am_idx, a.am_val, s);
    }
    if (am_mode) {
      // K is sliced: the fp32 outputs go to the workspace, then a per-row argmax over them
      a.y = a.cand;
      a.ldy = a.n;
      a.y_bf16 = 0;
      a.ws = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(a.cand) + am_outputs_bytes(a.n, a.m));
    }
  } else {
    if (am_mode) return hipErrorInvalidValue;
  }
  hipLaunchKernelGGL((mfma_gemv_kernel<FMT, NMAT, MT, XS, G>), grid, dim3(kWaves * 64), lds, s, a);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && a.ks > 1) {
    const int64_t mn = (int64_t)a.m * a.n;
    hipLaunchKernelGGL((slice_sum_kernel<NMAT>), dim3((unsigned)((mn + 255) / 256)), dim3(256), 0, s, a);
    e = hipGetLastError();
  }
  if (e != hipSuccess || !am_mode) return e;
  return am::launch_rows<true>(nullptr, static_cast<const float*>(a.y), a.n, a.n, a.m, a.am_idx, a.am_val, s);
}

template <int FMT, int XS>
hipError_t launch(const MgArgs& a, hipStream_t s) {
  const bool two = a.code[1] != nullptr;
  if (a.m <= 16) return two ? launch_mt<FMT, 2, 1, XS>(a, s) : launch_mt<FMT, 1, 1, XS>(a, s);
  return two ? launch_mt<FMT, 2, 2, XS>(a, s) : launch_mt<FMT, 1, 2, XS>(a, s);
}

}  // namespace mg
}  // namespace bfp
