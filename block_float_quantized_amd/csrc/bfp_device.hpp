// Device helpers shared by the libbfp kernels (gfx950 / CDNA4, wave64).
//
// Block format (model-card pages "Qwen3.8-27B — TT-native mixed BFP4/BFP8 (GPTQ)",
// revision gptq-ctx2-20261002, "What changed in this release": 16-value blocks with a
// shared exponent): per 16-value block one exponent byte E and per value a sign bit plus an
// m-bit magnitude (m = 7 for BFP8, 3 for BFP4); value = (-1)^sign * mag * 2^(E-127-(m-1)).
//
// Unpack strategy (all exact):
//  * BFP4: a nibble s|mmm is moved into a byte s000_0mmm, which is an OCP FP8 E4M3
//    subnormal of value (-1)^s * mmm * 2^-9; v_cvt_pk_f32_fp8 turns two such bytes into two
//    fp32 values. Eight nibbles cost 6 bit ops + 4 conversions. The 2^9 is folded into the
//    block scale 2^(E - 129 + 9) = 2^(E - 120).
//  * BFP8: a byte s|mmmmmmm -> v_cvt_f32_ubyte of the magnitude, sign bit OR-ed into bit 31.
//    The block scale is 2^(E - 133).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bfp {

constexpr int kBlock = 16;
constexpr int kWave = 64;

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Exponent offset that turns the raw block exponent E into the log2 of the per-block
// multiplier applied to the unpacked integers (see the file comment).
template <int FMT> struct FmtTraits;
template <> struct FmtTraits<4> {
  static constexpr int kMagBits = 3;
  static constexpr int kCodeBytes = 8;     // bytes of codes per 16-value block
  static constexpr int kScaleBias = 120;   // 127 + (3 - 1) - 9
};
template <> struct FmtTraits<8> {
  static constexpr int kMagBits = 7;
  static constexpr int kCodeBytes = 16;
  static constexpr int kScaleBias = 133;   // 127 + (7 - 1)
};

// ---- unpack ---------------------------------------------------------------------------

// Eight BFP4 nibbles (value i in bits [4i, 4i+4)) -> fp32 values (-1)^s * mag * 2^-9.
__device__ __forceinline__ void unpack8_bfp4(uint32_t c, float w[8]) {
  // even nibbles -> bytes s000_0mmm (values 0,2,4,6); odd nibbles likewise (1,3,5,7)
  const uint32_t ev = ((c << 4) & 0x80808080u) | (c & 0x07070707u);
  const uint32_t od = (c & 0x80808080u) | ((c >> 4) & 0x07070707u);
  const f32x2 e01 = __builtin_amdgcn_cvt_pk_f32_fp8(ev, false);
  const f32x2 e23 = __builtin_amdgcn_cvt_pk_f32_fp8(ev, true);
  const f32x2 o01 = __builtin_amdgcn_cvt_pk_f32_fp8(od, false);
  const f32x2 o23 = __builtin_amdgcn_cvt_pk_f32_fp8(od, true);
  w[0] = e01.x; w[2] = e01.y; w[4] = e23.x; w[6] = e23.y;
  w[1] = o01.x; w[3] = o01.y; w[5] = o23.x; w[7] = o23.y;
}

// Four BFP8 codes (value i in byte i) -> fp32 values (-1)^s * mag.
__device__ __forceinline__ void unpack4_bfp8(uint32_t c, float w[4]) {
  const uint32_t a = c & 0x7f7f7f7fu;
  // byte -> float conversions (the compiler selects v_cvt_f32_ubyte0..3)
  const float m0 = (float)(a & 0xffu);
  const float m1 = (float)((a >> 8) & 0xffu);
  const float m2 = (float)((a >> 16) & 0xffu);
  const float m3 = (float)(a >> 24);
  w[0] = __uint_as_float(__float_as_uint(m0) | ((c << 24) & 0x80000000u));
  w[1] = __uint_as_float(__float_as_uint(m1) | ((c << 16) & 0x80000000u));
  w[2] = __uint_as_float(__float_as_uint(m2) | ((c << 8) & 0x80000000u));
  w[3] = __uint_as_float(__float_as_uint(m3) | (c & 0x80000000u));
}

// Eight BFP4 nibbles -> four dwords of bf16 pairs (-1)^s * mag * 2^-9, in the pair order
// (v0,v2) (v4,v6) (v1,v3) (v5,v7); activations are staged in the same order.
__device__ __forceinline__ void unpack8_bfp4_bf16(uint32_t c, uint32_t w[4]) {
  const uint32_t ev = ((c << 4) & 0x80808080u) | (c & 0x07070707u);
  const uint32_t od = (c & 0x80808080u) | ((c >> 4) & 0x07070707u);
  w[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(ev, 1.0f, false));
  w[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(ev, 1.0f, true));
  w[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(od, 1.0f, false));
  w[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(od, 1.0f, true));
}

// Four BFP8 codes -> two dwords of bf16 pairs (-1)^s * mag in the order (v0,v2) (v1,v3).
// Integers up to 127 have at most 7 significant bits, so the top half of the fp32 is the
// exact bf16.
__device__ __forceinline__ void unpack4_bfp8_bf16(uint32_t c, uint32_t w[2]) {
  const uint32_t a = c & 0x7f7f7f7fu;
  const uint32_t f0 = __float_as_uint((float)(a & 0xffu));
  const uint32_t f1 = __float_as_uint((float)((a >> 8) & 0xffu));
  const uint32_t f2 = __float_as_uint((float)((a >> 16) & 0xffu));
  const uint32_t f3 = __float_as_uint((float)(a >> 24));
  // byte selectors: result = [hi16(second) : hi16(first)]
  w[0] = __builtin_amdgcn_perm(f2, f0, 0x07060302u) | ((c << 8) & 0x80008000u);
  w[1] = __builtin_amdgcn_perm(f3, f1, 0x07060302u) | (c & 0x80008000u);
}

// acc + a.lo * b.lo + a.hi * b.hi for two packed bf16 pairs (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), acc, false);
}

// log2 of the multiplier of a block's unpacked integers: E - kScaleBias. Applied with
// v_ldexp_f32 (apply_shift), which is exact for every E: a multiplier 2^(E - kScaleBias)
// held as a float would overflow for BFP4 blocks with E >= 248 (largest |w| >= 2^121).
template <int FMT>
__device__ __forceinline__ int block_shift(uint32_t e) { return (int)e - FmtTraits<FMT>::kScaleBias; }
__device__ __forceinline__ float apply_shift(float v, int sh) { return __builtin_amdgcn_ldexpf(v, sh); }
// Shift that turns any finite value into a signed zero (masks out a clamped, duplicate unit).
constexpr int kShiftToZero = -512;

// The multiplier itself, for BFP8 only: 2^(E - 133) lies in [2^-133, 2^121], always finite
// (ldexp gives the fp32 subnormal below 2^-126).
template <int FMT>
__device__ __forceinline__ float block_scale(uint32_t e) {
  static_assert(FMT == 8, "a BFP4 multiplier overflows for E >= 248: use block_shift");
  return __builtin_amdgcn_ldexpf(1.0f, (int)e - FmtTraits<FMT>::kScaleBias);
}

// ---- BFP4 to bf16 with the block scale applied (8 values -> 4 dwords of pairs) -------------

// BFP4, exponent in [8, 247]: 2^(E-120) is a normal fp32 and every result a normal bf16.
__device__ __forceinline__ u32x4 dq8_bfp4_fast(uint32_t c, float sc) {
  const uint32_t ev = ((c << 4) & 0x80808080u) | (c & 0x07070707u);
  const uint32_t od = (c & 0x80808080u) | ((c >> 4) & 0x07070707u);
  u32x4 o;
  o.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(ev, sc, false));   // (v0, v2)
  o.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(ev, sc, true));    // (v4, v6)
  o.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(od, sc, false));   // (v1, v3)
  o.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(od, sc, true));    // (v5, v7)
  return o;
}

// BFP4, any exponent: fp32 values scaled by ldexp (exact, subnormals included); a value with
// at most 3 significant bits and a multiple of 2^-133 is its own bf16, the top half of the fp32.
__device__ __forceinline__ u32x4 dq8_bfp4_any(uint32_t c, uint32_t e) {
  float w[8];
  unpack8_bfp4(c, w);
  const int sh = (int)e - FmtTraits<4>::kScaleBias;
  uint32_t b[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) b[i] = __float_as_uint(__builtin_amdgcn_ldexpf(w[i], sh));
  u32x4 o;
  o.x = __builtin_amdgcn_perm(b[2], b[0], 0x07060302u);
  o.y = __builtin_amdgcn_perm(b[6], b[4], 0x07060302u);
  o.z = __builtin_amdgcn_perm(b[3], b[1], 0x07060302u);
  o.w = __builtin_amdgcn_perm(b[7], b[5], 0x07060302u);
  return o;
}

// ---- bf16 -----------------------------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// ---- cross-lane reductions --------------------------------------------------------------

// DPP lane permutations inside a row of 16 lanes (gfx9 encodings).
constexpr int kDppQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;    // lane i <-> 7-i inside each 8-lane half row
constexpr int kDppRowRor8 = 0x128;       // lane i <-> i^8 inside a 16-lane row

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

// One halving step inside a 16-lane row: `v` holds N values; afterwards the first N/2
// entries hold sums over the lane pair, the lane whose selector bit is set keeping the
// upper half of the index range. PAIR is a DPP involution whose partner differs in `bit`.
template <int N, int CTRL>
__device__ __forceinline__ void halve_dpp(float* v, bool upper) {
#pragma unroll
  for (int i = 0; i < N / 2; ++i) {
    const float send = upper ? v[i] : v[i + N / 2];
    const float keep = upper ? v[i + N / 2] : v[i];
    v[i] = keep + dpp_mov<CTRL>(send);
  }
}

template <int N, int CTRL>
__device__ __forceinline__ void butterfly_dpp(float* v) {
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] += dpp_mov<CTRL>(v[i]);
}

// Halving step across the two 32-lane halves of the wave with v_permlane32_swap.
template <int N>
__device__ __forceinline__ void halve_x32(float* v) {
#pragma unroll
  for (int i = 0; i < N / 2; ++i) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[i]), __float_as_uint(v[i + N / 2]),
                                              false, false);
    v[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
}
// Halving step across 16-lane rows (lanes l and l^16) with v_permlane16_swap.
template <int N>
__device__ __forceinline__ void halve_x16(float* v) {
#pragma unroll
  for (int i = 0; i < N / 2; ++i) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[i]), __float_as_uint(v[i + N / 2]),
                                              false, false);
    v[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
}
template <int N>
__device__ __forceinline__ void butterfly_x32(float* v) {
#pragma unroll
  for (int i = 0; i < N; ++i) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[i]), __float_as_uint(v[i]), false, false);
    v[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
}
template <int N>
__device__ __forceinline__ void butterfly_x16(float* v) {
#pragma unroll
  for (int i = 0; i < N; ++i) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[i]), __float_as_uint(v[i]), false, false);
    v[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
}

// Sum C values over the LPR lanes of a lane group (LPR = 16 or 64), recursive halving:
// each step sends half of the current values to the partner lane and adds what comes
// back, so the total work is about 2C moves instead of C * log2(LPR). Halving stops once
// KEEP values are left per lane (the remaining steps are plain butterflies).
// Afterwards lane position p = lane % LPR holds `count` = max(KEEP, C/LPR) sums, for the
// value indices [(p >> (log2(LPR) - h)) * count, ... + count) where h is the number of
// halving steps (reduce_halvings<C, KEEP, LPR>()).
template <int C, int KEEP, int LPR>
struct LaneReduce {
  static constexpr int ilog2(int x) { return x <= 1 ? 0 : 1 + ilog2(x / 2); }
  static_assert(C >= 1 && (C & (C - 1)) == 0 && LPR >= 1 && (LPR & (LPR - 1)) == 0,
                "the halving tree takes a power-of-two count of values and lanes");
  static constexpr int kSteps = ilog2(LPR);
  static constexpr int kHalvings = (ilog2(C / KEEP) < kSteps) ? ilog2(C / KEEP) : kSteps;
  static constexpr int kCount = C >> kHalvings;

  template <int STEP, int CUR>
  __device__ __forceinline__ static void step(float* v, int lane) {
    if constexpr (STEP < kSteps) {
      // offset of this step in lanes: LPR/2, LPR/4, ..., 1
      constexpr int OFF = LPR >> (STEP + 1);
      const bool upper = (lane & OFF) != 0;
      constexpr bool HALVE = CUR > KEEP;
      if constexpr (OFF == 32) {
        if constexpr (HALVE) halve_x32<CUR>(v); else butterfly_x32<CUR>(v);
      } else if constexpr (OFF == 16) {
        if constexpr (HALVE) halve_x16<CUR>(v); else butterfly_x16<CUR>(v);
      } else if constexpr (OFF == 8) {
        if constexpr (HALVE) halve_dpp<CUR, kDppRowRor8>(v, upper); else butterfly_dpp<CUR, kDppRowRor8>(v);
      } else if constexpr (OFF == 4) {
        if constexpr (HALVE) halve_dpp<CUR, kDppHalfMirror>(v, upper); else butterfly_dpp<CUR, kDppHalfMirror>(v);
      } else if constexpr (OFF == 2) {
        if constexpr (HALVE) halve_dpp<CUR, kDppQuadXor2>(v, upper); else butterfly_dpp<CUR, kDppQuadXor2>(v);
      } else {
        if constexpr (HALVE) halve_dpp<CUR, kDppQuadXor1>(v, upper); else butterfly_dpp<CUR, kDppQuadXor1>(v);
      }
      step<STEP + 1, (HALVE ? CUR / 2 : CUR)>(v, lane);
    }
  }
  __device__ __forceinline__ static void run(float* v, int lane) { step<0, C>(v, lane); }
  // first value index held by lane position p (p = lane % LPR)
  __device__ __forceinline__ static int first_index(int p) {
    return (p >> (kSteps - kHalvings)) * kCount;
  }
  // lanes that hold a distinct copy (the others hold duplicates after butterflies)
  __device__ __forceinline__ static bool writer(int p) {
    return (p & ((1 << (kSteps - kHalvings)) - 1)) == 0;
  }
};

}  // namespace bfp
