#pragma once
// Encoding of one 16-value BFP block ("Qwen3.6-35B-A3B — TT-native mixed BFP4/BFP8",
// "Verification", Checkpoint bullet: BFP tensors are the bit-exact round-to-nearest
// conversion; "Qwen3.8-27B — TT-native mixed BFP4/BFP8 (GPTQ)", gptq-ctx2-20261002, "What
// changed in this release": 16-value blocks, representable values re-encode bit for bit).
// E = the largest fp32 exponent field of the block; each value keeps its sign bit and the
// magnitude |v| * 2^-(E - 127 - (m - 1)) rounded to nearest, ties to even, clamped to 2^m - 1.
//
// The rounding is done in integers on the 24-bit significand (no floating-point step), so it is
// exact for normal and subnormal inputs alike: with e_eff = max(e, 1) and the significand s24
// (implicit bit added for e > 0), the magnitude is s24 >> (24 + E - e_eff - m) rounded half to
// even on the bits shifted out.
#include "bfp_device.hpp"

namespace bfp {

template <int MAGBITS>
__device__ __forceinline__ uint32_t encode_value(uint32_t u, uint32_t big_e) {
  const uint32_t e = (u >> 23) & 0xffu;
  const uint32_t e_eff = e > 0 ? e : 1u;
  const uint32_t sig = (u & 0x7fffffu) | (e > 0 ? 0x800000u : 0u);
  // shift >= 24 - MAGBITS - 1 > 0 because e_eff <= max(big_e, 1)
  const int sh = 24 + (int)big_e - (int)e_eff - MAGBITS;
  uint32_t q;
  if (sh >= 26) {
    q = 0;                                    // below half of the smallest step
  } else {
    q = sig >> sh;
    const uint32_t rem = sig & ((1u << sh) - 1u);
    const uint32_t half = 1u << (sh - 1);
    q += (rem > half || (rem == half && (q & 1u))) ? 1u : 0u;
  }
  const uint32_t maxmag = (1u << MAGBITS) - 1u;
  q = q < maxmag ? q : maxmag;
  return ((u >> 31) << MAGBITS) | q;
}

// Encode 16 fp32 bit patterns: *exp = E, code = 16 bytes (BFP8) or 8 bytes (BFP4, value 2j in
// the low nibble of byte j). Returns true when a value is Inf or NaN (the codes are then
// meaningless).
template <int FMT>
__device__ __forceinline__ bool encode_block(const uint32_t (&u)[16], uint8_t* exp, uint8_t* code) {
  uint32_t big_e = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) big_e = max(big_e, (u[i] >> 23) & 0xffu);
  *exp = (uint8_t)big_e;
  constexpr int MB = FmtTraits<FMT>::kMagBits;
  uint32_t c[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) c[i] = encode_value<MB>(u[i], big_e);
  if constexpr (FMT == 8) {
    uint4 o;
    o.x = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
    o.y = c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24);
    o.z = c[8] | (c[9] << 8) | (c[10] << 16) | (c[11] << 24);
    o.w = c[12] | (c[13] << 8) | (c[14] << 16) | (c[15] << 24);
    *reinterpret_cast<uint4*>(code) = o;
  } else {
    uint2 o;
    o.x = 0; o.y = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) o.x |= c[i] << (4 * i);
#pragma unroll
    for (int i = 0; i < 8; ++i) o.y |= c[8 + i] << (4 * i);
    *reinterpret_cast<uint2*>(code) = o;
  }
  return big_e == 0xffu;
}

}  // namespace bfp
