// BFP4/BFP8 encode and decode kernels for gfx950.
//
// Encoding (model-card pages "Qwen3.6-35B-A3B — TT-native mixed BFP4/BFP8", "Verification",
// Checkpoint bullet: BFP tensors are the bit-exact round-to-nearest conversion; "Qwen3.8-27B
// — TT-native mixed BFP4/BFP8 (GPTQ)", gptq-ctx2-20261002, "What changed in this release":
// 16-value blocks, representable values re-encode bit for bit). Per 16-value block:
// E = the largest fp32 exponent field; each value keeps its sign bit and the magnitude
// |v| * 2^-(E - 127 - (m - 1)) rounded to nearest, ties to even, clamped to 2^m - 1.
//
// One thread encodes one block from four 16-byte loads. The rounding is done in integers on
// the 24-bit significand (no floating-point step), so it is exact for normal and subnormal
// inputs alike: with e_eff = max(e, 1) and the significand s24 (implicit bit added for
// e > 0), the magnitude is s24 >> (24 + E - e_eff - m) rounded half to even on the bits
// shifted out.
#include "bfp_device.hpp"
#include "bfp_internal.hpp"

namespace bfp {

namespace {

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

template <int FMT>
__global__ __launch_bounds__(256) void quantize_kernel(const float* __restrict__ w, int64_t nblocks,
                                                       uint8_t* __restrict__ exp,
                                                       uint8_t* __restrict__ code, int* flag) {
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= nblocks) return;
  const u32x4* src = reinterpret_cast<const u32x4*>(w + b * kBlock);
  uint32_t u[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    u[4 * i] = v.x; u[4 * i + 1] = v.y; u[4 * i + 2] = v.z; u[4 * i + 3] = v.w;
  }
  uint32_t big_e = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) big_e = max(big_e, (u[i] >> 23) & 0xffu);
  if (big_e == 0xffu) atomicOr(flag, 1);
  exp[b] = (uint8_t)big_e;
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
    reinterpret_cast<uint4*>(code)[b] = o;
  } else {
    uint2 o;
    o.x = 0; o.y = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) o.x |= c[i] << (4 * i);
#pragma unroll
    for (int i = 0; i < 8; ++i) o.y |= c[8 + i] << (4 * i);
    reinterpret_cast<uint2*>(code)[b] = o;
  }
}

// One thread decodes one block with the same unpack helpers the matmul kernels use, so the
// bit-exact decode test also checks the matmuls' in-register unpack.
template <int FMT>
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* __restrict__ exp,
                                                      const uint8_t* __restrict__ code,
                                                      int64_t nblocks, int out_bf16, void* out) {
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= nblocks) return;
  const float sc = block_scale<FMT>(exp[b]);
  float v[16];
  if constexpr (FMT == 4) {
    const uint2 c = reinterpret_cast<const uint2*>(code)[b];
    unpack8_bfp4(c.x, v);
    unpack8_bfp4(c.y, v + 8);
  } else {
    const uint4 c = reinterpret_cast<const uint4*>(code)[b];
    unpack4_bfp8(c.x, v);
    unpack4_bfp8(c.y, v + 4);
    unpack4_bfp8(c.z, v + 8);
    unpack4_bfp8(c.w, v + 12);
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] *= sc;
  if (out_bf16) {
    // every decoded value is bf16-representable, so dropping the low half is exact
    uint4* o = reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + b * kBlock);
    uint32_t h[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      h[i] = (__float_as_uint(v[2 * i]) >> 16) | (__float_as_uint(v[2 * i + 1]) & 0xffff0000u);
    o[0] = make_uint4(h[0], h[1], h[2], h[3]);
    o[1] = make_uint4(h[4], h[5], h[6], h[7]);
  } else {
    f32x4* o = reinterpret_cast<f32x4*>(static_cast<float*>(out) + b * kBlock);
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = f32x4{v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]};
  }
}

}  // namespace

hipError_t quantize_launch(int fmt, const float* w, int64_t n, int64_t k, uint8_t* exp,
                           uint8_t* code, int* flag, hipStream_t s) {
  const int64_t nb = n * (k / kBlock);
  if (nb == 0) return hipSuccess;
  const int64_t grid = (nb + 255) / 256;
  if (fmt == 8)
    hipLaunchKernelGGL(quantize_kernel<8>, dim3((unsigned)grid), dim3(256), 0, s, w, nb, exp, code, flag);
  else
    hipLaunchKernelGGL(quantize_kernel<4>, dim3((unsigned)grid), dim3(256), 0, s, w, nb, exp, code, flag);
  return hipGetLastError();
}

hipError_t dequant_launch(int fmt, const uint8_t* exp, const uint8_t* code, int64_t n, int64_t k,
                          int out_bf16, void* out, hipStream_t s) {
  const int64_t nb = n * (k / kBlock);
  if (nb == 0) return hipSuccess;
  const int64_t grid = (nb + 255) / 256;
  if (fmt == 8)
    hipLaunchKernelGGL(dequant_kernel<8>, dim3((unsigned)grid), dim3(256), 0, s, exp, code, nb, out_bf16, out);
  else
    hipLaunchKernelGGL(dequant_kernel<4>, dim3((unsigned)grid), dim3(256), 0, s, exp, code, nb, out_bf16, out);
  return hipGetLastError();
}

}  // namespace bfp
