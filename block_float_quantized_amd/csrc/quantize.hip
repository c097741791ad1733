// BFP4/BFP8 encode and decode kernels for gfx950 (the block encoding is in bfp_encode.hpp).
//
// One thread encodes one 16-value block from four 16-byte loads.
#include "bfp_device.hpp"
#include "bfp_encode.hpp"
#include "bfp_internal.hpp"

namespace bfp {

namespace {

// Block b is block b % nbk of row b / nbk; rows of w are ldw values apart.
template <int FMT>
__global__ __launch_bounds__(256) void quantize_kernel(const float* __restrict__ w, int64_t nblocks, int64_t nbk,
                                                       int64_t ldw, uint8_t* __restrict__ exp,
                                                       uint8_t* __restrict__ code, int* flag) {
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= nblocks) return;
  const u32x4* src = reinterpret_cast<const u32x4*>(w + (b / nbk) * ldw + (b % nbk) * kBlock);
  uint32_t u[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    u[4 * i] = v.x; u[4 * i + 1] = v.y; u[4 * i + 2] = v.z; u[4 * i + 3] = v.w;
  }
  if (encode_block<FMT>(u, exp + b, code + b * FmtTraits<FMT>::kCodeBytes)) atomicOr(flag, 1);
}

// One thread decodes one block with the same unpack helpers the matmul kernels use, so the
// bit-exact decode test also checks the matmuls' in-register unpack.
template <int FMT>
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* __restrict__ exp,
                                                      const uint8_t* __restrict__ code,
                                                      int64_t nblocks, int out_bf16, void* out) {
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= nblocks) return;
  const int sh = block_shift<FMT>(exp[b]);
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
  for (int i = 0; i < 16; ++i) v[i] = apply_shift(v[i], sh);
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

hipError_t quantize_launch(int fmt, const float* w, int64_t n, int64_t k, int64_t ldw, uint8_t* exp,
                           uint8_t* code, int* flag, hipStream_t s) {
  const int64_t nbk = k / kBlock;
  const int64_t nb = n * nbk;
  if (nb == 0) return hipSuccess;
  const int64_t grid = (nb + 255) / 256;
  if (fmt == 8)
    hipLaunchKernelGGL(quantize_kernel<8>, dim3((unsigned)grid), dim3(256), 0, s, w, nb, nbk, ldw, exp, code, flag);
  else
    hipLaunchKernelGGL(quantize_kernel<4>, dim3((unsigned)grid), dim3(256), 0, s, w, nb, nbk, ldw, exp, code, flag);
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
