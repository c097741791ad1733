// Skinny BFP4/BFP8 matmul dispatch: the matrix-core kernel (mfma_gemv.hpp) or the vector-ALU
// kernel (gemv_impl.hpp, compiled in four translation units).
#include <atomic>

#include "bfp_internal.hpp"
#include "gemv_row.hpp"
#include "mfma_gemv.hpp"

namespace bfp {

namespace rowk {

// Compute units per device, looked up once per device.
int device_cus() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cus[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int c = cus[dev].load(std::memory_order_relaxed);
  if (c <= 0) {
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0) c = 256;
    cus[dev].store(c, std::memory_order_relaxed);
  }
  return c;
}

}  // namespace rowk

hipError_t gemv_launch_b4_bf16x(const GemvParams& g, hipStream_t s);
hipError_t gemv_launch_b4_f32x(const GemvParams& g, hipStream_t s);
hipError_t gemv_launch_b8_bf16x(const GemvParams& g, hipStream_t s);
hipError_t gemv_launch_b8_f32x(const GemvParams& g, hipStream_t s);
hipError_t mfma_gemv_launch_b4(const mg::MgArgs& a, bool x_bf16, hipStream_t s);
hipError_t mfma_gemv_launch_b8(const mg::MgArgs& a, bool x_bf16, hipStream_t s);

namespace {

// One activation row runs the vector-ALU kernel (it streams the weights faster when there is
// a single row to multiply); 2..32 rows run the matrix-core kernel. Batch-invariant calls run
// the matrix-core kernel for every m, so that row i does not depend on m.
bool use_vector(int64_t m, bool invariant) { return !invariant && m == 1; }

hipError_t vector_launch(const GemvParams& g, hipStream_t s) {
  if (g.fmt == 4) return g.x_bf16 ? gemv_launch_b4_bf16x(g, s) : gemv_launch_b4_f32x(g, s);
  return g.x_bf16 ? gemv_launch_b8_bf16x(g, s) : gemv_launch_b8_f32x(g, s);
}

hipError_t mfma_launch(const GemvParams& g, hipStream_t s) {
  mg::MgArgs a{};
  a.exp[0] = g.w_exp; a.code[0] = g.w_code;
  a.exp[1] = g.u_exp; a.code[1] = g.u_code;
  a.x = g.x; a.ldx = g.ldx;
  a.y = g.y; a.ldy = g.ldy;
  a.n = (int)g.n; a.k = (int)g.k; a.m = (int)g.m;
  a.y_bf16 = g.y_bf16;
  a.ws = static_cast<float*>(g.ws);
  a.ks = 1; a.sps = 0; a.kc = 0; a.exp_vec = 0;
  a.code16 = (g.k % 32) == 0;
  if (g.am_idx != nullptr) {
    a.cand = static_cast<uint64_t*>(g.ws);
    a.am_idx = g.am_idx;
    a.am_val = g.am_val;
  }
  return g.fmt == 4 ? mfma_gemv_launch_b4(a, g.x_bf16 != 0, s) : mfma_gemv_launch_b8(a, g.x_bf16 != 0, s);
}

}  // namespace

size_t gemv_workspace_bytes(int fmt, bool swiglu, int64_t n, int64_t k, int64_t m, bool invariant) {
  if (use_vector(m, invariant)) return 0;
  const int N = (int)n, K = (int)k, M = (int)m;
  if (fmt == 4) return swiglu ? mg::workspace_bytes<4, 2>(N, K, M) : mg::workspace_bytes<4, 1>(N, K, M);
  return swiglu ? mg::workspace_bytes<8, 2>(N, K, M) : mg::workspace_bytes<8, 1>(N, K, M);
}

size_t gemv_argmax_workspace_bytes(int fmt, int64_t n, int64_t k, int64_t m, bool invariant) {
  if (use_vector(m, invariant)) return (size_t)m * ((n + kVectorMinRowsPerWg - 1) / kVectorMinRowsPerWg) * sizeof(uint64_t);
  const int N = (int)n, K = (int)k, M = (int)m;
  return fmt == 4 ? mg::argmax_workspace_bytes<4>(N, K, M) : mg::argmax_workspace_bytes<8>(N, K, M);
}

hipError_t gemv_launch(const GemvParams& g, hipStream_t s) {
  if (use_vector(g.m, g.invariant != 0)) return vector_launch(g, s);
  return mfma_launch(g, s);
}

}  // namespace bfp
