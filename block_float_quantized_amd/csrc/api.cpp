// C ABI of libbfp: argument checks, kernel selection and status codes.
//
// Every check runs on the host before anything is launched, so an error return means no
// device work was queued. No C++ exception crosses this boundary.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>
#include <unordered_map>

#include "../../include/libbfp.h"
#include "bfp_internal.hpp"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool valid_fmt(int32_t f) { return f == BFP_FMT_BFP4 || f == BFP_FMT_BFP8; }

// Checks a matrix view; `need_n`/`need_k` < 0 means "any".
int32_t check_tensor(const bfp_tensor* t) {
  if (!t) return BFP_E_ARG;
  if (!valid_fmt(t->fmt)) return BFP_E_ARG;
  if (t->n <= 0 || t->k <= 0 || (t->k % 16) != 0) return BFP_E_SHAPE;
  if (t->n > INT32_MAX || t->k > (int64_t)1 << 24) return BFP_E_SHAPE;   // kernels index rows with int
  if (!t->exp || !t->code) return BFP_E_ARG;
  if (!aligned16(t->code)) return BFP_E_ALIGN;
  return BFP_OK;
}

int32_t from_hip(hipError_t e) { return e == hipSuccess ? BFP_OK : BFP_E_DEVICE; }

// One 4-byte device flag per device for bfp_quantize's non-finite report, made on first use
// and kept until the process ends.
int* quantize_flag() {
  static std::mutex mu;
  static std::unordered_map<int, int*> flags;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  auto it = flags.find(dev);
  if (it != flags.end()) return it->second;
  int* p = nullptr;
  if (hipMalloc(&p, sizeof(int)) != hipSuccess) return nullptr;
  flags[dev] = p;
  return p;
}

}  // namespace

extern "C" {

int32_t bfp_version(void) { return 100; }

const char* bfp_status_str(int32_t s) {
  switch (s) {
    case BFP_OK: return "ok";
    case BFP_E_ARG: return "invalid argument";
    case BFP_E_SHAPE: return "invalid shape";
    case BFP_E_ALIGN: return "device pointer not 16-byte aligned";
    case BFP_E_NONFINITE: return "non-finite input (Inf or NaN)";
    case BFP_E_WORKSPACE: return "workspace missing or too small";
    case BFP_E_DEVICE: return "HIP runtime or launch failure";
    case BFP_E_UNSUPPORTED: return "unsupported request";
    default: return "unknown status";
  }
}

size_t bfp_exp_bytes(int64_t n, int64_t k) {
  if (n < 0 || k < 0) return 0;
  return (size_t)(n * (k / 16));
}

size_t bfp_code_bytes(int32_t fmt, int64_t n, int64_t k) {
  if (n < 0 || k < 0) return 0;
  if (fmt == BFP_FMT_BFP8) return (size_t)(n * k);
  if (fmt == BFP_FMT_BFP4) return (size_t)(n * (k / 2));
  return 0;
}

int32_t bfp_quantize(int32_t fmt, const float* w, int64_t n, int64_t k, int64_t ldw, uint8_t* exp,
                     uint8_t* code, void* stream) {
  if (!valid_fmt(fmt)) return BFP_E_ARG;
  if (!w || !exp || !code) return BFP_E_ARG;
  if (n <= 0 || k <= 0 || (k % 16) != 0 || ldw < k) return BFP_E_SHAPE;
  if (!aligned16(w) || !aligned16(code) || (ldw % 4) != 0) return BFP_E_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int* flag = quantize_flag();
  if (!flag) return BFP_E_DEVICE;
  if (hipMemsetAsync(flag, 0, sizeof(int), s) != hipSuccess) return BFP_E_DEVICE;
  if (bfp::quantize_launch(fmt, w, n, k, ldw, exp, code, flag, s) != hipSuccess) return BFP_E_DEVICE;
  int h = 0;
  if (hipMemcpyAsync(&h, flag, sizeof(int), hipMemcpyDeviceToHost, s) != hipSuccess) return BFP_E_DEVICE;
  if (hipStreamSynchronize(s) != hipSuccess) return BFP_E_DEVICE;
  return h ? BFP_E_NONFINITE : BFP_OK;
}

int32_t bfp_dequantize(const bfp_tensor* w, int32_t out_dtype, void* out, void* stream) {
  int32_t st = check_tensor(w);
  if (st != BFP_OK) return st;
  if (out_dtype != BFP_DT_F32 && out_dtype != BFP_DT_BF16) return BFP_E_ARG;
  if (!out) return BFP_E_ARG;
  if (!aligned16(out)) return BFP_E_ALIGN;
  return from_hip(bfp::dequant_launch(w->fmt, w->exp, w->code, w->n, w->k, out_dtype == BFP_DT_BF16,
                                      out, static_cast<hipStream_t>(stream)));
}

size_t bfp_gemm_workspace_bytes(const bfp_tensor* w, const bfp_tensor* w_up, int64_t m) {
  if (check_tensor(w) != BFP_OK || m < 1 || m > BFP_GEMM_MAX_M) return 0;
  // enough for both kernel choices (with and without BFP_GEMM_BATCH_INVARIANT)
  return std::max(bfp::gemv_workspace_bytes(w->fmt, w_up != nullptr, w->n, w->k, m, false),
                  bfp::gemv_workspace_bytes(w->fmt, w_up != nullptr, w->n, w->k, m, true));
}

int32_t bfp_gemm(const bfp_tensor* w, const bfp_tensor* w_up, int32_t epilogue, const void* x,
                 int32_t x_dtype, int64_t m, int64_t ldx, void* y, int32_t y_dtype, int64_t ldy,
                 void* ws, size_t ws_bytes, void* stream) {
  int32_t st = check_tensor(w);
  if (st != BFP_OK) return st;
  const int32_t flags = epilogue & ~0xff;
  epilogue &= 0xff;
  if ((flags & ~BFP_GEMM_BATCH_INVARIANT) != 0) return BFP_E_ARG;
  const bool invariant = (flags & BFP_GEMM_BATCH_INVARIANT) != 0;
  if (epilogue == BFP_EPI_NONE) {
    if (w_up) return BFP_E_ARG;
  } else if (epilogue == BFP_EPI_SWIGLU) {
    st = check_tensor(w_up);
    if (st != BFP_OK) return st;
    if (w_up->fmt != w->fmt) return BFP_E_ARG;
    if (w_up->n != w->n || w_up->k != w->k) return BFP_E_SHAPE;
  } else {
    return BFP_E_ARG;
  }
  if ((x_dtype != BFP_DT_F32 && x_dtype != BFP_DT_BF16) || (y_dtype != BFP_DT_F32 && y_dtype != BFP_DT_BF16))
    return BFP_E_ARG;
  if (!x || !y) return BFP_E_ARG;
  if (m < 1 || m > BFP_GEMM_MAX_M) return BFP_E_SHAPE;
  if (ldx < w->k || ldy < w->n) return BFP_E_SHAPE;
  const int64_t xs = x_dtype == BFP_DT_BF16 ? 2 : 4;
  if (!aligned16(x) || ((ldx * xs) % 16) != 0) return BFP_E_ALIGN;
  const size_t need = bfp::gemv_workspace_bytes(w->fmt, epilogue == BFP_EPI_SWIGLU, w->n, w->k, m, invariant);
  if (need > 0 && (!ws || ws_bytes < need)) return BFP_E_WORKSPACE;
  if (ws && !aligned16(ws)) return BFP_E_ALIGN;
  bfp::GemvParams g{};
  g.fmt = w->fmt;
  g.w_exp = w->exp; g.w_code = w->code;
  g.u_exp = epilogue == BFP_EPI_SWIGLU ? w_up->exp : nullptr;
  g.u_code = epilogue == BFP_EPI_SWIGLU ? w_up->code : nullptr;
  g.n = w->n; g.k = w->k;
  g.x = x; g.ldx = ldx; g.x_bf16 = x_dtype == BFP_DT_BF16;
  g.m = m; g.y = y; g.ldy = ldy; g.y_bf16 = y_dtype == BFP_DT_BF16;
  g.ws = ws;
  g.invariant = invariant;
  return from_hip(bfp::gemv_launch(g, static_cast<hipStream_t>(stream)));
}

size_t bfp_gemm_argmax_workspace_bytes(const bfp_tensor* w, int64_t m) {
  if (check_tensor(w) != BFP_OK || m < 1 || m > BFP_GEMM_MAX_M) return 0;
  return std::max(bfp::gemv_argmax_workspace_bytes(w->fmt, w->n, w->k, m, false),
                  bfp::gemv_argmax_workspace_bytes(w->fmt, w->n, w->k, m, true));
}

int32_t bfp_gemm_argmax(const bfp_tensor* w, const void* x, int32_t x_dtype, int64_t m, int64_t ldx,
                        int32_t flags, int32_t* idx, float* val, void* ws, size_t ws_bytes, void* stream) {
  int32_t st = check_tensor(w);
  if (st != BFP_OK) return st;
  if ((flags & ~BFP_GEMM_BATCH_INVARIANT) != 0) return BFP_E_ARG;
  const bool invariant = (flags & BFP_GEMM_BATCH_INVARIANT) != 0;
  if (x_dtype != BFP_DT_F32 && x_dtype != BFP_DT_BF16) return BFP_E_ARG;
  if (x_dtype != BFP_DT_BF16) return BFP_E_UNSUPPORTED;
  if (!x || !idx || !val || !ws) return BFP_E_ARG;
  if (m < 1 || m > BFP_GEMM_MAX_M) return BFP_E_SHAPE;
  if (ldx < w->k) return BFP_E_SHAPE;
  if (!aligned16(x) || ((ldx * 2) % 16) != 0) return BFP_E_ALIGN;
  if (!aligned16(ws)) return BFP_E_ALIGN;
  if (ws_bytes < bfp::gemv_argmax_workspace_bytes(w->fmt, w->n, w->k, m, invariant)) return BFP_E_WORKSPACE;
  bfp::GemvParams g{};
  g.fmt = w->fmt;
  g.w_exp = w->exp; g.w_code = w->code;
  g.n = w->n; g.k = w->k;
  g.x = x; g.ldx = ldx; g.x_bf16 = 1;
  g.m = m;
  g.ws = ws;
  g.am_idx = idx;
  g.am_val = val;
  g.invariant = invariant;
  return from_hip(bfp::gemv_launch(g, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

// MoE entry points are defined in moe_api.cpp.
