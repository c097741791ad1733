// C ABI of the MoE entry points: layer checks, workspace layout, and the decode pipelines:
// a few tokens: router logits -> per-token top-k + gate/up + SwiGLU -> down + combine; more:
// router logits -> top-k + dispatch -> grouped gate/up + SwiGLU -> grouped down -> combine.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "../../include/libbfp.h"
#include "bfp_moe.hpp"
#include "bfp_prefill.hpp"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int32_t check_mat(const bfp_tensor& t, int64_t n, int64_t k) {
  if (t.fmt != BFP_FMT_BFP4) return t.fmt == BFP_FMT_BFP8 ? BFP_E_UNSUPPORTED : BFP_E_ARG;
  if (t.n != n || t.k != k) return BFP_E_SHAPE;
  if (!t.exp || !t.code) return BFP_E_ARG;
  if (!aligned16(t.exp) || !aligned16(t.code)) return BFP_E_ALIGN;
  return BFP_OK;
}

int32_t check_router(const bfp_moe_layer* L) {
  if (!L) return BFP_E_ARG;
  if (L->n_experts < 1 || L->n_experts > 256) return BFP_E_SHAPE;
  if (L->top_k < 1 || L->top_k > 8 || L->top_k > L->n_experts) return BFP_E_SHAPE;
  if (L->hidden <= 0 || L->hidden % 32 != 0 || L->hidden > (1 << 16)) return BFP_E_SHAPE;
  if (!L->router_w) return BFP_E_ARG;
  if (!aligned16(L->router_w) || (L->sh_gate_w && !aligned16(L->sh_gate_w))) return BFP_E_ALIGN;
  return BFP_OK;
}

int32_t check_layer(const bfp_moe_layer* L) {
  int32_t st = check_router(L);
  if (st != BFP_OK) return st;
  if (L->inter <= 0 || L->inter % 32 != 0 || L->inter > (1 << 16)) return BFP_E_SHAPE;
  const int64_t E = L->n_experts, H = L->hidden, F = L->inter;
  if ((st = check_mat(L->gate, E * F, H)) != BFP_OK) return st;
  if ((st = check_mat(L->up, E * F, H)) != BFP_OK) return st;
  if ((st = check_mat(L->down, E * H, F)) != BFP_OK) return st;
  if (L->sh_gate.fmt != 0) {
    if ((st = check_mat(L->sh_gate, F, H)) != BFP_OK) return st;
    if ((st = check_mat(L->sh_up, F, H)) != BFP_OK) return st;
    if ((st = check_mat(L->sh_down, H, F)) != BFP_OK) return st;
  }
  return BFP_OK;
}

// Workspace regions, each 256-byte aligned.
struct Layout {
  size_t logits, ids, w, g, counts, offsets, perm, inv, active, nact, chunks, h, o, extra, total;
};

size_t place(size_t& off, size_t bytes) {
  const size_t at = off;
  off += (bytes + 255) / 256 * 256;
  return at;
}

Layout layout(const bfp_moe_layer* L, int64_t m, bool with_experts) {
  Layout y{};
  size_t off = 0;
  const int64_t E = L->n_experts, K = L->top_k, H = L->hidden, F = L->inter;
  const int64_t pairs = m * K + m;
  const bool prefill = m > BFP_GEMM_MAX_M;
  y.logits = place(off, bfp::route_workspace_bytes((int)m, (int)E));
  if (with_experts) {
    y.ids = place(off, (size_t)m * K * 4);
    y.w = place(off, (size_t)m * K * 4);
    y.g = place(off, (size_t)m * 4);
    y.counts = place(off, (size_t)E * 4);
    y.offsets = place(off, (size_t)(E + 1) * 4);
    y.perm = place(off, (size_t)m * K * 4);
    y.inv = place(off, (size_t)m * K * 4);
    y.active = place(off, (size_t)E * 4);
    y.nact = place(off, 16);
    if (prefill) {
      y.chunks = place(off, bfp::dispatch_scratch_bytes((int)m));
      y.h = place(off, (size_t)pairs * F * 2);       // bf16 h
      y.o = place(off, (size_t)pairs * H * 4);
      y.extra = off;
      y.total = off + bfp::prefill_workspace_extra_bytes((int)m, (int)E, (int)K, (int)H);
      return y;
    }
    y.h = place(off, (size_t)pairs * F * 4);
    y.o = place(off, (size_t)pairs * H * 4);
    y.extra = place(off, (size_t)(E + 2) * 4);      // row-tile starts of the groups
  }
  y.total = off;
  return y;
}

template <typename T>
T* at(void* ws, size_t off) { return reinterpret_cast<T*>(static_cast<char*>(ws) + off); }

int32_t from_hip(hipError_t e) { return e == hipSuccess ? BFP_OK : BFP_E_DEVICE; }

bfp::RouteArgs route_args(const bfp_moe_layer* L, const uint16_t* x, int64_t m, double* logits, int32_t* ids,
                          float* w, float* g) {
  bfp::RouteArgs r;
  r.x = x; r.m = (int)m; r.hidden = (int)L->hidden;
  r.router_w = L->router_w; r.bias = L->router_bias; r.sh_gate_w = L->sh_gate_w;
  r.n_exp = L->n_experts; r.top_k = L->top_k;
  r.logits = logits; r.ld_logits = L->n_experts + 1;
  r.ids = ids; r.w = w; r.g = g;
  return r;
}

}  // namespace

extern "C" {

size_t bfp_moe_route_workspace_bytes(const bfp_moe_layer* L, int64_t m) {
  if (check_router(L) != BFP_OK || m < 1 || m > BFP_MOE_MAX_M) return 0;
  return layout(L, m, false).total;
}

int32_t bfp_moe_route(const bfp_moe_layer* L, const uint16_t* x, int64_t m, int32_t* ids, float* w, float* g,
                      void* ws, size_t ws_bytes, void* stream) {
  int32_t st = check_router(L);
  if (st != BFP_OK) return st;
  if (m < 1 || m > BFP_MOE_MAX_M) return BFP_E_SHAPE;
  if (m > BFP_GEMM_MAX_M && L->hidden % 64 != 0) return BFP_E_UNSUPPORTED;   // many-token router tiles
  if (!x || !ids || !w) return BFP_E_ARG;
  if (!aligned16(x)) return BFP_E_ALIGN;
  const Layout y = layout(L, m, false);
  if (!ws || ws_bytes < y.total) return BFP_E_WORKSPACE;
  if (!aligned16(ws)) return BFP_E_ALIGN;
  return from_hip(bfp::router_launch(route_args(L, x, m, at<double>(ws, y.logits), ids, w, g),
                                     static_cast<hipStream_t>(stream)));
}

int32_t bfp_moe_dispatch(const int32_t* ids, int64_t m, int32_t top_k, int32_t n_experts, int32_t* counts,
                         int32_t* offsets, int32_t* perm, void* stream) {
  if (!ids || !counts || !offsets || !perm) return BFP_E_ARG;
  if (m < 1 || m > BFP_MOE_MAX_M || top_k < 1 || top_k > 8 || n_experts < 1 || n_experts > 256 ||
      top_k > n_experts)
    return BFP_E_SHAPE;
  bfp::DispatchArgs d{};
  d.ids = ids; d.m = (int)m; d.top_k = top_k; d.n_exp = n_experts;
  d.counts = counts; d.offsets = offsets; d.perm = perm;
  return from_hip(bfp::dispatch_launch(d, static_cast<hipStream_t>(stream)));
}

size_t bfp_moe_workspace_bytes(const bfp_moe_layer* L, int64_t m) {
  if (check_layer(L) != BFP_OK || m < 1 || m > BFP_MOE_MAX_M) return 0;
  return layout(L, m, true).total;
}

}  // extern "C"

namespace {

// Host checks of bfp_moe_forward that do not involve the workspace.
int32_t check_forward(const bfp_moe_layer* L, const uint16_t* x, int64_t m, const float* y) {
  int32_t st = check_layer(L);
  if (st != BFP_OK) return st;
  if (m < 1 || m > BFP_MOE_MAX_M) return BFP_E_SHAPE;
  // many-token path: 256-column down tiles over hidden, 128-column gate/up tiles and 128-value
  // K steps over inter
  if (m > BFP_GEMM_MAX_M && (L->hidden % 256 != 0 || L->inter % 128 != 0 || !bfp::prefill_supported(L, m)))
    return BFP_E_UNSUPPORTED;
  if (!x || !y) return BFP_E_ARG;
  if (!aligned16(x) || !aligned16(y)) return BFP_E_ALIGN;
  return BFP_OK;
}

// Largest batch whose grouped path ends with the per-token down + combine kernel: it reads
// an expert's down rows once per (token, slot) instead of once per expert, which costs more
// than the combine launch it saves once experts are shared by many tokens.
constexpr int kTokDownMaxM = 8;

// The layer's kernels on a checked call; ws holds at least layout(L, m, true).total bytes.
int32_t moe_forward(const bfp_moe_layer* L, const uint16_t* x, int64_t m, float* y, int32_t* topk_ids,
                    float* topk_w, void* ws, hipStream_t s) {
  const Layout ly = layout(L, m, true);
  const bool shared = L->sh_gate.fmt != 0;
  int32_t* ids = topk_ids ? topk_ids : at<int32_t>(ws, ly.ids);
  float* w = topk_w ? topk_w : at<float>(ws, ly.w);
  float* g = at<float>(ws, ly.g);
  const bfp::RouteArgs r = route_args(L, x, m, at<double>(ws, ly.logits), ids, w, g);
  hipError_t e = hipSuccess;
  if (bfp::moe_tok_supported((int)m, L->top_k, (int)L->inter)) {
    // few tokens: router logits, then top-k + gate/up, then down + combine, per token
    if (bfp::router_logits_launch(r, s) != hipSuccess) return BFP_E_DEVICE;
    bfp::MoeTokArgs a{};
    a.logits = r.logits; a.ld_logits = r.ld_logits;
    a.m = (int)m; a.n_exp = L->n_experts; a.top_k = L->top_k; a.gate_row = L->sh_gate_w != nullptr;
    a.x = x; a.hidden = (int)L->hidden; a.inter = (int)L->inter;
    a.g_exp = L->gate.exp; a.g_code = L->gate.code; a.u_exp = L->up.exp; a.u_code = L->up.code;
    a.d_exp = L->down.exp; a.d_code = L->down.code;
    if (shared) {
      a.sg_exp = L->sh_gate.exp; a.sg_code = L->sh_gate.code; a.su_exp = L->sh_up.exp; a.su_code = L->sh_up.code;
      a.sd_exp = L->sh_down.exp; a.sd_code = L->sh_down.code;
    }
    a.ids = ids; a.w = w; a.g = g;
    a.h = at<float>(ws, ly.h); a.y = y;
    return from_hip(bfp::moe_tok_launch(a, s));
  }
  bfp::DispatchArgs d{};
  d.ids = ids; d.m = (int)m; d.top_k = L->top_k; d.n_exp = L->n_experts;
  d.counts = at<int32_t>(ws, ly.counts); d.offsets = at<int32_t>(ws, ly.offsets);
  d.perm = at<int32_t>(ws, ly.perm); d.inv = at<int32_t>(ws, ly.inv);
  d.active = at<int32_t>(ws, ly.active); d.n_active = at<int32_t>(ws, ly.nact);
  if (m > BFP_GEMM_MAX_M) {
    d.tile_m = bfp::prefill_tile_rows();
    d.with_shared = shared;
    d.tile_start = at<int32_t>(ws, ly.extra);
    d.chunk_counts = at<int32_t>(ws, ly.chunks);
  } else if (m > 1) {
    d.tile_m = bfp::kDecodeTileRows;
    d.with_shared = shared;
    d.tile_start = at<int32_t>(ws, ly.extra);
  }
  if (m > BFP_GEMM_MAX_M) {
    if ((e = bfp::router_launch(r, s)) != hipSuccess) return BFP_E_DEVICE;
    if ((e = bfp::dispatch_launch(d, s)) != hipSuccess) return BFP_E_DEVICE;
  } else if ((e = bfp::route_dispatch_launch(r, d, s)) != hipSuccess) {
    return BFP_E_DEVICE;
  }

  if (m > BFP_GEMM_MAX_M) {
    bfp::PrefillArgs p{};
    p.L = L; p.x = x; p.m = (int)m; p.y = y;
    p.w = w; p.g = shared ? g : nullptr; p.inv = d.inv; p.perm = d.perm; p.offsets = d.offsets;
    p.counts = d.counts; p.active = d.active; p.n_active = d.n_active;
    p.h = at<uint16_t>(ws, ly.h); p.o = at<float>(ws, ly.o);
    p.extra = d.tile_start;
    return from_hip(bfp::prefill_launch(p, s));
  }

  float* h = at<float>(ws, ly.h);
  float* o = at<float>(ws, ly.o);
  bfp::MoeGemvArgs gu{};
  gu.exp0 = L->gate.exp; gu.code0 = L->gate.code; gu.exp1 = L->up.exp; gu.code1 = L->up.code;
  if (shared) {
    gu.sexp0 = L->sh_gate.exp; gu.scode0 = L->sh_gate.code; gu.sexp1 = L->sh_up.exp; gu.scode1 = L->sh_up.code;
  }
  gu.rows_per_expert = (int)L->inter; gu.k = (int)L->hidden;
  gu.active = d.active; gu.n_active = d.n_active; gu.offsets = d.offsets; gu.perm = d.perm;
  gu.m = (int)m; gu.top_k = L->top_k;
  gu.x = x; gu.ldx = L->hidden; gu.x_by_token = 1; gu.x_bf16 = 1;
  gu.y = h; gu.ldy = L->inter; gu.y_bf16 = 0;
  gu.tile_start = d.tile_start; gu.tile_m = d.tile_m;
  if ((e = bfp::moe_gemv_launch(gu, 2, s)) != hipSuccess) return BFP_E_DEVICE;

  if (m <= kTokDownMaxM && L->inter <= 2048) {
    // down projection and combine per token (the combine's order, one launch fewer)
    bfp::MoeTokArgs a{};
    a.m = (int)m; a.n_exp = L->n_experts; a.top_k = L->top_k;
    a.hidden = (int)L->hidden; a.inter = (int)L->inter;
    a.d_exp = L->down.exp; a.d_code = L->down.code;
    if (shared) { a.sd_exp = L->sh_down.exp; a.sd_code = L->sh_down.code; }
    a.ids = ids; a.w = w; a.g = g;
    a.h = h; a.inv = d.inv; a.y = y;
    return from_hip(bfp::moe_tok_down_launch(a, s));
  }
  bfp::MoeGemvArgs dn = gu;
  dn.exp0 = L->down.exp; dn.code0 = L->down.code; dn.exp1 = nullptr; dn.code1 = nullptr;
  dn.sexp0 = shared ? L->sh_down.exp : nullptr; dn.scode0 = shared ? L->sh_down.code : nullptr;
  dn.sexp1 = nullptr; dn.scode1 = nullptr;
  dn.rows_per_expert = (int)L->hidden; dn.k = (int)L->inter;
  dn.x = h; dn.ldx = L->inter; dn.x_by_token = 0; dn.x_bf16 = 0;
  dn.y = o; dn.ldy = L->hidden; dn.y_bf16 = 0;
  if ((e = bfp::moe_gemv_launch(dn, 1, s)) != hipSuccess) return BFP_E_DEVICE;

  bfp::CombineArgs c{};
  c.o = o; c.inv = d.inv; c.w = w; c.g = shared ? g : nullptr;
  c.m = (int)m; c.top_k = L->top_k; c.hidden = (int)L->hidden; c.y = y;
  return from_hip(bfp::combine_launch(c, s));
}

// Scratch of bfp_moe_forward_noalloc: the decode workspace in a file-scope device array, one
// copy per device, held until the process ends. In host code `scratch` only names the symbol:
// its device address comes from hipGetSymbolAddress, once per device (with that device
// current), and only that address is handed to kernels.
__device__ __align__(256) unsigned char scratch[BFP_MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of the current device's scratch (looked up on the first call on a device).
int32_t scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return BFP_E_DEVICE;
  if (dev < 0 || dev >= kMaxDevices) return BFP_E_UNSUPPORTED;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return BFP_E_DEVICE;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return BFP_OK;
}

}  // namespace

extern "C" {

int32_t bfp_moe_forward_noalloc(const bfp_moe_layer* L, const uint16_t* x, int64_t m, float* y,
                                int32_t* topk_ids, float* topk_w, void* stream) {
  int32_t st = check_forward(L, x, m, y);
  if (st != BFP_OK) return st;
  if (m > BFP_GEMM_MAX_M) return BFP_E_UNSUPPORTED;
  if (layout(L, m, true).total > BFP_MOE_NOALLOC_SCRATCH_BYTES) return BFP_E_WORKSPACE;
  void* ws = nullptr;
  if ((st = scratch_address(&ws)) != BFP_OK) return st;
  return moe_forward(L, x, m, y, topk_ids, topk_w, ws, static_cast<hipStream_t>(stream));
}

int32_t bfp_moe_forward(const bfp_moe_layer* L, const uint16_t* x, int64_t m, float* y, int32_t* topk_ids,
                        float* topk_w, void* ws, size_t ws_bytes, void* stream) {
  int32_t st = check_forward(L, x, m, y);
  if (st != BFP_OK) return st;
  if (!ws || ws_bytes < layout(L, m, true).total) return BFP_E_WORKSPACE;
  if (!aligned16(ws)) return BFP_E_ALIGN;
  return moe_forward(L, x, m, y, topk_ids, topk_w, ws, static_cast<hipStream_t>(stream));
}

}  // extern "C"
