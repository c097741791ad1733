// C ABI of the BFP KV cache (BFP8 K and V, or BFP8 K and rotated BFP4 V): argument checks for append and decode attention.
#include <hip/hip_runtime.h>

#include "../../include/libbfp.h"
#include "bfp_attn.hpp"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int32_t check_cache(const bfp_kv_cache* c) {
  if (!c) return BFP_E_ARG;
  if (c->kv_heads < 1 || c->kv_heads > 64 || c->max_tokens < 1 || c->max_tokens > (int64_t)1 << 24) return BFP_E_SHAPE;
  if (c->head_dim != 64 && c->head_dim != 128 && c->head_dim != 256) return BFP_E_SHAPE;
  if (!c->k_exp || !c->k_code || !c->v_exp || !c->v_code) return BFP_E_ARG;
  if (c->v_format != BFP_KV_V_BFP8 && c->v_format != BFP_KV_V_BFP4_HADAMARD) return BFP_E_ARG;
  if (!aligned16(c->k_code) || !aligned16(c->v_code)) return BFP_E_ALIGN;
  return BFP_OK;
}

int32_t from_hip(hipError_t e) { return e == hipSuccess ? BFP_OK : BFP_E_DEVICE; }

}  // namespace

extern "C" {

int32_t bfp_kv_append(const bfp_kv_cache* c, const void* k, const void* v, int32_t dtype, int64_t pos, int64_t n,
                      void* stream) {
  int32_t st = check_cache(c);
  if (st != BFP_OK) return st;
  if (dtype != BFP_DT_F32 && dtype != BFP_DT_BF16) return BFP_E_ARG;
  if (!k || !v) return BFP_E_ARG;
  if (n < 0 || pos < 0 || pos + n > c->max_tokens) return BFP_E_SHAPE;
  if (!aligned16(k) || !aligned16(v)) return BFP_E_ALIGN;
  bfp::KvAppendArgs a{};
  a.k = k; a.v = v; a.src_bf16 = dtype == BFP_DT_BF16;
  a.n = n; a.pos = pos;
  a.kv_heads = c->kv_heads; a.head_dim = c->head_dim; a.max_tokens = c->max_tokens;
  a.k_exp = c->k_exp; a.k_code = c->k_code; a.v_exp = c->v_exp; a.v_code = c->v_code;
  a.v_rot4 = c->v_format == BFP_KV_V_BFP4_HADAMARD;
  return from_hip(bfp::kv_append_launch(a, static_cast<hipStream_t>(stream)));
}

size_t bfp_attn_decode_workspace_bytes(const bfp_kv_cache* c, int32_t q_heads, int64_t seq_len) {
  if (check_cache(c) != BFP_OK || seq_len < 1 || seq_len > c->max_tokens) return 0;
  if (!bfp::attn_supported(c->kv_heads, c->head_dim, q_heads)) return 0;
  return bfp::attn_workspace_bytes(c->kv_heads, c->head_dim, q_heads, (int)seq_len);
}

int32_t bfp_attn_decode(const bfp_kv_cache* c, const void* q, int32_t q_dtype, int32_t q_heads, int64_t seq_len,
                        float scale, float* out, void* ws, size_t ws_bytes, void* stream) {
  int32_t st = check_cache(c);
  if (st != BFP_OK) return st;
  if (q_dtype != BFP_DT_F32 && q_dtype != BFP_DT_BF16) return BFP_E_ARG;
  if (!q || !out || !ws) return BFP_E_ARG;
  if (q_heads < 1 || q_heads % c->kv_heads != 0) return BFP_E_SHAPE;
  if (!bfp::attn_supported(c->kv_heads, c->head_dim, q_heads)) return BFP_E_UNSUPPORTED;
  if (seq_len < 1 || seq_len > c->max_tokens) return BFP_E_SHAPE;
  if (!(scale == scale) || scale == __builtin_inff() || scale == -__builtin_inff()) return BFP_E_ARG;
  if (!aligned16(q) || !aligned16(out) || !aligned16(ws)) return BFP_E_ALIGN;
  if (ws_bytes < bfp::attn_workspace_bytes(c->kv_heads, c->head_dim, q_heads, (int)seq_len)) return BFP_E_WORKSPACE;
  bfp::AttnArgs a{};
  a.k_exp = c->k_exp; a.k_code = c->k_code; a.v_exp = c->v_exp; a.v_code = c->v_code;
  a.kv_heads = c->kv_heads; a.head_dim = c->head_dim; a.max_tokens = c->max_tokens;
  a.v_rot4 = c->v_format == BFP_KV_V_BFP4_HADAMARD;
  a.q = q; a.q_bf16 = q_dtype == BFP_DT_BF16; a.q_heads = q_heads;
  a.L = (int)seq_len; a.scale = scale; a.out = out; a.ws = static_cast<float*>(ws);
  return from_hip(bfp::attn_decode_launch(a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
