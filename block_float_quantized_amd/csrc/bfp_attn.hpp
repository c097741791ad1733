// Internal interface of the BFP KV cache kernels (append, decode attention): BFP8 K and V, or
// BFP8 K and 4-bit V after a Hadamard rotation.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace bfp {

struct KvAppendArgs {
  const void* k;               // [n][kv_heads][head_dim], fp32 or bf16
  const void* v;
  int src_bf16;
  int64_t n, pos;              // rows appended, first token slot
  int kv_heads, head_dim;
  int64_t max_tokens;
  uint8_t *k_exp, *k_code, *v_exp, *v_code;   // cache planes (K BFP8; V BFP8 or rotated BFP4)
  int v_rot4;                  // V rotated and stored in BFP4
};
hipError_t kv_append_launch(const KvAppendArgs& a, hipStream_t s);

struct AttnArgs {
  const uint8_t *k_exp, *k_code, *v_exp, *v_code;
  int kv_heads, head_dim;
  int64_t max_tokens;
  int v_rot4;
  const void* q;               // [q_heads][head_dim], fp32 or bf16
  int q_bf16;
  int q_heads;
  int L;                       // tokens attended
  float scale;
  float* out;                  // [q_heads][head_dim]
  float* ws;                   // attn_workspace_bytes
};
size_t attn_workspace_bytes(int kv_heads, int head_dim, int q_heads, int L);
bool attn_supported(int kv_heads, int head_dim, int q_heads);
hipError_t attn_decode_launch(const AttnArgs& a, hipStream_t s);

}  // namespace bfp
