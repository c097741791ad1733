// Internal interface of the MoE kernels (routing, dispatch, grouped expert matmuls, combine).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bfp {

struct RouteArgs {
  const uint16_t* x;           // bf16 [m][hidden]
  int m, hidden;
  const uint16_t* router_w;    // bf16 [n_exp][hidden]
  const float* bias;           // fp32 [n_exp] or null
  const uint16_t* sh_gate_w;   // bf16 [hidden] or null
  int n_exp, top_k;
  double* logits;              // fp64 [m][ld_logits] (n_exp + 1 columns)
  int ld_logits;
  int32_t* ids;                // [m][top_k]
  float* w;                    // [m][top_k]
  float* g;                    // [m] or null
};
// Bytes of the logits workspace region for m tokens (shared by both routing methods).
size_t route_workspace_bytes(int m, int n_exp);
hipError_t router_launch(const RouteArgs& a, hipStream_t s);

struct DispatchArgs {
  const int32_t* ids;          // [m][top_k]
  int m, top_k, n_exp;
  int32_t* counts;             // [n_exp]
  int32_t* offsets;            // [n_exp + 1]
  int32_t* perm;               // [m * top_k]
  int32_t* inv;                // [m * top_k] position of each pair in perm, or null
  int32_t* active;             // [n_exp] experts with count > 0, ascending, or null
  int32_t* n_active;           // [1] or null
  int tile_m;                  // > 0: also write tile_start for row tiles of tile_m rows
  int with_shared;             // the tile list ends with a group of all m tokens
  int32_t* tile_start;         // [n_exp + 2]: first row tile of each group, then the total
  int32_t* chunk_counts;       // dispatch_scratch_bytes(m) of scratch: many-token sort over several
                               // workgroups; null: one workgroup
};
size_t dispatch_scratch_bytes(int m);
hipError_t dispatch_launch(const DispatchArgs& a, hipStream_t s);
// Decode (m <= 32): the router logits alone (fp64, n_exp + 1 columns per token).
hipError_t router_logits_launch(const RouteArgs& a, hipStream_t s);
// Decode (m <= 32): the router logits, then top-k and dispatch in one single-workgroup kernel
// (router_launch + dispatch_launch with one launch fewer; d.ids must be r.ids).
hipError_t route_dispatch_launch(const RouteArgs& r, const DispatchArgs& d, hipStream_t s);

// Expert-grouped skinny matmul for decode: workgroup row y picks the y-th active expert (or
// the shared expert right after the active ones) and streams that expert's rows once for all
// of its (token, slot) pairs.
struct MoeGemvArgs {
  const uint8_t *exp0, *code0, *exp1, *code1;       // routed experts, stacked along rows
  const uint8_t *sexp0, *scode0, *sexp1, *scode1;   // shared expert (null: none)
  int rows_per_expert;                              // N of one expert
  int k;                                            // K
  const int32_t* active;
  const int32_t* n_active;
  const int32_t* offsets;
  const int32_t* perm;
  int m, top_k;
  const void* x;                                    // x bf16 [m][k] (by token) or h fp32 [pairs][k]
  int64_t ldx;
  int x_by_token;                                   // 1: read the pair's token row, 0: its position row
  int x_bf16;
  void* y;                                          // [pairs][ldy], row = pair position
  int64_t ldy;
  int y_bf16;
  const int32_t* tile_start;                        // non-null: the groups cut into row tiles of
  int tile_m;                                       // tile_m pairs (dispatch's list), one per
                                                    // workgroup row; null: one group per row
};
// Row-tile height of the decode expert kernels when m > 1 (a kernel built for more rows per
// group holds more registers, and almost every group has one or two pairs).
constexpr int kDecodeTileRows = 2;
hipError_t moe_gemv_launch(const MoeGemvArgs& a, int nmat, hipStream_t s);

struct CombineArgs {
  const float* o;              // [m*top_k + m][hidden] per-pair expert outputs (+ shared rows)
  const int32_t* inv;          // [m*top_k]
  const float* w;              // [m][top_k]
  const float* g;              // [m] (shared gate) or null when there is no shared expert
  int m, top_k, hidden;
  float* y;                    // [m][hidden]
};
hipError_t combine_launch(const CombineArgs& a, hipStream_t s);

// Per-token path, two launches after the router logits: (1) every workgroup of the gate/up
// grid ranks its token's experts itself from the logits and streams its rows of the expert of
// its (token, slot) (slot top_k: the shared expert); one per token also writes that token's
// ids, w and g; (2) each workgroup of the down grid computes a few output columns of every
// slot of one token and combines them. No dispatch, no per-pair outputs: an expert chosen by
// several tokens is streamed once per token. The per-row arithmetic is that of the grouped
// kernels above (same tile, same lane split and order), so a token's output does not depend on
// the batch size or on which path ran.
struct MoeTokArgs {
  const double* logits;                             // [m][ld_logits] (column n_exp: shared gate)
  int ld_logits;
  int m, n_exp, top_k;
  int gate_row;                                     // a shared-gate logit is present
  const uint16_t* x;                                // bf16 [m][hidden]
  int hidden, inter;
  const uint8_t *g_exp, *g_code, *u_exp, *u_code, *d_exp, *d_code;       // routed, stacked
  const uint8_t *sg_exp, *sg_code, *su_exp, *su_code, *sd_exp, *sd_code; // shared (null: none)
  int32_t* ids;                                     // [m][top_k], rank order
  float* w;                                         // [m][top_k]
  float* g;                                         // [m] (written when there is a shared expert)
  float* h;                                         // fp32 h rows, see inv
  const int32_t* inv;                               // null: h row of (t, d) is t (top_k + 1) + d;
                                                    // else inv[t top_k + d], and m top_k + t for
                                                    // the shared expert (the grouped kernels' rows)
  float* y;                                         // fp32 [m][hidden]
};
// Largest batch the per-token path takes (beyond it the grouped kernels read each selected
// expert once for all of its tokens).
constexpr int kTokPathMaxM = 4;
// Whether the per-token kernels take this call (the down kernel stages every slot's h row).
bool moe_tok_supported(int m, int top_k, int inter);
hipError_t moe_tok_launch(const MoeTokArgs& a, hipStream_t s);
// The per-token down + combine kernel alone, on h rows written by the grouped gate/up kernel
// (a.inv set): the grouped path's last two launches in one (m <= 32, inter <= 2048).
hipError_t moe_tok_down_launch(const MoeTokArgs& a, hipStream_t s);

}  // namespace bfp
