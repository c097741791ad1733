/*
 * libbfp — block-floating-point (BFP4 / BFP8) weight-streaming matmuls for AMD MI355X (gfx950).
 *
 * The operations follow the model-card pages on the TT-native mixed BFP4/BFP8 Qwen
 * checkpoints:
 *  - "Qwen3.8-27B — TT-native mixed BFP4/BFP8 (GPTQ), single P150" (revision
 *    gptq-ctx2-20261002, "What changed in this release", GPTQ bullet): BFP4 matrices are
 *    made of 16-value blocks; values already representable re-encode bit for bit.
 *  - "Qwen3.6-35B-A3B — TT-native mixed BFP4/BFP8 (GPTQ experts), single P150"
 *    ("What is in this release", "Precision as served", "Fused decode kernels",
 *    "Verification"): routed and shared experts in BFP4, dense projections and the LM
 *    head in BFP8 (round to nearest), BF16 router, device top-k routing, BFP tensors
 *    converted bit-exactly by round to nearest.
 *  - "qwen3.6-a3b-blackhole" bundle page, introduction: a 256-expert top-8 MoE plus a
 *    shared expert in every layer.
 *  - "Qwen3.8-27B ..." ("What changed in this release (s27v6-20261024)", "Multi-user
 *    decode"): up to 32 rows share one pass over every weight; prefill in 2,048-token
 *    chunks.
 *
 * Format. A matrix W is stored [N][K] (N output rows, reduction along K, K a multiple of
 * 16) as two planes, row-major in block order:
 *   exp  : uint8 [N][K/16]   shared exponent E of each 16-value block
 *   code : BFP8 uint8 [N][K]   one byte per value, sign<<7 | magnitude (7 bits)
 *          BFP4 uint8 [N][K/2] value 2j in the low nibble of byte j, 2j+1 in the high
 *                              nibble, each nibble sign<<3 | magnitude (3 bits)
 * Value i of a block decodes to (-1)^sign_i * mag_i * 2^(E - 127 - (m - 1)), m = 7 or 3.
 * Encoding: E = the largest fp32 exponent field in the block; mag = |v| * 2^-(E-127-(m-1))
 * rounded to nearest, ties to even, clamped to 2^m - 1; the sign bit is copied (so -0.0
 * and values that round to 0 keep their sign). Inf/NaN are rejected.
 *
 * Conventions for every call:
 *  - Pointers named "device" are device memory owned by the caller; the library keeps no
 *    reference to them after the call returns. Host-side structs are read during the call.
 *  - `stream` is a hipStream_t (NULL = the default stream). Calls are stream-ordered and
 *    asynchronous except bfp_quantize, which synchronizes `stream` to report non-finite
 *    input.
 *  - Errors are returned as bfp_status codes; argument checks happen on the host before
 *    any launch, so an error means nothing was launched. No call aborts or throws.
 *  - Device pointers must be 16-byte aligned; leading dimensions are in elements.
 *  - Calls on different streams may run concurrently; calls that write the same output
 *    or workspace on different streams race.
 */
#ifndef LIBBFP_H
#define LIBBFP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  BFP_OK = 0,
  BFP_E_ARG = 1,          /* null pointer, unknown enum value, inconsistent struct */
  BFP_E_SHAPE = 2,        /* k not a multiple of 16, m or n out of range, mismatched shapes */
  BFP_E_ALIGN = 3,        /* a device pointer is not 16-byte aligned */
  BFP_E_NONFINITE = 4,    /* bfp_quantize met Inf or NaN (outputs are then unspecified) */
  BFP_E_WORKSPACE = 5,    /* workspace missing or smaller than the *_workspace_bytes query */
  BFP_E_DEVICE = 6,       /* a HIP runtime call or kernel launch failed */
  BFP_E_UNSUPPORTED = 7   /* a valid request this build does not implement */
} bfp_status;

enum { BFP_FMT_BFP4 = 4, BFP_FMT_BFP8 = 8 };
enum { BFP_DT_F32 = 0, BFP_DT_BF16 = 1 };
enum { BFP_EPI_NONE = 0, BFP_EPI_SWIGLU = 1 };
/*
 * Flag of bfp_gemm (or-ed into `epilogue`) and bfp_gemm_argmax: row i of the result is bit
 * for bit the same for every m in 1..BFP_GEMM_MAX_M, whatever the other rows hold
 * ("Qwen3.8-27B ...", "What changed in this release (s27v6-20261024)": each user's output in
 * a batch equals its single-user output bit for bit). Costs speed at m = 1 (the matrix-core
 * kernel runs where the vector kernel would be faster).
 */
#define BFP_GEMM_BATCH_INVARIANT 0x100

/* Non-owning view of one BFP matrix in device memory (layout above). */
typedef struct bfp_tensor {
  int32_t fmt;            /* BFP_FMT_BFP4 or BFP_FMT_BFP8; 0 marks an absent tensor */
  int64_t n;              /* rows (outputs) */
  int64_t k;              /* values per row, a multiple of 16 */
  const uint8_t *exp;     /* device, [n][k/16] */
  const uint8_t *code;    /* device, [n][k] (BFP8) or [n][k/2] (BFP4) */
} bfp_tensor;

/* Largest number of activation rows one bfp_gemm call streams the weights for. */
#define BFP_GEMM_MAX_M 32
/* Largest number of tokens one bfp_moe_forward call takes. */
#define BFP_MOE_MAX_M 8192

/* Library version (major*10000 + minor*100 + patch). */
int32_t bfp_version(void);

/* Human-readable name of a status code (a static string; never NULL). */
const char *bfp_status_str(int32_t status);

/* Bytes of the exponent plane of an n x k matrix: n * k / 16. */
size_t bfp_exp_bytes(int64_t n, int64_t k);

/* Bytes of the code plane: n * k (BFP8) or n * k / 2 (BFP4); 0 for an unknown format. */
size_t bfp_code_bytes(int32_t fmt, int64_t n, int64_t k);

/*
 * Encode (round to nearest, ties to even; see Format). w: device fp32 [n][ldw], the first k
 * values of each row are encoded (ldw >= k, ldw a multiple of 4 so that rows stay 16-byte
 * aligned; else BFP_E_SHAPE / BFP_E_ALIGN). exp, code: device outputs sized by bfp_exp_bytes /
 * bfp_code_bytes, written densely ([n][k/16] and [n][k] or [n][k/2]). Bit-exact: the same
 * input gives the same bytes on every run and device ("Qwen3.6-35B-A3B ...",
 * "Verification": the round-to-nearest conversion is bit-exact; "Qwen3.8-27B ...",
 * gptq-ctx2-20261002, "What changed in this release": values already representable
 * re-encode bit for bit). Synchronizes `stream`; returns BFP_E_NONFINITE if any input value
 * is Inf or NaN.
 */
int32_t bfp_quantize(int32_t fmt, const float *w, int64_t n, int64_t k, int64_t ldw,
                     uint8_t *exp, uint8_t *code, void *stream);

/*
 * Decode a whole matrix: out[n][k] = (-1)^sign * mag * 2^s, exact, in fp32
 * (out_dtype = BFP_DT_F32) or bf16 (BFP_DT_BF16; every BFP value is bf16-representable),
 * for every shared exponent E. The inverse of bfp_quantize on the values it represents
 * ("Qwen3.6-35B-A3B ...", "Verification": BFP tensors re-derived on the CPU and compared bit
 * for bit). out: device [n][k], 16-byte aligned.
 */
int32_t bfp_dequantize(const bfp_tensor *w, int32_t out_dtype, void *out, void *stream);

/*
 * Workspace bytes bfp_gemm needs for an m-row call on w (with w_up for SWIGLU, else NULL),
 * with or without BFP_GEMM_BATCH_INVARIANT; 0 when it needs none. Depends on the shapes only
 * (not on pointers or values).
 */
size_t bfp_gemm_workspace_bytes(const bfp_tensor *w, const bfp_tensor *w_up, int64_t m);

/*
 * Skinny matmul over streamed BFP weights, dequantized in registers ("Qwen3.6-35B-A3B ...",
 * "Precision as served": dense projections and LM head in BFP8, experts in BFP4; "Speed":
 * decode cost follows the weight bytes read; "Qwen3.8-27B ...", "What changed in this
 * release (s27v6-20261024)" and "Multi-user decode": up to 32 rows share one pass over every
 * weight, the MLP being gate/up with SwiGLU then down):
 *   epilogue NONE  : y[i][j] = sum_k x[i][k] * W[j][k]
 *   epilogue SWIGLU: y[i][j] = silu(sum_k x[i][k] * W[j][k]) * (sum_k x[i][k] * Wup[j][k])
 * with silu(g) = g / (1 + e^-g). i < m (1..BFP_GEMM_MAX_M rows share one pass over the
 * weights), j < w->n, k < w->k. x: device [m][ldx] of x_dtype (bf16 or fp32); y: device
 * [m][ldy] of y_dtype (fp32, or bf16 rounded to nearest even). Products of bf16 x with the
 * weights are exact and sums are fp32. m = 1 runs on the vector ALUs (fp32 x exact as well);
 * m >= 2 runs on the bf16 matrix cores, where fp32 x enters as the sum of two bf16 values
 * (about 16 significant bits) and row i of the result does not depend on m or on the other
 * rows (same reduction order for every m in 2..32). With BFP_GEMM_BATCH_INVARIANT or-ed into
 * `epilogue`, m = 1 runs on the matrix cores too, so that row i is the same for every m in
 * 1..32; other bits of `epilogue` above the low byte give BFP_E_ARG. w_up must be NULL for
 * NONE and match w's format and shape for SWIGLU. ws: device workspace of at least bfp_gemm_workspace_bytes(w, w_up, m) bytes (may
 * be NULL when that is 0; BFP_E_WORKSPACE if missing or smaller), 16-byte aligned, contents
 * on entry and on return unspecified. Calls sharing a workspace on different streams race.
 */
int32_t bfp_gemm(const bfp_tensor *w, const bfp_tensor *w_up, int32_t epilogue,
                 const void *x, int32_t x_dtype, int64_t m, int64_t ldx,
                 void *y, int32_t y_dtype, int64_t ldy, void *ws, size_t ws_bytes,
                 void *stream);

/* Workspace bytes bfp_gemm_argmax needs for an m-row call on w, with or without
 * BFP_GEMM_BATCH_INVARIANT (0 if w or m is invalid). */
size_t bfp_gemm_argmax_workspace_bytes(const bfp_tensor *w, int64_t m);

/*
 * Greedy pick over the outputs of a skinny matmul ("Qwen3.6-35B-A3B ...", "Fused decode
 * kernels": greedy argmax on the tiled LM-head logits, with no vocabulary-wide copy of
 * them). With y[i][j] the fp32 result bfp_gemm(w, NULL, BFP_EPI_NONE | flags, x,
 * BFP_DT_BF16, m, ...) would write, for every row i < m:
 *   idx[i] = the smallest j < w->n with y[i][j] maximal, NaN counting as larger than any
 *            number (the first NaN wins) and -0 as equal to +0;
 *   val[i] = y[i][idx[i]] (a -0 reported as +0, a NaN as the quiet NaN 0x7fc00000).
 * y itself is never written: each workgroup of the matmul reduces its own columns to one
 * candidate per row, and a second kernel reduces the candidates of each row. The outputs
 * are bit for bit those of this rule applied to bfp_gemm's y for the same m and flags.
 * flags: 0 or BFP_GEMM_BATCH_INVARIANT (other bits give BFP_E_ARG). x: device bf16
 * [m][ldx] (BFP_DT_F32 gives BFP_E_UNSUPPORTED); m in 1..BFP_GEMM_MAX_M; idx: device
 * int32 [m]; val: device fp32 [m]; ws: device workspace of at least
 * bfp_gemm_argmax_workspace_bytes(w, m) bytes (BFP_E_WORKSPACE if smaller), 16-byte
 * aligned, contents on entry and on return unspecified.
 */
int32_t bfp_gemm_argmax(const bfp_tensor *w, const void *x, int32_t x_dtype, int64_t m,
                        int64_t ldx, int32_t flags, int32_t *idx, float *val, void *ws,
                        size_t ws_bytes, void *stream);

/*
 * One MoE layer with BFP4 experts ("qwen3.6-a3b-blackhole", introduction; "Qwen3.6-35B-A3B
 * ...", "Precision as served" and "Fused decode kernels").
 * Routed experts are stacked along the rows: gate and up have n = n_experts * inter,
 * k = hidden (expert e owns rows [e*inter, (e+1)*inter)); down has n = n_experts * hidden,
 * k = inter. The shared expert has the same shapes for a single expert; set sh_gate.fmt = 0
 * for none. router_w: device bf16 [n_experts][hidden]; router_bias: device fp32
 * [n_experts] or NULL; sh_gate_w: device bf16 [hidden] (shared-expert sigmoid gate) or
 * NULL for a gate of 1.
 */
typedef struct bfp_moe_layer {
  int32_t n_experts;      /* routed experts, 1..256 */
  int32_t top_k;          /* experts per token, 1..8 */
  int64_t hidden;         /* model width (multiple of 32) */
  int64_t inter;          /* expert width (multiple of 32) */
  const uint16_t *router_w;
  const float *router_bias;
  bfp_tensor gate, up, down;
  bfp_tensor sh_gate, sh_up, sh_down;
  const uint16_t *sh_gate_w;
} bfp_moe_layer;

/* Workspace bytes bfp_moe_route needs for m tokens (the fp64 router logits). */
size_t bfp_moe_route_workspace_bytes(const bfp_moe_layer *L, int64_t m);

/*
 * Routing step of bfp_moe_forward, exposed on its own ("Qwen3.6-35B-A3B ...", "Precision as
 * served": BF16 router; "Fused decode kernels": device top-k routing; "qwen3.6-a3b-blackhole",
 * introduction: 256 experts, top-8, a shared expert). For each token t < m:
 *   l_e = sum_k x[t][k] * router_w[e][k] (+ router_bias[e]), exact bf16 products summed
 *         in fp64;
 *   ids[t][0..top_k) = the top_k experts by (l descending, e ascending), in that order;
 *   w[t][j] = softmax over all experts restricted to the selection and renormalised
 *             (= exp(l_ej - l_max) / sum over the selection), fp32;
 *   g[t] = sigmoid(x[t] . sh_gate_w) (1 if sh_gate_w is NULL), fp32.
 * x: device bf16 [m][hidden]; ids: device int32 [m][top_k]; w: device fp32 [m][top_k];
 * g: device fp32 [m] or NULL; ws: device workspace of at least
 * bfp_moe_route_workspace_bytes(L, m) bytes. Only the router fields of L are read.
 * m > BFP_GEMM_MAX_M needs hidden % 64 == 0 (else BFP_E_UNSUPPORTED). Non-finite inputs:
 * a NaN logit ranks below every number, so ids always hold top_k distinct experts in
 * [0, n_experts) in the rule's order; the weights of such a token are unspecified.
 */
int32_t bfp_moe_route(const bfp_moe_layer *L, const uint16_t *x, int64_t m,
                      int32_t *ids, float *w, float *g, void *ws, size_t ws_bytes, void *stream);

/*
 * Dispatch structure for expert-grouped execution (counting sort by expert), the grouping of
 * "batched expert streams" ("Qwen3.6-35B-A3B ...", "Fused decode kernels") and of a
 * 2,048-token prefill chunk run expert by expert ("Qwen3.8-27B ...", s27v6 bullets):
 *   counts[e]  = number of (token, slot) pairs routed to expert e;
 *   offsets[e] = sum of counts below e (n_experts + 1 entries, offsets[n_experts] = m*top_k);
 *   perm[p]    = pair ids top_k*t + j ordered by (expert ascending, token ascending).
 * ids: device int32 [m][top_k], every entry in [0, n_experts) and distinct within a row.
 * counts: device int32 [n_experts]; offsets: device int32 [n_experts + 1];
 * perm: device int32 [m * top_k]. Bit-exact (integer work).
 */
int32_t bfp_moe_dispatch(const int32_t *ids, int64_t m, int32_t top_k, int32_t n_experts,
                         int32_t *counts, int32_t *offsets, int32_t *perm, void *stream);

/* Workspace bytes bfp_moe_forward needs for m tokens (0 if the layer or m is invalid). */
size_t bfp_moe_workspace_bytes(const bfp_moe_layer *L, int64_t m);

/*
 * Full MoE layer: y[t] = sum_j w[t][j] * Down_ej(silu(Gate_ej x_t) * Up_ej x_t)
 *                        + g[t] * Shared(x_t),
 * routing as in bfp_moe_route. Every selected expert's weights are streamed once per call
 * for all tokens that chose it. m <= 32 runs the skinny decode path (h = silu(gate)*up kept
 * in fp32); larger m runs the prefill path, where tokens are grouped by expert and h is
 * rounded to bf16 (nearest even) before the down projection, which is then a bf16
 * matrix-core product with fp32 accumulation; it needs hidden % 256 == 0 and inter % 128 == 0
 * (else BFP_E_UNSUPPORTED).
 * x: device bf16 [m][hidden]; y: device fp32 [m][hidden]; topk_ids / topk_w: optional
 * device outputs [m][top_k] (NULL to skip); ws: device workspace of at least
 * bfp_moe_workspace_bytes(L, m) bytes (contents on return unspecified).
 */
int32_t bfp_moe_forward(const bfp_moe_layer *L, const uint16_t *x, int64_t m, float *y,
                        int32_t *topk_ids, float *topk_w, void *ws, size_t ws_bytes,
                        void *stream);

/*
 * bfp_moe_forward for decode (1..BFP_GEMM_MAX_M tokens) without a caller workspace and
 * without any allocation, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc). Same kernels and same
 * results, bit for bit, as bfp_moe_forward with a workspace. The workspace is a scratch array
 * of BFP_MOE_NOALLOC_SCRATCH_BYTES in the library's device code, one per device (held until
 * the process ends; its address is looked up on the first call on a device). Every call on a
 * device shares that device's scratch: calls that overlap on one device (other streams,
 * other host threads) race and must be serialised by the caller. Nothing in it needs to start
 * at zero. Errors: m > BFP_GEMM_MAX_M gives BFP_E_UNSUPPORTED; a layer whose decode
 * workspace (bfp_moe_workspace_bytes(L, m)) exceeds BFP_MOE_NOALLOC_SCRATCH_BYTES gives
 * BFP_E_WORKSPACE; all other arguments as bfp_moe_forward.
 */
#define BFP_MOE_NOALLOC_SCRATCH_BYTES (8u << 20)
int32_t bfp_moe_forward_noalloc(const bfp_moe_layer *L, const uint16_t *x, int64_t m, float *y,
                                int32_t *topk_ids, float *topk_w, void *stream);

/*
 * BFP8 KV cache for decode attention ("Qwen3.6-35B-A3B ...", "Precision as served": the KV
 * cache is BFP8; serving-settings table, KV-precision row: BFP8 halves the cache, 20.0 ->
 * 10.6 KiB per token, and decode attention, which reads the whole cache every step, gets
 * faster at long contexts). Every cached key or value vector (one token, one KV head,
 * head_dim values) is a BFP8 row encoded exactly as bfp_quantize encodes a weight row.
 * Layout (device memory owned by the caller), for K and for V alike:
 *   exp  : uint8 [kv_heads][max_tokens][head_dim/16]  (bfp_exp_bytes(kv_heads*max_tokens, head_dim))
 *   code : uint8 [kv_heads][max_tokens][head_dim]     (bfp_code_bytes(BFP_FMT_BFP8, ...))
 *
 * v_format BFP_KV_V_BFP4_HADAMARD is the long-context cache of "Qwen3.8-27B — TT-native mixed
 * BFP4/BFP8 (GPTQ)", changes in s27-20261005 (DFlash2 at 262K): K stays BFP8, V is stored in
 * 4-bit BFP4 after a Hadamard rotation. Each value vector v is replaced by H v / sqrt(head_dim)
 * (H the Sylvester Hadamard matrix, H_2n = [[H, H], [H, -H]]), computed in fp64 by the fast
 * transform (stages of span 1, 2, 4, ...: x_j, x_j+s <- x_j + x_j+s, x_j - x_j+s), times the
 * double nearest 1/sqrt(head_dim), rounded to fp32, then BFP4-encoded as bfp_quantize does. V
 * code plane: uint8 [kv_heads][max_tokens][head_dim/2] (value 2j in the low nibble of byte j).
 * The rotation is orthonormal and its own inverse: bfp_attn_decode rotates its output back.
 */
#define BFP_KV_V_BFP8 0
#define BFP_KV_V_BFP4_HADAMARD 1
typedef struct bfp_kv_cache {
  int32_t kv_heads;       /* 1..64 */
  int32_t head_dim;       /* 64, 128 or 256 */
  int64_t max_tokens;     /* token slots, 1..2^24 */
  uint8_t *k_exp, *k_code, *v_exp, *v_code;
  int32_t v_format;       /* BFP_KV_V_BFP8 (0) or BFP_KV_V_BFP4_HADAMARD */
} bfp_kv_cache;

/*
 * Encode n new tokens into slots pos .. pos+n-1 of every KV head. k, v: device
 * [n][kv_heads][head_dim] of dtype (fp32, or bf16 converted exactly). Inputs must be finite
 * (Inf/NaN, or a rotated value beyond the fp32 range, leave unspecified codes; no
 * synchronisation, unlike bfp_quantize). pos + n must not exceed max_tokens.
 */
int32_t bfp_kv_append(const bfp_kv_cache *c, const void *k, const void *v, int32_t dtype,
                      int64_t pos, int64_t n, void *stream);

/* Workspace bytes of bfp_attn_decode (0 if the arguments are invalid). */
size_t bfp_attn_decode_workspace_bytes(const bfp_kv_cache *c, int32_t q_heads, int64_t seq_len);

/*
 * Single-token decode attention over the first seq_len cached tokens, for one sequence:
 *   query head h reads KV head h / (q_heads / kv_heads);
 *   s_t = scale * q[h] . K[t] (decoded keys), p = softmax over t < seq_len,
 *   out[h] = sum_t p_t V[t] (decoded values; with BFP_KV_V_BFP4_HADAMARD the decoded rotated
 *   values, the sum rotated back by the same transform in fp32).
 * q: device [q_heads][head_dim], fp32 or bf16 (q_dtype); out: device fp32
 * [q_heads][head_dim]. q_heads / kv_heads must be 1, 2, 4 or 8 (else BFP_E_UNSUPPORTED).
 * Sums are fp32 (exp via the hardware exp2). With 8 query heads per KV head the products run
 * on the bf16 matrix instructions: cached values are exact in bf16, the scaled query is the sum
 * of three bf16 parts (~24 significant bits) and the probabilities of two (~16); otherwise the
 * products are fp32. The sequence is split into chunks merged in a fixed order, so results are
 * deterministic. ws: device workspace of at least bfp_attn_decode_workspace_bytes bytes.
 */
int32_t bfp_attn_decode(const bfp_kv_cache *c, const void *q, int32_t q_dtype, int32_t q_heads,
                        int64_t seq_len, float scale, float *out, void *ws, size_t ws_bytes,
                        void *stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBBFP_H */
