// BFP KV cache for decode attention (gfx950): append (encode) and single-token attention.
//
// "Qwen3.6-35B-A3B — TT-native mixed BFP4/BFP8", "Precision as served" (the KV cache is BFP8)
// and the serving-settings table, KV-precision row: BFP8 halves the cache (20.0 -> 10.6 KiB
// per token) and, because decode attention reads the whole cache every step, speeds it up at
// long contexts. Each cached key or value vector (one token, one KV head) is encoded like a
// weight row: 16-value blocks along head_dim with the weights' exact rounding (bfp_encode.hpp).
//
// The long-context cache ("Qwen3.8-27B — TT-native mixed BFP4/BFP8 (GPTQ)", changes in
// s27-20261005, DFlash2 at 262K) keeps K in BFP8 and stores V in BFP4 after a Hadamard
// rotation: v -> H v / sqrt(head_dim), H the Sylvester matrix, by the fast transform in fp64
// (one wave per row, stages of span below the values per lane in registers, the rest across
// lanes), rounded to fp32 and encoded. Attention then runs over the rotated values; the
// transform is linear, orthonormal and its own inverse, so each chunk's partial sum is rotated
// back (in fp32, in LDS) before the merge.
//
// Decode attention is split over the sequence (a workgroup per KV head and chunk of tokens); the
// G query heads of a KV head share every key and value row read from HBM. Each chunk yields
// its maximum m_c, sum l_c of exp(s - m_c) and unnormalised o_c = sum_t exp(s_t - m_c) v_t;
// attn_merge_kernel combines them, out = sum_c e^(m_c - M) o_c / sum_c e^(m_c - M) l_c.
// Every order is fixed, so results do not depend on scheduling. Two chunk kernels:
//  * G = 8 (attn_chunk_mfma_kernel): both products on the bf16 matrix instructions;
//  * G = 1, 2, 4 (attn_chunk_kernel): fp32 FMAs, head_dim / 8 lanes per cached row (8 values
//    each), a lane-group reduction per score, scores staged in LDS.
#include "bfp_attn.hpp"
#include "bfp_device.hpp"
#include "bfp_encode.hpp"

namespace bfp {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

// Magnitudes of the four BFP8 codes of c as fp32 (v_cvt_f32_ubyte0..3 of the masked word; the
// mask is opaque to the compiler so that it keeps the byte conversions).
__device__ __forceinline__ void mag4_bfp8(uint32_t c, float m[4]) {
  uint32_t t;
  asm("v_and_b32 %0, 0x7f7f7f7f, %1" : "=v"(t) : "v"(c));
  m[0] = (float)(t & 0xffu);
  m[1] = (float)((t >> 8) & 0xffu);
  m[2] = (float)((t >> 16) & 0xffu);
  m[3] = (float)(t >> 24);
}
// bf16 pair (lo = a, hi = b) of two fp32 values exact in bf16, with the sign bits of code bytes
// sa of ca and sb of cb (byte selectors of v_perm: sa in 0..3 of ca, sb in 4..7 of cb).
__device__ __forceinline__ uint32_t signed_pair(float a, float b, uint32_t ca, uint32_t cb, uint32_t sel) {
  const uint32_t p = __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u);
  return p ^ (__builtin_amdgcn_perm(cb, ca, sel) & 0x80008000u);
}
// selector placing byte ka of the low source at byte 1 and byte kb (4..7: of the high source)
// at byte 3, zeros elsewhere
__device__ __forceinline__ constexpr uint32_t sign_sel(int ka, int kb) {
  return ((uint32_t)kb << 24) | (0x0cu << 16) | ((uint32_t)ka << 8) | 0x0cu;
}

// ---- append ----------------------------------------------------------------------------

// One thread per 16-value block of K or V: rows [n][kv_heads][head_dim] -> token slots
// pos .. pos + n - 1 of every KV head.
// With v_rot4 only K is encoded here (kv_append_v4r_kernel writes V).
__global__ __launch_bounds__(256) void kv_append_kernel(KvAppendArgs a) {
  const int nb = a.head_dim / kBlock;
  const int64_t per = a.n * a.kv_heads * nb;
  int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (a.v_rot4 ? per : 2 * per)) return;
  const bool is_v = idx >= per;
  if (is_v) idx -= per;
  const int b = (int)(idx % nb);
  const int64_t r = idx / nb;                    // source row: token i, head g
  const int g = (int)(r % a.kv_heads);
  const int64_t i = r / a.kv_heads;
  uint32_t u[16];
  if (a.src_bf16) {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(is_v ? a.v : a.k) + r * a.head_dim +
                                                    b * kBlock);
    const uint4 lo = p[0], hi = p[1];
    const uint32_t w[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      u[2 * j] = w[j] << 16;
      u[2 * j + 1] = w[j] & 0xffff0000u;
    }
  } else {
    const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const float*>(is_v ? a.v : a.k) + r * a.head_dim +
                                                    b * kBlock);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u32x4 v = p[j];
      u[4 * j] = v.x; u[4 * j + 1] = v.y; u[4 * j + 2] = v.z; u[4 * j + 3] = v.w;
    }
  }
  const int64_t row = (int64_t)g * a.max_tokens + a.pos + i;
  uint8_t* exp = (is_v ? a.v_exp : a.k_exp) + row * nb + b;
  uint8_t* code = (is_v ? a.v_code : a.k_code) + (row * nb + b) * kBlock;
  encode_block<8>(u, exp, code);
}

// The double nearest 1 / sqrt(HD), and its fp32 rounding for the back rotation.
template <int HD>
constexpr double kInvSqrtHd = HD == 64 ? 0.125 : HD == 128 ? 0.08838834764831845 : 0.0625;

constexpr int kV4rWaves = 4;

// One wave per V row (token i, KV head g; rows past n idle): H v / sqrt(HD) in fp64, lane l
// holding elements l P .. l P + P - 1; rounded to fp32, staged in LDS, and encoded in BFP4 by
// HD / 16 lanes (one block each).
template <int HD>
__global__ __launch_bounds__(kV4rWaves * kWave) void kv_append_v4r_kernel(KvAppendArgs a) {
  constexpr int P = HD / kWave;
  constexpr int NB = HD / kBlock;
  __shared__ uint32_t rot[kV4rWaves][HD];
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int64_t r = (int64_t)blockIdx.x * kV4rWaves + wave;        // source row i * kv_heads + g
  const bool valid = r < a.n * a.kv_heads;
  const int64_t rr = valid ? r : 0;
  double x[P];
  if (a.src_bf16) {
    const uint16_t* src = static_cast<const uint16_t*>(a.v) + rr * HD + lane * P;
#pragma unroll
    for (int p = 0; p < P; ++p) x[p] = (double)__uint_as_float((uint32_t)src[p] << 16);
  } else {
    const float* src = static_cast<const float*>(a.v) + rr * HD + lane * P;
#pragma unroll
    for (int p = 0; p < P; ++p) x[p] = (double)src[p];
  }
  // stages of span s: the pair (j, j + s) becomes (x_j + x_j+s, x_j - x_j+s)
#pragma unroll
  for (int s = 1; s < P; s <<= 1)
#pragma unroll
    for (int p = 0; p < P; ++p)
      if ((p & s) == 0) {
        const double lo = x[p], hi = x[p + s];
        x[p] = lo + hi;
        x[p + s] = lo - hi;
      }
#pragma unroll
  for (int s = P; s < HD; s <<= 1) {
    const int m = s / P;                           // partner lane = lane ^ m
    const bool upper = (lane & m) != 0;
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const double o = __shfl_xor(x[p], m, kWave);
      x[p] = upper ? o - x[p] : x[p] + o;
    }
  }
#pragma unroll
  for (int p = 0; p < P; ++p) rot[wave][lane * P + p] = __float_as_uint((float)(x[p] * kInvSqrtHd<HD>));
  __syncthreads();
  if (!valid || lane >= NB) return;
  uint32_t u[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) u[i] = rot[wave][lane * kBlock + i];
  const int g = (int)(r % a.kv_heads);
  const int64_t row = (int64_t)g * a.max_tokens + a.pos + r / a.kv_heads;
  encode_block<4>(u, a.v_exp + row * NB + lane, a.v_code + row * (HD / 2) + lane * 8);
}

// ---- decode attention ------------------------------------------------------------------

constexpr int kAttnThreads = 256;
constexpr int kAttnWaves = kAttnThreads / kWave;
constexpr int kMaxChunk = 256;                   // tokens per workgroup at most

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// This lane's 8 values of cached rows: codes and exponent loaded first (kSteps rows in flight
// per lane), decoded to fp32 (block scale applied) when used.
constexpr int kSteps = 8;
struct Row8 {
  uint2 c;
  uint32_t e;
};
template <int HD>
__device__ __forceinline__ Row8 load_row8(const uint8_t* exp, const uint8_t* code, int64_t row, int sub) {
  Row8 r;
  r.c = *reinterpret_cast<const uint2*>(code + row * HD + sub * 8);
  r.e = exp[row * (HD / kBlock) + sub / 2];
  return r;
}
__device__ __forceinline__ void decode_row8(const Row8& r, float (&w)[8]) {
  const float sc = block_scale<8>(r.e);
  unpack4_bfp8(r.c.x, w);
  unpack4_bfp8(r.c.y, w + 4);
#pragma unroll
  for (int i = 0; i < 8; ++i) w[i] *= sc;
}
// The same for a BFP4 row (4 code bytes per lane; c.y unused).
template <int HD>
__device__ __forceinline__ Row8 load_row8_b4(const uint8_t* exp, const uint8_t* code, int64_t row, int sub) {
  Row8 r;
  r.c.x = *reinterpret_cast<const uint32_t*>(code + row * (HD / 2) + sub * 4);
  r.c.y = 0;
  r.e = exp[row * (HD / kBlock) + sub / 2];
  return r;
}
__device__ __forceinline__ void decode_row8_b4(const Row8& r, float (&w)[8]) {
  const int sh = block_shift<4>(r.e);
  unpack8_bfp4(r.c.x, w);
#pragma unroll
  for (int i = 0; i < 8; ++i) w[i] = apply_shift(w[i], sh);
}

struct ChunkArgs {
  AttnArgs a;
  int chunk;                   // tokens per workgroup (a multiple of the tokens per step)
  int nchunks;
};

// Workgroup (c, g): tokens [c chunk, (c + 1) chunk) of KV head g for its G query heads.
// Writes o_c (unnormalised), m_c and l_c to the workspace. With V4R the values are the rotated
// BFP4 ones and o_c is rotated back before it is written.
template <int HD, int G, bool V4R>
__global__ __launch_bounds__(kAttnThreads) void attn_chunk_kernel(ChunkArgs ca) {
  constexpr int LPT = HD / 8;                    // lanes per cached row
  constexpr int TPW = kWave / LPT;               // rows per wave step
  constexpr int TPS = kAttnWaves * TPW;          // rows per workgroup step
  using Red = LaneReduce<G, 1, LPT>;
  __shared__ float sc[G][kMaxChunk];
  __shared__ float red[kAttnWaves][G][HD];
  __shared__ float mrow[G], lrow[G];
  const AttnArgs& a = ca.a;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int grp = lane / LPT, sub = lane % LPT;
  const int c = blockIdx.x, g = blockIdx.y;
  const int t0 = c * ca.chunk;
  const int nt = min(ca.chunk, a.L - t0);
  const int64_t row0 = (int64_t)g * a.max_tokens + t0;

  // this lane's 8 dimensions of the group's query rows, times the scale
  float q[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const int64_t o = (int64_t)(g * G + h) * HD + sub * 8;
    if (a.q_bf16) {
      const uint4 v = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.q) + o);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        q[h][2 * j] = bf16_lo(w[j]) * a.scale;
        q[h][2 * j + 1] = bf16_hi(w[j]) * a.scale;
      }
    } else {
      const f32x4 v0 = *reinterpret_cast<const f32x4*>(static_cast<const float*>(a.q) + o);
      const f32x4 v1 = *reinterpret_cast<const f32x4*>(static_cast<const float*>(a.q) + o + 4);
      const float w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) q[h][i] = w[i] * a.scale;
    }
  }

  // scores (rows past the sequence re-read its last row and score -inf); kSteps wave steps of
  // loads are issued before their arithmetic
  for (int s0 = 0; s0 < ca.chunk; s0 += TPS * kSteps) {
    Row8 r[kSteps];
#pragma unroll
    for (int u = 0; u < kSteps; ++u) {
      const int tl = s0 + u * TPS + wave * TPW + grp;
      r[u] = load_row8<HD>(a.k_exp, a.k_code, row0 + min(tl, nt - 1), sub);
    }
#pragma unroll
    for (int u = 0; u < kSteps; ++u) {
      if (s0 + u * TPS >= ca.chunk) break;
      const int tl = s0 + u * TPS + wave * TPW + grp;
      float kv[8];
      decode_row8(r[u], kv);
      float v[G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) s = __builtin_fmaf(q[h][i], kv[i], s);
        v[h] = s;
      }
      Red::run(v, lane);
      if (Red::writer(sub)) sc[Red::first_index(sub)][tl] = tl < nt ? v[0] : -__builtin_inff();
    }
  }
  __syncthreads();

  // per head: the chunk's maximum, the probabilities exp(s - m) in place, their sum
  for (int h = wave; h < G; h += kAttnWaves) {
    float m = -__builtin_inff();
    for (int t = lane; t < ca.chunk; t += kWave) m = fmaxf(m, sc[h][t]);
    m = wave_max(m);
    float l = 0.f;
    for (int t = lane; t < ca.chunk; t += kWave) {
      const float p = __expf(sc[h][t] - m);
      sc[h][t] = p;
      l += p;
    }
    l = wave_sum(l);
    if (lane == 0) { mrow[h] = m; lrow[h] = l; }
  }
  __syncthreads();

  // sum_t p_t v_t
  float acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[h][i] = 0.f;
  for (int s0 = 0; s0 < ca.chunk; s0 += TPS * kSteps) {
    Row8 r[kSteps];
#pragma unroll
    for (int u = 0; u < kSteps; ++u) {
      const int tl = s0 + u * TPS + wave * TPW + grp;
      if constexpr (V4R) r[u] = load_row8_b4<HD>(a.v_exp, a.v_code, row0 + min(tl, nt - 1), sub);
      else r[u] = load_row8<HD>(a.v_exp, a.v_code, row0 + min(tl, nt - 1), sub);
    }
#pragma unroll
    for (int u = 0; u < kSteps; ++u) {
      if (s0 + u * TPS >= ca.chunk) break;
      const int tl = s0 + u * TPS + wave * TPW + grp;
      float vv[8];
      if constexpr (V4R) decode_row8_b4(r[u], vv);
      else decode_row8(r[u], vv);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float p = sc[h][tl];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[h][i] = __builtin_fmaf(p, vv[i], acc[h][i]);
      }
    }
  }
  // over the row groups of the wave, then over the waves in wave order
#pragma unroll
  for (int o = LPT; o < kWave; o <<= 1)
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[h][i] += __shfl_xor(acc[h][i], o, kWave);
  if (grp == 0)
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int i = 0; i < 8; ++i) red[wave][h][sub * 8 + i] = acc[h][i];
  __syncthreads();
  float* po = a.ws + ((int64_t)c * a.q_heads + g * G) * HD;
  if constexpr (V4R) {
    // the sums into sc (no longer read), then H o / sqrt(HD) in place, stage by stage
    for (int j = threadIdx.x; j < G * HD; j += kAttnThreads) {
      const int h = j / HD, d = j % HD;
      float s = red[0][h][d];
#pragma unroll
      for (int w = 1; w < kAttnWaves; ++w) s += red[w][h][d];
      sc[h][d] = s;
    }
    __syncthreads();
#pragma unroll
    for (int st = 1; st < HD; st <<= 1) {
      for (int j = threadIdx.x; j < G * HD / 2; j += kAttnThreads) {
        const int h = j / (HD / 2), pi = j % (HD / 2);
        const int lo = (pi / st) * 2 * st + pi % st;
        const float x = sc[h][lo], y = sc[h][lo + st];
        sc[h][lo] = x + y;
        sc[h][lo + st] = x - y;
      }
      __syncthreads();
    }
    constexpr float kInv = (float)kInvSqrtHd<HD>;
    for (int j = threadIdx.x; j < G * HD; j += kAttnThreads) po[j] = sc[j / HD][j % HD] * kInv;
  } else {
    for (int j = threadIdx.x; j < G * HD; j += kAttnThreads) {
      const int h = j / HD, d = j % HD;
      float s = red[0][h][d];
#pragma unroll
      for (int w = 1; w < kAttnWaves; ++w) s += red[w][h][d];
      po[(int64_t)h * HD + d] = s;
    }
  }
  if (threadIdx.x < G) {
    float* pml = a.ws + (int64_t)ca.nchunks * a.q_heads * HD + ((int64_t)c * a.q_heads + g * G + threadIdx.x) * 2;
    pml[0] = mrow[threadIdx.x];
    pml[1] = lrow[threadIdx.x];
  }
}

// Matrix-core chunk kernel for G = 8 query heads per KV head. A 16x16 product D += A B on the
// matrix instructions has lane l = 16 j + r (j < 4, r < 16) supply row r of A and column r of
// B for the k slots of lane group j, and hold D[4 j + i][r], i < 4. Each wave takes tiles of 16
// tokens (tiles wave, wave + 4, ... of the chunk):
//  * scores S^T = K Q^T on v_mfma_f32_16x16x32_bf16: lane (j, r) supplies token r's dimensions
//    [HD/4 j, HD/4 (j+1)), 8 per step (a contiguous HD/4-byte piece of its row), as A, and the
//    same dimensions of query head r (zero for r >= 8) as B; D gives lane (j, r) the scores of
//    tokens 4 j + i for head r. Decoded keys are exact in bf16; the scaled query is the sum of
//    three bf16 parts (about 24 significant bits), one product each;
//  * the wave's maximum per head (across the four lane groups), p = exp(s - m) in place;
//  * O = P V on v_mfma_f32_16x16x16_bf16, k = the tile's 16 tokens: lane (j, r) supplies its
//    own p (tokens 4 j + i, head r) as A, split into hi + lo bf16 parts, and as B the dims
//    [HD/16 r, HD/16 (r+1)) of those four tokens' value rows (one whole 16-value block at
//    HD = 256), one output tile per dimension of the piece.
// The waves' (m, l, O) are combined in wave order. The query parts and the waves' partial
// outputs share one LDS area (33 KB at head_dim 256), and at most two tiles of value rows are
// held in registers, so that the rotated-V kernel (4-bit value rows) runs 3 waves per SIMD;
// the BFP8 one, with twice the value bytes per lane, stays at 2 (at 3 it spills).
constexpr int kMfmaTile = 16;

// Raw cached rows of one lane: a tile's key piece, a value piece (codes and exponent bytes).
template <int HD>
struct KPiece {
  uint4 c[HD / 64];
  uint32_t e;
};
struct VPiece {
  uint4 c;
  uint32_t e;
};

// NT: tiles per wave (the chunk is 64 NT tokens).
template <int HD, bool V4R, int NT>
__global__ __launch_bounds__(kAttnThreads, V4R ? 3 : 2) void attn_chunk_mfma_kernel(ChunkArgs ca) {
  constexpr int G = 8;
  constexpr int QK = HD / 4;                     // score steps; dims per lane group
  constexpr int DPC = HD / 16;                   // value dims per lane column = output tiles
  constexpr int QS = HD + 8;                     // LDS row stride of the query parts (conflict-free b128 reads)
  // one LDS area: the query parts while scores run, then the waves' partial outputs
  constexpr int kQsBytes = 3 * 16 * QS * 2, kRedBytes = kAttnWaves * G * HD * 4;
  __shared__ __align__(16) unsigned char lds_area[kQsBytes > kRedBytes ? kQsBytes : kRedBytes];
  auto& qs = *reinterpret_cast<uint16_t (*)[3][16][QS]>(lds_area);
  auto& red = *reinterpret_cast<float (*)[kAttnWaves][G][HD]>(lds_area);
  __shared__ float wstat[kAttnWaves][16], wsum[kAttnWaves][16], wfac[kAttnWaves][G];
  __shared__ float mrow[G], lrow[G];
  const AttnArgs& a = ca.a;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int j = lane >> 4, r = lane & 15;
  const int c = blockIdx.x, g = blockIdx.y;
  const int t0 = c * ca.chunk;
  const int nt = min(ca.chunk, a.L - t0);
  const int64_t row0 = (int64_t)g * a.max_tokens + t0;

  auto kload = [&](int tile, KPiece<HD>& k) {
    const int64_t row = row0 + min(tile * kMfmaTile + r, nt - 1);
    const uint4* pc = reinterpret_cast<const uint4*>(a.k_code + row * HD + QK * j);
#pragma unroll
    for (int v = 0; v < HD / 64; ++v) k.c[v] = pc[v];
    const uint8_t* pe = a.k_exp + row * (HD / kBlock) + (QK / 16) * j;
    if constexpr (HD == 256) k.e = *reinterpret_cast<const uint32_t*>(pe);
    else if constexpr (HD == 128) k.e = *reinterpret_cast<const uint16_t*>(pe);
    else k.e = *pe;
  };
  // value piece of token tile * 16 + 4 j + u: dims [DPC r, DPC r + DPC)
  auto vload = [&](int tile, int u, VPiece& v) {
    const int64_t row = row0 + min(tile * kMfmaTile + 4 * j + u, nt - 1);
    v.e = a.v_exp[row * (HD / kBlock) + (DPC * r) / kBlock];
    constexpr int bytes = V4R ? DPC / 2 : DPC;
    const uint8_t* pc = a.v_code + row * (V4R ? HD / 2 : HD) + bytes * r;
    v.c = uint4{0u, 0u, 0u, 0u};
    if constexpr (bytes == 16) v.c = *reinterpret_cast<const uint4*>(pc);
    else if constexpr (bytes == 8) { const uint2 x = *reinterpret_cast<const uint2*>(pc); v.c.x = x.x; v.c.y = x.y; }
    else if constexpr (bytes == 4) v.c.x = *reinterpret_cast<const uint32_t*>(pc);
    else v.c.x = *reinterpret_cast<const uint16_t*>(pc);
  };

  // queries times the scale in LDS as three bf16 parts (hi + mid + lo, about 24 significant
  // bits together), rows 8..15 zero
  for (int x = threadIdx.x; x < 16 * HD; x += kAttnThreads) {
    const int h = x / HD, d = x % HD;
    float q = 0.f;
    if (h < G) {
      const int64_t o = (int64_t)(g * G + h) * HD + d;
      q = (a.q_bf16 ? __uint_as_float((uint32_t)static_cast<const uint16_t*>(a.q)[o] << 16)
                    : static_cast<const float*>(a.q)[o]) * a.scale;
    }
    const uint32_t hi = f32_to_bf16_rne(q);
    const float r1 = q - __uint_as_float(hi << 16);
    const uint32_t mid = f32_to_bf16_rne(r1);
    const uint32_t lo = f32_to_bf16_rne(r1 - __uint_as_float(mid << 16));
    qs[0][h][d] = (uint16_t)hi;
    qs[1][h][d] = (uint16_t)mid;
    qs[2][h][d] = (uint16_t)lo;
  }

  // the wave's tiles in two phases: all scores (each tile's value rows load as soon as its key
  // rows are used), the wave's maximum m (head r) and, per lane, the sum l of its own
  // probabilities, then O = P V
  KPiece<HD> kb[NT];
  VPiece vb[NT][4];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) kload(wave + tt * kAttnWaves, kb[tt]);
  __syncthreads();                               // query parts in LDS

  float S[NT][4];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
    const int tile = wave + tt * kAttnWaves;
    // scores of tokens 4 j + i, head r: bf16 products (v_mfma_f32_16x16x32_bf16, A = 8 key
    // values of lane group j, B = the same dims of query head r): the keys are exact in bf16
    // (at most 8 significant bits, the block scale a power of two), the query is the sum of
    // its three parts; per part an accumulator of its own, added at the end
    const uint32_t* code = reinterpret_cast<const uint32_t*>(kb[tt].c);
    f32x4 acc[3];
#pragma unroll
    for (int e = 0; e < 3; ++e) acc[e] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < QK / 8; ++st) {
      const float scl = block_scale<8>((kb[tt].e >> (8 * (st / 2))) & 0xffu);
      const uint32_t c0 = code[2 * st], c1 = code[2 * st + 1];
      float kv[8];
      mag4_bfp8(c0, kv);
      mag4_bfp8(c1, kv + 4);
#pragma unroll
      for (int e = 0; e < 8; ++e) kv[e] *= scl;
      uint32_t kp2[4];
      kp2[0] = signed_pair(kv[0], kv[1], c0, c0, sign_sel(0, 5));
      kp2[1] = signed_pair(kv[2], kv[3], c0, c0, sign_sel(2, 7));
      kp2[2] = signed_pair(kv[4], kv[5], c1, c1, sign_sel(0, 5));
      kp2[3] = signed_pair(kv[6], kv[7], c1, c1, sign_sel(2, 7));
      const bf16x8 kbf = __builtin_bit_cast(bf16x8, kp2);
#pragma unroll
      for (int e = 0; e < 3; ++e) {
        const bf16x8 qb = *reinterpret_cast<const bf16x8*>(&qs[e][r][QK * j + 8 * st]);
        acc[e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kbf, qb, acc[e], 0, 0, 0);
      }
    }
    if (tt == (NT >= 2 ? NT - 2 : 0))          // the first tile's value rows, shortly before P V
#pragma unroll
      for (int u = 0; u < 4; ++u) vload(wave, u, vb[0][u]);
    const f32x4 as = acc[0] + (acc[1] + acc[2]);
    const float av[4] = {as.x, as.y, as.z, as.w};
#pragma unroll
    for (int i = 0; i < 4; ++i)
      S[tt][i] = (r < G && tile * kMfmaTile + 4 * j + i < nt) ? av[i] : -__builtin_inff();
  }
  float m = -__builtin_inff();
#pragma unroll
  for (int tt = 0; tt < NT; ++tt)
#pragma unroll
    for (int i = 0; i < 4; ++i) m = fmaxf(m, S[tt][i]);
  m = fmaxf(m, __shfl_xor(m, 16, kWave));
  m = fmaxf(m, __shfl_xor(m, 32, kWave));
  float l = 0.f;
#pragma unroll
  for (int tt = 0; tt < NT; ++tt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      S[tt][i] = S[tt][i] == -__builtin_inff() ? 0.f : __expf(S[tt][i] - m);
      l += S[tt][i];
    }

  f32x4 O[DPC];
#pragma unroll
  for (int n = 0; n < DPC; ++n) O[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
    if (tt + 1 < NT)                             // the next tile's value rows load during this one
#pragma unroll
      for (int u = 0; u < 4; ++u) vload(wave + (tt + 1) * kAttnWaves, u, vb[tt + 1][u]);
    const VPiece (&vc)[4] = vb[tt];
    // O += P V on v_mfma_f32_16x16x16_bf16 over the tile's 16 tokens: lane (j, r) supplies as
    // A its own probabilities (tokens 4 j + i, head r) as hi + lo bf16 parts, and as B the
    // value dims DPC r + n of those four tokens (exact in bf16), one product per n
    uint32_t ph[2], pl[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const uint32_t h0 = __float_as_uint(S[tt][2 * e]) & 0xffff0000u;
      const uint32_t h1 = __float_as_uint(S[tt][2 * e + 1]) & 0xffff0000u;
      ph[e] = h1 | (h0 >> 16);
      const uint32_t l0 = f32_to_bf16_rne(S[tt][2 * e] - __uint_as_float(h0));
      const uint32_t l1 = f32_to_bf16_rne(S[tt][2 * e + 1] - __uint_as_float(h1));
      pl[e] = (l1 << 16) | l0;
    }
    const s16x4 pah = __builtin_bit_cast(s16x4, ph), pal = __builtin_bit_cast(s16x4, pl);
    float vv[4][DPC];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t cw[4] = {vc[u].c.x, vc[u].c.y, vc[u].c.z, vc[u].c.w};
      if constexpr (V4R) {
        const int sh = block_shift<4>(vc[u].e);
        if constexpr (DPC >= 8) {
#pragma unroll
          for (int b = 0; b < DPC / 8; ++b) unpack8_bfp4(cw[b], vv[u] + 8 * b);
        } else {
          float t8[8];
          unpack8_bfp4(cw[0], t8);
#pragma unroll
          for (int e = 0; e < 4; ++e) vv[u][e] = t8[e];
        }
#pragma unroll
        for (int e = 0; e < DPC; ++e) vv[u][e] = apply_shift(vv[u][e], sh);
      } else {
        const float sc = block_scale<8>(vc[u].e);
#pragma unroll
        for (int b = 0; b < DPC / 4; ++b) mag4_bfp8(cw[b], vv[u] + 4 * b);   // signs added below
#pragma unroll
        for (int e = 0; e < DPC; ++e) vv[u][e] *= sc;
      }
    }
#pragma unroll
    for (int n = 0; n < DPC; ++n) {
      uint32_t vbf[2];
      if constexpr (V4R) {
        vbf[0] = __builtin_amdgcn_perm(__float_as_uint(vv[1][n]), __float_as_uint(vv[0][n]), 0x07060302u);
        vbf[1] = __builtin_amdgcn_perm(__float_as_uint(vv[3][n]), __float_as_uint(vv[2][n]), 0x07060302u);
      } else {
        const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&vc[0].c);
        const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&vc[1].c);
        const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&vc[2].c);
        const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&vc[3].c);
        const uint32_t sel = sign_sel(n % 4, 4 + n % 4);
        vbf[0] = signed_pair(vv[0][n], vv[1][n], w0[n / 4], w1[n / 4], sel);
        vbf[1] = signed_pair(vv[2][n], vv[3][n], w2[n / 4], w3[n / 4], sel);
      }
      const s16x4 bv = __builtin_bit_cast(s16x4, vbf);
      O[n] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pah, bv, O[n], 0, 0, 0);
      O[n] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pal, bv, O[n], 0, 0, 0);
    }
  }
  l += __shfl_xor(l, 16, kWave);
  l += __shfl_xor(l, 32, kWave);

  // the waves' (m, l, O) combined in wave order: M = max m_w, O = sum_w e^(m_w - M) O_w
  __syncthreads();                               // every wave is done with the query parts
  if (j == 0) {
    wstat[wave][r] = m;
    wsum[wave][r] = l;
  }
  if (j < 2)
#pragma unroll
    for (int n = 0; n < DPC; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wave][4 * j + i][DPC * r + n] = O[n][i];
  __syncthreads();
  if (threadIdx.x < G) {
    const int h = threadIdx.x;
    float M = wstat[0][h];
#pragma unroll
    for (int w = 1; w < kAttnWaves; ++w) M = fmaxf(M, wstat[w][h]);
    float ls = 0.f;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) {
      const float f = wstat[w][h] == -__builtin_inff() ? 0.f : __expf(wstat[w][h] - M);
      wfac[w][h] = f;
      ls += f * wsum[w][h];
    }
    mrow[h] = M;
    lrow[h] = ls;
  }
  __syncthreads();
  float* po = a.ws + ((int64_t)c * a.q_heads + g * G) * HD;
  if constexpr (V4R) {
    for (int x = threadIdx.x; x < G * HD; x += kAttnThreads) {
      const int h = x / HD, d = x % HD;
      float s2 = wfac[0][h] * red[0][h][d];
#pragma unroll
      for (int w = 1; w < kAttnWaves; ++w) s2 = __builtin_fmaf(wfac[w][h], red[w][h][d], s2);
      red[0][h][d] = s2;
    }
    __syncthreads();
#pragma unroll
    for (int st = 1; st < HD; st <<= 1) {
      for (int x = threadIdx.x; x < G * HD / 2; x += kAttnThreads) {
        const int h = x / (HD / 2), pi = x % (HD / 2);
        const int lo = (pi / st) * 2 * st + pi % st;
        const float y0 = red[0][h][lo], y1 = red[0][h][lo + st];
        red[0][h][lo] = y0 + y1;
        red[0][h][lo + st] = y0 - y1;
      }
      __syncthreads();
    }
    constexpr float kInv = (float)kInvSqrtHd<HD>;
    for (int x = threadIdx.x; x < G * HD; x += kAttnThreads) po[x] = red[0][x / HD][x % HD] * kInv;
  } else {
    for (int x = threadIdx.x; x < G * HD; x += kAttnThreads) {
      const int h = x / HD, d = x % HD;
      float s2 = wfac[0][h] * red[0][h][d];
#pragma unroll
      for (int w = 1; w < kAttnWaves; ++w) s2 = __builtin_fmaf(wfac[w][h], red[w][h][d], s2);
      po[(int64_t)h * HD + d] = s2;
    }
  }
  __syncthreads();
  if (threadIdx.x < G) {
    float* pml = a.ws + (int64_t)ca.nchunks * a.q_heads * HD + ((int64_t)c * a.q_heads + g * G + threadIdx.x) * 2;
    pml[0] = mrow[threadIdx.x];
    pml[1] = lrow[threadIdx.x];
  }
}

// Workgroup (h, j): dimensions [64 j, 64 j + 64) of query head h, merged over the chunks.
// kMergeGroups thread groups of 16 threads (four dimensions each, one 16-byte load per chunk)
// each fold a fixed residue class of chunks in chunk order into a running (m, l, o) (eight
// chunks' loads in flight per thread); the groups' results are then combined in group order,
// so the result does not depend on scheduling.
constexpr int kMergeThreads = 1024;
constexpr int kMergeDims = 64;
constexpr int kMergeTpr = kMergeDims / 4;                 // threads per chunk row
constexpr int kMergeGroups = kMergeThreads / kMergeTpr;
template <int HD>
__global__ __launch_bounds__(kMergeThreads) void attn_merge_kernel(ChunkArgs ca) {
  constexpr int U = 8;
  __shared__ float gm[kMergeGroups], gl[kMergeGroups];
  __shared__ __align__(16) float go[kMergeGroups][kMergeDims];
  const AttnArgs& a = ca.a;
  const int h = blockIdx.x, tid = threadIdx.x;
  const int d0 = blockIdx.y * kMergeDims;
  const int grp = tid / kMergeTpr, qd = 4 * (tid % kMergeTpr);
  const float* ml = a.ws + (int64_t)ca.nchunks * a.q_heads * HD;
  float m = -__builtin_inff(), l = 0.f;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  for (int c0 = grp; c0 < ca.nchunks; c0 += kMergeGroups * U) {
    float mc[U], lc[U];
    f32x4 oc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = min(c0 + u * kMergeGroups, ca.nchunks - 1);
      const int64_t row = (int64_t)c * a.q_heads + h;
      mc[u] = ml[row * 2];
      lc[u] = ml[row * 2 + 1];
      oc[u] = *reinterpret_cast<const f32x4*>(a.ws + row * HD + d0 + qd);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (c0 + u * kMergeGroups >= ca.nchunks) break;
      const float mn = fmaxf(m, mc[u]);              // every chunk's maximum is finite
      const float fa = __expf(m - mn), fb = __expf(mc[u] - mn);
      l = l * fa + lc[u] * fb;
      o = o * fa + oc[u] * fb;
      m = mn;
    }
  }
  if (tid % kMergeTpr == 0) {
    gm[grp] = m;
    gl[grp] = l;
  }
  *reinterpret_cast<f32x4*>(&go[grp][qd]) = o;
  __syncthreads();
  if (tid < kMergeDims) {
    float M = gm[0];
    for (int g = 1; g < kMergeGroups; ++g) M = fmaxf(M, gm[g]);
    float os = 0.f, ls = 0.f;
    for (int g = 0; g < kMergeGroups; ++g) {
      const float f = gm[g] == -__builtin_inff() ? 0.f : __expf(gm[g] - M);
      os = __builtin_fmaf(f, go[g][tid], os);
      ls = __builtin_fmaf(f, gl[g], ls);
    }
    a.out[(int64_t)h * HD + d0 + tid] = os / ls;
  }
}

// Tokens per workgroup: about 256 workgroups in all, a multiple of 64 between 64 and kMaxChunk
// (a whole number of steps of either kernel).
inline int pick_chunk(int head_dim, int kv_heads, int L) {
  (void)head_dim;
  int ch = (int)(((int64_t)L * kv_heads + 255) / 256);
  ch = ch < 64 ? 64 : ch > kMaxChunk ? kMaxChunk : ch;
  return (ch + 63) / 64 * 64;
}

template <int HD, int NT>
void launch_mfma(const ChunkArgs& ca, dim3 grid, hipStream_t s) {
  if (ca.a.v_rot4) hipLaunchKernelGGL((attn_chunk_mfma_kernel<HD, true, NT>), grid, dim3(kAttnThreads), 0, s, ca);
  else hipLaunchKernelGGL((attn_chunk_mfma_kernel<HD, false, NT>), grid, dim3(kAttnThreads), 0, s, ca);
}

template <int HD, int G>
hipError_t launch_hd_g(const AttnArgs& a, hipStream_t s) {
  ChunkArgs ca;
  ca.a = a;
  ca.chunk = pick_chunk(HD, a.kv_heads, a.L);
  ca.nchunks = (a.L + ca.chunk - 1) / ca.chunk;
  const dim3 grid(ca.nchunks, a.kv_heads);
  if constexpr (G == 8) {
    switch (ca.chunk / (kAttnWaves * kMfmaTile)) {
      case 1: launch_mfma<HD, 1>(ca, grid, s); break;
      case 2: launch_mfma<HD, 2>(ca, grid, s); break;
      case 3: launch_mfma<HD, 3>(ca, grid, s); break;
      default: launch_mfma<HD, 4>(ca, grid, s); break;
    }
  } else {
    if (a.v_rot4) hipLaunchKernelGGL((attn_chunk_kernel<HD, G, true>), grid, dim3(kAttnThreads), 0, s, ca);
    else hipLaunchKernelGGL((attn_chunk_kernel<HD, G, false>), grid, dim3(kAttnThreads), 0, s, ca);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_merge_kernel<HD>), dim3(a.q_heads, HD / kMergeDims), dim3(kMergeThreads), 0, s, ca);
  return hipGetLastError();
}

template <int HD>
hipError_t launch_hd(const AttnArgs& a, hipStream_t s) {
  switch (a.q_heads / a.kv_heads) {
    case 1: return launch_hd_g<HD, 1>(a, s);
    case 2: return launch_hd_g<HD, 2>(a, s);
    case 4: return launch_hd_g<HD, 4>(a, s);
    case 8: return launch_hd_g<HD, 8>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t kv_append_launch(const KvAppendArgs& a, hipStream_t s) {
  const int64_t blocks = (a.v_rot4 ? 1 : 2) * a.n * a.kv_heads * (a.head_dim / kBlock);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(kv_append_kernel, dim3((unsigned)((blocks + 255) / 256)), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !a.v_rot4) return e;
  const dim3 grid((unsigned)((a.n * a.kv_heads + kV4rWaves - 1) / kV4rWaves));
  const dim3 block(kV4rWaves * kWave);
  if (a.head_dim == 64) hipLaunchKernelGGL((kv_append_v4r_kernel<64>), grid, block, 0, s, a);
  else if (a.head_dim == 128) hipLaunchKernelGGL((kv_append_v4r_kernel<128>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((kv_append_v4r_kernel<256>), grid, block, 0, s, a);
  return hipGetLastError();
}

bool attn_supported(int kv_heads, int head_dim, int q_heads) {
  if (kv_heads < 1 || q_heads < kv_heads || q_heads % kv_heads != 0) return false;
  const int g = q_heads / kv_heads;
  if (g != 1 && g != 2 && g != 4 && g != 8) return false;
  return head_dim == 64 || head_dim == 128 || head_dim == 256;
}

size_t attn_workspace_bytes(int kv_heads, int head_dim, int q_heads, int L) {
  if (L < 1) return 0;
  const int chunk = pick_chunk(head_dim, kv_heads, L);
  const int64_t nchunks = (L + chunk - 1) / chunk;
  return (size_t)nchunks * q_heads * (head_dim + 2) * sizeof(float);
}

hipError_t attn_decode_launch(const AttnArgs& a, hipStream_t s) {
  if (!attn_supported(a.kv_heads, a.head_dim, a.q_heads) || a.L < 1) return hipErrorInvalidValue;
  if (a.head_dim == 64) return launch_hd<64>(a, s);
  if (a.head_dim == 128) return launch_hd<128>(a, s);
  return launch_hd<256>(a, s);
}

}  // namespace bfp
