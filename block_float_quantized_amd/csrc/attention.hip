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
// Decode attention is split over the sequence (a workgroup per KV head and chunk of tokens):
//  * the G query heads of a KV head share every key and value row read from HBM;
//  * head_dim / 8 lanes hold one cached row, 8 values each (one 8-byte code load and one
//    exponent byte per lane: a wave load covers whole consecutive rows);
//  * scores: 8 products per query head per lane, then a lane-group reduction that leaves one
//    head's score per writer lane (stored in LDS with the chunk's other scores);
//  * per head the chunk's maximum m and sum l of exp(s - m), then sum_t exp(s_t - m) v_t;
//  * attn_merge_kernel combines the chunks in chunk order: out = sum_c e^(m_c - M) o_c /
//    sum_c e^(m_c - M) l_c. Every order is fixed, so results do not depend on scheduling.
#include "bfp_attn.hpp"
#include "bfp_device.hpp"
#include "bfp_encode.hpp"

namespace bfp {

namespace {

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
  const float sc = block_scale<4>(r.e);
  unpack8_bfp4(r.c.x, w);
#pragma unroll
  for (int i = 0; i < 8; ++i) w[i] *= sc;
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

// Workgroup (h, j): dimensions [64 j, 64 j + 64) of query head h, merged over the chunks. The
// maximum M of the chunk maxima first; then kMergeGroups thread groups (one thread per
// dimension) each add a fixed residue class of chunks in chunk order, eight chunks' loads in
// flight per thread, and the groups' sums are added in group order: the result does not
// depend on scheduling.
constexpr int kMergeThreads = 1024;
constexpr int kMergeDims = 64;
constexpr int kMergeGroups = kMergeThreads / kMergeDims;
template <int HD>
__global__ __launch_bounds__(kMergeThreads) void attn_merge_kernel(ChunkArgs ca) {
  constexpr int GT = kMergeDims;                     // threads per group
  constexpr int U = 8;
  __shared__ float wmax[kMergeThreads / kWave];
  __shared__ float po[kMergeGroups][GT], pl[kMergeGroups];
  const AttnArgs& a = ca.a;
  const int h = blockIdx.x, tid = threadIdx.x;
  const int d0 = blockIdx.y * kMergeDims;
  const float* ml = a.ws + (int64_t)ca.nchunks * a.q_heads * HD;
  float mx = -__builtin_inff();
  for (int c = tid; c < ca.nchunks; c += kMergeThreads) mx = fmaxf(mx, ml[((int64_t)c * a.q_heads + h) * 2]);
  mx = wave_max(mx);
  if ((tid & (kWave - 1)) == 0) wmax[tid / kWave] = mx;
  __syncthreads();
  mx = wmax[0];
#pragma unroll
  for (int w = 1; w < kMergeThreads / kWave; ++w) mx = fmaxf(mx, wmax[w]);
  const int grp = tid / GT, d = d0 + tid % GT;
  float l = 0.f, o = 0.f;
  {
    for (int c0 = grp; c0 < ca.nchunks; c0 += kMergeGroups * U) {
      float m[U], lv[U], ov[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = min(c0 + u * kMergeGroups, ca.nchunks - 1);
        m[u] = ml[((int64_t)c * a.q_heads + h) * 2];
        lv[u] = ml[((int64_t)c * a.q_heads + h) * 2 + 1];
        ov[u] = a.ws[((int64_t)c * a.q_heads + h) * HD + d];
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (c0 + u * kMergeGroups >= ca.nchunks) break;
        const float w = __expf(m[u] - mx);
        l = __builtin_fmaf(w, lv[u], l);
        o = __builtin_fmaf(w, ov[u], o);
      }
    }
    po[grp][tid % GT] = o;
    if (tid % GT == 0) pl[grp] = l;
  }
  __syncthreads();
  if (tid < GT) {
    float os = po[0][tid], ls = pl[0];
#pragma unroll
    for (int j = 1; j < kMergeGroups; ++j) {
      os += po[j][tid];
      ls += pl[j];
    }
    a.out[(int64_t)h * HD + d0 + tid] = os / ls;
  }
}

template <int HD>
constexpr int tokens_per_step() { return kAttnWaves * (kWave / (HD / 8)); }

// Tokens per workgroup: about 256 workgroups in all, between 64 and kMaxChunk tokens.
inline int pick_chunk(int head_dim, int kv_heads, int L) {
  const int tps = kAttnWaves * (kWave / (head_dim / 8));
  int ch = (int)(((int64_t)L * kv_heads + 255) / 256);
  ch = ch < 64 ? 64 : ch > kMaxChunk ? kMaxChunk : ch;
  return (ch + tps - 1) / tps * tps;
}

template <int HD, int G>
hipError_t launch_hd_g(const AttnArgs& a, hipStream_t s) {
  ChunkArgs ca;
  ca.a = a;
  ca.chunk = pick_chunk(HD, a.kv_heads, a.L);
  ca.nchunks = (a.L + ca.chunk - 1) / ca.chunk;
  if (a.v_rot4)
    hipLaunchKernelGGL((attn_chunk_kernel<HD, G, true>), dim3(ca.nchunks, a.kv_heads), dim3(kAttnThreads), 0, s, ca);
  else
    hipLaunchKernelGGL((attn_chunk_kernel<HD, G, false>), dim3(ca.nchunks, a.kv_heads), dim3(kAttnThreads), 0, s, ca);
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
