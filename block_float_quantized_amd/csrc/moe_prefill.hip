// MoE prefill for gfx950: expert-grouped GEMMs on the bf16 matrix cores.
//
// A 2,048-token prefill chunk ("Qwen3.8-27B — TT-native mixed BFP4/BFP8", section "What
// changed in this release (s27v6-20261024)": prompts prefill in 2,048-token chunks) routes
// 16,384 (token, slot) pairs through the 256 BFP4 experts ("qwen3.6-a3b-blackhole",
// introduction). With the pairs sorted by expert (dispatch), each expert is a dense GEMM:
//   h = silu(X_e Wg_e^T) * (X_e Wu_e^T)   rounded to bf16,
//   o = h Wd_e^T                           fp32 per pair,
// and the shared expert is one more group holding every token. y is then the weighted sum
// of each token's pair rows (the decode combine kernel).
//
// Kernel design:
//  * One workgroup (4 waves) computes a TM x TN tile of one group. The tile list (row tiles
//    of every group) comes from the dispatch kernel; workgroups are mapped so that each XCD
//    takes a contiguous range of tiles, ordered (group, column tile, row tile): the tiles
//    that reuse one expert's weights share an L2.
//  * Per K step of 64: the activation rows are gathered (token rows of x, or pair rows of h)
//    into LDS; each lane loads and dequantizes its own weight values straight into MFMA B
//    operands (the weights never go through LDS); the next step's global loads are issued
//    before the current step's MFMAs.
//  * v_mfma_f32_32x32x16_bf16 with fp32 accumulation; each wave owns all 64 rows of the tile
//    and 64 output columns.
//    A and B share one permutation of K inside every 8-value group (the order the BFP4
//    unpack produces pairs in), which leaves every dot product unchanged.
//  * Dequantization is exact: a nibble becomes an FP8 E4M3 subnormal (mag * 2^-9) and the
//    conversion to bf16 applies the block scale 2^(E-120); blocks whose scale falls outside
//    the conversion's exact range go through an fp32 path.
#include "bfp_device.hpp"
#include "bfp_moe.hpp"
#include "bfp_prefill.hpp"

#include <type_traits>

namespace bfp {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kTM = 128;         // rows (pairs) per tile
constexpr int kRT = kTM / 32;    // 32-row MFMA fragments per tile
constexpr int kTK = 64;          // K per step
constexpr int kLDK = kTK + 8;    // bf16 per LDS row (padding spreads banks)
constexpr int kPT = 256;         // threads per workgroup

struct PfArgs {
  const uint8_t *exp0, *code0, *exp1, *code1;       // routed (stacked) matrices
  const uint8_t *sexp0, *scode0, *sexp1, *scode1;   // shared expert
  int rows_per_expert;                              // N of one expert
  int k;                                            // K
  const int32_t* active;
  const int32_t* n_active;
  const int32_t* offsets;
  const int32_t* perm;
  const int32_t* tile_start;
  int with_shared;
  int m, top_k;
  const uint16_t* a;                                // A rows (bf16): x by token, or h by position
  int64_t lda;
  int a_by_token;
  void* c;                                          // output rows by pair position
  int64_t ldc;
};

// 8 BFP4 values (one dword) with exponent E -> 4 dwords of bf16 pairs in the permuted order
// (v0,v2)(v4,v6)(v1,v3)(v5,v7). Fast form, for E in [8, 247]: the scaled FP8 conversion
// applies 2^(E-120) (a normal fp32) and every result is a normal bf16.
__device__ __forceinline__ u32x4 dequant8_fast(uint32_t c, uint32_t e) {
  const float sc = __uint_as_float((e + 7u) << 23);           // 2^(E - 120)
  const uint32_t ev = ((c << 4) & 0x80808080u) | (c & 0x07070707u);
  const uint32_t od = (c & 0x80808080u) | ((c >> 4) & 0x07070707u);
  u32x4 o;
  o.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(ev, sc, false));
  o.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(ev, sc, true));
  o.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(od, sc, false));
  o.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(od, sc, true));
  return o;
}

// Any exponent: fp32 values scaled by ldexp (exact, subnormals included), top halves packed.
__device__ __forceinline__ u32x4 dequant8_any(uint32_t c, uint32_t e) {
  const int sh = (int)e - 120;
  float w[8];
  unpack8_bfp4(c, w);
  auto b = [&](int i) { return __float_as_uint(__builtin_amdgcn_ldexpf(w[i], sh)) >> 16; };
  return u32x4{b(0) | (b(2) << 16), b(4) | (b(6) << 16), b(1) | (b(3) << 16), b(5) | (b(7) << 16)};
}

// 8 bf16 activations (natural order) -> the same permutation as the weights.
__device__ __forceinline__ uint4 permute8(uint4 v) {
  uint4 o;
  o.x = __builtin_amdgcn_perm(v.y, v.x, 0x05040100u);   // (x0, x2)
  o.y = __builtin_amdgcn_perm(v.w, v.z, 0x05040100u);   // (x4, x6)
  o.z = __builtin_amdgcn_perm(v.y, v.x, 0x07060302u);   // (x1, x3)
  o.w = __builtin_amdgcn_perm(v.w, v.z, 0x07060302u);   // (x5, x7)
  return o;
}

struct TileInfo {
  int shared;       // shared-expert group
  int e;            // routed expert id
  int p0, n;        // first pair position and rows of the group
  int row0;         // first row of the tile inside the group
  int col0;         // first output column
};

// Maps this workgroup to a tile; false when it has none. Each XCD (workgroups bid % 8) takes a
// contiguous range of the tiles that exist.
template <int TN>
__device__ __forceinline__ bool find_tile(const PfArgs& a, TileInfo& t) {
  const int na = *a.n_active;
  const int ng = na + (a.with_shared ? 1 : 0);
  const int nct = a.rows_per_expert / TN;
  const int total = a.tile_start[ng] * nct;
  const int per = (total + 7) / 8;
  const int local = blockIdx.x / 8;
  if (local >= per) return false;
  const int tile = (blockIdx.x % 8) * per + local;
  if (tile >= total) return false;
  // group: last g with tile_start[g] * nct <= tile
  int lo = 0, hi = ng - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (a.tile_start[mid] * nct <= tile) lo = mid; else hi = mid - 1;
  }
  const int g = lo;
  const int mtiles = a.tile_start[g + 1] - a.tile_start[g];
  const int loc = tile - a.tile_start[g] * nct;
  const int ct = loc / mtiles, mt = loc % mtiles;
  t.shared = g == na;
  if (t.shared) {
    t.e = -1;
    t.p0 = a.m * a.top_k;
    t.n = a.m;
  } else {
    t.e = a.active[g];
    t.p0 = a.offsets[t.e];
    t.n = a.offsets[t.e + 1] - t.p0;
  }
  t.row0 = mt * kTM;
  t.col0 = ct * TN;
  return true;
}

typedef float f32x16 __attribute__((ext_vector_type(16)));

// Grouped GEMM C[pos][col] = A[row(pos)] . W_e[col] for one tile of kTM rows, on
// v_mfma_f32_32x32x16_bf16. Each of the 4 waves owns all kTM rows (kRT 32-row A fragments)
// and NB = 2 B tiles of 32 columns: NMAT = 2 -> the same 32 columns of gate and of up (the
// SwiGLU pair lands in one lane), NMAT = 1 -> 64 adjacent columns. A workgroup therefore
// covers TN = 4 * 32 * 2 / NMAT columns of each matrix.
//
// Per K step of 64: the gathered A rows go through LDS (shared by the 4 waves); every lane
// loads the 16 code bytes (32 values) of each of its B rows directly and dequantizes them
// in registers, so the weights never touch LDS. Lane group g = lane / 32 takes K values
// [32g, 32g + 32) of the step, 8 per MFMA; its A fragment reads the same K values from LDS.
template <int NMAT>
__global__ __launch_bounds__(kPT, 2) void grouped_gemm_kernel(PfArgs a) {
  constexpr int NB = 2;                            // 32-column B tiles per wave
  constexpr int TN = 4 * 32 * NB / NMAT;           // columns per matrix per workgroup
  __shared__ __align__(16) uint16_t As[2][kTM][kLDK];
  __shared__ int arow[kTM];
  TileInfo t;
  if (!find_tile<TN>(a, t)) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane / 32, lc = lane % 32;
  if (tid < kTM) {
    const int r = t.row0 + tid;
    int row = -1;
    if (r < t.n) {
      const int pos = t.p0 + r;
      const int tok = t.shared ? r : a.perm[pos] / a.top_k;
      row = a.a_by_token ? tok : pos;
    }
    arow[tid] = row;
  }
  __syncthreads();

  const int64_t nbk = a.k / kBlock;
  const int64_t rows0 = t.shared ? 0 : (int64_t)t.e * a.rows_per_expert;
  const uint8_t* expb[2] = {(t.shared ? a.sexp0 : a.exp0) + rows0 * nbk,
                            NMAT == 2 ? (t.shared ? a.sexp1 : a.exp1) + rows0 * nbk : nullptr};
  const uint8_t* codeb[2] = {(t.shared ? a.scode0 : a.code0) + rows0 * (a.k / 2),
                             NMAT == 2 ? (t.shared ? a.scode1 : a.code1) + rows0 * (a.k / 2) : nullptr};
  // B row (output column) of tile b of this lane, and the matrix it belongs to
  const uint8_t* bcode[NB];
  const uint8_t* bexp[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int mat = NMAT == 2 ? b : 0;
    const int col = NMAT == 2 ? t.col0 + wave * 32 + lc : t.col0 + wave * 64 + b * 32 + lc;
    bcode[b] = codeb[mat] + (int64_t)col * (a.k / 2);
    bexp[b] = expb[mat] + (int64_t)col * nbk;
  }
  // A staging: kTM rows x 64 values = 256 threads x 32 values
  constexpr int kAQ = kPT / kTM;                   // threads per row
  constexpr int kAH = 64 / kAQ / 8;                // 8-value pieces per thread
  const int ar = tid / kAQ, aq = tid % kAQ;
  const int arow_this = arow[ar];
  // rows of this tile that exist (wave-uniform): MFMAs of fragments past them are skipped
  const int nrt = (min(kTM, t.n - t.row0) + 31) / 32;

  // weight loads of one K step (issued two steps ahead), kept in registers until consumed;
  // activation loads of the next step (one step ahead) go to one register set
  struct StepRegs {
    u32x4 rc[NB];
    uint32_t re[NB];
  };
  auto load_step = [&](StepRegs& R, int k0) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      R.rc[b] = *reinterpret_cast<const u32x4*>(bcode[b] + (k0 + 32 * g) / 2);
      R.re[b] = *reinterpret_cast<const uint16_t*>(bexp[b] + (k0 + 32 * g) / 16);
    }
  };
  uint4 ra[kAH];
  auto load_a = [&](int k0) {
#pragma unroll
    for (int h = 0; h < kAH; ++h) {
      ra[h] = make_uint4(0, 0, 0, 0);
      if (arow_this >= 0)
        ra[h] = *reinterpret_cast<const uint4*>(a.a + (int64_t)arow_this * a.lda + k0 + aq * 8 * kAH + h * 8);
    }
  };

  f32x16 acc[kRT][NB];
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt)
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[rt][b] = f32x16{};

  // consume step k0: stage its activations into LDS buffer `buf`, one barrier, then issue the
  // loads of the next step's activations and of the weights two steps ahead, then dequantize
  // and run the MFMAs of the NRT fragments that hold rows
  auto consume = [&](StepRegs& R, int buf, int k0, auto NC) __attribute__((always_inline)) {
    constexpr int NRT = decltype(NC)::value;
    // one decision per wave and step: all exponents inside the fast conversion's range?
    bool ok = true;
#pragma unroll
    for (int b = 0; b < NB; ++b) ok = ok && ((R.re[b] & 0xffu) - 8u) <= 239u && ((R.re[b] >> 8) - 8u) <= 239u;
    const bool fast = __builtin_amdgcn_ballot_w64(!ok) == 0;
#pragma unroll
    for (int h = 0; h < kAH; ++h) *reinterpret_cast<uint4*>(&As[buf][ar][aq * 8 * kAH + h * 8]) = permute8(ra[h]);
    u32x4 cw[NB];
    uint32_t ew[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) { cw[b] = R.rc[b]; ew[b] = R.re[b]; }
    __syncthreads();
    if (k0 + kTK < a.k) load_a(k0 + kTK);
    if (k0 + 2 * kTK < a.k) load_step(R, k0 + 2 * kTK);
    // per 16-value MFMA slice: dequantize 8 values of each B tile, then the MFMAs
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      bf16x8 bf[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const uint32_t e = (ew[b] >> (8 * (st / 2))) & 0xffu;
        u32x4 d;
        if (fast) d = dequant8_fast(cw[b][st], e);
        else d = dequant8_any(cw[b][st], e);
        bf[b] = __builtin_bit_cast(bf16x8, d);
      }
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        const bf16x8 af = *reinterpret_cast<const bf16x8*>(&As[buf][rt * 32 + lc][32 * g + 8 * st]);
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[rt][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bf[b], acc[rt][b], 0, 0, 0);
      }
    }
  };

  // two register sets, two LDS buffers: step s uses set s % 2 and buffer s % 2. Writing
  // buffer s % 2 at step s is safe: every wave finished reading it (step s - 2) before the
  // barrier of step s - 1. K is a multiple of 2 kTK, so the loop body is the same for every
  // iteration; one copy of the loop per count of row fragments.
  auto run = [&](auto NC) __attribute__((always_inline)) {
    StepRegs r0, r1;
    load_step(r0, 0);
    load_a(0);
    load_step(r1, kTK);
    for (int k0 = 0; k0 < a.k; k0 += 2 * kTK) {
      consume(r0, 0, k0, NC);
      consume(r1, 1, k0 + kTK, NC);
    }
  };
  switch (nrt) {
    case 1: run(std::integral_constant<int, 1>{}); break;
    case 2: run(std::integral_constant<int, 2>{}); break;
    case 3: run(std::integral_constant<int, 3>{}); break;
    default: run(std::integral_constant<int, 4>{}); break;
  }

  // epilogue: element i of a 32x32 tile sits at row (i/4)*8 + g*4 + i%4, column lc
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = rt * 32 + (i / 4) * 8 + g * 4 + (i % 4);
      if (t.row0 + r >= t.n) continue;
      const int64_t pos = t.p0 + t.row0 + r;
      if constexpr (NMAT == 2) {
        const float gv = acc[rt][0][i], uv = acc[rt][1][i];
        const float hv = gv / (1.0f + __expf(-gv)) * uv;
        static_cast<uint16_t*>(a.c)[pos * a.ldc + t.col0 + wave * 32 + lc] = (uint16_t)f32_to_bf16_rne(hv);
      } else {
#pragma unroll
        for (int b = 0; b < NB; ++b)
          static_cast<float*>(a.c)[pos * a.ldc + t.col0 + wave * 64 + b * 32 + lc] = acc[rt][b][i];
      }
    }
}

// y[t] = sum_j w[t][j] * o[inv[t*K+j]] + g[t] * o[m*K + t]
__global__ __launch_bounds__(256) void pf_combine_kernel(const float* o, const int32_t* inv, const float* w,
                                                         const float* g, int m, int top_k, int hidden, float* y) {
  const int t = blockIdx.y;
  const int n4 = blockIdx.x * 256 + threadIdx.x;
  if (n4 * 4 >= hidden) return;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < top_k; ++j) {
    const float wj = w[(int64_t)t * top_k + j];
    const f32x4 v = *reinterpret_cast<const f32x4*>(o + (int64_t)inv[(int64_t)t * top_k + j] * hidden + n4 * 4);
    acc.x = __builtin_fmaf(wj, v.x, acc.x);
    acc.y = __builtin_fmaf(wj, v.y, acc.y);
    acc.z = __builtin_fmaf(wj, v.z, acc.z);
    acc.w = __builtin_fmaf(wj, v.w, acc.w);
  }
  if (g) {
    const float gt = g[t];
    const f32x4 v = *reinterpret_cast<const f32x4*>(o + ((int64_t)m * top_k + t) * hidden + n4 * 4);
    acc.x = __builtin_fmaf(gt, v.x, acc.x);
    acc.y = __builtin_fmaf(gt, v.y, acc.y);
    acc.z = __builtin_fmaf(gt, v.z, acc.z);
    acc.w = __builtin_fmaf(gt, v.w, acc.w);
  }
  *reinterpret_cast<f32x4*>(y + (int64_t)t * hidden + n4 * 4) = acc;
}

constexpr int kTNGate = 128;     // columns per matrix in the gate/up tiles
constexpr int kTNDown = 256;     // columns in the down tiles

int grid_for(int m, int top_k, int n_exp, int shared, int nct) {
  // upper bound of row tiles: every group may waste one partial tile
  const int pairs = m * top_k + (shared ? m : 0);
  const int groups = (n_exp < m * top_k ? n_exp : m * top_k) + (shared ? 1 : 0);
  const int tiles = (pairs / kTM + groups) * nct;
  return (tiles + 7) / 8 * 8;
}

}  // namespace

size_t prefill_workspace_extra_bytes(int, int n_exp, int) { return (size_t)(n_exp + 2) * 4; }

hipError_t prefill_launch(const PrefillArgs& p, hipStream_t s) {
  const bfp_moe_layer* L = p.L;
  const int shared = L->sh_gate.fmt != 0;
  const int H = (int)L->hidden, F = (int)L->inter, K = L->top_k;
  if (F % kTNGate != 0 || H % kTNDown != 0 || H % kTK != 0 || F % kTK != 0) return hipErrorNotSupported;
  const int32_t* tile_start = p.tile_start;
  PfArgs a{};
  a.active = p.active; a.n_active = p.n_active; a.offsets = p.offsets; a.perm = p.perm;
  a.tile_start = tile_start; a.with_shared = shared; a.m = p.m; a.top_k = K;
  // gate/up + SwiGLU -> h (bf16)
  a.exp0 = L->gate.exp; a.code0 = L->gate.code; a.exp1 = L->up.exp; a.code1 = L->up.code;
  if (shared) {
    a.sexp0 = L->sh_gate.exp; a.scode0 = L->sh_gate.code; a.sexp1 = L->sh_up.exp; a.scode1 = L->sh_up.code;
  }
  a.rows_per_expert = F; a.k = H;
  a.a = p.x; a.lda = H; a.a_by_token = 1;
  a.c = p.h; a.ldc = F;
  hipLaunchKernelGGL((grouped_gemm_kernel<2>), dim3(grid_for(p.m, K, L->n_experts, shared, F / kTNGate)),
                     dim3(kPT), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // down -> o (fp32)
  PfArgs b = a;
  b.exp0 = L->down.exp; b.code0 = L->down.code; b.exp1 = nullptr; b.code1 = nullptr;
  b.sexp0 = shared ? L->sh_down.exp : nullptr; b.scode0 = shared ? L->sh_down.code : nullptr;
  b.sexp1 = nullptr; b.scode1 = nullptr;
  b.rows_per_expert = H; b.k = F;
  b.a = p.h; b.lda = F; b.a_by_token = 0;
  b.c = p.o; b.ldc = H;
  hipLaunchKernelGGL((grouped_gemm_kernel<1>), dim3(grid_for(p.m, K, L->n_experts, shared, H / kTNDown)),
                     dim3(kPT), 0, s, b);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  dim3 grid((H / 4 + 255) / 256, p.m);
  hipLaunchKernelGGL(pf_combine_kernel, grid, dim3(256), 0, s, p.o, p.inv, p.w, p.g, p.m, K, H, p.y);
  return hipGetLastError();
}

int prefill_tile_rows() { return kTM; }

}  // namespace bfp
