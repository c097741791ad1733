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
//  * One workgroup (4 waves, two workgroups per CU) computes a 128-row x TN tile of one
//    group. The row tiles of every group come from the dispatch kernel; a small pass sorts
//    them heaviest first (row fragments that hold rows), and workgroup j takes column tile
//    j % nct of sorted row tile j / nct, so that the long tiles start first.
//  * Every operand reaches LDS by buffer loads that write LDS directly (no registers, no
//    waits in the issuing wave): activation rows per K step of 64 (two steps in flight),
//    weight codes per block of two steps with 4 lanes per column (every load instruction
//    touches 16 lines and uses 64 bytes of each), the block exponents into registers. Each
//    ring slot is a separate LDS array named at compile time (the loop is unrolled over a
//    4-step cycle), so the compiler can tell the slot being read from those being filled;
//    one barrier per step, after a counted wait for the step's own loads and for the
//    wave's LDS reads of the slots refilled next.
//  * v_mfma_f32_32x32x16_bf16 with fp32 accumulation; each wave owns all 128 rows of the
//    tile and 64 output columns.
//    A and B share one permutation of K inside every 8-value group (the order the BFP4
//    unpack produces pairs in), which leaves every dot product unchanged: x is permuted once
//    before the gate/up GEMM, and h is written permuted by its epilogue.
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
constexpr int kPT = 256;         // threads per workgroup (two workgroups per CU)
constexpr int kWaves = kPT / 64;
constexpr int kNB = 2;           // 32-column B tiles per wave
constexpr int kWaveCols = 32 * kNB;
constexpr int kStagesA = 2;      // activation steps in the LDS ring
constexpr int kAStageBytes = kTM * kTK * 2;
constexpr int kBBlk = 2;         // K steps per weight-code block
constexpr int kBRing = 2;        // weight-code blocks in the LDS ring
constexpr int kBColBytes = kTK * kBBlk / 2;             // code bytes of one column per block
constexpr int kBWaveBytes = kWaveCols * kBColBytes;
constexpr int kBBlockBytes = kWaves * kBWaveBytes;

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
  const int32_t* items;                             // row tiles, heaviest first: group << 16 | tile
  int with_shared;
  int m, top_k;
  const uint16_t* a;                                // A rows (bf16): x by token, or h by position
  int64_t lda;
  uint32_t a_bytes;                                 // bytes of A (below 2 GiB)
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

// Maps this workgroup to a tile; false when it has none. Workgroup j takes column tile j % nct
// of row tile j / nct in the sorted list: the heaviest tiles start first (list scheduling,
// longest first, as workgroups are dispatched in index order), and the XCDs (workgroups j % 8)
// each get a share of every class.
template <int TN>
__device__ __forceinline__ bool find_tile(const PfArgs& a, TileInfo& t) {
  const int na = *a.n_active;
  const int ng = na + (a.with_shared ? 1 : 0);
  const int nct = (a.rows_per_expert + TN - 1) / TN;
  const int j = blockIdx.x;
  if (j >= a.tile_start[ng] * nct) return false;
  const int item = a.items[j / nct];
  const int g = item >> 16, mt = item & 0xffff, ct = j % nct;
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
// and kNB = 2 B tiles of 32 columns: NMAT = 2 -> the same 32 columns of gate and of up (the
// SwiGLU pair lands in one lane), NMAT = 1 -> 64 adjacent columns. A workgroup therefore
// covers TN = 4 * 64 / NMAT columns of each matrix (two workgroups per CU: the LDS rings
// below take 64 KB each).
//
// Every operand goes through LDS, loaded by buffer loads straight into LDS (no registers):
//  * activations, per K step of 64: kTM rows of 128 bytes, gathered by row, in a ring of
//    kStagesA steps;
//  * weight codes, per block of kBBlk steps: each wave's 64 columns x 64 bytes, in a ring of
//    kBRing blocks. A load instruction covers 16 columns with 4 lanes each, so it touches 16
//    lines and uses 64 bytes of each (with one lane per column, 32 lines and 32 bytes);
//  * the block exponents go to registers, 16 bytes per column per 4 steps.
// Lane group g = lane / 32 takes K values [32g, 32g + 32) of a step, 8 per MFMA; its A
// fragment reads the same K values. Both operand reads use XOR-swizzled 16-byte slots, so
// the 8 lanes a read serves at once hit distinct banks.

// A pointer every lane holds the same value of, moved to scalar registers.
__device__ __forceinline__ void* uniform_ptr(const void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
}

// s_waitcnt vmcnt(n) lgkmcnt(0), expcnt left alone. Before the step's barrier a wave needs
// both: its own loads of the step landed, and its LDS reads of the previous step returned.
// The slot those reads used is refilled right after the barrier, and a read still queued in
// the LDS unit can be overtaken by another wave's load-to-LDS write arriving on the memory
// return path (the compiler waits for a read only where its MFMA consumes it, often after
// the barrier).
template <int N>
__device__ __forceinline__ void wait_vm_lds() {
  static_assert(N >= 0 && N <= 63, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0070 | (N & 0xF) | ((N >> 4) << 14));
}

// keeps the compiler from moving memory accesses across this point
__device__ __forceinline__ void mem_order() { asm volatile("" ::: "memory"); }

template <int NMAT>
__global__ __launch_bounds__(kPT, 2) void grouped_gemm_kernel(PfArgs a) {
  constexpr int TN = kWaves * kWaveCols / NMAT;   // columns per matrix per workgroup
  // one array per ring slot: each gets its own alias scope, so the compiler can tell a read
  // of one slot from the loads still filling another and waits only for the right ones
  __shared__ __align__(16) uint8_t As0[kAStageBytes], As1[kAStageBytes];
  __shared__ __align__(16) uint8_t Bs0[kBBlockBytes], Bs1[kBBlockBytes];
  static_assert(kStagesA == 2 && kBRing == 2, "ring slots are named arrays");
  auto a_slot = [&](auto I) -> uint8_t* {
    if constexpr (decltype(I)::value % 2 == 0) return As0; else return As1;
  };
  auto b_slot = [&](auto I) -> uint8_t* {
    if constexpr (decltype(I)::value % 2 == 0) return Bs0; else return Bs1;
  };
  TileInfo t;
  if (!find_tile<TN>(a, t)) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave wave-uniform
  const int g = lane / 32, lc = lane % 32;
  // A row (token row of x, or pair row of h) of tile row rr; rows past the group read the
  // group's first row: their results are never stored
  auto arow = [&](int rr) {
    const int r = t.row0 + rr < t.n ? t.row0 + rr : t.row0;
    const int pos = t.p0 + r;
    const int tok = t.shared ? r : a.perm[pos] / a.top_k;
    return a.a_by_token ? tok : pos;
  };

  const int nbk = a.k / kBlock;
  const int64_t rows0 = t.shared ? 0 : (int64_t)t.e * a.rows_per_expert;
  const uint8_t* expb[2] = {(t.shared ? a.sexp0 : a.exp0) + rows0 * nbk,
                            NMAT == 2 ? (t.shared ? a.sexp1 : a.exp1) + rows0 * nbk : nullptr};
  const uint8_t* codeb[2] = {(t.shared ? a.scode0 : a.code0) + rows0 * (a.k / 2),
                             NMAT == 2 ? (t.shared ? a.scode1 : a.code1) + rows0 * (a.k / 2) : nullptr};
  // one buffer descriptor per matrix over this group's rows: loads past them (columns past
  // N in the last column tile) return zeros
  // (named descriptors, not an array: the host pass rejects array elements as operands of
  // the load-to-LDS builtin and silently drops the kernel)
  const int cbytes = a.rows_per_expert * (a.k / 2), ebytes = a.rows_per_expert * nbk;
  const __amdgpu_buffer_rsrc_t crs0 = __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(codeb[0]), (short)0, cbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t crs1 = __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(codeb[NMAT - 1]), (short)0, cbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t ers0 = __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(expb[0]), (short)0, ebytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t ers1 = __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(expb[NMAT - 1]), (short)0, ebytes, 0x00020000);
  // this wave's weight rows c = 0..63: matrix and output column
  auto wcol = [&](int c) { return NMAT == 2 ? t.col0 + 32 * wave + c % 32 : t.col0 + 64 * wave + c; };

  // activation loads: 16 instructions per step, 4 per wave, each filling 8 rows (1 KB);
  // lane i brings 16 bytes of row 8 (4 wave + q) + i / 8, source chunk (i % 8) ^ (row % 8),
  // to byte 16 i of the instruction's 1 KB (the activations are stored pre-permuted)
  const __amdgpu_buffer_rsrc_t arsrc = __builtin_amdgcn_make_buffer_rsrc((void*)a.a, (short)0, (int)a.a_bytes, 0x00020000);
  constexpr int kAQ = kTM / 8 / kWaves;  // activation instructions per wave and step
  uint32_t asrc[kAQ];
#pragma unroll
  for (int q = 0; q < kAQ; ++q) {
    const int rr = 8 * (kAQ * wave + q) + lane / 8;
    const int chunk = (lane % 8) ^ (rr % 8);
    asrc[q] = (uint32_t)(((int64_t)arow(rr) * a.lda + chunk * 8) * 2);
  }
  auto load_a = [&](auto STAGE, int step) __attribute__((always_inline)) {
    uint8_t* dst = a_slot(STAGE) + kAQ * wave * 1024;
#pragma unroll
    for (int q = 0; q < kAQ; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(arsrc, (__attribute__((address_space(3))) void*)(dst + q * 1024), 16,
                                               asrc[q], step * kTK * 2, 0, 0);
  };
  // weight-code loads: 4 instructions per block, instruction q covering this wave's columns
  // c = 16 q + 2 p + u / 4 (p = lane / 8, u = lane % 8); the lane brings 16-byte chunk
  // (u % 4) ^ (p % 4) of the column's 64-byte block to byte 16 lane of the instruction's 1 KB,
  // so that chunk j of column c sits at byte (c / 2) 128 + ((c % 2) 4 + (j ^ (c / 2) % 4)) 16
  uint32_t bsrc[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int c = 16 * q + 2 * (lane / 8) + (lane % 8) / 4;
    const int j = (lane % 4) ^ ((lane / 8) % 4);
    bsrc[q] = (uint32_t)(wcol(c) * (a.k / 2) + 16 * j);
  }
  auto load_b = [&](auto SLOT, int blk) __attribute__((always_inline)) {
    uint8_t* dst = b_slot(SLOT) + wave * kBWaveBytes;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(q < 2 ? crs0 : crs1, (__attribute__((address_space(3))) void*)(dst + q * 1024),
                                               16, bsrc[q], blk * kBColBytes, 0, 0);
  };
  // exponent loads: per B tile, the 16 bytes of this lane's column covering 4 steps
  uint32_t eoff[kNB];
#pragma unroll
  for (int b = 0; b < kNB; ++b) eoff[b] = (uint32_t)(wcol(b * 32 + lc) * nbk);
  auto load_e = [&](u32x4* E, int grp) __attribute__((always_inline)) {
#pragma unroll
    for (int b = 0; b < kNB; ++b) E[b] = __builtin_amdgcn_raw_buffer_load_b128(b == 0 ? ers0 : ers1, eoff[b], grp * 16, 0);
  };

  // operand reads, ordinary LDS loads. A: row rt * 32 + lc of the step's stage, chunk 4 g + st
  // at slot (4 g + st) ^ (lc % 8). B: this lane's column b * 32 + lc, chunk j = 2 (step % 2) + g
  // at byte (c / 2) 128 + ((c % 2) 4 + (j ^ (c / 2) % 4)) 16 of the wave's part of the block.
  const int a_off = lc * kTK * 2, a_g4 = 4 * g, a_sw = lc % 8;
  const int b_off = wave * kBWaveBytes + (lc / 2) * 128 + (lc % 2) * 64, b_sw = (lc / 2) % 4;

  // rows of this tile that exist (wave-uniform): MFMAs of fragments past them are skipped
  const int nrt = (min(kTM, t.n - t.row0) + 31) / 32;
  const int nsteps = a.k / kTK;          // even
  const int nblk = nsteps / kBBlk;
  const int ngrp = (nsteps + 3) / 4;

  f32x16 acc[kRT][kNB];
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt)
#pragma unroll
    for (int b = 0; b < kNB; ++b) acc[rt][b] = f32x16{};

  // Step s (I = SP = s % 4 at compile time): wait until this wave's loads of step s have
  // landed (and its LDS reads are done), one barrier (every wave's have; every wave is done
  // with the slots refilled next), issue the activations of step s + 1, on even steps the
  // weight block of steps s + 2 and s + 3, on SP = 0 the exponents of steps s + 4 .. s + 7, then
  // compute. Loads past the end repeat the last step, block or group, so every step issues
  // the same loads. Per wave a step issues 4 activation loads, 4 weight loads on even steps
  // and 2 exponent loads on SP = 0, in that order; counting those issued after the ones step s
  // needs (its activations, issued one step earlier, and on even steps its weight block,
  // issued two steps earlier) gives the wait below.
  u32x4 ecur[kNB], enext[kNB];
  auto step = [&](int s, auto IC, auto NC) __attribute__((always_inline)) {
    constexpr int I = decltype(IC)::value;
    constexpr int SP = I % 4;
    constexpr int NRT = decltype(NC)::value;
    wait_vm_lds<SP == 0 ? 0 : SP == 1 ? 6 : SP == 2 ? 0 : 4>();
    mem_order();
    __builtin_amdgcn_s_barrier();
    mem_order();
    load_a(std::integral_constant<int, (I + 1) % 2>{}, min(s + 1, nsteps - 1));
    mem_order();
    if constexpr (SP % 2 == 0) {
      load_b(std::integral_constant<int, (I / 2 + 1) % 2>{}, min(s / 2 + 1, nblk - 1));
      mem_order();
    }
    if constexpr (SP == 0) {
      load_e(enext, min(s / 4 + 1, ngrp - 1));
      mem_order();
    }
    // this step's code chunks (16 bytes = 32 values per column) and exponents
    const uint8_t* bb = b_slot(std::integral_constant<int, I / 2>{}) + b_off + (((2 * (SP % 2) + g) ^ b_sw) << 4);
    u32x4 cw[kNB];
#pragma unroll
    for (int b = 0; b < kNB; ++b) cw[b] = *reinterpret_cast<const u32x4*>(bb + b * 16 * 128);
    uint32_t ew[kNB];
#pragma unroll
    for (int b = 0; b < kNB; ++b) ew[b] = (ecur[b][SP] >> (16 * g)) & 0xffffu;
    bool ok = true;
#pragma unroll
    for (int b = 0; b < kNB; ++b) ok = ok && ((ew[b] & 0xffu) - 8u) <= 239u && ((ew[b] >> 8) - 8u) <= 239u;
    const bool fast = __builtin_amdgcn_ballot_w64(!ok) == 0;
    // the step's weights dequantized first (one fast/slow decision per slice pair), then the
    // MFMAs and their LDS reads as one straight-line stretch the scheduler can interleave
    bf16x8 bf[4][kNB];
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int b = 0; b < kNB; ++b) {
        const uint32_t e = (ew[b] >> (8 * (st / 2))) & 0xffu;
        u32x4 d;
        if (fast) d = dequant8_fast(cw[b][st], e);
        else d = dequant8_any(cw[b][st], e);
        bf[st][b] = __builtin_bit_cast(bf16x8, d);
      }
    const uint8_t* at = a_slot(IC) + a_off;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const uint8_t* as = at + (((a_g4 + st) ^ a_sw) << 4);
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        const bf16x8 af = *reinterpret_cast<const bf16x8*>(as + rt * 32 * kTK * 2);
#pragma unroll
        for (int b = 0; b < kNB; ++b) acc[rt][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bf[st][b], acc[rt][b], 0, 0, 0);
      }
    }
    if constexpr (SP == 3) {
#pragma unroll
      for (int b = 0; b < kNB; ++b) ecur[b] = enext[b];
    }
  };

  // four steps per iteration (the ring slots of every step known at compile time), then the
  // two steps left when the step count is not a multiple of 4. One copy of the loop per count
  // of row fragments.
  auto run = [&](auto NC) __attribute__((always_inline)) {
    // the first loads in the order the steps issue theirs: exponent group 0, weight block 0,
    // activations 0
    load_e(ecur, 0);
    mem_order();
    load_b(std::integral_constant<int, 0>{}, 0);
    mem_order();
    load_a(std::integral_constant<int, 0>{}, 0);
    mem_order();
    int s = 0;
    for (; s + 4 <= nsteps; s += 4) {
      step(s + 0, std::integral_constant<int, 0>{}, NC);
      step(s + 1, std::integral_constant<int, 1>{}, NC);
      step(s + 2, std::integral_constant<int, 2>{}, NC);
      step(s + 3, std::integral_constant<int, 3>{}, NC);
    }
    if (s < nsteps) {   // nsteps is even
      step(s + 0, std::integral_constant<int, 0>{}, NC);
      step(s + 1, std::integral_constant<int, 1>{}, NC);
    }
  };
  switch (nrt) {
    case 1: run(std::integral_constant<int, 1>{}); break;
    case 2: run(std::integral_constant<int, 2>{}); break;
    case 3: run(std::integral_constant<int, 3>{}); break;
    default: run(std::integral_constant<int, 4>{}); break;
  }

  // epilogue: element i of a 32x32 tile sits at row (i/4)*8 + g*4 + i%4, column lc. h goes
  // out in the permuted pair order of each 8 columns (the down projection reads it as is).
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = rt * 32 + (i / 4) * 8 + g * 4 + (i % 4);
      if (t.row0 + r >= t.n) continue;
      const int64_t pos = t.p0 + t.row0 + r;
      if constexpr (NMAT == 2) {
        const int col = wcol(lc);
        if (col >= a.rows_per_expert) continue;
        const float gv = acc[rt][0][i], uv = acc[rt][1][i];
        const float hv = gv / (1.0f + __expf(-gv)) * uv;
        const int j = col & 7;
        const int pcol = (col & ~7) | ((j & 1) ? 4 + (j >> 1) : (j >> 1));
        static_cast<uint16_t*>(a.c)[pos * a.ldc + pcol] = (uint16_t)f32_to_bf16_rne(hv);
      } else {
#pragma unroll
        for (int b = 0; b < kNB; ++b) {
          const int col = wcol(b * 32 + lc);
          if (col < a.rows_per_expert) static_cast<float*>(a.c)[pos * a.ldc + col] = acc[rt][b][i];
        }
      }
    }
}

// Row-tile classes of a group of n > 0 rows: x = tiles with 4 row fragments (the full ones,
// and a last one of more than 96 rows), y / z / w = 1 if the last tile has 3 / 2 / 1.
__device__ __forceinline__ int4 tile_classes(int n) {
  const int full = n / kTM, rem = n % kTM;
  const int c = (rem > 0 && rem <= 96) ? (rem + 31) / 32 : 0;
  return make_int4(full + (rem > 96 ? 1 : 0), c == 3, c == 2, c == 1);
}

struct PermArgs {
  const uint16_t* x;          // bf16 [m][hidden]
  int64_t n8;                 // m * hidden / 8
  uint16_t* xp;
  const int32_t* offsets;     // dispatch results
  const int32_t* active;
  const int32_t* n_active;
  int m, with_shared;
  int32_t* items;             // out: row tiles, heaviest first
};

// The last workgroup (256 threads) writes the sorted row-tile list: every tile with 4 row
// fragments, then the last tiles with 3, 2 and 1, groups in order within each class. The
// other workgroups permute x -> xp: every 8 values in the pair order (x0,x2)(x4,x6)(x1,x3)
// (x5,x7) of the weight unpack (the gate/up activations, copied as they are into LDS by the
// grouped GEMM).
__global__ __launch_bounds__(256) void permute_rows_kernel(PermArgs p) {
  if (blockIdx.x + 1 < gridDim.x) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < p.n8) *reinterpret_cast<uint4*>(p.xp + i * 8) = permute8(*reinterpret_cast<const uint4*>(p.x + i * 8));
    return;
  }
  __shared__ int4 wtot[4];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int na = *p.n_active, ng = na + p.with_shared;
  auto rows_of = [&](int g) { return g < na ? p.offsets[p.active[g] + 1] - p.offsets[p.active[g]] : p.m; };
  // exclusive block scan of v (tot: the block's sum)
  auto scan = [&](int4 v, int4& tot) {
    int4 inc = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int a0 = __shfl_up(inc.x, o), a1 = __shfl_up(inc.y, o), a2 = __shfl_up(inc.z, o), a3 = __shfl_up(inc.w, o);
      if (lane >= o) { inc.x += a0; inc.y += a1; inc.z += a2; inc.w += a3; }
    }
    if (lane == 63) wtot[w] = inc;
    __syncthreads();
    int4 base = make_int4(0, 0, 0, 0);
    tot = make_int4(0, 0, 0, 0);
    for (int i = 0; i < 4; ++i) {
      const int4 t = wtot[i];
      if (i < w) { base.x += t.x; base.y += t.y; base.z += t.z; base.w += t.w; }
      tot.x += t.x; tot.y += t.y; tot.z += t.z; tot.w += t.w;
    }
    __syncthreads();
    return make_int4(base.x + inc.x - v.x, base.y + inc.y - v.y, base.z + inc.z - v.z, base.w + inc.w - v.w);
  };
  int4 T = make_int4(0, 0, 0, 0);
  for (int g0 = 0; g0 < ng; g0 += 256) {
    const int g = g0 + tid;
    int4 tot;
    scan(g < ng ? tile_classes(rows_of(g)) : make_int4(0, 0, 0, 0), tot);
    T.x += tot.x; T.y += tot.y; T.z += tot.z; T.w += tot.w;
  }
  int4 run = make_int4(0, T.x, T.x + T.y, T.x + T.y + T.z);   // where each class starts
  for (int g0 = 0; g0 < ng; g0 += 256) {
    const int g = g0 + tid;
    const int n = g < ng ? rows_of(g) : 0;
    const int4 v = g < ng ? tile_classes(n) : make_int4(0, 0, 0, 0);
    int4 tot;
    const int4 ex = scan(v, tot);
    if (g < ng) {
      for (int mt = 0; mt < v.x; ++mt) p.items[run.x + ex.x + mt] = g << 16 | mt;
      const int last = g << 16 | (n / kTM);
      if (v.y) p.items[run.y + ex.y] = last;
      if (v.z) p.items[run.z + ex.z] = last;
      if (v.w) p.items[run.w + ex.w] = last;
    }
    run.x += tot.x; run.y += tot.y; run.z += tot.z; run.w += tot.w;
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

constexpr int kTNGate = kWaves * kWaveCols / 2;   // columns per matrix in the gate/up tiles
constexpr int kTNDown = kWaves * kWaveCols;       // columns in the down tiles

int grid_for(int m, int top_k, int n_exp, int shared, int nct) {
  // upper bound of row tiles: every group may waste one partial tile
  const int pairs = m * top_k + (shared ? m : 0);
  const int groups = (n_exp < m * top_k ? n_exp : m * top_k) + (shared ? 1 : 0);
  const int tiles = (pairs / kTM + groups) * nct;
  return (tiles + 7) / 8 * 8;
}

}  // namespace

// extra region: the dispatch kernel's tile starts [n_exp + 2], the sorted row tiles (at most
// one partial tile per group beyond the full ones), then the permuted activations; each part
// 256-byte aligned
static size_t round256(size_t b) { return (b + 255) / 256 * 256; }
static size_t items_offset(int n_exp) { return round256((size_t)(n_exp + 2) * 4); }
static size_t max_items(int m, int n_exp, int top_k) { return (size_t)(m * top_k + m) / kTM + n_exp + 1; }
static size_t xp_offset(int m, int n_exp, int top_k) { return items_offset(n_exp) + round256(max_items(m, n_exp, top_k) * 4); }

bool prefill_supported(const bfp_moe_layer* L, int64_t m) {
  const int64_t H = L->hidden, F = L->inter, K = L->top_k;
  // K steps come in weight blocks of two; the last column tile may be partial
  if (H % (kTK * kBBlk) != 0 || F % (kTK * kBBlk) != 0 || F % 8 != 0) return false;
  // activations and one expert's weights are addressed with 32-bit byte offsets
  if (F * H / 2 >= (1ll << 31)) return false;
  if (m * H * 2 >= (1ll << 31) || (m * K + m) * F * 2 >= (1ll << 31)) return false;
  return true;
}

hipError_t prefill_launch(const PrefillArgs& p, hipStream_t s) {
  const bfp_moe_layer* L = p.L;
  const int shared = L->sh_gate.fmt != 0;
  const int H = (int)L->hidden, F = (int)L->inter, K = L->top_k;
  if (!prefill_supported(L, p.m)) return hipErrorNotSupported;
  const int32_t* tile_start = p.extra;
  char* extra = reinterpret_cast<char*>(p.extra);
  int32_t* items = reinterpret_cast<int32_t*>(extra + items_offset(L->n_experts));
  uint16_t* xp = reinterpret_cast<uint16_t*>(extra + xp_offset(p.m, L->n_experts, K));
  PermArgs pa{};
  pa.x = p.x; pa.n8 = (int64_t)p.m * H / 8; pa.xp = xp;
  pa.offsets = p.offsets; pa.active = p.active; pa.n_active = p.n_active;
  pa.m = p.m; pa.with_shared = shared; pa.items = items;
  hipLaunchKernelGGL(permute_rows_kernel, dim3((unsigned)((pa.n8 + 255) / 256 + 1)), dim3(256), 0, s, pa);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  PfArgs a{};
  a.active = p.active; a.n_active = p.n_active; a.offsets = p.offsets; a.perm = p.perm;
  a.tile_start = tile_start; a.items = items; a.with_shared = shared; a.m = p.m; a.top_k = K;
  // gate/up + SwiGLU -> h (bf16)
  a.exp0 = L->gate.exp; a.code0 = L->gate.code; a.exp1 = L->up.exp; a.code1 = L->up.code;
  if (shared) {
    a.sexp0 = L->sh_gate.exp; a.scode0 = L->sh_gate.code; a.sexp1 = L->sh_up.exp; a.scode1 = L->sh_up.code;
  }
  a.rows_per_expert = F; a.k = H;
  a.a = xp; a.lda = H; a.a_by_token = 1; a.a_bytes = (uint32_t)((int64_t)p.m * H * 2);
  a.c = p.h; a.ldc = F;
  hipLaunchKernelGGL((grouped_gemm_kernel<2>), dim3(grid_for(p.m, K, L->n_experts, shared, (F + kTNGate - 1) / kTNGate)),
                     dim3(kPT), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // down -> o (fp32)
  PfArgs b = a;
  b.exp0 = L->down.exp; b.code0 = L->down.code; b.exp1 = nullptr; b.code1 = nullptr;
  b.sexp0 = shared ? L->sh_down.exp : nullptr; b.scode0 = shared ? L->sh_down.code : nullptr;
  b.sexp1 = nullptr; b.scode1 = nullptr;
  b.rows_per_expert = H; b.k = F;
  b.a = p.h; b.lda = F; b.a_by_token = 0; b.a_bytes = (uint32_t)(((int64_t)p.m * K + shared * p.m) * F * 2);
  b.c = p.o; b.ldc = H;
  hipLaunchKernelGGL((grouped_gemm_kernel<1>), dim3(grid_for(p.m, K, L->n_experts, shared, (H + kTNDown - 1) / kTNDown)),
                     dim3(kPT), 0, s, b);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  dim3 grid((H / 4 + 255) / 256, p.m);
  hipLaunchKernelGGL(pf_combine_kernel, grid, dim3(256), 0, s, p.o, p.inv, p.w, p.g, p.m, K, H, p.y);
  return hipGetLastError();
}

int prefill_tile_rows() { return kTM; }

size_t prefill_workspace_extra_bytes(int m, int n_exp, int top_k, int hidden) {
  return xp_offset(m, n_exp, top_k) + (size_t)m * hidden * sizeof(uint16_t);
}

}  // namespace bfp
