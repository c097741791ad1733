#pragma once
// Skinny BFP4/BFP8 matmul for one activation row (decode GEMV at m = 1) on gfx950: one wave per
// weight row, activations held in registers.
//
// What it computes ("Qwen3.6-35B-A3B — TT-native mixed BFP4/BFP8 (GPTQ experts)", sections
// "Precision as served" and "Speed": dense projections, LM head and experts stream their BFP
// weights every decode step, so the step costs what its weight bytes cost to read):
// y[j] = sum_k x[k] * W[j][k] (optionally SwiGLU over two matrices, or the greedy pick of the
// largest y[j]), W stored [N][K] as 16-value blocks along K.
//
// Design (bound by HBM; the vector ALUs do the unpack and the products):
//  * K is cut into steps of 1024 values, one 16-value block per lane of a wave, and the steps
//    into slices of J steps (J from K alone). A task is one (row, slice) pair: lane p of the
//    wave computes the blocks p, p + 64, ..., p + 64 (J - 1) of the slice, so every load
//    instruction reads 64 consecutive blocks of one row (512 B of BFP4 codes or 1 KiB of BFP8
//    codes, 64 B of exponents).
//  * One workgroup of twelve waves per compute unit (its LDS request keeps a second one off the
//    unit), each owning an equal share of the rows: every unit streams the same weight bytes.
//    The workgroup stages x in LDS once, by load-to-LDS buffer loads issued before the first
//    weight loads (a register copy issued after them had to wait for them: loads complete
//    in order); a wave keeps its lanes' x values of the current slice
//    in registers (bf16 pairs in the unpack's pair order, or fp32), so no weight is ever
//    matched against x read back from LDS.
//  * A workgroup's tasks are cut into batches of B rows of one slice (slice by slice), handed to
//    the waves in order from a counter in LDS as they ask for them (the waves sharing a SIMD
//    do not progress evenly; with a fixed share each, the compute unit would run the end of
//    the call with fewer loads in flight); each wave keeps the loads of the next D - 1 batches
//    in flight while it computes one (a ring of register buffers, loaded without branches, so
//    that the compiler's wait counts stay exact; the rows of a short batch are clamped to its
//    last row).
//  * A batch's B x NMAT lane sums are reduced over the 64 lanes by recursive halving
//    (v_permlane32_swap, v_permlane16_swap, then DPP), the same tree (lane pairs at distance
//    32, 16, ..., 1) for every value; the results go to LDS as partials[row][slice][matrix].
//  * After a barrier one thread per row adds its slices in slice order and applies the
//    epilogue, or (argmax mode) the workgroup's largest (value, column) key goes to the
//    candidate list that argmax_rows_kernel reduces.
//  * Every output's order of operations (blocks in order inside a lane, the lane tree, slices in
//    order) depends on K only.
#include "argmax.hpp"
#include "bfp_device.hpp"

namespace bfp {
namespace rowk {

constexpr int kWaves = 12;                    // three waves per SIMD
constexpr int kThreads = kWaves * kWave;
constexpr int kStepValues = kWave * kBlock;   // 1024 K values per step
constexpr size_t kLdsFloor = 96 * 1024;       // LDS requested per workgroup: one per compute unit
constexpr size_t kLdsMax = 160 * 1024;

struct RowArgs {
  const uint8_t* exp[2];
  const uint8_t* code[2];
  const void* x;                              // one activation row, bf16 or fp32
  void* y;                                    // one output row, fp32 or bf16
  int y_bf16;
  int n, k;
  int rows;                                   // weight rows per workgroup
  int slices;                                 // K / (J * 1024)
  uint64_t* cand;                             // argmax mode: one key per workgroup, else null
};

template <int FMT> struct BlockCodes;
template <> struct BlockCodes<4> { using T = u32x2; };    // 16 nibbles
template <> struct BlockCodes<8> { using T = u32x4; };    // 16 bytes

// Batch size and ring depth from the task shape (tasks of two matrices are five times the bytes
// of one-step tasks). A one-matrix launch whose workgroups would have fewer batches than waves
// (a short matrix) uses one row per batch instead.
template <int NMAT, int J> constexpr int kBatch = NMAT == 2 ? 1 : (J >= 3 ? 2 : 4);
template <int NMAT, int J> constexpr int kDepth = (NMAT == 1 && J == 1) ? 3 : 2;

template <int FMT, int NMAT, int J, int B>
struct Batch {
  typename BlockCodes<FMT>::T c[B][NMAT][J];
  uint8_t e[B][NMAT][J];                       // kept as bytes: widened where used
};

// x values of one slice for one lane: per step, the lane's 16-value block.
template <bool XB, int J> struct XRegs;
template <int J> struct XRegs<true, J> { uint32_t v[J][8]; };   // bf16 pairs, unpack order
template <int J> struct XRegs<false, J> { float v[J][16]; };

// Batch bi of the workgroup: slice s = bi / nbs, rows r0 .. r0 + count - 1 (relative).
struct BatchPos {
  int s, r0, count;
};
__device__ __forceinline__ BatchPos batch_pos(int bi, int nbs, int nr, int B) {
  BatchPos p;
  p.s = bi / nbs;
  p.r0 = (bi - p.s * nbs) * B;
  p.count = min(B, nr - p.r0);
  return p;
}

// Codes are streamed with nontemporal loads; exponents with ordinary (cached) loads: a row's
// 64 exponent bytes per step are half a 128-byte line whose other half the next step of the
// same batch reads, so keeping the line saves that second fetch (gate/up 19.6-20.2 ->
// 18.9-19.5 us; caching the codes as well was slower).
template <int FMT, int NMAT, int J, int B>
__device__ __forceinline__ void load_batch(Batch<FMT, NMAT, J, B>& g, const RowArgs& a, int row0, const BatchPos& p,
                                           int lane) {
  using T = typename BlockCodes<FMT>::T;
  const int64_t nbk = a.k / kBlock;
  const int64_t cpr = FMT == 8 ? (int64_t)a.k : (int64_t)a.k / 2;
#pragma unroll
  for (int b = 0; b < B; ++b) {
    const int64_t row = row0 + p.r0 + min(b, p.count - 1);      // clamped: no branch
    const int64_t blk0 = (int64_t)p.s * J * kWave;
#pragma unroll
    for (int t = 0; t < NMAT; ++t)
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int64_t blk = blk0 + j * kWave + lane;
        g.c[b][t][j] = __builtin_nontemporal_load(reinterpret_cast<const T*>(a.code[t] + row * cpr) + blk);
        g.e[b][t][j] = a.exp[t][row * nbk + blk];        // cached: see load_batch
      }
  }
}

// The lane's x values of slice s from the staged row (xs: bf16 or fp32 values of all of K).
template <int FMT, bool XB, int J>
__device__ __forceinline__ void load_x(XRegs<XB, J>& xr, const void* xs, int s, int lane) {
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int blk = s * J * kWave + j * kWave + lane;
    if constexpr (XB) {
      const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(xs) + blk * kBlock);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint4 v = src[h];
        uint32_t* o = xr.v[j] + 4 * h;
        if constexpr (FMT == 4) {                                 // (x0,x2) (x4,x6) (x1,x3) (x5,x7)
          o[0] = __builtin_amdgcn_perm(v.y, v.x, 0x05040100u);
          o[1] = __builtin_amdgcn_perm(v.w, v.z, 0x05040100u);
          o[2] = __builtin_amdgcn_perm(v.y, v.x, 0x07060302u);
          o[3] = __builtin_amdgcn_perm(v.w, v.z, 0x07060302u);
        } else {                                                  // (x0,x2) (x1,x3) (x4,x6) (x5,x7)
          o[0] = __builtin_amdgcn_perm(v.y, v.x, 0x05040100u);
          o[1] = __builtin_amdgcn_perm(v.y, v.x, 0x07060302u);
          o[2] = __builtin_amdgcn_perm(v.w, v.z, 0x05040100u);
          o[3] = __builtin_amdgcn_perm(v.w, v.z, 0x07060302u);
        }
      }
    } else {
      const f32x4* src = reinterpret_cast<const f32x4*>(static_cast<const float*>(xs) + blk * kBlock);
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const f32x4 v = src[h];
        xr.v[j][4 * h] = v.x; xr.v[j][4 * h + 1] = v.y; xr.v[j][4 * h + 2] = v.z; xr.v[j][4 * h + 3] = v.w;
      }
    }
  }
}

// Sum over one 16-value block of the lane: products of the unpacked weights (exact small
// integers times 2^-9 for BFP4) with x, in a fixed order.
template <int FMT, bool XB, int J>
__device__ __forceinline__ float block_dot(const typename BlockCodes<FMT>::T& c, const XRegs<XB, J>& xr, int j) {
  float part = 0.f;
  if constexpr (XB) {
    uint32_t w[8];
    if constexpr (FMT == 4) {
      unpack8_bfp4_bf16(c.x, w);
      unpack8_bfp4_bf16(c.y, w + 4);
    } else {
      unpack4_bfp8_bf16(c.x, w);
      unpack4_bfp8_bf16(c.y, w + 2);
      unpack4_bfp8_bf16(c.z, w + 4);
      unpack4_bfp8_bf16(c.w, w + 6);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) part = dot2_bf16(w[i], xr.v[j][i], part);
  } else {
    float w[16];
    if constexpr (FMT == 4) {
      unpack8_bfp4(c.x, w);
      unpack8_bfp4(c.y, w + 8);
    } else {
      unpack4_bfp8(c.x, w);
      unpack4_bfp8(c.y, w + 4);
      unpack4_bfp8(c.z, w + 8);
      unpack4_bfp8(c.w, w + 12);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) part = __builtin_fmaf(w[i], xr.v[j][i], part);
  }
  return part;
}

// Lane sum of one (row, matrix, step) unit of a batch: the block's products, scaled by 2^shift.
template <int FMT, int NMAT, bool XB, int J, int B>
__device__ __forceinline__ float unit_sum(const Batch<FMT, NMAT, J, B>& g, const XRegs<XB, J>& xr, int b, int t,
                                          int j) {
  return apply_shift(block_dot<FMT, XB, J>(g.c[b][t][j], xr, j), block_shift<FMT>(g.e[b][t][j]));
}

// Lane sums of batch g (v[b * NMAT + t], steps in order) while the loads of batch pl go into ld,
// unit by unit: one unit's loads, then one unit's arithmetic. A wave thus never queues a whole
// batch of loads at once (with the memory queue full it would stall there, arithmetic and all);
// the scheduling barriers keep that order.
template <int FMT, int NMAT, bool XB, int J, int B>
__device__ __forceinline__ void load_and_sum(Batch<FMT, NMAT, J, B>& ld, const RowArgs& a, int row0,
                                             const BatchPos& pl, const Batch<FMT, NMAT, J, B>& g,
                                             const XRegs<XB, J>& xr, float (&v)[B * NMAT], int lane) {
  using T = typename BlockCodes<FMT>::T;
  const int64_t nbk = a.k / kBlock;
  const int64_t cpr = FMT == 8 ? (int64_t)a.k : (int64_t)a.k / 2;
#pragma unroll
  for (int b = 0; b < B; ++b) {
    const int64_t row = row0 + pl.r0 + min(b, pl.count - 1);
    const int64_t blk0 = (int64_t)pl.s * J * kWave;
#pragma unroll
    for (int t = 0; t < NMAT; ++t) {
      float acc;
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int64_t blk = blk0 + j * kWave + lane;
        ld.c[b][t][j] = __builtin_nontemporal_load(reinterpret_cast<const T*>(a.code[t] + row * cpr) + blk);
        ld.e[b][t][j] = a.exp[t][row * nbk + blk];        // cached: see load_batch
        __builtin_amdgcn_sched_barrier(0);
        const float u = unit_sum<FMT, NMAT, XB, J, B>(g, xr, b, t, j);
        acc = j == 0 ? u : acc + u;
        __builtin_amdgcn_sched_barrier(0);
      }
      v[b * NMAT + t] = acc;
    }
  }
}

// Lane sums of batch g without loads (the wave's last rounds).
template <int FMT, int NMAT, bool XB, int J, int B>
__device__ __forceinline__ void sum_batch(const Batch<FMT, NMAT, J, B>& g, const XRegs<XB, J>& xr,
                                          float (&v)[B * NMAT]) {
#pragma unroll
  for (int b = 0; b < B; ++b)
#pragma unroll
    for (int t = 0; t < NMAT; ++t) {
      float acc;
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const float u = unit_sum<FMT, NMAT, XB, J, B>(g, xr, b, t, j);
        acc = j == 0 ? u : acc + u;
      }
      v[b * NMAT + t] = acc;
    }
}

// A batch's lane sums reduced over the wave and written to the workgroup's partials.
template <int NMAT, int B>
__device__ __forceinline__ void reduce_store(float (&v)[B * NMAT], const BatchPos& p, float* part, int slices,
                                             int lane) {
  constexpr int C = B * NMAT;
  using Red = LaneReduce<C, 1, kWave>;
  Red::run(v, lane);
  if (Red::writer(lane)) {
    const int idx = Red::first_index(lane);          // one value per writer lane
    const int b = idx / NMAT, t = idx % NMAT;
    if (b < p.count) part[((p.r0 + b) * slices + p.s) * NMAT + t] = v[0];
  }
}

template <int FMT, int NMAT, bool XB, int J, bool AM, int B = kBatch<NMAT, J>>
__global__ __launch_bounds__(kThreads) void row_gemv_kernel(RowArgs a) {
  constexpr int D = kDepth<NMAT, J>;
  using BatchT = Batch<FMT, NMAT, J, B>;
  extern __shared__ __align__(16) unsigned char smem[];
  const size_t xbytes = ((size_t)a.k * (XB ? 2 : 4) + 15) / 16 * 16;
  void* xs = smem;
  float* part = reinterpret_cast<float*>(smem + xbytes);

  const int lane = threadIdx.x & (kWave - 1);
  // wave-uniform (readfirstlane): batch indices, rows and load bases then live in scalar
  // registers, and the vector unit only does the per-lane work
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int row0 = blockIdx.x * a.rows;
  const int nr = min(a.rows, a.n - row0);
  const int nbs = (nr + B - 1) / B;                  // batches per slice
  const int nb = nbs * a.slices;

  // Batches are handed out in order from a workgroup counter in LDS, so a wave that runs ahead
  // (the three waves of a SIMD progress unevenly) takes more of them and all waves finish
  // together. The first D batches of each wave are dealt round-robin (index wave + kWaves d):
  // D - 1 loaded while x is staged (an index past the last batch loads the last one, with no
  // branch, so that the wait counts stay exact, and is never computed), the D-th the wave's
  // first ticket. Each ticket after that is taken from the counter one batch ahead, so that
  // its round trip overlaps the batch being summed.
  __shared__ int next_batch;
  // The activation row goes straight into LDS (load-to-LDS buffer loads: no registers),
  // issued before the weight ring, so that the wave's wait for it does not include the
  // weights: each instruction moves 64 chunks of 16 bytes, and the row is a whole number of
  // such groups (K is a multiple of 1024).
  {
    const int n16 = a.k * (XB ? 2 : 4) / 16;
    const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(a.x), (short)0, n16 * 16,
                                                                         0x00020000);
    for (int c0 = wave * kWave; c0 < n16; c0 += kThreads)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xrs, (__attribute__((address_space(3))) void*)(smem + c0 * 16), 16,
                                               (uint32_t)(c0 + lane) * 16u, 0, 0, 0);
  }
  asm volatile("" ::: "memory");
  BatchT ring[D];
  int idx[D];
#pragma unroll
  for (int d = 0; d < D - 1; ++d) {
    idx[d] = wave + kWaves * d;
    load_batch<FMT, NMAT, J, B>(ring[d], a, row0, batch_pos(min(idx[d], nb - 1), nbs, nr, B), lane);
  }
  asm volatile("" ::: "memory");
  if (threadIdx.x == 0) next_batch = kWaves * D;
  // vmcnt(ring loads): every load issued before the ring (the wave's x chunks) has landed
  {
    constexpr int kRingLoads = (D - 1) * B * NMAT * J * 2;
    static_assert(kRingLoads <= 63, "vmcnt field");
    __builtin_amdgcn_s_waitcnt((0x0F70 & ~0xF) | (kRingLoads & 0xF) | ((kRingLoads >> 4) << 14));
  }
  __syncthreads();

  XRegs<XB, J> xr;
  int cur = -1;
  auto x_for = [&](const BatchPos& p) {
    if (p.s != cur) {
      load_x<FMT, XB, J>(xr, xs, p.s, lane);
      cur = p.s;
    }
  };
  int ticket = wave + kWaves * (D - 1);               // the batch after the ring's, same in every lane
  // Steady state: slot d holds a loaded batch; while the ticket is a batch, its loads go into
  // the free slot as slot d is computed (no load is conditional on this path) and the next
  // ticket is fetched. Indices only grow, so once one is past the end the wave computes the
  // D - 1 slots still in flight that hold a batch, in order, and stops.
  bool live = true;
  while (live) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      if (!live) break;
      const int nxt = ticket;
      if (nxt >= nb) {
#pragma unroll
        for (int e = 0; e < D - 1; ++e) {
          const int sl = (d + e) % D;
          if (idx[sl] < nb) {
            const BatchPos p = batch_pos(idx[sl], nbs, nr, B);
            x_for(p);
            float v[B * NMAT];
            sum_batch<FMT, NMAT, XB, J, B>(ring[sl], xr, v);
            reduce_store<NMAT, B>(v, p, part, a.slices, lane);
          }
        }
        live = false;
        break;
      }
      // here idx[d] < nb too: every index dealt before nxt is smaller than it
      int pending = 0;                                // read back only after this batch is summed
      if (lane == 0)                                  // increment (not add): kept as one LDS op whose result is read late
        pending = (int)__builtin_amdgcn_atomic_inc32(reinterpret_cast<uint32_t*>(&next_batch), 0x7fffffffu, __ATOMIC_RELAXED, "workgroup");
      const BatchPos p = batch_pos(idx[d], nbs, nr, B);
      x_for(p);
      float v[B * NMAT];
      load_and_sum<FMT, NMAT, XB, J, B>(ring[(d + D - 1) % D], a, row0, batch_pos(nxt, nbs, nr, B), ring[d], xr,
                                        v, lane);
      reduce_store<NMAT, B>(v, p, part, a.slices, lane);
      idx[(d + D - 1) % D] = nxt;
      ticket = __builtin_amdgcn_readfirstlane(pending);
    }
  }
  __syncthreads();

  // finalize: slices in order, then the epilogue (or the workgroup's argmax candidate)
  if constexpr (AM) {
    __shared__ uint64_t wbest[kWaves];
    uint64_t best = am::kNone;
    for (int i = threadIdx.x; i < nr; i += kThreads) {
      float s = 0.f;
      for (int sl = 0; sl < a.slices; ++sl) s += part[i * a.slices + sl];
      best = am::kmax(best, am::key_of(s, row0 + i));
    }
    best = am::lane_max<kWave>(best);
    if (lane == 0) wbest[wave] = best;
    __syncthreads();
    if (threadIdx.x == 0) {
#pragma unroll
      for (int w = 1; w < kWaves; ++w) best = am::kmax(best, wbest[w]);
      a.cand[blockIdx.x] = best;
    }
  } else {
    for (int i = threadIdx.x; i < nr; i += kThreads) {
      float v[NMAT];
#pragma unroll
      for (int t = 0; t < NMAT; ++t) {
        float s = 0.f;
        for (int sl = 0; sl < a.slices; ++sl) s += part[(i * a.slices + sl) * NMAT + t];
        v[t] = s;
      }
      float out = v[0];
      if constexpr (NMAT == 2) out = v[0] / (1.0f + __expf(-v[0])) * v[1];
      if (a.y_bf16) static_cast<uint16_t*>(a.y)[row0 + i] = (uint16_t)f32_to_bf16_rne(out);
      else static_cast<float*>(a.y)[row0 + i] = out;
    }
  }
}

// ---- launch (host) --------------------------------------------------------------------------

// Compute units of the current device (cached per device).
int device_cus();

// Largest J <= jmax dividing the number of 1024-value steps.
inline int pick_j(int steps, int jmax) {
  for (int j = jmax; j > 1; --j)
    if (steps % j == 0) return j;
  return 1;
}

// Rows per workgroup and the grid: every compute unit gets the same share (at least 8 rows, the
// bound the argmax workspace assumes).
inline void pick_rows(int n, int& rows, int& grid) {
  const int cus = device_cus();
  rows = (n + cus - 1) / cus;
  if (rows < 8) rows = 8;
  grid = (n + rows - 1) / rows;
}

inline size_t lds_bytes(int k, bool xb, int rows, int slices, int nmat) {
  const size_t xbytes = ((size_t)k * (xb ? 2 : 4) + 15) / 16 * 16;
  return xbytes + (size_t)rows * slices * nmat * sizeof(float);
}

// Whether this kernel takes the shape (K a multiple of 1024, x and partials fit in LDS).
inline bool supported(int n, int k, bool xb, int nmat) {
  if (k % kStepValues != 0 || n < 1) return false;
  int rows, grid;
  pick_rows(n, rows, grid);
  const int steps = k / kStepValues;
  const int slices = steps / pick_j(steps, xb ? 5 : 2);
  return lds_bytes(k, xb, rows, slices, nmat) <= kLdsMax;
}

template <int FMT, int NMAT, bool XB, int J, bool AM>
hipError_t launch_j(RowArgs a, hipStream_t s) {
  int grid;
  pick_rows(a.n, a.rows, grid);
  a.slices = a.k / kStepValues / J;
  size_t lds = lds_bytes(a.k, XB, a.rows, a.slices, NMAT);
  if (lds > kLdsMax) return hipErrorNotSupported;
  if (lds < kLdsFloor) lds = kLdsFloor;
  if constexpr (NMAT == 1 && !AM && kBatch<NMAT, J> > 1) {
    // few tasks per workgroup (a short matrix): one row per batch, so that every wave has one
    if ((a.rows * a.slices + kBatch<NMAT, J> - 1) / kBatch<NMAT, J> < kWaves) {
      hipLaunchKernelGGL((row_gemv_kernel<FMT, NMAT, XB, J, AM, 1>), dim3(grid), dim3(kThreads), lds, s, a);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((row_gemv_kernel<FMT, NMAT, XB, J, AM>), dim3(grid), dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

// Entry for one (format, activation type): m = 1, NMAT matrices (2: SwiGLU), or argmax mode
// (a.cand set; the caller reduces the candidates, one per workgroup, with argmax_rows_kernel).
template <int FMT, bool XB>
hipError_t launch(const RowArgs& a, int nmat, int* grid_out, hipStream_t s) {
  const int steps = a.k / kStepValues;
  const int j = pick_j(steps, XB ? 5 : 2);
  int rows;
  pick_rows(a.n, rows, *grid_out);
  const bool am = a.cand != nullptr;
  if (nmat == 2) {
    switch (j) {
      case 1: return launch_j<FMT, 2, XB, 1, false>(a, s);
      case 2: return launch_j<FMT, 2, XB, 2, false>(a, s);
      default: break;
    }
    if constexpr (XB) {
      switch (j) {
        case 3: return launch_j<FMT, 2, XB, 3, false>(a, s);
        case 4: return launch_j<FMT, 2, XB, 4, false>(a, s);
        case 5: return launch_j<FMT, 2, XB, 5, false>(a, s);
        default: break;
      }
    }
    return hipErrorNotSupported;
  }
  if constexpr (XB) {
    if (am) {
      switch (j) {
        case 1: return launch_j<FMT, 1, XB, 1, true>(a, s);
        case 2: return launch_j<FMT, 1, XB, 2, true>(a, s);
        case 3: return launch_j<FMT, 1, XB, 3, true>(a, s);
        case 4: return launch_j<FMT, 1, XB, 4, true>(a, s);
        case 5: return launch_j<FMT, 1, XB, 5, true>(a, s);
        default: return hipErrorNotSupported;
      }
    }
    switch (j) {
      case 1: return launch_j<FMT, 1, XB, 1, false>(a, s);
      case 2: return launch_j<FMT, 1, XB, 2, false>(a, s);
      case 3: return launch_j<FMT, 1, XB, 3, false>(a, s);
      case 4: return launch_j<FMT, 1, XB, 4, false>(a, s);
      case 5: return launch_j<FMT, 1, XB, 5, false>(a, s);
      default: return hipErrorNotSupported;
    }
  } else {
    if (am) return hipErrorNotSupported;
    switch (j) {
      case 1: return launch_j<FMT, 1, XB, 1, false>(a, s);
      case 2: return launch_j<FMT, 1, XB, 2, false>(a, s);
      default: return hipErrorNotSupported;
    }
  }
}

}  // namespace rowk
}  // namespace bfp
