// "Team" layout: each XCD runs one batch row's whole recurrence.
//
// The grid is 8 teams of P workgroups; the workgroups of one team share
// blockIdx % 8 and therefore one XCD (workgroups are dealt to the 8 XCDs
// round-robin; checked once per handle).  Team x serves batch row x % B.
// With B < 8 the teams x >= B compute nothing: they stamp their region with
// the tags of the call's last two steps and leave (team_stamp_tail).
//
// Within a team, the N rows of W are split over its P * V waves (balanced to
// within one row; V = 8 waves per workgroup, 12 or 16 for sparse layers with
// many rows per wave); a wave keeps its rows in registers for all T steps.  Per
// step the team exchanges h_{t-1} through its own XCD's region of the ring,
// ring[xcd][2][Npad], with ordinary stores and loads that stay in the XCD's
// L2: no data crosses between XCDs inside the time loop.  Words carry the
// same step tag as in the other layout (bit 31 = (S >> 1) & 1, slot S & 1).
// Region x is indexed by the hardware XCD id, written and read only by the
// workgroups running on XCD x (and reset by them), and written for every
// step of every call, so it always holds steps S-1 and S-2 when step S
// starts, whatever batch row the team on it serves.
//
// Per step each of the V waves stages its share of h_{t-1} (chunks w, w+V,
// ...) from the region into a double-buffered LDS row, spinning on the tags;
// one workgroup barrier later every wave multiplies its rows with the whole
// row from LDS.  A wave whose wait expires raises a workgroup abort flag but
// still reaches the barrier; the workgroup then leaves together.
#pragma once

#include <type_traits>

#include "device_common.h"
#include "team_pinned.h"
#include "kernels.h"
#include "dense_kernel.h"
#include "sparse_kernel.h"

namespace prnn {

constexpr int kTeamWaves = 8;

struct TeamPos {
  int team, rank, b, wave, lane, q;  // q = global wave index inside the team
  bool primary;
  int nr, r0;                        // this wave's rows
};

template <int W = kTeamWaves>
__device__ __forceinline__ TeamPos team_pos(const StepArgs& a) {
  TeamPos p;
  p.team = blockIdx.x & 7;
  p.rank = blockIdx.x >> 3;
  p.b = p.team % a.B;
  p.primary = p.team < a.B;
  p.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform for the compiler
  p.lane = threadIdx.x & 63;
  p.q = p.rank * W + p.wave;
  p.nr = a.base_rows + (p.q < a.extra_rows ? 1 : 0);
  p.r0 = p.q * a.base_rows + min(p.q, a.extra_rows);
  return p;
}

// This XCD's region of the team ring: [2][Npad] words.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t team_region(const StepArgs& a) {
  const uint32_t xcc = __builtin_amdgcn_s_getreg((20) | (31 << 11)) & 7u;  // HW_REG_XCC_ID
  return make_rsrc(a.ring + (size_t)xcc * 2 * a.Npad, 2u * a.Npad * 4u);
}

// 1 if f is finite and rounds to an fp16 infinity (|f| >= 65520), from the
// magnitude bits alone (one unsigned compare, no branch).
__device__ __forceinline__ uint32_t beyond_fp16(float f) {
  const uint32_t m = __float_as_uint(f) & 0x7fffffffu;
  return (m - 0x477FF000u) < (0x7F800000u - 0x477FF000u) ? 1u : 0u;  // [65520, inf)
}

// One staged 4-word chunk into the LDS row: fp32 as is, or rounded to fp16
// (round to nearest even) for the half-h dense path, which also records in
// `bad` a finite value beyond the fp16 range.
__device__ __forceinline__ void store_chunk(float* d, const float4& f, uint32_t&) {
  *reinterpret_cast<float4*>(d) = f;
}
__device__ __forceinline__ void store_chunk(_Float16* d, const float4& f, uint32_t& bad) {
  const f16x2 a = {(_Float16)f.x, (_Float16)f.y};
  const f16x2 b = {(_Float16)f.z, (_Float16)f.w};
  bad |= beyond_fp16(f.x) | beyond_fp16(f.y) | beyond_fp16(f.z) | beyond_fp16(f.w);
  *reinterpret_cast<uint2*>(d) = make_uint2(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b));
}

// Stages chunks w, w + 8, ... of ring slot `slot` into the LDS row `dst`
// (Npad elements), waiting until every word carries `tag`; W = waves per
// workgroup.  Returns false if the wait expired (the caller must still reach
// the workgroup barrier).
template <int W = kTeamWaves, typename HT>
__device__ __forceinline__ bool team_stage(__amdgpu_buffer_rsrc_t region, uint32_t slot, int npad, int n, int jn,
                                           int wave, int lane, uint32_t tag, uint64_t deadline, HT* dst,
                                           uint32_t& bad) {
  const uint32_t base = slot * (uint32_t)npad * 4u;
  bool ok = true;
  for (int j = wave; j < jn; j += W) {
    const int c = 256 * j + 4 * lane;
    u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(region, base + 4u * c, 0, kCoherent);
    const uint64_t t0 = now_ticks();
    while (true) {
      const bool mine = chunk_ready(v, tag, c, n);
      if (!wave_any(!mine)) break;
      // Re-issue before reading the clock: the clock read then overlaps the
      // load instead of adding its latency to every poll.
      if (!mine) v = __builtin_amdgcn_raw_buffer_load_b128(region, base + 4u * c, 0, kCoherent);
      if (now_ticks() - t0 > deadline) { ok = false; break; }
    }
    if (!ok) break;
    if (c < n) store_chunk(dst + c, chunk_values(v, c, n), bad);
  }
  return ok;
}

// h0 (or zeros) into the LDS row, all threads of the workgroup.
template <typename HT>
__device__ __forceinline__ void team_stage_h0(const float* h0, int b, int n, int npad, HT* dst, uint32_t& bad) {
  for (int c = threadIdx.x; c < npad; c += blockDim.x) {
    const float f = (h0 != nullptr && c < n) ? h0[(size_t)b * n + c] : 0.f;
    if (std::is_same<HT, _Float16>::value) bad |= beyond_fp16(f);
    dst[c] = (HT)f;
  }
}

// Phase timing for the trace instances; compiles to nothing otherwise.  The
// shader clock is read with s_memtime, whose result the next use waits for,
// so a traced run is a little slower than an untraced one.
template <bool ON>
struct PhaseClock {
  __device__ __forceinline__ void start() {}
  __device__ __forceinline__ void mark(int) {}
  __device__ __forceinline__ void finish(uint64_t*, int) {}
};
template <>
struct PhaseClock<true> {
  uint64_t acc[5], last, c0, r0;
  __device__ __forceinline__ void start() {
    for (int k = 0; k < 5; ++k) acc[k] = 0;
    r0 = __builtin_amdgcn_s_memrealtime();
    c0 = last = __builtin_amdgcn_s_memtime();
  }
  __device__ __forceinline__ void mark(int k) {
    const uint64_t now = __builtin_amdgcn_s_memtime();
    acc[k] += now - last;
    last = now;
  }
  // out = this wave's record; lane 0 writes it.
  __device__ __forceinline__ void finish(uint64_t* out, int steps) {
    const uint64_t c1 = __builtin_amdgcn_s_memtime();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    if ((threadIdx.x & 63) == 0) {
      for (int k = 0; k < 5; ++k) out[k] = acc[k];
      out[kTrLoopCycles] = c1 - c0;
      out[kTrLoopTicks] = r1 - r0;
      out[kTrSteps] = (uint64_t)steps;
    }
  }
};

template <int W = kTeamWaves>
__device__ __forceinline__ uint64_t* trace_record(const StepArgs& a, const TeamPos& p) {
  return a.trace + ((size_t)blockIdx.x * W + (size_t)p.wave) * kTraceWords;
}

// The dense recurrence in the team layout.  RW = rows per wave (capacity),
// J = 256-column chunks per row (capacity).
// Register form of a 4-weight chunk for each weight type: fp32 as is, fp16
// either packed (v_fma_mix_f32) or widened to fp32 in the prologue.
template <typename WT, bool WIDE>
struct TeamChunk { using type = WChunk<WT>; };
template <>
struct TeamChunk<_Float16, true> { using type = WChunkWide; };

// Widened instances keep as many of their rows widened as 196 weight VGPRs
// hold (the 7 x 7 instance: every row) and the rest packed.  Both forms do one
// fused multiply-add per weight with one rounding, so the split changes no
// result, only how fast the rows issue.
constexpr int kWideWeightRegs = 196;
constexpr int team_wide_rows(bool wide, int rw, int j) {
  const int fit = (kWideWeightRegs / j - 2 * rw) / 2;  // 4 registers widened, 2 packed per chunk
  return !wide ? 0 : fit < 0 ? 0 : fit < rw ? fit : rw;
}

// Keeps this XCD's region continuous when the team serves no batch row of its
// own (B < 8): the next call only needs the tags of this call's last two
// steps, so the team stamps those on its rows and leaves.  No one reads the
// region during this call.
__device__ __forceinline__ void team_stamp_tail(const StepArgs& a, const TeamPos& p,
                                                __amdgpu_buffer_rsrc_t region) {
  const uint32_t last = a.step0 + (uint32_t)(a.T - 1);
  for (int k = 0; k < 2 && k < a.T; ++k) {
    const uint32_t S = last - (uint32_t)k;
    for (int r = p.lane; r < p.nr; r += 64)
      __builtin_amdgcn_raw_buffer_store_b32(tag_bit(S), region, ((S & 1u) * a.Npad + p.r0 + r) * 4u, 0, kPlain);
  }
}

// Widened weights at fixed registers (team_pinned.h) for the instances that
// have them.  Left to itself the register allocator scattered the widened
// weights (two components of a chunk near v20-v100, the other two near
// v110-v190), and the step's multiply-add stream then issued at 2.6-2.7
// cycles per instruction per SIMD against 2.07 with a regular assignment
// (the same instructions replayed in a probe, every CU busy, two waves per
// SIMD).  The order of the products in each sum does not change.
constexpr bool kPinnedWeights = true;

//
// HALF (fp16 W only): the staged row holds h_{t-1} rounded to fp16 and every
// instruction adds two exact fp16 x fp16 products to the fp32 sums (dot4);
// a finite h outside the fp16 range raises kStatusRange.
template <typename WT, int RW, int J, bool WIDE = false, bool TRACE = false, bool HALF = false>
__global__ void __launch_bounds__(512) dense_team_kernel(StepArgs a) {
  static_assert(!HALF || (std::is_same<WT, _Float16>::value && !WIDE), "half-h needs packed fp16 weights");
  using HT = typename std::conditional<HALF, _Float16, float>::type;
  constexpr int M = pow2_at_least(RW);
  constexpr int kRow = 256 * J;   // LDS row: every chunk the instance can hold
  // 16-byte aligned: the row is read and written in 16- (8-) byte pieces, and
  // the static abort flag would otherwise leave the dynamic block at byte 4.
  extern __shared__ __attribute__((aligned(16))) float lds_words[];
  HT* const lds = reinterpret_cast<HT*>(lds_words);  // [2][kRow] double-buffered h row
  __shared__ int abort_flag;
  const TeamPos p = team_pos(a);
  // A failed run stays failed until reported.  One thread reads the status
  // word so that the whole workgroup takes the same decision.
  if (threadIdx.x == 0) abort_flag = __builtin_nontemporal_load(a.status) != 0u;
  // Words past the row stay zero (their weights are zero too), so every chunk
  // below is read and multiplied without a bounds test and the compiler can
  // issue all the LDS reads of a step together.
  for (int c = a.Npad + (int)threadIdx.x; c < 2 * kRow; c += blockDim.x)
    if (c % kRow >= a.Npad) lds[c] = (HT)0.f;
  __syncthreads();
  if (abort_flag) return;

  const int N = a.N;
  const int jn = a.chunks;
  const bool vec = (N & 3) == 0 && a.w_vec != 0;
  uint32_t range_bad = 0;  // half-h: a staged value beyond the fp16 range
  if (!p.primary) {
    team_stamp_tail(a, p, team_region(a));
    return;
  }
  // rows [0, WR) widened, [WR, RW) packed; the indexes below are constants
  // once the loops are unrolled
  constexpr int WR = team_wide_rows(WIDE, RW, J);
  typename TeamChunk<WT, WIDE>::type ww[WR > 0 ? WR : 1][J];
  WChunk<WT> wp[RW > WR ? RW - WR : 1][J];
#pragma unroll
  for (int r = 0; r < RW; ++r)
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const bool live = r < p.nr && j < jn;
      if (r < WR)
        ww[r < WR ? r : 0][j].load(a.W, (size_t)(p.r0 + r) * N, 256 * j + 4 * p.lane, N, live, vec);
      else
        wp[r < WR ? 0 : r - WR][j].load(a.W, (size_t)(p.r0 + r) * N, 256 * j + 4 * p.lane, N, live, vec);
    }

  const __amdgpu_buffer_rsrc_t region = team_region(a);
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.X, a.x_bytes);
  const int my_row = RowReduce<M>::owner_row(p.lane);
  const bool owner = my_row >= 0 && my_row < p.nr;

  // x of the row this lane owns.  The load for step t + 1 is issued right
  // after step t's staging: the next step's polls, whose waits also drain
  // every earlier load of the wave, then find it long finished.
  const uint32_t xstep = (uint32_t)a.B * (uint32_t)N * 4u;
  uint32_t xoff = ((uint32_t)p.b * (uint32_t)N + (uint32_t)(p.r0 + (owner ? my_row : 0))) * 4u;
  float x_next = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(xr, xoff, 0, kPlain));
  PhaseClock<TRACE> clk;
  clk.start();

  for (int t = 0; t < a.T; ++t) {
    const uint32_t S = a.step0 + (uint32_t)t;
    HT* hrow = lds + (t & 1) * kRow;
    bool ok = true;
    if (t == 0) {
      team_stage_h0(a.h0, p.b, N, a.Npad, hrow, range_bad);
    } else {
      const uint32_t prev = S - 1u;
      ok = team_stage(region, prev & 1u, a.Npad, N, jn, p.wave, p.lane, tag_bit(prev), a.deadline, hrow, range_bad);
    }
    if (!ok && p.lane == 0) {
      abort_flag = 1;
      report_failure(a.status, a.status_host, kStatusTimeout);
    }
    clk.mark(kTrStage);
    __syncthreads();
    clk.mark(kTrBarrier);
    // Waves 4-7 share their SIMDs with waves 0-3, which win the issue
    // arbitration at equal priority and leave their partners to finish the
    // step's arithmetic alone.  Raising the later waves for the arithmetic
    // evens the pairs out: 1.32 -> 1.28 us per step at N = 1792 (exact), the
    // same results.
    if (p.wave >= kTeamWaves / 2) __builtin_amdgcn_s_setprio(2);
    // The abort flag is read together with the row and tested only before
    // the stores, so it adds no LDS round trip to the step's path.
    int aborted_now = abort_flag;
    const float x = x_next;
    xoff += xstep;
    if (t + 1 < a.T) x_next = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(xr, xoff, 0, kPlain));

    float acc[M];
#pragma unroll
    for (int r = 0; r < M; ++r) acc[r] = 0.f;
    if constexpr (HALF) {
      uint2 h[J];
#pragma unroll
      for (int j = 0; j < J; ++j) h[j] = *reinterpret_cast<const uint2*>(hrow + 256 * j + 4 * p.lane);
#pragma unroll
      for (int j = 0; j < J; ++j)
#pragma unroll
        for (int r = 0; r < RW; ++r) wp[r][j].dot4(acc[r], h[j]);
    } else {
      float4 h[J];
#pragma unroll
      for (int j = 0; j < J; ++j) h[j] = *reinterpret_cast<const float4*>(hrow + 256 * j + 4 * p.lane);
      if constexpr (kPinnedWeights && PinnedFma<RW, J>::kAvailable && WR == RW) {
        // every read in flight before the first product, as in the loop below
        __builtin_amdgcn_sched_barrier(0);
        PinnedFma<RW, J>::run(acc, ww, h);
      } else {
#pragma unroll
        for (int j = 0; j < J; ++j)
#pragma unroll
          for (int r = 0; r < RW; ++r) {
            if (r < WR)
              ww[r < WR ? r : 0][j].fma4(acc[r], h[j]);
            else
              wp[r < WR ? 0 : r - WR][j].fma4(acc[r], h[j]);
          }
      }
    }
    if constexpr (TRACE) {
      // the products in asm blocks may otherwise sink past the clock read
#pragma unroll
      for (int r = 0; r < M; ++r) asm volatile("" : : "v"(acc[r]));
    }
    clk.mark(kTrCompute);
    const float sum = RowReduce<M>::reduce(acc, p.lane);
    clk.mark(kTrReduce);
    __builtin_amdgcn_s_setprio(0);
    asm volatile("" : "+v"(aborted_now) : "v"(sum));  // keep the test after the arithmetic
    if (aborted_now) return;
    debug_jitter(a.jitter_seed, a.jitter_span, p.wave, t);
    if (owner && !(p.rank == a.skip_wg && t == a.skip_step)) {
      const uint32_t hb = relu_bits(sum + x);
      const int row = p.r0 + my_row;
      // the exchange store first: the next step waits for it, not for H
      __builtin_amdgcn_raw_buffer_store_b32(hb | tag_bit(S), region, ((S & 1u) * a.Npad + row) * 4u, 0, kPlain);
      a.H[((size_t)t * a.B + p.b) * N + row] = __uint_as_float(hb);
    }
    clk.mark(kTrEpilogue);
  }
  if (HALF && wave_any(range_bad != 0) && p.lane == 0) report_failure(a.status, a.status_host, kStatusRange);
  if (TRACE) clk.finish(trace_record(a, p), a.T);
}

// Rows [0, C) of slot S: every gather first, so their LDS latencies overlap,
// then the multiply-adds (the FMA is inline asm, which the compiler does not
// move loads across).
template <int C, int S, typename P, int RW, int SPR>
__device__ __forceinline__ void gather_fma_rows(P (&pr)[RW][SPR], const float* hrow, float (&acc)[pow2_at_least(RW)]) {
  float hv[C > 0 ? C : 1];
#pragma unroll
  for (int r = 0; r < C; ++r) hv[r] = hrow[pr[r][S].column()];
#pragma unroll
  for (int r = 0; r < C; ++r) pr[r][S].fma(acc[r], hv[r]);
}

// The sparse recurrence in the team layout: the h row is staged once per
// workgroup (all its waves serve the same batch row) and every wave gathers
// from it for its own rows.  RW = rows per wave, SPR = 64-pair slots per row,
// WAVES = waves per workgroup (8; 12 or 16 for layers with many rows per wave).
//
// RAGGED: rows of unequal length (a.row_len), for the unbalanced sparsity the
// pages set against load-balanced pruning ("Sparse Persistent RNNs", table
// "Measured effects reported in the paper", load-balanced pruning row).  The
// rows are ordered by slot count (a.sorted, most first) and dealt to the
// team's Q waves in snake order: round r of the deal gives wave q the row at
// r Q + q for even r and r Q + Q - 1 - q for odd r, so every wave's rows add
// up to about the same number of slots.  A wave places each row's pairs over
// that row's own slots and runs each slot for all its rows up to the slots of
// its longest row (the slots a row does not have are zero pairs): a step
// costs the wave's longest row times its rows, not the layer's.  Running each
// slot only for the rows that have it (one dispatch per slot on their count)
// was slower: 1.92 against 1.76 us per step at 10 %, N = 2304.
template <typename VT, int RW, int SPR, bool TRACE = false, int WAVES = kTeamWaves, bool RAGGED = false>
__global__ void __launch_bounds__(64 * WAVES) sparse_team_kernel(StepArgs a) {
  constexpr int M = pow2_at_least(RW);
  // The two LDS rows of h are `stride` words apart, a bound the instance fixes
  // (N <= RW rows x at most 32 WAVES waves per team; the host passes the same
  // value).  Where the registers allow one more per pair (kTwoSteps), the loop
  // runs two steps per iteration: a gather's address is then the same at every
  // step and the step's row is an immediate offset of the LDS read, instead of
  // an address computed per pair and step (N = 1792, 10 %: 23 -> 1 address
  // instructions per step).  Rows of more than 5 slots (25 % at N = 2304:
  // 2.01 -> 2.08 us per step) and the blocks that would run out of registers
  // keep one step per iteration.
  constexpr int stride = sparse_team_stride(RW, WAVES);
  constexpr bool kTwoSteps = SPR <= 5 && 2 * RW * SPR + 40 <= 512 / (WAVES / 4);
  extern __shared__ __attribute__((aligned(16))) float lds[];  // [2][stride]: word N of each row stays 0
  __shared__ int abort_flag;
  __shared__ uint2 place_scratch[WAVES][64 * SPR];  // prologue only: pair placement
  const TeamPos p = team_pos<WAVES>(a);
  const int N = a.N;
  const int K = a.K;
  if (threadIdx.x == 0) abort_flag = __builtin_nontemporal_load(a.status) != 0u;
  for (int c = N + (int)threadIdx.x; c < 2 * stride; c += blockDim.x)
    if (c % stride >= N) lds[c] = 0.f;
  __syncthreads();
  if (abort_flag) return;
  if (!p.primary) {
    team_stamp_tail(a, p, team_region(a));
    return;
  }

  // The owned rows' pairs into registers, each row in bank-aware order so
  // that the gathers below hit distinct LDS banks.
  Pair<VT> pr[RW][SPR];
  int cnt_max = 0;       // RAGGED: slots of the wave's longest row (wave-uniform)
  int nr = p.nr;         // rows this wave owns
  int my_layer_row = 0;  // the layer row whose sum this lane owns
  const int my_row = RowReduce<M>::owner_row(p.lane);
  const int Q = a.G * WAVES;  // waves of the team
  auto snake = [&](int r) { return r * Q + ((r & 1) ? Q - 1 - p.q : p.q); };
  if constexpr (RAGGED) {
    int rows[RW], lens[RW], ns[RW];
    nr = 0;
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      const int idx = snake(r);
      const int row = idx < N ? a.sorted[idx] : 0;
      const int len = idx < N ? min(max(a.row_len[row], 0), K) : 0;
      rows[r] = __builtin_amdgcn_readfirstlane(row);
      lens[r] = __builtin_amdgcn_readfirstlane(len);
      ns[r] = (lens[r] + 63) >> 6;
      if (idx < N) nr = r + 1;
    }
    load_place_rows_ragged<0, RW, Pair<VT>, SPR>(pr, reinterpret_cast<const int16_t*>(a.W), a.V, rows, lens, ns, K, N,
                                                 p.lane, place_scratch[p.wave]);
    cnt_max = ns[0];  // the wave's rows come longest first
    if (my_row >= 0 && my_row < nr) my_layer_row = a.sorted[snake(my_row)];
  } else {
    load_place_rows<0, RW, Pair<VT>, SPR>(pr, reinterpret_cast<const int16_t*>(a.W), a.V, p.r0, p.nr, a.spr, K, N,
                                          p.lane, place_scratch[p.wave]);
    my_layer_row = p.r0 + (my_row >= 0 && my_row < p.nr ? my_row : 0);
  }

  const __amdgpu_buffer_rsrc_t region = team_region(a);
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.X, a.x_bytes);
  const bool owner = my_row >= 0 && my_row < nr;
  const int jn = a.chunks;
  // Two-step instances of row-balanced fp16 layers keep each pair as its
  // column and its value widened to fp32 (exact): the loop then needs no
  // packed pair at all, and each product is a v_fmac_f32 instead of a
  // v_fma_mix_f32 (the same fused multiply-add with one rounding).
  constexpr bool kWidened = kTwoSteps && !RAGGED && std::is_same<VT, _Float16>::value;
  int wcol[kWidened ? RW : 1][kWidened ? SPR : 1];
  float wval[kWidened ? RW : 1][kWidened ? SPR : 1];
  if constexpr (kWidened) {
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
      for (int s = 0; s < SPR; ++s) {
        wcol[r][s] = pr[r][s].column();
        wval[r][s] = pr[r][s].value();
      }
  }

  // x of the row this lane owns.  The load for step t + 1 is issued right
  // after step t's staging: the next step's polls, whose waits also drain
  // every earlier load of the wave, then find it long finished.
  const uint32_t xstep = (uint32_t)a.B * (uint32_t)N * 4u;
  uint32_t xoff = ((uint32_t)p.b * (uint32_t)N + (uint32_t)my_layer_row) * 4u;
  float x_next = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(xr, xoff, 0, kPlain));
  PhaseClock<TRACE> clk;
  clk.start();

  // One step into the LDS row hrow; false when the run stops (a failure).
  auto step = [&](int t, float* hrow) -> bool {
    const uint32_t S = a.step0 + (uint32_t)t;
    bool ok = true;
    if (t == 0) {
      for (int c = threadIdx.x; c < N; c += blockDim.x) hrow[c] = a.h0 != nullptr ? a.h0[(size_t)p.b * N + c] : 0.f;
    } else {
      const uint32_t prev = S - 1u;
      uint32_t unused = 0;
      ok = team_stage<WAVES>(region, prev & 1u, a.Npad, N, jn, p.wave, p.lane, tag_bit(prev), a.deadline, hrow, unused);
    }
    if (!ok && p.lane == 0) {
      abort_flag = 1;
      report_failure(a.status, a.status_host, kStatusTimeout);
    }
    clk.mark(kTrStage);
    __syncthreads();
    clk.mark(kTrBarrier);
    // Three or four waves per SIMD (12- and 16-wave workgroups): the later
    // waves of each SIMD are raised for the gathers, as in the dense kernel
    // (N = 5760: 1 % 1.78 -> 1.68, 5 % 2.99 -> 2.86 us per step, the same
    // results).  With 8 waves it did not pay (N = 1152: 0.90 -> 0.95).
    if constexpr (WAVES > kTeamWaves) {
      if (p.wave >= 8) __builtin_amdgcn_s_setprio(3);
      else if (p.wave >= 4) __builtin_amdgcn_s_setprio(2);
    }
    // The abort flag is read together with the row and tested only before
    // the stores, so it adds no LDS round trip to the step's path.
    int aborted_now = abort_flag;
    const float x = x_next;
    xoff += xstep;
    if (t + 1 < a.T) x_next = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(xr, xoff, 0, kPlain));

    float acc[M];
#pragma unroll
    for (int r = 0; r < M; ++r) acc[r] = 0.f;
#pragma unroll
    for (int s = 0; s < SPR; ++s) {
      if (RAGGED && s < cnt_max) {
        // every row of the wave for the slots of its longest row (a row's
        // slots past its own are zero pairs)
        float hv[RW];
#pragma unroll
        for (int r = 0; r < RW; ++r) hv[r] = hrow[pr[r][s].column()];
#pragma unroll
        for (int r = 0; r < RW; ++r) pr[r][s].fma(acc[r], hv[r]);
      } else if (kWidened && s < a.spr) {
        float hv[RW];
#pragma unroll
        for (int r = 0; r < RW; ++r) hv[r] = hrow[wcol[r][s]];
#pragma unroll
        for (int r = 0; r < RW; ++r) acc[r] = fmaf(wval[r][s], hv[r], acc[r]);
      } else if (!RAGGED && s < a.spr) {
        // All of the slot's gathers are issued before its first FMA, so
        // their LDS latencies overlap (the FMA is inline asm, which the
        // compiler does not move loads across).
        float hv[RW];
#pragma unroll
        for (int r = 0; r < RW; ++r) hv[r] = hrow[pr[r][s].column()];
#pragma unroll
        for (int r = 0; r < RW; ++r) pr[r][s].fma(acc[r], hv[r]);
      }
    }
    clk.mark(kTrCompute);
    const float sum = RowReduce<M>::reduce(acc, p.lane);
    clk.mark(kTrReduce);
    if constexpr (WAVES > kTeamWaves) __builtin_amdgcn_s_setprio(0);
    asm volatile("" : "+v"(aborted_now) : "v"(sum));  // keep the test after the arithmetic
    if (aborted_now) return false;
    debug_jitter(a.jitter_seed, a.jitter_span, p.wave, t);
    if (owner && !(p.rank == a.skip_wg && t == a.skip_step)) {
      const uint32_t hb = relu_bits(sum + x);
      const int row = my_layer_row;
      // the exchange store first: the next step waits for it, not for H
      __builtin_amdgcn_raw_buffer_store_b32(hb | tag_bit(S), region, ((S & 1u) * a.Npad + row) * 4u, 0, kPlain);
      a.H[((size_t)t * a.B + p.b) * N + row] = __uint_as_float(hb);
    }
    clk.mark(kTrEpilogue);
    return true;
  };
  if constexpr (kTwoSteps) {
    for (int t = 0; t < a.T; t += 2) {
      if (!step(t, lds)) return;
      if (t + 1 < a.T && !step(t + 1, lds + stride)) return;
    }
  } else {
    for (int t = 0; t < a.T; ++t)
      if (!step(t, lds + (t & 1) * a.lds_stride)) return;
  }
  if (TRACE) clk.finish(trace_record<WAVES>(a, p), a.T);
}


#define PRNN_DENSE_TEAM(WT, WTAG, R, JJ) {WTAG, R, JJ, reinterpret_cast<const void*>(&dense_team_kernel<WT, R, JJ>)}
#define PRNN_DENSE_TEAM_WIDE(R, JJ) {kF16, R, JJ, reinterpret_cast<const void*>(&dense_team_kernel<_Float16, R, JJ, true>)}
#define PRNN_SPARSE_TEAM(VT, VTAG, R, S) {VTAG, R, S, reinterpret_cast<const void*>(&sparse_team_kernel<VT, R, S>)}
#define PRNN_DENSE_TEAM_TRACE(WT, WTAG, R, JJ) \
  {WTAG, R, JJ, reinterpret_cast<const void*>(&dense_team_kernel<WT, R, JJ, false, true>)}
#define PRNN_DENSE_TEAM_HALF(R, JJ) \
  {kF16, R, JJ, reinterpret_cast<const void*>(&dense_team_kernel<_Float16, R, JJ, false, false, true>)}
#define PRNN_DENSE_TEAM_HALF_TRACE(R, JJ) \
  {kF16, R, JJ, reinterpret_cast<const void*>(&dense_team_kernel<_Float16, R, JJ, false, true, true>)}
#define PRNN_DENSE_TEAM_WIDE_TRACE(R, JJ) \
  {kF16, R, JJ, reinterpret_cast<const void*>(&dense_team_kernel<_Float16, R, JJ, true, true>)}
#define PRNN_SPARSE_TEAM12(VT, VTAG, R, S) \
  {VTAG, R, S, reinterpret_cast<const void*>(&sparse_team_kernel<VT, R, S, false, 12>), 12}
#define PRNN_SPARSE_TEAM16(VT, VTAG, R, S) \
  {VTAG, R, S, reinterpret_cast<const void*>(&sparse_team_kernel<VT, R, S, false, 16>), 16}
#define PRNN_SPARSE_TEAM16_TRACE(VT, VTAG, R, S) \
  {VTAG, R, S, reinterpret_cast<const void*>(&sparse_team_kernel<VT, R, S, true, 16>), 16}
#define PRNN_SPARSE_ROWS(R, S) \
  {kF16, R, S, reinterpret_cast<const void*>(&sparse_team_kernel<_Float16, R, S, false, 8, true>)}
#define PRNN_SPARSE_ROWS12(R, S) \
  {kF16, R, S, reinterpret_cast<const void*>(&sparse_team_kernel<_Float16, R, S, false, 12, true>), 12}
#define PRNN_SPARSE_TEAM_TRACE(VT, VTAG, R, S) \
  {VTAG, R, S, reinterpret_cast<const void*>(&sparse_team_kernel<VT, R, S, true>)}

}  // namespace prnn
