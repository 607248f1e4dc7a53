// Dense fp16 layers larger than one XCD's register files hold: each batch row
// is served by XP = 2 or 4 XCDs, each holding one part of the rows of W.
//
// "persistent-rnn" ("What This Project Does") keeps the weights in the
// register files; its "Important Constraints" put a limit on the layer size.
// One XCD holds 16 MB of registers, and from N = 2560 on (13.1 MB of fp16 W)
// the rows no longer fit one team of the team layout.  Here the 8 XCDs form
// 8 / XP teams of XP parts: XCD x serves batch row x % (8 / XP) with part
// x / (8 / XP) of the rows, [part * part_rows, part * part_rows + part_rows).
// part_rows is a multiple of 256, so every 256-column chunk of h_{t-1} is
// produced by exactly one part.
//
// Exchange.  Each row's owner publishes h_t twice, with the same step tag as
// the team layout (bit 31 = (S >> 1) & 1, slot S & 1): into its own XCD's
// region of the ring with plain stores (read by the XCD's other workgroups
// through its L2), and into a shared ring[batch row][2][Npad] with stores
// that reach the device coherence point (read by the other parts' XCDs with
// loads that observe it).  Staging takes a chunk from the XCD's own region
// when its part produced it and from the shared ring otherwise; the choice is
// the same for the whole wave.
//
// Weights: fp16, as many rows widened to fp32 as 192 weight registers hold,
// the rest packed (v_fma_mix_f32); one fused multiply-add per weight either
// way, so the split changes no result.  h_{t-1} is read from LDS one chunk at
// a time, which leaves the registers to the weights.
#include "team_kernel.h"

namespace prnn {

namespace {

constexpr int kSplitWeightRegs = 192;
constexpr int split_wide_rows(int rw, int j) {
  const int fit = (kSplitWeightRegs / j - 2 * rw) / 2;  // 4 registers widened, 2 packed per chunk
  return fit < 0 ? 0 : fit < rw ? fit : rw;
}

struct SplitPos {
  int b, part, rank, wave, lane;
  bool primary;
  int nr, r0;  // this wave's rows (r0: row index in the layer)
};

template <int WAVES = kTeamWaves>
__device__ __forceinline__ SplitPos split_pos(const StepArgs& a) {
  SplitPos p;
  const int xp = a.xcds_per_row;
  const int bc = 8 / xp;  // batch rows the grid can serve
  // The team is the hardware XCD (the workgroups sharing blockIdx % 8 all run
  // on one XCD), so an XCD serves the same batch row and part in every call and
  // its region always holds its own part's rows of the last two steps.
  const int team = (int)(__builtin_amdgcn_s_getreg((20) | (31 << 11)) & 7u);  // HW_REG_XCC_ID
  p.b = team % bc;
  p.part = team / bc;
  p.primary = p.b < a.B;
  p.rank = blockIdx.x >> 3;
  p.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  p.lane = threadIdx.x & 63;
  const int part_r0 = p.part * a.part_rows;
  const int len = max(0, min(a.part_rows, a.N - part_r0));
  const int Q = a.G * WAVES;
  const int q = p.rank * WAVES + p.wave;
  const int base = len / Q, extra = len % Q;
  p.nr = base + (q < extra ? 1 : 0);
  p.r0 = part_r0 + q * base + min(q, extra);
  return p;
}

// Shared ring of batch row b: [2][Npad] words after the team ring's 16 Npad.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t split_shared(const StepArgs& a, int b) {
  return make_rsrc(a.ring + 16ull * a.Npad + (size_t)b * 2 * a.Npad, 2u * a.Npad * 4u);
}

// Stages chunks w, w + 8, ... of slot `slot` into the LDS row, each from the
// XCD's region (its own part's chunks) or from the shared ring.  Returns false
// if a wait expired.
template <int WAVES = kTeamWaves>
__device__ __forceinline__ bool split_stage(__amdgpu_buffer_rsrc_t region, __amdgpu_buffer_rsrc_t shared,
                                            int part, int part_chunks, uint32_t slot, int npad, int n, int jn,
                                            int wave, int lane, uint32_t tag, uint64_t deadline, float* dst) {
  const uint32_t base = slot * (uint32_t)npad * 4u;
  bool ok = true;
  for (int j = wave; j < jn; j += WAVES) {
    const __amdgpu_buffer_rsrc_t src = (j / part_chunks == part) ? region : shared;
    const int c = 256 * j + 4 * lane;
    u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(src, base + 4u * c, 0, kCoherent);
    const uint64_t t0 = now_ticks();
    while (true) {
      const bool mine = chunk_ready(v, tag, c, n);
      if (!wave_any(!mine)) break;
      if (!mine) v = __builtin_amdgcn_raw_buffer_load_b128(src, base + 4u * c, 0, kCoherent);
      if (now_ticks() - t0 > deadline) { ok = false; break; }
    }
    if (!ok) break;
    if (c < n) *reinterpret_cast<float4*>(dst + c) = chunk_values(v, c, n);
  }
  return ok;
}

// A team without a batch row of its own stamps its rows, in both rings, with
// the tags of the call's last two steps, so that the next call finds every
// word continuous (as team_stamp_tail does for the team layout).
__device__ __forceinline__ void split_stamp_tail(const StepArgs& a, const SplitPos& p,
                                                 __amdgpu_buffer_rsrc_t region, __amdgpu_buffer_rsrc_t shared) {
  const uint32_t last = a.step0 + (uint32_t)(a.T - 1);
  for (int k = 0; k < 2 && k < a.T; ++k) {
    const uint32_t S = last - (uint32_t)k;
    for (int r = p.lane; r < p.nr; r += 64) {
      const uint32_t off = ((S & 1u) * a.Npad + p.r0 + r) * 4u;
      __builtin_amdgcn_raw_buffer_store_b32(tag_bit(S), shared, off, 0, kCoherent);
      __builtin_amdgcn_raw_buffer_store_b32(tag_bit(S), region, off, 0, kPlain);
    }
  }
}

// RW = rows per wave (capacity), J = 256-column chunks of the whole row.
template <int RW, int J>
__global__ void __launch_bounds__(512) dense_split_kernel(StepArgs a) {
  constexpr int M = pow2_at_least(RW);
  constexpr int kRow = 256 * J;
  extern __shared__ __attribute__((aligned(16))) float lds[];  // [2][kRow] double-buffered h row
  __shared__ int abort_flag;
  const SplitPos p = split_pos(a);
  if (threadIdx.x == 0) abort_flag = __builtin_nontemporal_load(a.status) != 0u;
  for (int c = a.Npad + (int)threadIdx.x; c < 2 * kRow; c += blockDim.x)
    if (c % kRow >= a.Npad) lds[c] = 0.f;
  __syncthreads();
  if (abort_flag) return;

  const int N = a.N;
  const int jn = a.chunks;
  const bool vec = (N & 3) == 0 && a.w_vec != 0;
  const __amdgpu_buffer_rsrc_t region = team_region(a);
  const __amdgpu_buffer_rsrc_t shared = split_shared(a, p.b);
  if (!p.primary) {
    split_stamp_tail(a, p, region, shared);
    return;
  }
  constexpr int WR = split_wide_rows(RW, J);
  WChunkWide ww[WR > 0 ? WR : 1][J];
  WChunk<_Float16> wp[RW > WR ? RW - WR : 1][J];
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

  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.X, a.x_bytes);
  const int my_row = RowReduce<M>::owner_row(p.lane);
  const bool owner = my_row >= 0 && my_row < p.nr;
  const int part_chunks = a.part_rows / 256;

  const uint32_t xstep = (uint32_t)a.B * (uint32_t)N * 4u;
  uint32_t xoff = ((uint32_t)p.b * (uint32_t)N + (uint32_t)(p.r0 + (owner ? my_row : 0))) * 4u;
  float x_next = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(xr, xoff, 0, kPlain));

  for (int t = 0; t < a.T; ++t) {
    const uint32_t S = a.step0 + (uint32_t)t;
    float* hrow = lds + (t & 1) * kRow;
    bool ok = true;
    if (t == 0) {
      uint32_t unused = 0;
      team_stage_h0(a.h0, p.b, N, a.Npad, hrow, unused);
    } else {
      const uint32_t prev = S - 1u;
      ok = split_stage(region, shared, p.part, part_chunks, prev & 1u, a.Npad, N, jn, p.wave, p.lane, tag_bit(prev),
                       a.deadline, hrow);
    }
    if (!ok && p.lane == 0) {
      abort_flag = 1;
      report_failure(a.status, a.status_host, kStatusTimeout);
    }
    __syncthreads();
    if (p.wave >= kTeamWaves / 2) __builtin_amdgcn_s_setprio(2);  // as in the team kernel
    int aborted_now = abort_flag;
    const float x = x_next;
    xoff += xstep;
    if (t + 1 < a.T) x_next = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(xr, xoff, 0, kPlain));

    float acc[M];
#pragma unroll
    for (int r = 0; r < M; ++r) acc[r] = 0.f;
    if constexpr (kPinnedWeights && PinnedFma<RW, J>::kAvailable && WR == RW) {
      // the weights at fixed registers, as in the team kernel
      float4 h[J];
#pragma unroll
      for (int j = 0; j < J; ++j) h[j] = *reinterpret_cast<const float4*>(hrow + 256 * j + 4 * p.lane);
      __builtin_amdgcn_sched_barrier(0);
      PinnedFma<RW, J>::run(acc, ww, h);
    } else {
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const float4 h = *reinterpret_cast<const float4*>(hrow + 256 * j + 4 * p.lane);
#pragma unroll
        for (int r = 0; r < RW; ++r) {
          if (r < WR)
            ww[r < WR ? r : 0][j].fma4(acc[r], h);
          else
            wp[r < WR ? 0 : r - WR][j].fma4(acc[r], h);
        }
      }
    }
    const float sum = RowReduce<M>::reduce(acc, p.lane);
    __builtin_amdgcn_s_setprio(0);
    asm volatile("" : "+v"(aborted_now) : "v"(sum));  // keep the test after the arithmetic
    if (aborted_now) return;
    debug_jitter(a.jitter_seed, a.jitter_span, p.wave, t);
    if (owner && !(p.rank == a.skip_wg && t == a.skip_step)) {
      const uint32_t hb = relu_bits(sum + x) | tag_bit(S);
      const int row = p.r0 + my_row;
      const uint32_t off = ((S & 1u) * a.Npad + row) * 4u;
      // the other parts' copy first: their next step waits on the longer path
      __builtin_amdgcn_raw_buffer_store_b32(hb, shared, off, 0, kCoherent);
      __builtin_amdgcn_raw_buffer_store_b32(hb, region, off, 0, kPlain);
      a.H[((size_t)t * a.B + p.b) * N + row] = __uint_as_float(hb & 0x7fffffffu);
    }
  }
}

// The step protocol of the split layout without weights or arithmetic (the
// per-step floor of a split layer): the same grid, staging from both rings,
// barrier and double publication; each wave publishes t + 1 for its rows
// (at most 64 per wave).
template <int WAVES>
__global__ void __launch_bounds__(64 * WAVES) floor_split_kernel(StepArgs a) {
  extern __shared__ __attribute__((aligned(16))) float lds[];  // [2][Npad]
  __shared__ int abort_flag;
  const SplitPos p = split_pos<WAVES>(a);
  if (threadIdx.x == 0) abort_flag = __builtin_nontemporal_load(a.status) != 0u;
  __syncthreads();
  if (abort_flag) return;
  const int N = a.N;
  const __amdgpu_buffer_rsrc_t region = team_region(a);
  const __amdgpu_buffer_rsrc_t shared = split_shared(a, p.b);
  if (!p.primary) {
    split_stamp_tail(a, p, region, shared);
    return;
  }
  const int part_chunks = a.part_rows / 256;
  for (int t = 0; t < a.T; ++t) {
    const uint32_t S = a.step0 + (uint32_t)t;
    float* hrow = lds + (t & 1) * a.Npad;
    bool ok = true;
    if (t > 0) {
      const uint32_t prev = S - 1u;
      ok = split_stage<WAVES>(region, shared, p.part, part_chunks, prev & 1u, a.Npad, N, a.chunks, p.wave, p.lane,
                              tag_bit(prev), a.deadline, hrow);
    }
    if (!ok && p.lane == 0) {
      abort_flag = 1;
      report_failure(a.status, a.status_host, kStatusTimeout);
    }
    __syncthreads();
    int aborted_now = abort_flag;
    const float seen = t > 0 ? hrow[p.lane] : 0.f;
    asm volatile("" : "+v"(aborted_now) : "v"(seen));
    if (aborted_now) return;
    if (p.lane < p.nr) {
      const uint32_t hb = relu_bits((float)(t + 1) + seen * 0.f) | tag_bit(S);
      const int row = p.r0 + p.lane;
      const uint32_t off = ((S & 1u) * a.Npad + row) * 4u;
      __builtin_amdgcn_raw_buffer_store_b32(hb, shared, off, 0, kCoherent);
      __builtin_amdgcn_raw_buffer_store_b32(hb, region, off, 0, kPlain);
      a.H[((size_t)t * a.B + p.b) * N + row] = __uint_as_float(hb & 0x7fffffffu);
    }
  }
}

// Row-balanced sparse layers split the same way (XP = 2 XCDs per batch row):
// the sparse team kernel's pairs, placement and gathers over the rows of
// this XCD's part, the split layout's staging and double publication.  The
// LDS row holds all N values, at most XP x RW x 32 WAVES words; where the
// registers allow, two steps per iteration with each pair as its column and
// its value widened to fp32 (as in the sparse team kernel).
// RAGGED: rows of unequal length (a.row_len), as in the sparse team kernel,
// over the part: the part's rows ordered by slot count (a.sorted holds each
// part's order in its own range) and dealt to the XCD's waves in snake order;
// each row's pairs over its own slots, each slot run for all the wave's rows
// up to the slots of its longest row.
template <int RW, int SPR, int WAVES, int XP, bool RAGGED = false>
__global__ void __launch_bounds__(64 * WAVES) sparse_split_kernel(StepArgs a) {
  constexpr int M = pow2_at_least(RW);
  constexpr int stride = XP * RW * 32 * WAVES + 4;
  constexpr bool kTwoSteps = !RAGGED && SPR <= 5 && 2 * RW * SPR + 40 <= 512 / (WAVES / 4);
  extern __shared__ __attribute__((aligned(16))) float lds[];  // [2][stride]: word N of each row stays 0
  __shared__ int abort_flag;
  __shared__ uint2 place_scratch[WAVES][64 * SPR];  // prologue only: pair placement
  const SplitPos p = split_pos<WAVES>(a);
  const int N = a.N;
  const int K = a.K;
  if (threadIdx.x == 0) abort_flag = __builtin_nontemporal_load(a.status) != 0u;
  for (int c = N + (int)threadIdx.x; c < 2 * stride; c += blockDim.x)
    if (c % stride >= N) lds[c] = 0.f;
  __syncthreads();
  if (abort_flag) return;
  const __amdgpu_buffer_rsrc_t region = team_region(a);
  const __amdgpu_buffer_rsrc_t shared = split_shared(a, p.b);
  if (!p.primary) {
    split_stamp_tail(a, p, region, shared);
    return;
  }
  Pair<_Float16> pr[RW][SPR];
  int cnt_max = 0;  // RAGGED: slots of the wave's longest row (wave-uniform)
  int nr = p.nr;    // rows this wave owns
  const int my_row = RowReduce<M>::owner_row(p.lane);
  int my_layer_row = p.r0 + (my_row >= 0 && my_row < p.nr ? my_row : 0);  // the row whose sum this lane owns
  if constexpr (RAGGED) {
    const int part_r0 = p.part * a.part_rows;
    const int len = max(0, min(a.part_rows, N - part_r0));
    const int Q = a.G * WAVES;  // waves of the XCD
    const int q = p.rank * WAVES + p.wave;
    auto snake = [&](int r) { return r * Q + ((r & 1) ? Q - 1 - q : q); };
    int rows[RW], lens[RW], ns[RW];
    nr = 0;
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      const int idx = snake(r);
      const int row = idx < len ? a.sorted[part_r0 + idx] : 0;
      const int rl = idx < len ? min(max(a.row_len[row], 0), K) : 0;
      rows[r] = __builtin_amdgcn_readfirstlane(row);
      lens[r] = __builtin_amdgcn_readfirstlane(rl);
      ns[r] = (lens[r] + 63) >> 6;
      if (idx < len) nr = r + 1;
    }
    load_place_rows_ragged<0, RW, Pair<_Float16>, SPR>(pr, reinterpret_cast<const int16_t*>(a.W), a.V, rows, lens, ns,
                                                       K, N, p.lane, place_scratch[p.wave]);
    cnt_max = ns[0];  // the wave's rows come longest first
    if (my_row >= 0 && my_row < nr) my_layer_row = a.sorted[part_r0 + snake(my_row)];
  } else {
    load_place_rows<0, RW, Pair<_Float16>, SPR>(pr, reinterpret_cast<const int16_t*>(a.W), a.V, p.r0, p.nr, a.spr, K,
                                                N, p.lane, place_scratch[p.wave]);
  }
  int wcol[kTwoSteps ? RW : 1][kTwoSteps ? SPR : 1];
  float wval[kTwoSteps ? RW : 1][kTwoSteps ? SPR : 1];
  if constexpr (kTwoSteps) {
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
      for (int s = 0; s < SPR; ++s) {
        wcol[r][s] = pr[r][s].column();
        wval[r][s] = pr[r][s].value();
      }
  }
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.X, a.x_bytes);
  const bool owner = my_row >= 0 && my_row < nr;
  const int part_chunks = a.part_rows / 256;
  const uint32_t xstep = (uint32_t)a.B * (uint32_t)N * 4u;
  uint32_t xoff = ((uint32_t)p.b * (uint32_t)N + (uint32_t)my_layer_row) * 4u;
  float x_next = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(xr, xoff, 0, kPlain));

  auto step = [&](int t, float* hrow) -> bool {
    const uint32_t S = a.step0 + (uint32_t)t;
    bool ok = true;
    if (t == 0) {
      for (int c = threadIdx.x; c < N; c += blockDim.x) hrow[c] = a.h0 != nullptr ? a.h0[(size_t)p.b * N + c] : 0.f;
    } else {
      const uint32_t prev = S - 1u;
      ok = split_stage<WAVES>(region, shared, p.part, part_chunks, prev & 1u, a.Npad, N, a.chunks, p.wave, p.lane,
                              tag_bit(prev), a.deadline, hrow);
    }
    if (!ok && p.lane == 0) {
      abort_flag = 1;
      report_failure(a.status, a.status_host, kStatusTimeout);
    }
    __syncthreads();
    if constexpr (WAVES > kTeamWaves) {
      if (p.wave >= 8) __builtin_amdgcn_s_setprio(3);
      else if (p.wave >= 4) __builtin_amdgcn_s_setprio(2);
    }
    int aborted_now = abort_flag;
    const float x = x_next;
    xoff += xstep;
    if (t + 1 < a.T) x_next = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(xr, xoff, 0, kPlain));
    float acc[M];
#pragma unroll
    for (int r = 0; r < M; ++r) acc[r] = 0.f;
#pragma unroll
    for (int s = 0; s < SPR; ++s) {
      if (RAGGED ? s < cnt_max : s < a.spr) {
        float hv[RW];
        if constexpr (kTwoSteps) {
#pragma unroll
          for (int r = 0; r < RW; ++r) hv[r] = hrow[wcol[r][s]];
#pragma unroll
          for (int r = 0; r < RW; ++r) acc[r] = fmaf(wval[r][s], hv[r], acc[r]);
        } else {
#pragma unroll
          for (int r = 0; r < RW; ++r) hv[r] = hrow[pr[r][s].column()];
#pragma unroll
          for (int r = 0; r < RW; ++r) pr[r][s].fma(acc[r], hv[r]);
        }
      }
    }
    const float sum = RowReduce<M>::reduce(acc, p.lane);
    if constexpr (WAVES > kTeamWaves) __builtin_amdgcn_s_setprio(0);
    asm volatile("" : "+v"(aborted_now) : "v"(sum));  // keep the test after the arithmetic
    if (aborted_now) return false;
    debug_jitter(a.jitter_seed, a.jitter_span, p.wave, t);
    if (owner && !(p.rank == a.skip_wg && t == a.skip_step)) {
      const uint32_t hb = relu_bits(sum + x) | tag_bit(S);
      const int row = my_layer_row;
      const uint32_t off = ((S & 1u) * a.Npad + row) * 4u;
      __builtin_amdgcn_raw_buffer_store_b32(hb, shared, off, 0, kCoherent);
      __builtin_amdgcn_raw_buffer_store_b32(hb, region, off, 0, kPlain);
      a.H[((size_t)t * a.B + p.b) * N + row] = __uint_as_float(hb & 0x7fffffffu);
    }
    return true;
  };
  if constexpr (kTwoSteps) {
    for (int t = 0; t < a.T; t += 2) {
      if (!step(t, lds)) return;
      if (t + 1 < a.T && !step(t + 1, lds + stride)) return;
    }
  } else {
    for (int t = 0; t < a.T; ++t)
      if (!step(t, lds + (t & 1) * stride)) return;
  }
}

}  // namespace

const void* kFloorSplitKernel = reinterpret_cast<const void*>(&floor_split_kernel<8>);
const void* kFloorSplitKernel12 = reinterpret_cast<const void*>(&floor_split_kernel<12>);

#define PRNN_DENSE_SPLIT(R, JJ) {kF16, R, JJ, reinterpret_cast<const void*>(&dense_split_kernel<R, JJ>)}

// (rows per wave, 256-column chunks of the row) on 256 waves per XCD: two XCDs
// per batch row (B <= 4) up to N = 2048, 2560, 3072, 3584; four (B <= 2) up to
// N = 2048, 2560, 3072, 4096, 5120.
const KernelEntry kDenseSplitF16Kernels[] = {
    PRNN_DENSE_SPLIT(4, 8), PRNN_DENSE_SPLIT(5, 10), PRNN_DENSE_SPLIT(6, 12), PRNN_DENSE_SPLIT(7, 14),
    PRNN_DENSE_SPLIT(2, 8), PRNN_DENSE_SPLIT(3, 10), PRNN_DENSE_SPLIT(3, 12), PRNN_DENSE_SPLIT(4, 16),
    PRNN_DENSE_SPLIT(5, 20),
    {0, 0, 0, nullptr},
};

#define PRNN_SPARSE_SPLIT(R, S, W) \
  {kF16, R, S, reinterpret_cast<const void*>(&sparse_split_kernel<R, S, W, 2>), W}
// Sparse fp16 layers on two XCDs per batch row: (rows per wave, 64-pair slots)
// for the 2304- and 5760-neuron layers at 8 and 12 waves per workgroup; the
// 16-slot ones hold rows of up to 1024 pairs at N = 2304 (the 25 % layer with
// unbalanced rows, stored at its longest row's width), which no one-XCD
// instance holds without spilling.
const KernelEntry kSparseSplitF16Kernels[] = {
    PRNN_SPARSE_SPLIT(5, 4, 8), PRNN_SPARSE_SPLIT(5, 9, 8), PRNN_SPARSE_SPLIT(5, 10, 8), PRNN_SPARSE_SPLIT(12, 1, 8),
    PRNN_SPARSE_SPLIT(12, 5, 8), PRNN_SPARSE_SPLIT(8, 5, 12), PRNN_SPARSE_SPLIT(4, 9, 12), PRNN_SPARSE_SPLIT(4, 10, 12),
    PRNN_SPARSE_SPLIT(5, 16, 8), PRNN_SPARSE_SPLIT(4, 16, 12),
    {0, 0, 0, nullptr},
};
// Rows of unequal length on two XCDs per batch row: rows of up to 1024 pairs
// at N = 2304 (the unbalanced 25 % layer), 5 rows per wave at 8 waves.
const KernelEntry kSparseRowsSplitF16Kernels[] = {
    {kF16, 5, 16, reinterpret_cast<const void*>(&sparse_split_kernel<5, 16, 8, 2, true>), 8},
    {0, 0, 0, nullptr},
};

}  // namespace prnn
