// A stack of L dense fp16 layers as a wavefront ("Optimizing Performance of
// Recurrent Neural Networks on GPUs", Abstract, entire-network stage: layer
// l + 1's step t depends only on layer l's step t and on its own step t - 1,
// so the layers run at the same time, each behind the one below, on their
// own compute units).
//
// The grid is the team layout's (8 teams of P workgroups, team x on XCD x);
// team x serves layer x / B and batch row x % B, so L B <= 8.  Team (l, b)
// runs Tl[l] steps of its layer from its own pre-activations X[l] (0 steps:
// it only keeps its region current).  Two ways to feed the layers:
//
// Blocked (FUSED = false): the host cuts the sequence into blocks and launch
// i runs layer l on block i - l, so layer l + 1 runs one block behind layer
// l.  A launch starts with each layer's input product for its block (U_0 x +
// bias_0, U_l H_{l-1} + bias_l; H_{l-1}'s block was finished by the launch
// before): each workgroup computes, on the matrix cores, the product for the
// rows it owns at every step of the block (project_tile) and writes it in
// place into H_l's block, which the recurrence then reads (each element by
// the lane that later overwrites it).  Only then are the weights loaded into
// the registers the product used.
//
// Fused (FUSED = true): layer 0 adds X[0][t]; a layer l >= 1 keeps the rows
// of [U_l | W_l] in
// registers (widened to fp32) and multiplies them with the staged row
// [H_{l-1}[t] ; h_l[t-1]]:
//
//   h_l[t] = max(0, bias_l + U_l H_{l-1}[t] + W_l h_l[t-1]).
//
// h_l[t-1] comes from the team's own XCD region, as in the team layout.
// H_{l-1}[t] comes straight from layer l - 1's output sequence in memory:
// the host fills H_0 .. H_{L-2} with 0xFFFFFFFF before the launch, layer
// l - 1 stores its outputs written through to memory (never with bit 31 set:
// ReLU outputs are cleared of it), and layer l polls each word until bit 31
// is clear.  Every step has its own words, so a lower layer may run any
// number of steps ahead and nothing is ever overwritten: no backpressure.
#include "project_tile.h"
#include "team_kernel.h"

namespace prnn {
namespace {

template <int RW, int J, bool FUSED>
__global__ void __launch_bounds__(512) stack_team_kernel(StackArgs a) {
  constexpr int M = pow2_at_least(RW);
  constexpr int kHalf = 256 * J;  // one half of an LDS row: input part, then state part
  constexpr int kParts = FUSED ? 2 : 1;
  extern __shared__ __attribute__((aligned(16))) float lds[];  // [2 steps][kParts][kHalf]
  __shared__ int abort_flag;
  const int team = blockIdx.x & 7;
  const int rank = blockIdx.x >> 3;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int layer = team / a.B;
  const int b = team % a.B;
  const bool primary = team < a.L * a.B && a.Tl[team / a.B] > 0;
  const int q = rank * kTeamWaves + wave;
  const int nr = a.base_rows + (q < a.extra_rows ? 1 : 0);
  const int r0 = q * a.base_rows + min(q, a.extra_rows);
  const int N = a.N;
  const int jn = a.chunks;

  if (threadIdx.x == 0) abort_flag = __builtin_nontemporal_load(a.status) != 0u;
  __syncthreads();
  if (abort_flag) return;
  const uint32_t xcc = __builtin_amdgcn_s_getreg((20) | (31 << 11)) & 7u;  // HW_REG_XCC_ID
  const __amdgpu_buffer_rsrc_t region = make_rsrc(a.ring + (size_t)xcc * 2 * a.Npad, 2u * a.Npad * 4u);
  // Keeps the region continuous for the next launch: the tags of this
  // launch's last two steps on this wave's rows (teams that run no step, or
  // fewer steps than the launch).
  auto stamp_tail = [&]() {
    const uint32_t last = a.step0 + (uint32_t)(a.T - 1);
    for (int k = 0; k < 2 && k < a.T; ++k) {
      const uint32_t S = last - (uint32_t)k;
      for (int r = lane; r < nr; r += 64)
        __builtin_amdgcn_raw_buffer_store_b32(tag_bit(S), region, ((S & 1u) * a.Npad + r0 + r) * 4u, 0, kPlain);
    }
  };
  if (!primary) {
    stamp_tail();
    return;
  }

  const int Tl = a.Tl[layer];
  if (!FUSED && a.P[layer] != nullptr) {
    // This workgroup's rows [n0, n1) of the block's input product, 64 steps
    // of the block at a time (8 waves x RW rows fit one 64-row tile).  Two
    // k-steps of loads in flight: 2-layer stacks took 554 (N = 1792) and
    // 431 us (N = 1152) per call against 571 and 443 with four and 583 and
    // 454 with eight.
    static_assert(FUSED || kTeamWaves * RW <= proj::kBM, "a workgroup's rows must fit one tile");
    static_assert(kStackProjLds >= proj::lds_bytes<64>(), "LDS of the in-launch product");
    constexpr int kInLaunchDepth = 2;
    const int q0 = rank * kTeamWaves;
    const int n0 = q0 * a.base_rows + min(q0, a.extra_rows);
    const int n1 = n0 + kTeamWaves * a.base_rows + max(0, min(kTeamWaves, a.extra_rows - q0));
    const int I = a.p_cols[layer];
    const bool f32 = a.p_f32[layer] != 0, pv = a.p_vec[layer] != 0;
    const uint32_t esize = f32 ? 4u : 2u;
    const __amdgpu_buffer_rsrc_t pr = make_rsrc(a.P[layer], (uint32_t)Tl * (uint32_t)a.B * (uint32_t)I * esize);
    const __amdgpu_buffer_rsrc_t ur = make_rsrc(a.U[layer], (uint32_t)N * (uint32_t)I * 2u);
    const proj::TileRows rows{Tl, a.B, b};
    const float* pb = a.bias[layer];
    _Float16* plds = reinterpret_cast<_Float16*>(lds);
    bool range_ok = true;
    for (int mb = 0; mb < Tl; mb += proj::kBM) {
      bool ok;
      if (f32)
        ok = pv ? proj::project_tile<true, true, 64, kInLaunchDepth>(pr, ur, pb, a.H[layer], N, rows, mb, n0, n1, I, plds)
                : proj::project_tile<true, false, 64, kInLaunchDepth>(pr, ur, pb, a.H[layer], N, rows, mb, n0, n1, I, plds);
      else
        ok = pv ? proj::project_tile<false, true, 64, kInLaunchDepth>(pr, ur, pb, a.H[layer], N, rows, mb, n0, n1, I, plds)
                : proj::project_tile<false, false, 64, kInLaunchDepth>(pr, ur, pb, a.H[layer], N, rows, mb, n0, n1, I, plds);
      range_ok = range_ok && ok;
    }
    if (wave_any(!range_ok) && lane == 0) report_failure(a.status, a.status_host, kStatusRange);
  }
  // Words past N in each half stay zero (their weights are zero too).  The
  // barrier also orders the product's stores before the recurrence's loads.
  for (int c = threadIdx.x; c < 2 * kParts * kHalf; c += blockDim.x)
    if (c % kHalf >= N) lds[c] = 0.f;
  __syncthreads();
  const bool has_input = FUSED && layer > 0;
  const bool vec = (N & 3) == 0;
  // w[r][j]: (fused) j < J the input part (U_l), then the state part (W_l);
  // fp16 widened to fp32 registers once.
  WChunkWide w[RW][kParts * J];
#pragma unroll
  for (int r = 0; r < RW; ++r)
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const size_t off = (size_t)(r0 + r) * N;
      const bool live = r < nr && j < jn;
      if (FUSED) w[r][j].load(a.U[layer], off, 256 * j + 4 * lane, N, live && has_input, vec);
      w[r][(kParts - 1) * J + j].load(a.W[layer], off, 256 * j + 4 * lane, N, live, vec);
    }

  const int my_row = RowReduce<M>::owner_row(lane);
  const bool owner = my_row >= 0 && my_row < nr;
  const int row = r0 + (owner ? my_row : 0);
  const uint32_t hbytes = a.x_bytes;  // every [T][B][N] sequence has this size
  const __amdgpu_buffer_rsrc_t in = make_rsrc(has_input ? a.H[layer - 1] : a.X[layer], hbytes);
  const __amdgpu_buffer_rsrc_t out = make_rsrc(a.H[layer], hbytes);
  const bool feeds_next = FUSED && layer + 1 < a.L;
  // Layer 0 adds X0[t] (loaded a step ahead); the others add their bias.
  const float bias = (has_input && owner && a.bias[layer] != nullptr) ? a.bias[layer][row] : 0.f;
  const uint32_t xstep = (uint32_t)a.B * (uint32_t)N * 4u;
  uint32_t xoff = ((uint32_t)b * (uint32_t)N + (uint32_t)row) * 4u;
  float x_next = has_input ? 0.f : __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(in, xoff, 0, kPlain));
  const float* h0 = a.h0[layer];

  for (int t = 0; t < Tl; ++t) {
    const uint32_t S = a.step0 + (uint32_t)t;
    float* inrow = lds + (t & 1) * kParts * kHalf;
    float* strow = inrow + (kParts - 1) * kHalf;
    bool ok = true;
    // Staging tasks: the state part's chunks, then (layers >= 1) the input
    // part's, dealt over the 8 waves.
    const int tasks = has_input ? 2 * jn : jn;
    for (int k = wave; k < tasks && ok; k += kTeamWaves) {
      const bool state = k < jn;
      const int c = 256 * (state ? k : k - jn) + 4 * lane;
      if (state && t == 0) {
        if (c < N) {
          float4 f;
          f.x = (h0 != nullptr && c + 0 < N) ? h0[(size_t)b * N + c + 0] : 0.f;
          f.y = (h0 != nullptr && c + 1 < N) ? h0[(size_t)b * N + c + 1] : 0.f;
          f.z = (h0 != nullptr && c + 2 < N) ? h0[(size_t)b * N + c + 2] : 0.f;
          f.w = (h0 != nullptr && c + 3 < N) ? h0[(size_t)b * N + c + 3] : 0.f;
          *reinterpret_cast<float4*>(strow + c) = f;
        }
        continue;
      }
      // State: own region, slot (S-1) & 1, tag of step S-1.  Input: the
      // layer below's H[t][b][c..c+3], written once bit 31 is clear.
      const uint32_t prev = S - 1u;
      const __amdgpu_buffer_rsrc_t src = state ? region : in;
      const uint32_t off = state ? ((prev & 1u) * (uint32_t)a.Npad + (uint32_t)c) * 4u
                                 : (((uint32_t)t * (uint32_t)a.B + (uint32_t)b) * (uint32_t)N + (uint32_t)c) * 4u;
      const uint32_t tag = state ? tag_bit(prev) : 0u;
      u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(src, off, 0, kCoherent);
      const uint64_t t0 = now_ticks();
      while (true) {
        const bool mine = chunk_ready(v, tag, c, N);
        if (!wave_any(!mine)) break;
        if (!mine) v = __builtin_amdgcn_raw_buffer_load_b128(src, off, 0, kCoherent);
        if (now_ticks() - t0 > a.deadline) { ok = false; break; }
      }
      if (ok && c < N) *reinterpret_cast<float4*>((state ? strow : inrow) + c) = chunk_values(v, c, N);
    }
    if (!ok && lane == 0) {
      abort_flag = 1;
      report_failure(a.status, a.status_host, kStatusTimeout);
    }
    __syncthreads();
    int aborted_now = abort_flag;
    const float x = has_input ? bias : x_next;
    xoff += xstep;
    if (!has_input && t + 1 < Tl) x_next = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(in, xoff, 0, kPlain));

    float acc[M];
#pragma unroll
    for (int r = 0; r < M; ++r) acc[r] = 0.f;
    if constexpr (!FUSED && kPinnedWeights && PinnedFma<RW, J>::kAvailable) {
      // the weights at fixed registers, as in the layer kernel
      float4 h[J];
#pragma unroll
      for (int j = 0; j < J; ++j) h[j] = *reinterpret_cast<const float4*>(inrow + 256 * j + 4 * lane);
      __builtin_amdgcn_sched_barrier(0);
      PinnedFma<RW, J>::run(acc, w, h);
    } else {
#pragma unroll
      for (int j = 0; j < kParts * J; ++j) {
        if (FUSED && j < J && !has_input) continue;  // layer 0 has no input part
        const float4 h = *reinterpret_cast<const float4*>(inrow + 256 * j + 4 * lane);
#pragma unroll
        for (int r = 0; r < RW; ++r) w[r][j].fma4(acc[r], h);
      }
    }
    const float sum = RowReduce<M>::reduce(acc, lane);
    asm volatile("" : "+v"(aborted_now) : "v"(sum));  // keep the test after the arithmetic
    if (aborted_now) return;
    debug_jitter(a.jitter_seed, a.jitter_span, wave, t);
    if (owner) {
      const uint32_t hb = relu_bits(sum + x);
      __builtin_amdgcn_raw_buffer_store_b32(hb | tag_bit(S), region, ((S & 1u) * a.Npad + row) * 4u, 0, kPlain);
      const uint32_t hoff = (((uint32_t)t * (uint32_t)a.B + (uint32_t)b) * (uint32_t)N + (uint32_t)row) * 4u;
      if (feeds_next)
        __builtin_amdgcn_raw_buffer_store_b32(hb, out, hoff, 0, kCoherent);
      else
        __builtin_amdgcn_raw_buffer_store_b32(hb, out, hoff, 0, kPlain);
    }
  }
  if (Tl < a.T) stamp_tail();
}

}  // namespace

#define PRNN_STACK(R, JJ, F) {kF16, R, JJ, reinterpret_cast<const void*>(&stack_team_kernel<R, JJ, F>)}
// (rows per wave, 256-column chunks of each part), weights widened to fp32.
const KernelEntry kStackFusedKernels[] = {
    PRNN_STACK(1, 1, true), PRNN_STACK(2, 2, true), PRNN_STACK(4, 4, true), PRNN_STACK(5, 5, true),
    {0, 0, 0, nullptr},
};
const KernelEntry kStackBlockedKernels[] = {
    PRNN_STACK(1, 1, false), PRNN_STACK(2, 2, false), PRNN_STACK(4, 4, false), PRNN_STACK(5, 5, false),
    PRNN_STACK(7, 7, false),
    {0, 0, 0, nullptr},
};

}  // namespace prnn
