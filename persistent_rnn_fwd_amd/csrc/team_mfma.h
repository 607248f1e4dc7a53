// Dense fp16 recurrence in the team layout on the matrix cores.
//
// Each workgroup owns R = 16 TR consecutive rows of W (TR tiles of 16 rows);
// wave w owns the 256-column chunk w of every tile, kept in registers in the
// A-operand layout of v_mfma_f32_16x16x32_f16 (8 fp16 per lane per 16x32
// block, 8 blocks per tile).  A step multiplies the 16-row tiles by h_{t-1}
// given as two fp16 columns, hi = fp16(h) and lo = fp16(h - hi): the products
// are exact in the fp32 accumulators, so W h = W hi + W lo is formed to about
// 2^-22 of |h| (fp32 h carries 2^-24), provided |h| < 65504; a larger value
// raises kStatusRange and the call reports EXECUTION_FAILED.  Column 0 of
// the 16-wide result holds W hi, column 1 W lo, the other 14 stay zero.
//
// Per step: wave w polls its own chunk of h_{t-1} from the XCD's region (no
// LDS broadcast of the whole row), splits its four values per lane into hi
// and lo, writes them as fp16 to a wave-private LDS slot (next to a 16-byte
// zero word), reads each k-step's B operand back with one 16-byte LDS read
// per lane (column-0 lanes read hi, column-1 lanes lo, the rest the zeros),
// runs 8 TR MFMAs, and writes its partial row sums (W hi + W lo, over its 256
// columns; zeros for a wave without a chunk) to LDS.  One workgroup barrier later
// every row's owner lane adds the waves' partials in a fixed order, adds x,
// applies ReLU and publishes.  The partial sums are double-buffered by step
// parity: a wave may start the next step while owners still read this one,
// but not the one after (that needs this workgroup's rows, stored after the
// reads).
#pragma once

#include "team_kernel.h"

namespace prnn {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4v __attribute__((ext_vector_type(4)));
typedef float float4v __attribute__((ext_vector_type(4)));

// Value of the neighbouring lane in each pair (DPP quad_perm [1,0,3,2]).
__device__ __forceinline__ float swap_pairs(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
}

template <int TR, bool TRACE = false>
__global__ void __launch_bounds__(512) dense_team_mfma_kernel(StepArgs a) {
  constexpr int KS = 8;        // 32-column k-steps per wave (one 256-column chunk)
  constexpr int R = 16 * TR;   // rows per workgroup
  constexpr int RPW = R / 8;   // rows whose epilogue each wave runs
  // LDS: per wave [256 hi][256 lo][8 zero] fp16 (1040 bytes), then [2][8][R] fp32 partials
  constexpr int kSlot = 520;   // fp16 words per wave slot
  extern __shared__ __attribute__((aligned(16))) float lds[];
  __shared__ int abort_flag;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int team = blockIdx.x & 7;
  const int rank = blockIdx.x >> 3;
  const int b = team % a.B;
  const int N = a.N;
  const int jn = a.chunks;  // <= 8
  const int row0 = rank * R;
  if (threadIdx.x == 0) abort_flag = __builtin_nontemporal_load(a.status) != 0u;
  __syncthreads();
  if (abort_flag) return;
  const __amdgpu_buffer_rsrc_t region = team_region(a);
  if (team >= a.B) {
    // No batch row of its own: stamp this workgroup's rows for the call's
    // last two steps (see team_stamp_tail) and leave.
    const uint32_t last = a.step0 + (uint32_t)(a.T - 1);
    if (wave == 0 && lane < R && row0 + lane < N)
      for (int k = 0; k < 2 && k < a.T; ++k) {
        const uint32_t S = last - (uint32_t)k;
        __builtin_amdgcn_raw_buffer_store_b32(tag_bit(S), region, ((S & 1u) * a.Npad + row0 + lane) * 4u, 0, kPlain);
      }
    return;
  }

  _Float16* slot = reinterpret_cast<_Float16*>(lds) + wave * kSlot;  // this wave's chunk as hi, lo
  float* part = lds + 8 * kSlot / 2;                                 // [2][8][R]
  if (lane < 8) slot[512 + lane] = (_Float16)0.f;                    // the zero word
  const int n16 = lane & 15;      // MFMA column of this lane (B and D)
  const int q = lane >> 4;        // 8-wide k group (A, B) / 4-row group (D)

  // W in the A layout: tile i, k-step s, lane: row 16 i + n16, columns
  // 256 wave + 32 s + 8 q + e, e < 8.  Zero outside the matrix.
  half8 w[TR][KS];
  const uint16_t* W16 = reinterpret_cast<const uint16_t*>(a.W);
  const bool vec = (N & 7) == 0 && a.w_vec != 0;
#pragma unroll
  for (int i = 0; i < TR; ++i)
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int row = row0 + 16 * i + n16;
      const int c = 256 * wave + 32 * s + 8 * q;
      half8 v = {};
      if (row < N && c < N) {
        if (vec) {
          v = __builtin_bit_cast(half8, *reinterpret_cast<const uint4*>(W16 + (size_t)row * N + c));
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (c + e < N) v[e] = __builtin_bit_cast(_Float16, W16[(size_t)row * N + c + e]);
        }
      }
      w[i][s] = v;
    }

  // the rows whose epilogue this lane runs
  const int my_local = wave * RPW + lane;
  const int my_row = row0 + my_local;
  const bool owner = lane < RPW && my_row < N;
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.X, a.x_bytes);
  const uint32_t xstep = (uint32_t)a.B * (uint32_t)N * 4u;
  uint32_t xoff = ((uint32_t)b * (uint32_t)N + (uint32_t)(owner ? my_row : 0)) * 4u;
  float x_next = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(xr, xoff, 0, kPlain));
  bool range_ok = true;
  PhaseClock<TRACE> clk;
  clk.start();

  // this lane's B operand source: column 0 reads hi, column 1 lo, the rest zeros
  const _Float16* bsrc = n16 == 0 ? slot + 8 * q : n16 == 1 ? slot + 256 + 8 * q : slot + 512;
  const int bstep = n16 < 2 ? 32 : 0;

  for (int t = 0; t < a.T; ++t) {
    const uint32_t S = a.step0 + (uint32_t)t;
    float* pbuf = part + (t & 1) * 8 * R;
    bool ok = true;
    // 1. this wave's chunk of h_{t-1}, zero past N, as fp16 hi and lo
    if (wave < jn) {
      const int c = 256 * wave + 4 * lane;
      float4 f;
      if (t == 0) {
        f = load_h0(a.h0, b, N, c);
      } else {
        const uint32_t prev = S - 1u, tag = tag_bit(prev);
        const uint32_t off = ((prev & 1u) * (uint32_t)a.Npad + (uint32_t)c) * 4u;
        u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(region, off, 0, kCoherent);
        const uint64_t t0 = now_ticks();
        while (true) {
          const bool mine = chunk_ready(v, tag, c, N);
          if (!wave_any(!mine)) break;
          if (!mine) v = __builtin_amdgcn_raw_buffer_load_b128(region, off, 0, kCoherent);
          if (now_ticks() - t0 > a.deadline) { ok = false; break; }
        }
        f = chunk_values(v, c, N);
      }
      const float fv[4] = {f.x, f.y, f.z, f.w};
      half4v hi, lo;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        hi[e] = (_Float16)fv[e];
        lo[e] = (_Float16)(fv[e] - (float)hi[e]);  // the difference is exact in fp32
        range_ok = range_ok && !(__builtin_isinf((float)hi[e]) && __builtin_isfinite(fv[e]));
      }
      *reinterpret_cast<half4v*>(slot + 4 * lane) = hi;
      *reinterpret_cast<half4v*>(slot + 256 + 4 * lane) = lo;
    }
    if (!ok && lane == 0) {
      abort_flag = 1;
      report_failure(a.status, a.status_host, kStatusTimeout);
    }
    clk.mark(kTrStage);

    // 2. B operands and the products (waves past the last chunk add nothing)
    float4v d[TR];
#pragma unroll
    for (int i = 0; i < TR; ++i) d[i] = float4v{0.f, 0.f, 0.f, 0.f};
    if (wave < jn && ok) {
      half8 bm[KS];
#pragma unroll
      for (int s = 0; s < KS; ++s) bm[s] = *reinterpret_cast<const half8*>(bsrc + bstep * s);
      // all eight B operands in their own registers before the first product:
      // the matrix cores then run 8 TR products without an LDS wait between
      asm volatile("" : "+v"(bm[0]), "+v"(bm[1]), "+v"(bm[2]), "+v"(bm[3]), "+v"(bm[4]), "+v"(bm[5]), "+v"(bm[6]),
                   "+v"(bm[7]));
#pragma unroll
      for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int i = 0; i < TR; ++i) d[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(w[i][s], bm[s], d[i], 0, 0, 0);
      // column 1 (W lo) onto column 0 (W hi): quad_perm [1,0,3,2] gives lane
      // n16 = 0 the value of lane n16 = 1
#pragma unroll
      for (int i = 0; i < TR; ++i) {
        float4 sum;
        sum.x = d[i][0] + swap_pairs(d[i][0]);
        sum.y = d[i][1] + swap_pairs(d[i][1]);
        sum.z = d[i][2] + swap_pairs(d[i][2]);
        sum.w = d[i][3] + swap_pairs(d[i][3]);
        if (n16 == 0) *reinterpret_cast<float4*>(pbuf + wave * R + 16 * i + 4 * q) = sum;
      }
    } else if (lane < R / 4) {
      *reinterpret_cast<float4*>(pbuf + wave * R + 4 * lane) = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    clk.mark(kTrCompute);
    __syncthreads();
    clk.mark(kTrBarrier);
    int aborted_now = abort_flag;
    const float x = x_next;
    xoff += xstep;
    if (t + 1 < a.T) x_next = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(xr, xoff, 0, kPlain));

    // 3. owners: the waves' partials in a fixed order, x, ReLU, publish
    float sum = 0.f;
    if (owner) {
      float pv[8];
#pragma unroll
      for (int ww = 0; ww < 8; ++ww) pv[ww] = pbuf[ww * R + my_local];
#pragma unroll
      for (int ww = 0; ww < 8; ++ww) sum += pv[ww];
    }
    clk.mark(kTrReduce);
    asm volatile("" : "+v"(aborted_now) : "v"(sum));  // keep the test after the reads
    if (aborted_now) return;
    debug_jitter(a.jitter_seed, a.jitter_span, wave, t);
    if (owner && !(rank == a.skip_wg && t == a.skip_step)) {
      const uint32_t hb = relu_bits(sum + x);
      __builtin_amdgcn_raw_buffer_store_b32(hb | tag_bit(S), region, ((S & 1u) * a.Npad + my_row) * 4u, 0, kPlain);
      a.H[((size_t)t * a.B + b) * N + my_row] = __uint_as_float(hb);
    }
    clk.mark(kTrEpilogue);
  }
  if (wave_any(!range_ok) && lane == 0) report_failure(a.status, a.status_host, kStatusRange);
  if (TRACE) {
    TeamPos p;
    p.wave = wave;
    clk.finish(trace_record(a, p), a.T);
  }
}

#define PRNN_DENSE_TEAM_MFMA(TR) {kF16, 16 * TR, 8, reinterpret_cast<const void*>(&dense_team_mfma_kernel<TR>)}
#define PRNN_DENSE_TEAM_MFMA_TRACE(TR) {kF16, 16 * TR, 8, reinterpret_cast<const void*>(&dense_team_mfma_kernel<TR, true>)}

}  // namespace prnn
