// Dense persistent kernel: H[t] = relu(X[t] + W h_{t-1}) with W resident in
// registers for all T steps ("persistent-rnn", "What This Project Does":
// weights stay in the register files instead of being reloaded every step).
//
// Decomposition (one launch, one workgroup per compute unit):
//   * workgroup g owns rows [row0, row0 + nr) of W, balanced to within one
//     row across the grid;
//   * wave w of the workgroup serves batch row b = 4 * batch_group + w, so the
//     four batch rows run as independent recurrences that share W and never
//     synchronise with each other;
//   * lane l of a wave holds the columns 256 j + 4 l + {0,1,2,3}, j < J, of
//     every owned row: W takes RMAX * J * 4 values per lane (fp16 packed in
//     pairs and multiplied with v_fma_mix_f32, or fp32), loaded once in the
//     prologue;
//   * per step a lane loads its 4 J values of h_{t-1}[b] from the exchange
//     ring (16-byte coherent loads, one 1 KiB coalesced request per chunk per
//     wave), multiplies them into RMAX partial sums as soon as each chunk
//     carries the expected step tag, then the 64 partial sums of each row are
//     added across lanes (permlane swaps + DPP) and the owner lane of each row
//     adds X, applies ReLU, writes H and publishes the tagged value.
#pragma once

#include "device_common.h"
#include "kernels.h"

namespace prnn {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __fp16 fp16x2 __attribute__((ext_vector_type(2)));  // operand type of the dot2 builtin


template <typename WT>
struct WChunk;  // four consecutive weights of one row

template <>
struct WChunk<float> {
  float4 w;
  // vec: n % 4 == 0 and W 16-byte aligned, so a chunk is either entirely
  // inside the row or outside, and its load is naturally aligned.
  __device__ __forceinline__ void load(const void* W, size_t row_off, int c, int n, bool live, bool vec) {
    const float* p = reinterpret_cast<const float*>(W) + row_off;
    if (vec) {
      w = (live && c < n) ? *reinterpret_cast<const float4*>(p + c) : make_float4(0.f, 0.f, 0.f, 0.f);
      return;
    }
    w.x = (live && c + 0 < n) ? p[c + 0] : 0.f;
    w.y = (live && c + 1 < n) ? p[c + 1] : 0.f;
    w.z = (live && c + 2 < n) ? p[c + 2] : 0.f;
    w.w = (live && c + 3 < n) ? p[c + 3] : 0.f;
  }
  __device__ __forceinline__ void fma4(float& acc, const float4& h) const {
    acc = fmaf(w.x, h.x, acc);
    acc = fmaf(w.y, h.y, acc);
    acc = fmaf(w.z, h.z, acc);
    acc = fmaf(w.w, h.w, acc);
  }
};

template <>
struct WChunk<_Float16> {
  uint32_t lo, hi;  // (w0, w1), (w2, w3) as fp16 pairs
  __device__ __forceinline__ void load(const void* W, size_t row_off, int c, int n, bool live, bool vec) {
    const uint16_t* p = reinterpret_cast<const uint16_t*>(W) + row_off;
    if (vec) {
      const uint2 q = (live && c < n) ? *reinterpret_cast<const uint2*>(p + c) : make_uint2(0u, 0u);
      lo = q.x;
      hi = q.y;
      return;
    }
    uint32_t e0 = (live && c + 0 < n) ? p[c + 0] : 0u;
    uint32_t e1 = (live && c + 1 < n) ? p[c + 1] : 0u;
    uint32_t e2 = (live && c + 2 < n) ? p[c + 2] : 0u;
    uint32_t e3 = (live && c + 3 < n) ? p[c + 3] : 0u;
    lo = e0 | (e1 << 16);
    hi = e2 | (e3 << 16);
  }
  // fp16 x fp32 products accumulated in fp32: the fp16 weight is widened
  // exactly, h keeps full fp32 precision.
  __device__ __forceinline__ void fma4(float& acc, const float4& h) const {
    fma_mix_lo(acc, lo, h.x);
    fma_mix_hi(acc, lo, h.y);
    fma_mix_lo(acc, hi, h.z);
    fma_mix_hi(acc, hi, h.w);
  }
  // Half-h form: h as four fp16 values (h01, h23 packed).  Each instruction
  // (v_dot2_f32_f16) adds two fp16 x fp16 products, exact in fp32, to the
  // fp32 sum: half the multiply-add instructions of the fp32-h forms.
  __device__ __forceinline__ void dot4(float& acc, const uint2& h) const {
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(fp16x2, lo), __builtin_bit_cast(fp16x2, h.x), acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(fp16x2, hi), __builtin_bit_cast(fp16x2, h.y), acc, false);
  }
};

// fp16 weights widened once to fp32 in the prologue: twice the registers of
// the packed form, but the time loop then runs v_fmac_f32, which issues about
// 1.7x faster than v_fma_mix_f32 on gfx950 (measured).  Widening is exact.
struct WChunkWide {
  float4 w;
  __device__ __forceinline__ void load(const void* W, size_t row_off, int c, int n, bool live, bool vec) {
    WChunk<_Float16> p;
    p.load(W, row_off, c, n, live, vec);
    const f16x2 a = __builtin_bit_cast(f16x2, p.lo);
    const f16x2 b = __builtin_bit_cast(f16x2, p.hi);
    w = make_float4((float)a.x, (float)a.y, (float)b.x, (float)b.y);
  }
  __device__ __forceinline__ void fma4(float& acc, const float4& h) const {
    acc = fmaf(w.x, h.x, acc);
    acc = fmaf(w.y, h.y, acc);
    acc = fmaf(w.z, h.z, acc);
    acc = fmaf(w.w, h.w, acc);
  }
};

// Loads h0[b][c..c+3] (or zeros), with per-element bounds.
__device__ __forceinline__ float4 load_h0(const float* h0, int b, int n, int c) {
  float4 f = make_float4(0.f, 0.f, 0.f, 0.f);
  if (h0 != nullptr) {
    const float* p = h0 + (size_t)b * n;
    f.x = (c + 0 < n) ? p[c + 0] : 0.f;
    f.y = (c + 1 < n) ? p[c + 1] : 0.f;
    f.z = (c + 2 < n) ? p[c + 2] : 0.f;
    f.w = (c + 3 < n) ? p[c + 3] : 0.f;
  }
  return f;
}

// RMAX rows per workgroup are computed (rows beyond the owned nr carry zero
// weights and are never stored); the cross-lane sum runs over M = RMAX rounded
// up to a power of two.
template <typename WT, int RMAX, int J>
__global__ void __launch_bounds__(256) dense_kernel(StepArgs a) {
  constexpr int M = pow2_at_least(RMAX);
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int g = blockIdx.x % a.G;
  const int b = (blockIdx.x / a.G) * 4 + wave;
  if (b >= a.B) return;
  if (__builtin_nontemporal_load(a.status) != 0u) return;  // a failed run stays failed until reported

  const int N = a.N;
  const int nr = a.base_rows + (g < a.extra_rows ? 1 : 0);
  const int row0 = g * a.base_rows + min(g, a.extra_rows);
  const int jn = a.chunks;

  // Prologue: this workgroup's rows of W into registers, once per call.
  const bool vec = (N & 3) == 0 && a.w_vec != 0;
  WChunk<WT> w[RMAX][J];
#pragma unroll
  for (int r = 0; r < RMAX; ++r)
#pragma unroll
    for (int j = 0; j < J; ++j)
      w[r][j].load(a.W, (size_t)(row0 + r) * N, 256 * j + 4 * lane, N, r < nr && j < jn, vec);

  const Exchange ex = make_exchange(a.ring, a.relay, a.ring_bytes, a.relay_slice, g, N);
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.X, a.x_bytes);
  const int my_row = RowReduce<M>::owner_row(lane);
  const bool owner = my_row >= 0 && my_row < nr;
  const bool skipper = (g == a.skip_wg);

  for (int t = 0; t < a.T; ++t) {
    const uint32_t S = a.step0 + (uint32_t)t;
    const uint32_t xoff = (uint32_t)(((size_t)t * a.B + b) * N + row0 + (owner ? my_row : 0)) * 4u;
    const float x = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(xr, xoff, 0, kPlain));

    float acc[M];
#pragma unroll
    for (int r = 0; r < M; ++r) acc[r] = 0.f;

    if (t == 0) {
#pragma unroll
      for (int j = 0; j < J; ++j) {
        if (j < jn) {
          const float4 h = load_h0(a.h0, b, N, 256 * j + 4 * lane);
#pragma unroll
          for (int r = 0; r < RMAX; ++r) w[r][j].fma4(acc[r], h);
        }
      }
    } else {
      const uint32_t prev = S - 1u;
      const uint32_t row_bytes = (uint32_t)(((prev & 1u) * a.B + b) * a.Npad) * 4u;
      const uint32_t tag = tag_bit(prev);
      u32x4 v[J];
      bool done = false;
      if (a.relay_slice > 0) {
        // Relay: every slice is in this XCD's copy once its last word is.
        // Then read the row once and multiply each 1 KiB chunk as it lands.
        if (!relay_slice(ex, row_bytes, lane, N, tag, a.deadline) ||
            !wait_slices(ex, a.relay_slice, row_bytes, lane, N, tag, a.deadline)) {
          if (lane == 0) report_failure(a.status, a.status_host, kStatusTimeout);
          return;
        }
#pragma unroll
        for (int j = 0; j < J; ++j)
          if (j < jn) v[j] = __builtin_amdgcn_raw_buffer_load_b128(ex.local, row_bytes + 4u * (256 * j + 4 * lane), 0, kCoherent);
        done = true;
#pragma unroll
        for (int j = 0; j < J; ++j) {
          if (j < jn) {
            done = done && !wave_any(!chunk_ready(v[j], tag, 256 * j + 4 * lane, N));
            if (done) {
              const float4 h = chunk_values(v[j], 256 * j + 4 * lane, N);
#pragma unroll
              for (int r = 0; r < RMAX; ++r) w[r][j].fma4(acc[r], h);
            }
          }
        }
      }
      if (!done) {
        // Direct exchange, or a relayed row that was not complete yet: wait
        // for the whole row, then (re)compute the sums from scratch.
        if (!gather_row<J>(v, ex.local, row_bytes, lane, jn, N, tag, a.deadline)) {
          if (lane == 0) report_failure(a.status, a.status_host, kStatusTimeout);
          return;
        }
#pragma unroll
        for (int r = 0; r < M; ++r) acc[r] = 0.f;
#pragma unroll
        for (int j = 0; j < J; ++j) {
          if (j < jn) {
            const float4 h = chunk_values(v[j], 256 * j + 4 * lane, N);
#pragma unroll
            for (int r = 0; r < RMAX; ++r) w[r][j].fma4(acc[r], h);
          }
        }
      }
    }

    const float sum = RowReduce<M>::reduce(acc, lane);
    debug_jitter(a.jitter_seed, a.jitter_span, wave, t);
    if (owner && !(skipper && t == a.skip_step)) {
      const uint32_t hb = relu_bits(sum + x);
      const int row = row0 + my_row;
      a.H[((size_t)t * a.B + b) * N + row] = __uint_as_float(hb);
      const uint32_t roff = (uint32_t)(((S & 1u) * a.B + b) * a.Npad + row) * 4u;
      __builtin_amdgcn_raw_buffer_store_b32(hb | tag_bit(S), ex.ring, roff, 0, kCoherent);
    }
  }

  // Relay mode: hand the last step to this XCD's copy as well, so that the
  // copies hold steps S-1 and S-2 when the next call starts at step S (its
  // first step reads h0, not the ring).
  if (a.T > 0) {
    const uint32_t last = a.step0 + (uint32_t)(a.T - 1);
    if (!relay_slice(ex, (uint32_t)(((last & 1u) * a.B + b) * a.Npad) * 4u, lane, N, tag_bit(last), a.deadline)) {
      if (lane == 0) report_failure(a.status, a.status_host, kStatusTimeout);
    }
  }
}

// The same grid, exchange and step protocol without weights or arithmetic:
// each owner lane publishes (t + 1) once it has seen all of h_{t-1}.
template <int J>
__global__ void __launch_bounds__(256) floor_kernel(StepArgs a) {
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int g = blockIdx.x % a.G;
  const int b = (blockIdx.x / a.G) * 4 + wave;
  if (b >= a.B) return;
  if (__builtin_nontemporal_load(a.status) != 0u) return;
  const int N = a.N;
  const int nr = a.base_rows + (g < a.extra_rows ? 1 : 0);
  const int row0 = g * a.base_rows + min(g, a.extra_rows);
  const int jn = a.chunks;
  const Exchange ex = make_exchange(a.ring, a.relay, a.ring_bytes, a.relay_slice, g, N);
  for (int t = 0; t < a.T; ++t) {
    const uint32_t S = a.step0 + (uint32_t)t;
    float acc = 0.f;
    if (t > 0) {
      const uint32_t prev = S - 1u;
      const uint32_t row_bytes = (uint32_t)(((prev & 1u) * a.B + b) * a.Npad) * 4u;
      u32x4 v[J];
      if (!relay_slice(ex, row_bytes, lane, N, tag_bit(prev), a.deadline) ||
          (a.relay_slice > 0 && !wait_slices(ex, a.relay_slice, row_bytes, lane, N, tag_bit(prev), a.deadline)) ||
          !gather_row<J>(v, ex.local, row_bytes, lane, jn, N, tag_bit(prev), a.deadline)) {
        if (lane == 0) report_failure(a.status, a.status_host, kStatusTimeout);
        return;
      }
#pragma unroll
      for (int j = 0; j < J; ++j) {
        if (j < jn) {
          const float4 h = chunk_values(v[j], 256 * j + 4 * lane, N);
          acc += h.x + h.y + h.z + h.w;
        }
      }
    }
    // rows are published by lanes 0 .. nr-1 (nr <= 64)
    if (lane < nr) {
      const uint32_t hb = relu_bits((float)(t + 1) + acc * 0.f);
      const int row = row0 + lane;
      a.H[((size_t)t * a.B + b) * N + row] = __uint_as_float(hb);
      const uint32_t roff = (uint32_t)(((S & 1u) * a.B + b) * a.Npad + row) * 4u;
      __builtin_amdgcn_raw_buffer_store_b32(hb | tag_bit(S), ex.ring, roff, 0, kCoherent);
    }
  }

  // Relay mode: hand the last step to this XCD's copy as well, so that the
  // copies hold steps S-1 and S-2 when the next call starts at step S (its
  // first step reads h0, not the ring).
  if (a.T > 0) {
    const uint32_t last = a.step0 + (uint32_t)(a.T - 1);
    if (!relay_slice(ex, (uint32_t)(((last & 1u) * a.B + b) * a.Npad) * 4u, lane, N, tag_bit(last), a.deadline)) {
      if (lane == 0) report_failure(a.status, a.status_host, kStatusTimeout);
    }
  }
}

#define PRNN_DENSE(WT, WTAG, R, JJ) {WTAG, R, JJ, reinterpret_cast<const void*>(&dense_kernel<WT, R, JJ>)}
#define PRNN_FLOOR(JJ) {0, 64, JJ, reinterpret_cast<const void*>(&floor_kernel<JJ>)}

}  // namespace prnn
