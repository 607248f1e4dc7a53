// Device-side building blocks shared by the persistent kernels (gfx950 only).
//
// Exchange of h_{t-1} between workgroups
// --------------------------------------
// Every workgroup owns some rows of W and, at each step, produces those rows of
// h_t for every batch row; every workgroup needs all of h_{t-1}.  The values
// travel through a two-slot ring of 32-bit words, ring[slot][b][Npad], written
// with device-coherent stores and read with device-coherent loads.  Each word
// carries its own step tag in bit 31, in the spirit of the Lamport timestamps
// of "Sparse Persistent RNNs: Squeezing Large Recurrent Networks On-Chip"
// (table "Measured effects reported in the paper", Lamport timestamps row):
//
//   * h = relu(.) is never negative, so its sign bit is free.  The value is
//     stored with bit 31 = ((S >> 1) & 1), S = global step counter, in slot
//     S & 1.
//   * The previous content of that slot is step S-2, whose tag bit differs, so
//     a reader compares bit 31 with the tag it expects and knows whether the
//     word is already the new value.  A 32-bit aligned store is single-copy
//     atomic, so a word is either entirely old or entirely new.
//   * Slot reuse is safe with two slots: before any workgroup writes step S+1
//     into the slot of step S-1, it has read all of step S, which every
//     workgroup wrote only after it had finished reading step S-1.
//   * No barrier, no flag array and no reset between steps are needed; the
//     handle resets the ring (to tag 1 = "step -2 / -1") only when its
//     footprint changes or after a failed run.
//
// Every wait is bounded by a deadline on the constant 100 MHz clock; a wave
// that times out sets the status word and leaves the kernel, so every wave of
// every launch always exits.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace prnn {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Cache-policy bits of the buffer instructions (gfx950): sc0 = 1, nt = 2, sc1 = 16.
// sc0|sc1 makes a load observe, and a store reach, the device coherence point,
// across the L2 caches of all XCDs.
constexpr int kCoherent = 16 | 1;
constexpr int kPlain = 0;

constexpr uint32_t kStatusTimeout = 1u;
constexpr uint32_t kStatusRange = 2u;  // a value reached the fp16 range of an hi + lo split

// A failed run: sets `bits` in the device status word, which every later
// kernel on the handle reads at entry (and then does nothing until the
// failure has been reported), and marks the host-visible mirror of the
// handle (pinned host memory: word 0 for an expired wait, word 1 for a value
// out of range) with a system-scope store, so that the host learns of the
// failure at its next call without waiting for the GPU.  Every writer of a
// mirror word stores the same value, so no atomic is needed there.
__device__ __forceinline__ void report_failure(uint32_t* status, uint32_t* host, uint32_t bits) {
  atomicOr(status, bits);
  if (host != nullptr) {
    if (bits & kStatusTimeout) __hip_atomic_store(host + 0, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    if (bits & kStatusRange) __hip_atomic_store(host + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  }
}

// Raw buffer resource over [p, p + bytes): out-of-range accesses read 0 and
// drop writes instead of faulting.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, bytes, 0x00020000);
}

__device__ __forceinline__ uint64_t now_ticks() { return __builtin_amdgcn_s_memrealtime(); }

// Test-only delay before a wave publishes its rows (span = 0: off, one
// scalar compare).  The wave sleeps n periods of s_sleep 1 (64 shader clocks
// each), n < span drawn from (seed, workgroup, wave, step) by a 32-bit integer
// hash (xor-shift-multiply rounds), the same for every lane.  It changes when
// rows arrive, never what they hold: results must not depend on it.
__device__ __forceinline__ void debug_jitter(uint32_t seed, uint32_t span, uint32_t wave, uint32_t t) {
  if (span == 0u) return;
  uint32_t x = seed ^ (blockIdx.x * 0x9E3779B1u) ^ (wave * 0x85EBCA77u) ^ (t * 0xC2B2AE3Du);
  x ^= x >> 16;
  x *= 0x7FEB352Du;
  x ^= x >> 15;
  x *= 0x846CA68Bu;
  x ^= x >> 16;
  for (uint32_t n = __builtin_amdgcn_readfirstlane(x % span); n > 0u; --n) __builtin_amdgcn_s_sleep(1);
}

// ReLU that keeps NaN (a < 0 is false for NaN) and returns +0 for any zero.
__device__ __forceinline__ uint32_t relu_bits(float a) {
  return (a < 0.f) ? 0u : (__float_as_uint(a) & 0x7fffffffu);
}

__device__ __forceinline__ uint32_t tag_bit(uint32_t step) { return ((step >> 1) & 1u) << 31; }

// Word-level validity of one 16-byte chunk: bit 31 must equal the tag, except
// for words at or beyond the row length (never written, always "valid").
__device__ __forceinline__ bool chunk_ready(const u32x4& v, uint32_t tag, int c, int n) {
  uint32_t bad = 0;
  bad |= ((v.x ^ tag) & 0x80000000u);
  bad |= (c + 1 < n) ? ((v.y ^ tag) & 0x80000000u) : 0u;
  bad |= (c + 2 < n) ? ((v.z ^ tag) & 0x80000000u) : 0u;
  bad |= (c + 3 < n) ? ((v.w ^ tag) & 0x80000000u) : 0u;
  return (c >= n) || bad == 0;
}

__device__ __forceinline__ float4 chunk_values(const u32x4& v, int c, int n) {
  float4 f;
  f.x = (c + 0 < n) ? __uint_as_float(v.x & 0x7fffffffu) : 0.f;
  f.y = (c + 1 < n) ? __uint_as_float(v.y & 0x7fffffffu) : 0.f;
  f.z = (c + 2 < n) ? __uint_as_float(v.z & 0x7fffffffu) : 0.f;
  f.w = (c + 3 < n) ? __uint_as_float(v.w & 0x7fffffffu) : 0.f;
  return f;
}

__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

constexpr int pow2_at_least(int x) { return x <= 1 ? 1 : 2 * pow2_at_least((x + 1) / 2); }

// acc += fp16(lo or hi half of w) * h, in fp32 (v_fma_mix_f32).  Written as
// inline asm so the compiler cannot hoist an fp16 -> fp32 widening of the
// resident weights out of the time loop, which would double their registers.
__device__ __forceinline__ void fma_mix_lo(float& acc, uint32_t w, float h) {
  asm("v_fma_mix_f32 %0, %1, %2, %0 op_sel_hi:[1,0,0]" : "+v"(acc) : "v"(w), "v"(h));
}
__device__ __forceinline__ void fma_mix_hi(float& acc, uint32_t w, float h) {
  asm("v_fma_mix_f32 %0, %1, %2, %0 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "+v"(acc) : "v"(w), "v"(h));
}

// Loads chunks [0, jn) of one ring row (lane l takes words 256 j + 4 l .. +3
// of chunk j) and waits until every word carries `tag`.  Each round re-issues
// only the chunks that are not complete yet, so the polling traffic shrinks as
// the producers' rows arrive.  Returns false if the wait exceeded `deadline`.
template <int J>
__device__ __forceinline__ bool gather_row(u32x4 (&v)[J], __amdgpu_buffer_rsrc_t ring, uint32_t row_bytes,
                                           int lane, int jn, int n, uint32_t tag, uint64_t deadline) {
#pragma unroll
  for (int j = 0; j < J; ++j)
    if (j < jn) v[j] = __builtin_amdgcn_raw_buffer_load_b128(ring, row_bytes + 4u * (256 * j + 4 * lane), 0, kCoherent);
  const uint64_t t0 = now_ticks();
  while (true) {
    bool ok = true;
#pragma unroll
    for (int j = 0; j < J; ++j)
      if (j < jn) ok = ok && chunk_ready(v[j], tag, 256 * j + 4 * lane, n);
    if (!wave_any(!ok)) return true;
    if (now_ticks() - t0 > deadline) return false;
#pragma unroll
    for (int j = 0; j < J; ++j)
      if (j < jn && !chunk_ready(v[j], tag, 256 * j + 4 * lane, n))
        v[j] = __builtin_amdgcn_raw_buffer_load_b128(ring, row_bytes + 4u * (256 * j + 4 * lane), 0, kCoherent);
  }
}

// ---------------------------------------------------------------------------
// Two-level exchange ("relay").  Polling the device-coherent ring from every
// compute unit makes each of the 8 XCDs fetch the same row 32 times per step
// across the fabric.  In relay mode each workgroup first copies one slice of
// the row (relay_slice words) from the ring into its own XCD's copy of the
// ring with ordinary stores, which stay in that XCD's L2; the workgroups of
// the XCD then read the whole row from there.  The row crosses the fabric
// once per XCD, and the 32 readers of an XCD hit its L2.  The copy keeps the
// words' step tags, so readers validate it exactly like the ring itself.
// Which XCD a workgroup runs on is read from the hardware (XCC_ID); the
// slices of one XCD are covered because workgroups are dealt to XCDs
// round-robin (checked once when a handle is created).
// ---------------------------------------------------------------------------
struct Exchange {
  __amdgpu_buffer_rsrc_t ring;   // written by every producer, device-coherent
  __amdgpu_buffer_rsrc_t local;  // where this wave reads h_{t-1}: the ring, or this XCD's copy
  int slice_lo;                  // first word of the slice this workgroup relays
  int slice_len;                 // words it relays (0: direct mode)
};

__device__ __forceinline__ Exchange make_exchange(uint32_t* ring, uint32_t* relay, uint32_t ring_bytes,
                                                  int relay_slice, int g, int n) {
  Exchange e;
  e.ring = make_rsrc(ring, ring_bytes);
  e.local = e.ring;
  e.slice_lo = 0;
  e.slice_len = 0;
  if (relay_slice > 0) {
    const uint32_t xcc = __builtin_amdgcn_s_getreg((20) | (31 << 11)) & 7u;  // HW_REG_XCC_ID
    e.local = make_rsrc(relay + (size_t)xcc * (ring_bytes / 4u), ring_bytes);
    e.slice_lo = (g >> 3) * relay_slice;
    e.slice_len = max(0, min(relay_slice, n - e.slice_lo));
  }
  return e;
}

// Relay mode, after relay_slice: wait until every slice of the row has
// reached this XCD's copy, watching only the last word of each slice (one
// 4-byte load per slice instead of re-reading the whole row while it is
// incomplete).  The row is then read once; its step tags still decide.
__device__ __forceinline__ bool wait_slices(const Exchange& e, int relay_slice, uint32_t row_bytes, int lane, int n,
                                            uint32_t tag, uint64_t deadline) {
  const int slices = (n + relay_slice - 1) / relay_slice;  // <= 64
  const bool mine = lane < slices;
  const int word = min((lane + 1) * relay_slice, n) - 1;
  uint32_t f = mine ? __builtin_amdgcn_raw_buffer_load_b32(e.local, row_bytes + 4u * word, 0, kCoherent) : tag;
  const uint64_t t0 = now_ticks();
  while (wave_any(((f ^ tag) & 0x80000000u) != 0u)) {
    if (now_ticks() - t0 > deadline) return false;
    if ((f ^ tag) & 0x80000000u) f = __builtin_amdgcn_raw_buffer_load_b32(e.local, row_bytes + 4u * word, 0, kCoherent);
  }
  return true;
}

// Relay mode: wait until this workgroup's slice of the ring row carries `tag`
// and copy it into the XCD-local copy.  Direct mode: nothing to do.
__device__ __forceinline__ bool relay_slice(const Exchange& e, uint32_t row_bytes, int lane, int n, uint32_t tag,
                                            uint64_t deadline) {
  if (e.slice_len == 0) return true;
  const int c = e.slice_lo + 4 * lane;
  const bool mine = 4 * lane < e.slice_len;
  u32x4 q = {0u, 0u, 0u, 0u};
  if (mine) q = __builtin_amdgcn_raw_buffer_load_b128(e.ring, row_bytes + 4u * c, 0, kCoherent);
  const uint64_t t0 = now_ticks();
  while (wave_any(mine && !chunk_ready(q, tag, c, n))) {
    if (now_ticks() - t0 > deadline) return false;
    if (mine && !chunk_ready(q, tag, c, n)) q = __builtin_amdgcn_raw_buffer_load_b128(e.ring, row_bytes + 4u * c, 0, kCoherent);
  }
  if (mine) __builtin_amdgcn_raw_buffer_store_b128(q, e.local, row_bytes + 4u * c, 0, kPlain);
  return true;
}

// ---------------------------------------------------------------------------
// Cross-lane sum of M per-lane partial values (M = 1, 2, 4, ... 32), one per
// row.  After the call, lane `owner_row(lane)` (if owner(lane)) holds the sum
// over all 64 lanes of value owner_row.  The order of additions is fixed, so
// results are bitwise reproducible.
//
//   stage 32: v_permlane32_swap pairs value i of lanes 0..31 with value
//             i + M/2 of lanes 32..63: one swap and one add per pair halves M;
//   stage 16: v_permlane16_swap does the same between 16-lane rows;
//   then each remaining value is summed inside its 16-lane row with DPP
//   (quad_perm xor1, xor2, row_half_mirror, row_mirror).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float dpp_row_sum(float x) {
  x += __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(x), 0xB1, 0xF, 0xF, false));
  x += __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(x), 0x4E, 0xF, 0xF, false));
  x += __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(x), 0x141, 0xF, 0xF, false));
  x += __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(x), 0x140, 0xF, 0xF, false));
  return x;
}

__device__ __forceinline__ void swap32_add(float& a, float& b) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  a = __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ void swap16_add(float& a, float& b) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  a = __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int M>
struct RowReduce {
  static_assert(M == 1 || M == 2 || M == 4 || M == 8 || M == 16 || M == 32, "M must be a power of two <= 32");
  // Row whose total this lane ends up owning, or -1.
  __device__ static __forceinline__ int owner_row(int lane) {
    if (M >= 4) {
      int i = lane & 15;
      return i < M / 4 ? (lane >> 4) * (M / 4) + i : -1;
    } else if (M == 2) {
      return (lane & 31) == 0 ? (lane >> 5) : -1;
    } else {
      return lane == 0 ? 0 : -1;
    }
  }
  // Reduces v in place; returns the value of owner_row(lane) (garbage if -1).
  __device__ static __forceinline__ float reduce(float (&v)[M], int lane) {
    if constexpr (M >= 4) {
#pragma unroll
      for (int i = 0; i < M / 2; ++i) swap32_add(v[i], v[i + M / 2]);
#pragma unroll
      for (int i = 0; i < M / 4; ++i) swap16_add(v[i], v[i + M / 4]);
      float out = 0.f;
      const int sel = lane & 15;
#pragma unroll
      for (int i = 0; i < M / 4; ++i) {
        float s = dpp_row_sum(v[i]);
        out = (sel == i) ? s : out;
      }
      return out;
    } else if constexpr (M == 2) {
      swap32_add(v[0], v[1]);
      float x = v[0];
      float y = x;
      swap16_add(x, y);
      return dpp_row_sum(x);
    } else {
      float x = v[0], y = v[0];
      swap32_add(x, y);
      float z = x;
      swap16_add(x, z);
      return dpp_row_sum(x);
    }
  }
};

}  // namespace prnn
