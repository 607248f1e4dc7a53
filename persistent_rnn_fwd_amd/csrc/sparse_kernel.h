// Row-balanced sparse persistent kernel: every row of W has exactly K
// nonzeros ("Sparse Persistent RNNs: Squeezing Large Recurrent Networks
// On-Chip", table "Measured effects reported in the paper": load-balanced
// pruning row), so every workgroup gets the same work per row and the
// nonzeros of its rows stay in registers for all T steps.
//
// Decomposition: as the dense kernel (workgroup = rows, wave = batch row).
// Per owned row r, its K (value, column) pairs are spread over the 64 lanes:
// lane l, slot s holds pair k = 64 s + l (zero value beyond K).  fp16 values
// and int16 columns are packed into one 32-bit register per pair.
// Per step each wave copies h_{t-1}[b] from the exchange ring into its own LDS
// row with 16-byte coherent loads ("wide memory loads" row of the same
// table) and 16-byte LDS writes, then every pair reads h[col] from LDS.
#pragma once

#include "device_common.h"
#include "kernels.h"

namespace prnn {


template <typename VT>
struct Pair;

template <>
struct Pair<_Float16> {
  uint32_t p;  // value bits | column << 16
  // Padding slots and columns outside [0, n) point at the zero word n.
  __device__ __forceinline__ void load(const int16_t* col, const void* val, size_t idx, bool live, int n) {
    uint32_t c = live ? (uint32_t)(uint16_t)col[idx] : (uint32_t)n;
    uint32_t v = live ? (uint32_t)reinterpret_cast<const uint16_t*>(val)[idx] : 0u;
    if (c >= (uint32_t)n) { c = (uint32_t)n; v = 0u; }
    p = v | (c << 16);
  }
  __device__ __forceinline__ int column() const { return (int)(p >> 16); }
  __device__ __forceinline__ float value() const {  // the fp16 value, widened exactly
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(p & 0xffffu));
  }
  __device__ __forceinline__ void fma(float& acc, float h) const { fma_mix_lo(acc, p, h); }
  __device__ __forceinline__ uint2 raw() const { return make_uint2(p, 0u); }
  __device__ __forceinline__ void set_raw(uint2 r) { p = r.x; }
};

template <>
struct Pair<float> {
  float v;
  int c;
  __device__ __forceinline__ void load(const int16_t* col, const void* val, size_t idx, bool live, int n) {
    c = live ? (int)(uint16_t)col[idx] : n;
    v = live ? reinterpret_cast<const float*>(val)[idx] : 0.f;
    if (c >= n) { c = n; v = 0.f; }
  }
  __device__ __forceinline__ int column() const { return c; }
  __device__ __forceinline__ void fma(float& acc, float h) const { acc = fmaf(v, h, acc); }
  __device__ __forceinline__ uint2 raw() const { return make_uint2(__float_as_uint(v), (uint32_t)c); }
  __device__ __forceinline__ void set_raw(uint2 r) {
    v = __uint_as_float(r.x);
    c = (int)r.y;
  }
};

// LDS: 32 banks of 4-byte words; each half of a wave (lanes 0-31, 32-63) is
// served on its own, one word per bank per cycle, all lanes that read the
// same word at once.  A gather whose 32 lanes hit b distinct words in one
// bank takes b cycles for that half (measured on gfx950).
constexpr int kLdsBanks = 32;
// Ranks with every slot's masks and counts in registers for pair blocks of up
// to 4 slots and 32 pairs per lane; larger blocks stage them in LDS, slot by
// slot (held in registers they made those blocks spill).
constexpr int kBitSlicedSlots = 4;
constexpr int kBitSlicedPairs = 32;
// Small blocks of 3 slots or more: ranks from per-bank counts and a scan,
// linear in the slots.  With 1 or 2 slots the scan costs more than it saves
// (launch prologue, 1 % at N = 1792: 9.4 us bit-sliced, 11.3 with counts;
// 10 % at N = 1792, 3 slots: 24.6 and 19.3; 10 % at N = 2304, 4 slots: 41
// and 26).
constexpr int kHistogramSlots = 3;
constexpr bool bit_sliced(int rw, int spr) { return spr <= kBitSlicedSlots && rw * spr <= kBitSlicedPairs; }

// Bank-aware placement of one row's pairs (the pages' bank-aware layout,
// our reading: every gather instruction should touch each LDS bank once).
// On entry lane l of slot s holds pair 64 s + l (s < spr, pairs >= K are
// padding that points at the zero word).  On exit the same K pairs sit so
// that each group (slot, half-wave) holds at most one pair per bank whenever
// no bank holds more than 2 * spr of the row's pairs: the pairs are ranked by
// bank (ties in their original order, so the placement and hence the
// summation order are deterministic) and dealt round-robin over the 2 * spr
// groups.  The sum is order-free, so any placement computes the same row.
// `scratch` is this wave's LDS area of SPR * 64 entries.
// A wave-uniform 64-bit value copied to vector registers (an empty asm the
// compiler cannot see through).
__device__ __forceinline__ uint64_t in_vgprs(uint64_t x) {
  uint32_t lo = (uint32_t)x, hi = (uint32_t)(x >> 32);
  asm("" : "+v"(lo), "+v"(hi));
  return ((uint64_t)hi << 32) | lo;
}

template <typename P, int SPR, bool BIT_SLICED>
__device__ __forceinline__ void place_row_bank_aware(P (&row)[SPR], int spr, int K, int n, int lane, uint2* scratch) {
  P pad;
  pad.load(nullptr, nullptr, 0, false, n);
  int rank[SPR];
#pragma unroll
  for (int s = 0; s < SPR; ++s) rank[s] = 0;
  // rank = number of pairs in lower banks + earlier pairs of the same bank
  if constexpr (BIT_SLICED && SPR >= kHistogramSlots) {
    // Five ballots per slot hold the slot's banks bit by bit; from them each
    // lane tells which of a slot's lanes share any one bank (match).  Lane b
    // (and b + 32) counts bank b in every slot; a scan over lanes 0-31 turns
    // the counts into the pairs of lower banks; each pair then reads from
    // lane `bank` the pairs before its slot and adds its slot's earlier lanes
    // of the same bank.  Linear in the slots, no scalar chain.
    int bk[SPR], cnt[SPR];
#pragma unroll
    for (int s = 0; s < SPR; ++s) bk[s] = row[s].column() & (kLdsBanks - 1);
    const uint64_t lanes_below = (1ull << lane) - 1ull;
    const int lane_bank = lane & (kLdsBanks - 1);
    auto masks = [&](int s, uint64_t& live, uint64_t (&bit)[5]) {
      const bool v = s < spr && 64 * s + lane < K;
      // in vector registers: held in scalar ones they pushed the kernel's own
      // scalars out to spill slots that the time loop reloads
      live = in_vgprs(__builtin_amdgcn_ballot_w64(v));
#pragma unroll
      for (int i = 0; i < 5; ++i) bit[i] = in_vgprs(__builtin_amdgcn_ballot_w64(v && ((bk[s] >> i) & 1)));
    };
    auto match = [](uint64_t live, const uint64_t (&bit)[5], int b) {
      uint64_t eq = live;
#pragma unroll
      for (int i = 0; i < 5; ++i) eq &= ~(bit[i] ^ (0ull - (uint64_t)((b >> i) & 1)));
      return eq;
    };
    int total = 0;
#pragma unroll
    for (int s = 0; s < SPR; ++s) {
      uint64_t live, bit[5];
      masks(s, live, bit);
      cnt[s] = __builtin_popcountll(match(live, bit, lane_bank));
      total += cnt[s];
    }
    int incl = total;  // inclusive scan of the bank totals over lanes 0-31 (and 32-63)
#pragma unroll
    for (int d = 1; d < kLdsBanks; d <<= 1) {
      const int y = __shfl_up(incl, d, kLdsBanks);
      if (lane_bank >= d) incl += y;
    }
    int off = incl - total;  // lane b: pairs in banks below b, then also in the slots done
#pragma unroll
    for (int s = 0; s < SPR; ++s) {
      uint64_t live, bit[5];
      masks(s, live, bit);
      rank[s] = __shfl(off, bk[s]) + __builtin_popcountll(match(live, bit, bk[s]) & lanes_below);
      off += cnt[s];
    }
  } else if constexpr (BIT_SLICED) {
    // Five ballots per slot hold its banks bit by bit.  Each lane then
    // compares its own bank with a whole slot at once: a walk from the top
    // bit down keeps the lanes still equal to it (eq) and collects those
    // found lower (lt).  Cheaper than the counts above for 1 or 2 slots; one
    // slot's masks are live at a time.
    int bk[SPR];
#pragma unroll
    for (int s = 0; s < SPR; ++s) bk[s] = row[s].column() & (kLdsBanks - 1);
    const uint64_t lanes_below = (1ull << lane) - 1ull;
#pragma unroll
    for (int s2 = 0; s2 < SPR; ++s2) {
      const bool v = s2 < spr && 64 * s2 + lane < K;
      // The masks move to vector registers: held in scalar ones they pushed
      // the kernel's own scalars out to spill slots that the time loop reloads.
      const uint64_t live = in_vgprs(__builtin_amdgcn_ballot_w64(v));
      uint64_t bit[5];
#pragma unroll
      for (int i = 0; i < 5; ++i) bit[i] = in_vgprs(__builtin_amdgcn_ballot_w64(v && ((bk[s2] >> i) & 1)));
#pragma unroll
      for (int s = 0; s < SPR; ++s) {
        uint64_t eq = live, lt = 0;
#pragma unroll
        for (int i = 4; i >= 0; --i) {
          const uint64_t m = 0ull - (uint64_t)((bk[s] >> i) & 1);  // all ones where my bit i is set
          lt |= eq & ~bit[i] & m;
          eq &= ~(bit[i] ^ m);
        }
        rank[s] += __builtin_popcountll(lt);
        if (s2 < s) rank[s] += __builtin_popcountll(eq);
        if (s2 == s) rank[s] += __builtin_popcountll(eq & lanes_below);
      }
    }
  } else {
    // Larger blocks: the same counts and scan, one slot at a time through
    // this wave's scratch (.x the pair's bank, .y its bank's count in the
    // slot, then its rank), so that no per-slot array but the ranks lives in
    // registers; held there, the masks and counts made these blocks spill.
    const uint64_t lanes_below = (1ull << lane) - 1ull;
    const int lane_bank = lane & (kLdsBanks - 1);
#pragma unroll
    for (int s = 0; s < SPR; ++s)
      if (s < spr) scratch[64 * s + lane] = make_uint2((uint32_t)(row[s].column() & (kLdsBanks - 1)), 0u);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    auto match_in = [&](int s, int b) {  // the lanes of slot s whose pair is in bank b
      const uint32_t bs = scratch[64 * s + lane].x;
      const bool v = 64 * s + lane < K;
      uint64_t eq = in_vgprs(__builtin_amdgcn_ballot_w64(v));
#pragma unroll
      for (int i = 0; i < 5; ++i) {
        const uint64_t bit = in_vgprs(__builtin_amdgcn_ballot_w64(v && ((bs >> i) & 1u)));
        eq &= ~(bit ^ (0ull - (uint64_t)((b >> i) & 1)));
      }
      return eq;
    };
    int total = 0;
    for (int s = 0; s < spr; ++s) {
      const int c = __builtin_popcountll(match_in(s, lane_bank));
      scratch[64 * s + lane].y = (uint32_t)c;
      total += c;
    }
    int incl = total;  // inclusive scan of the bank totals over lanes 0-31 (and 32-63)
#pragma unroll
    for (int d = 1; d < kLdsBanks; d <<= 1) {
      const int y = __shfl_up(incl, d, kLdsBanks);
      if (lane_bank >= d) incl += y;
    }
    int off = incl - total;
    for (int s = 0; s < spr; ++s) {
      const uint2 e = scratch[64 * s + lane];
      const int r = __shfl(off, (int)e.x) + __builtin_popcountll(match_in(s, (int)e.x) & lanes_below);
      off += (int)e.y;
      scratch[64 * s + lane].y = (uint32_t)r;
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int s = 0; s < SPR; ++s)
      if (s < spr) rank[s] = (int)scratch[64 * s + lane].y;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }
#pragma unroll
  for (int s = 0; s < SPR; ++s)
    if (s < spr) scratch[64 * s + lane] = pad.raw();
  const int groups = 2 * spr;
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // padding written before the pairs
#pragma unroll
  for (int s = 0; s < SPR; ++s) {
    if (s < spr && 64 * s + lane < K) {
      const int g = rank[s] % groups, q = rank[s] / groups;  // q < 32: K <= 32 * groups
      scratch[64 * (g >> 1) + 32 * (g & 1) + q] = row[s].raw();
    }
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // all lanes' writes before the reads
#pragma unroll
  for (int s = 0; s < SPR; ++s)
    if (s < spr) row[s].set_raw(scratch[64 * s + lane]);
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // scratch free for the next row
}

// Rows [R, RW) of a register-resident pair block, unrolled at compile time
// (a runtime row index would force the block out of registers).
template <int R, int RW, typename P, int SPR>
__device__ __forceinline__ void place_rows_bank_aware(P (&pr)[RW][SPR], int nr, int spr, int K, int n, int lane,
                                                      uint2* scratch) {
  if constexpr (R < RW) {
    if (R < nr) place_row_bank_aware<P, SPR, bit_sliced(RW, SPR)>(pr[R], spr, K, n, lane, scratch);
    place_rows_bank_aware<R + 1, RW, P, SPR>(pr, nr, spr, K, n, lane, scratch);
  }
}

constexpr int kLoadAllPairs = 48;  // pairs per lane up to which a block's loads are issued together

// Loads rows [R, RW) of a register-resident pair block and places each one
// before the next row's loads are issued: with every row's loads in flight
// at once the largest blocks would not fit the registers.
template <int R, int RW, typename P, int SPR>
__device__ __forceinline__ void load_place_rows(P (&pr)[RW][SPR], const int16_t* col, const void* val, int r0, int nr,
                                                int spr, int K, int n, int lane, uint2* scratch) {
  if constexpr (R == 0 && RW * SPR <= kLoadAllPairs) {
    // small blocks: every row's loads in flight at once, then the placements
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
      for (int s = 0; s < SPR; ++s) {
        const int k = 64 * s + lane;
        const bool live = r < nr && s < spr && k < K;
        pr[r][s].load(col, val, live ? (size_t)(r0 + r) * K + k : 0, live, n);
      }
    place_rows_bank_aware<0, RW, P, SPR>(pr, nr, spr, K, n, lane, scratch);
  } else if constexpr (R < RW) {
#pragma unroll
    for (int s = 0; s < SPR; ++s) {
      const int k = 64 * s + lane;
      const bool live = R < nr && s < spr && k < K;
      pr[R][s].load(col, val, live ? (size_t)(r0 + R) * K + k : 0, live, n);
    }
    if (R < nr) place_row_bank_aware<P, SPR, bit_sliced(RW, SPR)>(pr[R], spr, K, n, lane, scratch);
    asm volatile("" ::: "memory");
    load_place_rows<R + 1, RW, P, SPR>(pr, col, val, r0, nr, spr, K, n, lane, scratch);
  }
}

// Rows of unequal length: row R of the block is layer row rows[R] with
// lens[R] pairs in ns[R] = ceil(lens[R] / 64) slots (all wave-uniform); its
// pairs are placed over those slots only, and slots beyond stay padding.
template <int R, int RW, typename P, int SPR>
__device__ __forceinline__ void load_place_rows_ragged(P (&pr)[RW][SPR], const int16_t* col, const void* val,
                                                       const int (&rows)[RW], const int (&lens)[RW],
                                                       const int (&ns)[RW], int K, int n, int lane, uint2* scratch) {
  if constexpr (R < RW) {
#pragma unroll
    for (int s = 0; s < SPR; ++s) {
      const int k = 64 * s + lane;
      const bool live = k < lens[R];
      pr[R][s].load(col, val, live ? (size_t)rows[R] * K + k : 0, live, n);
    }
    if (ns[R] > 0) place_row_bank_aware<P, SPR, bit_sliced(RW, SPR)>(pr[R], ns[R], lens[R], n, lane, scratch);
    asm volatile("" ::: "memory");
    load_place_rows_ragged<R + 1, RW, P, SPR>(pr, col, val, rows, lens, ns, K, n, lane, scratch);
  }
}

constexpr int kStageChunks = 8;  // 16-byte loads in flight per lane while staging h

// RMAX rows per workgroup are computed (padding rows carry zero values and
// are never stored); the cross-lane sum runs over M = RMAX rounded up to a
// power of two.
template <typename VT, int RMAX, int SPR>
__global__ void __launch_bounds__(256) sparse_kernel(StepArgs a) {
  constexpr int M = pow2_at_least(RMAX);
  extern __shared__ float lds[];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int g = blockIdx.x % a.G;
  const int b = (blockIdx.x / a.G) * 4 + wave;
  if (b >= a.B) return;
  if (__builtin_nontemporal_load(a.status) != 0u) return;

  const int N = a.N;
  const int K = a.K;
  const int nr = a.base_rows + (g < a.extra_rows ? 1 : 0);
  const int row0 = g * a.base_rows + min(g, a.extra_rows);
  const int spr = a.spr;
  // This wave's copy of h_{t-1}[b].  The row is lds_stride >= N + 1 words
  // long; word N stays 0 and absorbs the pairs that carry no nonzero.
  float* hb = lds + wave * a.lds_stride;
  if (N + lane < a.lds_stride) hb[N + lane] = 0.f;

  // Prologue: the nonzeros of the owned rows into registers, once per call.
  Pair<VT> pr[RMAX][SPR];
#pragma unroll
  for (int r = 0; r < RMAX; ++r)
#pragma unroll
    for (int s = 0; s < SPR; ++s) {
      const int k = 64 * s + lane;
      const bool live = r < nr && s < spr && k < K;
      pr[r][s].load(reinterpret_cast<const int16_t*>(a.W), a.V, live ? (size_t)(row0 + r) * K + k : 0, live, N);
    }
  // Bank-aware order of each row's pairs (the same placement as the team
  // layout, so both layouts sum in the same order).
  __shared__ uint2 place_scratch[4][64 * SPR];
  place_rows_bank_aware<0, RMAX, Pair<VT>, SPR>(pr, nr, spr, K, N, lane, place_scratch[wave]);

  const Exchange ex = make_exchange(a.ring, a.relay, a.ring_bytes, a.relay_slice, g, N);
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.X, a.x_bytes);
  const int my_row = RowReduce<M>::owner_row(lane);
  const bool owner = my_row >= 0 && my_row < nr;
  const bool skipper = (g == a.skip_wg);
  const int jn = a.chunks;

  for (int t = 0; t < a.T; ++t) {
    const uint32_t S = a.step0 + (uint32_t)t;
    const uint32_t xoff = (uint32_t)(((size_t)t * a.B + b) * N + row0 + (owner ? my_row : 0)) * 4u;
    const float x = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(xr, xoff, 0, kPlain));

    // All lanes finished the previous step's LDS reads before hb is rewritten.
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();

    if (t == 0) {
      for (int j = 0; j < jn; ++j) {
        const int c = 256 * j + 4 * lane;
        if (c < N) {
          float4 f = make_float4(0.f, 0.f, 0.f, 0.f);
          if (a.h0 != nullptr) {
            const float* p = a.h0 + (size_t)b * N;
            f.x = (c + 0 < N) ? p[c + 0] : 0.f;
            f.y = (c + 1 < N) ? p[c + 1] : 0.f;
            f.z = (c + 2 < N) ? p[c + 2] : 0.f;
            f.w = (c + 3 < N) ? p[c + 3] : 0.f;
          }
          *reinterpret_cast<float4*>(hb + c) = f;
        }
      }
    } else {
      const uint32_t prev = S - 1u;
      const uint32_t tag = tag_bit(prev);
      const uint32_t row0_bytes = (uint32_t)(((prev & 1u) * a.B + b) * a.Npad) * 4u;
      if (!relay_slice(ex, row0_bytes, lane, N, tag, a.deadline) ||
          (a.relay_slice > 0 && !wait_slices(ex, a.relay_slice, row0_bytes, lane, N, tag, a.deadline))) {
        if (lane == 0) report_failure(a.status, a.status_host, kStatusTimeout);
        return;
      }
      for (int j0 = 0; j0 < jn; j0 += kStageChunks) {
        // chunks j0 .. j0 + 7 of the row, 256 words each
        const uint32_t row_bytes = (uint32_t)(((prev & 1u) * a.B + b) * a.Npad + 256 * j0) * 4u;
        const int n = N - 256 * j0;
        u32x4 v[kStageChunks];
        if (!gather_row<kStageChunks>(v, ex.local, row_bytes, lane, jn - j0, n, tag, a.deadline)) {
          if (lane == 0) report_failure(a.status, a.status_host, kStatusTimeout);
          return;
        }
#pragma unroll
        for (int q = 0; q < kStageChunks; ++q) {
          const int c = 256 * q + 4 * lane;
          if (q < jn - j0 && c < n) *reinterpret_cast<float4*>(hb + 256 * j0 + c) = chunk_values(v[q], c, n);
        }
      }
    }

    // h_{t-1}[b] is complete in this wave's LDS row before any lane gathers.
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();

    float acc[M];
#pragma unroll
    for (int r = 0; r < M; ++r) acc[r] = 0.f;
#pragma unroll
    for (int s = 0; s < SPR; ++s) {
      if (s < spr) {
        // The slot's gathers all go out before its first FMA (inline asm,
        // which the compiler does not move loads across).
        float hv[RMAX];
#pragma unroll
        for (int r = 0; r < RMAX; ++r) hv[r] = hb[pr[r][s].column()];
#pragma unroll
        for (int r = 0; r < RMAX; ++r) pr[r][s].fma(acc[r], hv[r]);
      }
    }

    const float sum = RowReduce<M>::reduce(acc, lane);
    debug_jitter(a.jitter_seed, a.jitter_span, wave, t);
    if (owner && !(skipper && t == a.skip_step)) {
      const uint32_t hbits = relu_bits(sum + x);
      const int row = row0 + my_row;
      a.H[((size_t)t * a.B + b) * N + row] = __uint_as_float(hbits);
      const uint32_t roff = (uint32_t)(((S & 1u) * a.B + b) * a.Npad + row) * 4u;
      __builtin_amdgcn_raw_buffer_store_b32(hbits | tag_bit(S), ex.ring, roff, 0, kCoherent);
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

#define PRNN_SPARSE(VT, VTAG, R, S) {VTAG, R, S, reinterpret_cast<const void*>(&sparse_kernel<VT, R, S>)}

}  // namespace prnn
