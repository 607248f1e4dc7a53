// Host side of the C ABI declared in include/prnn.h: handle, argument
// checks, launch plan (layout, grid, kernel instance, exchange), exchange-ring
// bookkeeping and the launches (plain or cooperative).
#include "prnn.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>

#include "host_internal.h"
#include "kernels.h"

using prnn::KernelEntry;
using prnn::StepArgs;

struct prnnContext {
  int device = 0;
  int num_cu = 0;
  size_t lds_per_block = 0;
  uint32_t* d_status = nullptr;
  // Host-visible mirror of failures (pinned host memory: word 0 = a wait
  // expired, word 1 = a value outside the fp16 range), written by the failing
  // kernel; h_status_dev is its address on the device.  The next call on the
  // handle reads it without waiting for the GPU.
  volatile uint32_t* h_status = nullptr;
  uint32_t* h_status_dev = nullptr;
  // A reported failure leaves the device status word set until the next
  // enqueued call clears it (first, on that call's stream).
  bool status_dirty = false;
  // Exchange memory.  Spread layout: [2][B][Npad] ring followed by 8
  // XCD-local copies of it.  Team layout: [8][2][Npad], one region per XCD.
  uint32_t* d_ring = nullptr;
  size_t ring_cap_words = 0;
  bool placement_round_robin = false;  // workgroup i runs on XCD (i + c) % 8
  // Dispatch of the persistent kernels (prnn_set_launch), and whether each
  // kind deals workgroups to the XCDs round-robin (placement_round_robin is
  // the chosen kind's).
  int launch_kind = PRNN_LAUNCH_COOPERATIVE;
  bool coop_placement = false;
  bool plain_placement = false;
  // Workgroups per compute unit of the kernels launched plainly, at their
  // block and LDS sizes (occupancy queries are not free).
  struct Fit {
    const void* fn;
    int block, lds, per_cu;
  };
  Fit fits[48] = {};
  int nfits = 0;
  int exchange = PRNN_EXCHANGE_AUTO;
  int layout = PRNN_LAYOUT_AUTO;
  int ring_layout = -1;  // layout the ring was last reset for
  int ring_xp = -1;      // ... and its XCDs per batch row (team layouts)
  int ring_B = -1;
  int ring_Npad = -1;
  bool ring_valid = false;
  uint64_t step = 0;  // ring step counter of the next timestep
  // Spread layout, relay exchange: the XCD-local copies hold steps S-1 and S-2
  // (as a relay call starting at step S needs) only for S == relay_next_step:
  // after a reset and after a relay call.  Elsewhere the ring is reset first.
  uint64_t relay_next_step = 0;
  int forced_grid = 0;
  int team_waves = 0;  // TEAM layout waves per workgroup: 0 = automatic, 8, 12 or 16
  int xcds_per_row = 0;  // TEAM layout, dense fp16: XCDs per batch row, 0 = automatic, 1, 2 or 4
  bool log = false;    // PRNN_LOG set (and not "0") when the handle was created: plans to stderr
  // A call was captured into a HIP graph: replays may run at any time, so from
  // then on every call starts from a reset ring (one fill kernel per call).
  bool captured = false;
  uint32_t watchdog_us = 200000;
  int math = PRNN_MATH_AUTO;
  int stack_mode = PRNN_STACK_AUTO;
  int skip_wg = -1;
  int skip_step = -1;
  uint32_t jitter_seed = 0;
  uint32_t jitter_span = 0;  // 0: no publish delays
  prnnPlanInfo_t last_plan{};
  bool have_plan = false;
  // Phase tracing: [grid][waves per workgroup][kTraceWords] of the last traced call.
  bool trace = false;
  uint64_t* d_trace = nullptr;
  // Sparse rows of unequal length: the rows ordered by slot count, [N].
  int32_t* d_sorted = nullptr;
  size_t sorted_cap = 0;
  int trace_records = 0;  // records written by the last traced call (0: none)
};

namespace {

constexpr uint32_t kRingResetWord = 0xFFFFFFFFu;  // tag 1 = "written at step -2 / -1"
constexpr int kTeamMaxWgPerXcd = 32;

enum Kind { kDense, kSparse, kFloor, kSparseRows };  // kSparseRows: rows of unequal length

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool overlap(const void* a, size_t an, const void* b, size_t bn) {
  const char* pa = static_cast<const char*>(a);
  const char* pb = static_cast<const char*>(b);
  return pa < pb + bn && pb < pa + an;
}

struct Plan {
  const char* what = "recurrence";  // log label
  int layout = PRNN_LAYOUT_SPREAD;
  int math = PRNN_MATH_EXACT;
  int grid = 0, block = 0;
  int G = 0;                 // spread: workgroups per batch group; team: workgroups per XCD
  int waves = 0;             // waves per workgroup
  int base_rows = 0, extra_rows = 0, max_rows = 0;  // spread: per workgroup; team: per wave
  int chunks = 0;            // 256-column chunks of a row
  int spr = 0;               // sparse: 64-pair slots per row
  int relay_slice = 0;       // spread: words each workgroup relays (0 = direct)
  int lds_stride = 0;        // sparse: words per LDS row
  int xcds_per_row = 1;      // team: XCDs per batch row (2 or 4: split team layout)
  int part_rows = 0;         // split team layout: rows per part
  const KernelEntry* k = nullptr;
  int lds_bytes = 0;
};

// Smallest kernel instance that covers (rows, cap).
const KernelEntry* pick(const KernelEntry* table, int rows, int cap) {
  const KernelEntry* best = nullptr;
  for (const KernelEntry* e = table; e->fn != nullptr; ++e) {
    if (e->rmax < rows || e->cap < cap) continue;
    if (best == nullptr || e->rmax < best->rmax || (e->rmax == best->rmax && e->cap < best->cap)) best = e;
  }
  return best;
}

int sparse_lds_stride(int N) { return (N + 1 + 3) & ~3; }

// Split team layout (dense fp16): the instance holding rows of an xp-way part
// on P workgroups of 8 waves per XCD, or null.  Parts are whole 256-column
// chunks, ceil(chunks / xp) of them each (the last part takes the rest).
const KernelEntry* split_instance(int N, int P, int xp, int* part_rows) {
  const int chunks = (N + 255) / 256;
  *part_rows = 256 * ((chunks + xp - 1) / xp);
  const int Q = P * 8;
  return pick(prnn::kDenseSplitF16Kernels, (std::min(*part_rows, N) + Q - 1) / Q, chunks);
}

// Sparse fp16 layer on two XCDs per batch row (B <= 4): each XCD holds a
// part of whole 256-column chunks of rows.  12 waves per workgroup where a
// part would hold more than 8 rows per wave at 8 waves, else 8 (a forced
// count: that one only).  Fills the split fields, waves, rows and instance of
// p; false when no instance holds the part.  `table`: row-balanced
// instances, or those of rows of unequal length.
bool plan_sparse_split(const prnnContext* h, int N, int P, int spr, Plan* p,
                       const KernelEntry* table = prnn::kSparseSplitF16Kernels) {
  const int chunks = (N + 255) / 256;
  const int part_rows = 256 * ((chunks + 1) / 2);
  const int rows8 = (std::min(part_rows, N) + 8 * P - 1) / (8 * P);
  const int order[2] = {rows8 > 8 ? 12 : 8, rows8 > 8 ? 8 : 12};
  for (int w : order) {
    if (h->team_waves != 0 && h->team_waves != w) continue;
    const int rows = (std::min(part_rows, N) + P * w - 1) / (P * w);
    const KernelEntry* k = nullptr;
    for (const KernelEntry* e = table; e->fn != nullptr; ++e)
      if (e->waves == w && e->rmax >= rows && e->cap >= spr &&
          (k == nullptr || e->rmax < k->rmax || (e->rmax == k->rmax && e->cap < k->cap)))
        k = e;
    if (k == nullptr) continue;
    p->k = k;
    p->waves = w;
    p->block = 64 * w;
    p->max_rows = rows;
    p->base_rows = p->extra_rows = 0;  // per part, derived on the device
    p->part_rows = part_rows;
    p->xcds_per_row = 2;
    p->spr = spr;
    p->lds_stride = 2 * k->rmax * 32 * w + 4;
    p->lds_bytes = 2 * p->lds_stride * 4;
    return true;
  }
  return false;
}

// XCDs per batch row of a dense fp16 layer in the team layout: 1 (the whole
// row on one XCD), or 2 / 4 (split: B <= 4 / B <= 2), or 0 when no form fits.
// A forced value (prnn_set_xcds_per_row) is taken as it is.  Automatically:
// one XCD up to N = 1792, where every row of a wave stays widened to fp32;
// beyond that a split, whose exchange costs 0.4-0.9 us per step more but whose
// waves hold fewer rows, all or mostly widened.  Measured (B = 4 / B = 2, us
// per step, 1 / 2 / 4 XCDs): N = 1792 1.29 / 1.55 / 1.85; N = 2048 1.81 / 1.50
// / 1.62; N = 2304 2.45 / 2.09 / 1.81; N = 2560 2.87 / 2.08 / 2.00; N = 3072
// - / 2.69 / 2.23.  So four XCDs where B <= 2 and N > 2048, else two.
int choose_xcds_per_row(const prnnContext* h, int N, int B, int P, bool single_fits) {
  int part_rows = 0;
  auto split_ok = [&](int xp) {
    return !h->trace && h->math != PRNN_MATH_SPLIT && h->math != PRNN_MATH_HALF && B <= 8 / xp &&
           split_instance(N, P, xp, &part_rows) != nullptr;
  };
  if (h->xcds_per_row == 1) return single_fits ? 1 : 0;
  if (h->xcds_per_row > 1) return split_ok(h->xcds_per_row) ? h->xcds_per_row : 0;
  if (single_fits && N <= 1792) return 1;
  if (N > 2048 && split_ok(4)) return 4;
  if (split_ok(2)) return 2;
  if (split_ok(4)) return 4;
  return single_fits ? 1 : 0;
}

// Spread layout: up to one workgroup per compute unit, each batch group of
// four batch rows on its own set of workgroups, one wave per batch row.
bool plan_spread(const prnnContext* h, Kind kind, int N, int B, int K, int wt, Plan* p) {
  p->layout = PRNN_LAYOUT_SPREAD;
  const int groups = (B + 3) / 4;
  p->waves = std::min(B, 4);
  int G = h->forced_grid > 0 ? h->forced_grid : std::max(1, h->num_cu / groups);
  G = std::min(G, N);
  if (G < 1) return false;
  p->G = G;
  p->grid = G * groups;
  p->block = 64 * p->waves;
  p->base_rows = N / G;
  p->extra_rows = N % G;
  p->max_rows = (N + G - 1) / G;
  p->chunks = (N + 255) / 256;
  if (kind == kDense) {
    p->k = pick(wt == prnn::kF32 ? prnn::kDenseF32Kernels : prnn::kDenseF16Kernels, p->max_rows, p->chunks);
  } else if (kind == kSparse) {
    p->spr = (K + 63) / 64;
    p->k = pick(wt == prnn::kF32 ? prnn::kSparseF32Kernels : prnn::kSparseF16Kernels, p->max_rows, p->spr);
    p->lds_stride = sparse_lds_stride(N);
    p->lds_bytes = p->waves * p->lds_stride * 4;
  } else {
    if (p->max_rows > 64) return false;
    p->k = pick(prnn::kFloorKernels, p->max_rows, p->chunks);
  }
  if (p->k == nullptr) return false;
  // static LDS: the sparse kernel's per-wave pair placement scratch
  const size_t static_lds = kind == kSparse ? (size_t)4 * 64 * p->k->cap * 8 : 0;
  if ((size_t)p->lds_bytes + static_lds > h->lds_per_block) return false;
  // Relay exchange when the grid spreads evenly over the 8 XCDs and is large
  // enough that per-XCD fan-in pays (measured: direct polling from 256
  // workgroups about 4 us per step; relay with slice sentinels about 3.2 us).
  p->relay_slice = 0;
  if (h->exchange != PRNN_EXCHANGE_DIRECT && h->placement_round_robin && G % 8 == 0) {
    const int Npad = (N + 3) & ~3;
    const int per_xcd = G / 8;
    const int slice = (((Npad / 4) + per_xcd - 1) / per_xcd) * 4;  // words, multiple of 4
    if (slice <= 256 && (h->exchange == PRNN_EXCHANGE_RELAY || G >= 192)) p->relay_slice = slice;
  }
  return !(h->exchange == PRNN_EXCHANGE_RELAY && p->relay_slice == 0);
}

// Team layout: each XCD runs one batch row with P workgroups of 8 waves.
bool plan_team(const prnnContext* h, Kind kind, int N, int B, int K, int wt, Plan* p) {
  p->layout = PRNN_LAYOUT_TEAM;
  if (!h->placement_round_robin || B > 8 || h->num_cu < 8) return false;
  int P;
  if (h->forced_grid > 0) {
    if (h->forced_grid % 8 != 0) return false;
    P = h->forced_grid / 8;
  } else {
    P = std::min(kTeamMaxWgPerXcd, h->num_cu / 8);
  }
  P = std::min(P, (N + 7) / 8);  // at least one row per workgroup on average
  if (P < 1 || 8 * P > h->num_cu) return false;
  // Sparse fp16 layers (and their floor) with more than 8 rows per wave at 8
  // waves per workgroup run 12-wave workgroups (3 waves per SIMD), above 16
  // rows 16-wave ones (4 per SIMD) first, where an instance fits: fewer rows
  // per wave.  Measured, us per step: 1 % at N = 5760 2.05 (8 waves), 1.85
  // (16), 1.82 (12); 5 % at N = 5760 3.44 -> 2.89 (12); 10 % at N = 2304
  // 1.70 -> 1.48 (12).  At 7 rows per wave (N = 1792) more waves were slower.
  const int rows8 = (N + 8 * P - 1) / (8 * P);
  // The floor of a dense fp16 layer that runs split over several XCDs per
  // batch row is the split layout's protocol (8-wave workgroups).
  if (kind == kFloor && (h->team_waves == 0 || h->xcds_per_row > 1)) {
    const int chunks = (N + 255) / 256;
    // a forced width (the protocol needs no weight instance), else the width
    // of the dense fp16 layer of the same N and B (one XCD per batch row when
    // no dense form fits either)
    if (h->xcds_per_row > 1 && B > 8 / h->xcds_per_row) return false;
    const int xp = h->xcds_per_row > 1 ? h->xcds_per_row
                                       : choose_xcds_per_row(h, N, B, P, pick(prnn::kDenseTeamF16Kernels, rows8, chunks) != nullptr);
    if (xp > 1) {
      static const KernelEntry floor_split = {0, 64, 1 << 30, nullptr};  // the caller substitutes the kernel
      const int w = h->team_waves != 0 ? h->team_waves : 8;  // 12: the floor of a 12-wave split sparse layer
      if (w != 8 && w != 12) return false;
      int part_rows = 0;
      (void)split_instance(N, P, xp, &part_rows);
      p->G = P;
      p->grid = 8 * P;
      p->waves = w;
      p->block = 64 * w;
      p->chunks = chunks;
      p->xcds_per_row = xp;
      p->part_rows = part_rows;
      p->max_rows = (std::min(part_rows, N) + w * P - 1) / (w * P);
      p->base_rows = p->extra_rows = 0;
      p->k = &floor_split;
      p->lds_bytes = 2 * ((N + 3) & ~3) * 4;
      return p->max_rows <= 64 && (size_t)p->lds_bytes + 256 <= h->lds_per_block;
    }
  }
  const bool wide_ok = ((kind == kSparse || kind == kSparseRows) && wt == prnn::kF16) || kind == kFloor;
  if (h->team_waves > 8 && !wide_ok) return false;
  auto set_waves = [&](int W) {
    const int Q = P * W;  // waves per team
    p->waves = W;
    p->block = 64 * W;
    p->base_rows = N / Q;
    p->extra_rows = N % Q;
    p->max_rows = (N + Q - 1) / Q;
  };
  int W = h->team_waves != 0 ? h->team_waves : (!wide_ok || rows8 <= 8 ? 8 : rows8 > 16 ? 16 : 12);
  p->G = P;
  p->grid = 8 * P;
  set_waves(W);
  p->chunks = (N + 255) / 256;
  const int Npad = (N + 3) & ~3;
  if (kind == kDense && wt == prnn::kF16 && h->math == PRNN_MATH_SPLIT) {
    // Matrix cores: 16 TR rows per workgroup, one 256-column chunk per wave.
    if (p->chunks > 8) return false;
    const int cap = h->forced_grid > 0 ? h->forced_grid / 8 : std::min(kTeamMaxWgPerXcd, h->num_cu / 8);
    int TR = 1;
    while (TR <= 4 && (N + 16 * TR - 1) / (16 * TR) > cap) ++TR;
    if (TR > 4) return false;
    const int Pm = h->forced_grid > 0 ? cap : (N + 16 * TR - 1) / (16 * TR);
    p->math = PRNN_MATH_SPLIT;
    p->G = Pm;
    p->grid = 8 * Pm;
    p->max_rows = 16 * TR;
    p->k = pick(h->trace ? prnn::kDenseTeamMfmaTraceKernels : prnn::kDenseTeamMfmaKernels, 16 * TR, 8);
    if (p->k == nullptr) return false;
    p->lds_bytes = 8 * 520 * 2 + 2 * 8 * p->k->rmax * 4;  // per-wave fp16 hi/lo/zero slots + partials
    return (size_t)p->lds_bytes + 256 <= h->lds_per_block;
  }
  if (kind == kDense && wt == prnn::kF16 && h->math == PRNN_MATH_HALF) {
    // h_{t-1} staged as fp16: packed weights, two rows of fp16 values
    p->math = PRNN_MATH_HALF;
    p->k = pick(h->trace ? prnn::kDenseTeamHalfTraceKernels : prnn::kDenseTeamHalfKernels, p->max_rows, p->chunks);
    if (p->k == nullptr) return false;
    p->lds_bytes = 2 * 256 * p->k->cap * 2;
  } else if (kind == kDense) {
    const KernelEntry* table = h->trace ? (wt == prnn::kF32 ? prnn::kDenseTeamF32TraceKernels : prnn::kDenseTeamF16TraceKernels)
                                        : (wt == prnn::kF32 ? prnn::kDenseTeamF32Kernels : prnn::kDenseTeamF16Kernels);
    const KernelEntry* single = pick(table, p->max_rows, p->chunks);
    const int xp = wt == prnn::kF16 ? choose_xcds_per_row(h, N, B, P, single != nullptr) : 1;
    if (xp == 0) return false;
    if (xp == 1) {
      p->k = single;
    } else {  // (split_instance is not null: choose_xcds_per_row checked it)
      int part_rows = 0;
      p->k = split_instance(N, P, xp, &part_rows);
      p->xcds_per_row = xp;
      p->part_rows = part_rows;
      p->max_rows = (std::min(part_rows, N) + 8 * P - 1) / (8 * P);
      p->base_rows = p->extra_rows = 0;  // per part, derived on the device
    }
    if (p->k == nullptr) return false;
    p->lds_bytes = 2 * 256 * p->k->cap * 4;  // two rows of every chunk the instance holds
  } else if (kind == kSparseRows) {
    // rows of unequal length: fp16 values, 12-wave workgroups where a 16-wave
    // one would be taken for row-balanced layers, else 8
    if (wt != prnn::kF16 || h->trace || h->team_waves == 16) return false;
    p->spr = (K + 63) / 64;
    if (W == 16) set_waves(W = 12);
    if (W == 12) {
      p->k = pick(prnn::kSparseRowsF16Kernels12, p->max_rows, p->spr);
      if (p->k == nullptr && h->team_waves == 12) return false;
      if (p->k == nullptr) set_waves(W = 8);
    }
    if (W == 8) p->k = pick(prnn::kSparseRowsF16Kernels, p->max_rows, p->spr);
    if (p->k == nullptr || h->xcds_per_row == 2) {
      // Rows of more slots than a one-XCD instance holds (or a forced width
      // of two): two XCDs per batch row, where B <= 4 and an instance holds
      // the part.
      if (B > 4 || h->xcds_per_row == 4 || (h->xcds_per_row == 1 && p->k == nullptr)) return false;
      Plan s = *p;
      if (!plan_sparse_split(h, N, P, p->spr, &s, prnn::kSparseRowsSplitF16Kernels)) return false;
      *p = s;
      W = p->waves;
    } else {
      if (h->xcds_per_row == 4) return false;
      p->lds_stride = prnn::sparse_team_stride(p->k->rmax, W);
      p->lds_bytes = 2 * p->lds_stride * 4;
    }
  } else if (kind == kSparse && wt == prnn::kF16 && h->xcds_per_row == 4) {
    return false;  // sparse layers split over two XCDs at most
  } else if (kind == kSparse && wt == prnn::kF16 && h->xcds_per_row == 2) {
    if (h->trace || B > 4 || h->team_waves == 16) return false;
    if (!plan_sparse_split(h, N, P, (K + 63) / 64, p)) return false;
    W = p->waves;
  } else if (kind == kSparse) {
    p->spr = (K + 63) / 64;
    const KernelEntry* table = h->trace ? (wt == prnn::kF32 ? prnn::kSparseTeamF32TraceKernels : prnn::kSparseTeamF16TraceKernels)
                                        : (wt == prnn::kF32 ? prnn::kSparseTeamF32Kernels : prnn::kSparseTeamF16Kernels);
    // 16 waves, else 12, else 8 (a forced count: that one only)
    if (W == 16) {
      p->k = pick(h->trace ? prnn::kSparseTeamF16TraceKernels16 : prnn::kSparseTeamF16Kernels16, p->max_rows, p->spr);
      if (p->k == nullptr && h->team_waves == 16) return false;
      if (p->k == nullptr) set_waves(W = 12);
    }
    if (W == 12) {
      p->k = h->trace ? nullptr : pick(prnn::kSparseTeamF16Kernels12, p->max_rows, p->spr);
      if (p->k == nullptr && h->team_waves == 12) return false;
      if (p->k == nullptr) set_waves(W = 8);
    }
    if (W == 8) p->k = pick(table, p->max_rows, p->spr);
    const bool may_split = wt == prnn::kF16 && h->xcds_per_row == 0 && h->team_waves == 0 && !h->trace && B <= 4;
    if (p->k == nullptr) {
      // No one-XCD instance holds the rows (more slots than any has): two
      // XCDs per batch row, where an instance holds the part.
      Plan s = *p;
      if (!may_split || !plan_sparse_split(h, N, P, p->spr, &s)) return false;
      *p = s;
      W = p->waves;
      const size_t static_lds = 256 + (size_t)W * 64 * p->k->cap * 8;
      return (size_t)p->lds_bytes + static_lds <= h->lds_per_block;
    }
    p->lds_stride = prnn::sparse_team_stride(p->k->rmax, W);  // the instance's fixed row distance
    p->lds_bytes = 2 * p->lds_stride * 4;
    // Automatically, fp16 layers whose rows of one wave hold more than 60
    // 64-pair slots (too many registers for the widened two-step loop) run on
    // two XCDs per batch row where B <= 4: fewer rows per wave, widened, at the
    // price of the cross-XCD exchange.  Measured, us per step (one XCD -> two):
    // 5 % at N = 5760 (15 x 5 slots) 2.86 -> 2.42; lighter layers lose (10 % at
    // N = 2304 1.36 -> 1.87, 1 % at N = 5760 1.47 -> 1.71), 25 % at N = 2304
    // (6 x 9) stays the same.
    if (may_split && p->k->rmax * p->k->cap > 60) {
      Plan s = *p;
      if (plan_sparse_split(h, N, P, p->spr, &s)) {
        *p = s;
        W = p->waves;
      }
    }
  } else {
    static const KernelEntry floor_team = {0, 64, 1 << 30, nullptr};
    static const KernelEntry floor_team12 = {0, 64, 1 << 30, nullptr, 12};
    static const KernelEntry floor_team16 = {0, 64, 1 << 30, nullptr, 16};
    if (p->max_rows > 64) return false;
    p->k = W == 16 ? &floor_team16 : W == 12 ? &floor_team12 : &floor_team;  // the caller substitutes the kernel
    p->lds_bytes = 2 * Npad * 4;
  }
  if (p->k == nullptr) return false;
  // static LDS of the team kernels: flags, and for sparse the per-wave pair
  // placement scratch (waves x 64 x slots x 8 bytes)
  const size_t static_lds = 256 + (kind == kSparse || kind == kSparseRows ? (size_t)W * 64 * p->k->cap * 8 : 0);
  return (size_t)p->lds_bytes + static_lds <= h->lds_per_block;
}

bool plan(const prnnContext* h, Kind kind, int N, int B, int K, int wt, Plan* p) {
  if (h->layout != PRNN_LAYOUT_SPREAD) {
    Plan t;
    if (plan_team(h, kind, N, B, K, wt, &t)) {
      *p = t;
      return true;
    }
    if (h->layout == PRNN_LAYOUT_TEAM || kind == kSparseRows) return false;
  }
  if (kind == kSparseRows) return false;  // the team layout only
  // the matrix-core and half-h forms exist in the team layout only
  if (kind == kDense && wt == prnn::kF16 && (h->math == PRNN_MATH_SPLIT || h->math == PRNN_MATH_HALF)) return false;
  if (h->trace) return false;  // trace instances exist for the team layout only
  return plan_spread(h, kind, N, B, K, wt, p);
}

prnnStatus_t hip_status(hipError_t e) {
  if (e == hipSuccess) return PRNN_STATUS_SUCCESS;
  if (e == hipErrorCooperativeLaunchTooLarge || e == hipErrorInvalidConfiguration ||
      e == hipErrorOutOfMemory)
    return PRNN_STATUS_NOT_SUPPORTED;
  return PRNN_STATUS_INTERNAL_ERROR;
}

// A failed run whose mirror reached the host, reported once: the mirror is
// cleared, the device status word is cleared by the next enqueued call, and
// the ring is reset before the next launch.
bool take_failure(prnnContext* h) {
  const uint32_t timeout = h->h_status[0], range = h->h_status[1];
  if ((timeout | range) == 0u) return false;
  h->h_status[0] = 0u;
  h->h_status[1] = 0u;
  h->status_dirty = true;
  h->ring_valid = false;
  if (h->log)
    std::fprintf(stderr, "prnn: run failed:%s%s\n", timeout ? " a wait for h_{t-1} expired (watchdog)" : "",
                 range ? " a value outside the fp16 range" : "");
  return true;
}

// Clears the device status word of a reported failure, on `stream`, before
// the call's own kernels.
prnnStatus_t clear_reported_status(prnnContext* h, hipStream_t stream) {
  if (!h->status_dirty) return PRNN_STATUS_SUCCESS;
  prnn::launch_fill(h->d_status, 64, 0u, stream);
  if (hipGetLastError() != hipSuccess) return PRNN_STATUS_INTERNAL_ERROR;
  h->status_dirty = false;
  return PRNN_STATUS_SUCCESS;
}

// Makes the exchange memory fit the plan's layout and, when the layout or its
// shape changed, a run failed, or relay continuity was broken, resets it on
// `stream` and restarts the step counter.
prnnStatus_t ensure_ring(prnnContext* h, const Plan& p, int B, int Npad, hipStream_t stream) {
  const bool team = p.layout == PRNN_LAYOUT_TEAM;
  if (clear_reported_status(h, stream) != PRNN_STATUS_SUCCESS) return PRNN_STATUS_INTERNAL_ERROR;
  // team: [8][2][Npad] (+ the split layout's shared ring, as large)
  const size_t words = team ? (p.xcds_per_row > 1 ? 32ull : 16ull) * (size_t)Npad : 18ull * (size_t)B * (size_t)Npad;
  if (words * 4ull > 0xFFFFFFF0ull) return PRNN_STATUS_NOT_SUPPORTED;
  // Under stream capture the call becomes a graph node that may be replayed
  // at any time, after any other call: its ring is reset inside the captured
  // sequence (a fill kernel) and its steps count from 0, and every later call
  // on the handle resets the ring as well.  Nothing may be allocated here
  // while capturing.
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cs) != hipSuccess) return PRNN_STATUS_INTERNAL_ERROR;
  const bool capturing = cs != hipStreamCaptureStatusNone;
  if (capturing) h->captured = true;
  if (h->captured) h->ring_valid = false;
  if (words > h->ring_cap_words && capturing) return PRNN_STATUS_NOT_SUPPORTED;
  if (words > h->ring_cap_words) {
    if (h->d_ring != nullptr) {
      if (hipDeviceSynchronize() != hipSuccess) return PRNN_STATUS_INTERNAL_ERROR;
      (void)hipFree(h->d_ring);
      h->d_ring = nullptr;
      h->ring_cap_words = 0;
    }
    void* mem = nullptr;
    if (hipMalloc(&mem, words * 4) != hipSuccess) return PRNN_STATUS_ALLOC_FAILED;
    h->d_ring = static_cast<uint32_t*>(mem);
    h->ring_cap_words = words;
    h->ring_valid = false;
  }
  if (!team && p.relay_slice > 0 && h->step != h->relay_next_step) h->ring_valid = false;
  const bool same = h->ring_layout == p.layout && h->ring_Npad == Npad && (team || h->ring_B == B) &&
                    (!team || h->ring_xp == p.xcds_per_row);
  if (!h->ring_valid || !same) {
    if (team) {
      prnn::launch_team_fill(h->d_ring, Npad, kRingResetWord, stream);
      if (p.xcds_per_row > 1) prnn::launch_fill(h->d_ring + 16ull * Npad, 16ull * Npad, kRingResetWord, stream);
    } else
      prnn::launch_fill(h->d_ring, words, kRingResetWord, stream);
    if (hipGetLastError() != hipSuccess) return PRNN_STATUS_INTERNAL_ERROR;
    h->ring_layout = p.layout;
    h->ring_xp = p.xcds_per_row;
    h->ring_B = B;
    h->ring_Npad = Npad;
    h->ring_valid = true;
    h->step = 0;
    h->relay_next_step = 0;
  }
  return PRNN_STATUS_SUCCESS;
}

// Shape checks, then (for T > 0) pointer checks.  *empty is set when there is
// nothing to do (T == 0): the call then succeeds without touching any buffer.
prnnStatus_t check_common(prnnHandle_t h, int N, int B, int T, const float* X, const float* h0, float* H,
                          bool* empty) {
  *empty = false;
  if (h == nullptr) return PRNN_STATUS_BAD_PARAM;
  if (N < 1 || B < 1 || B > 8 || T < 0) return PRNN_STATUS_BAD_PARAM;
  if (T == 0) {
    *empty = true;
    return PRNN_STATUS_SUCCESS;
  }
  if (X == nullptr || H == nullptr) return PRNN_STATUS_BAD_PARAM;
  if (!aligned(X, 4) || !aligned(H, 4) || (h0 != nullptr && !aligned(h0, 4))) return PRNN_STATUS_BAD_PARAM;
  const size_t xb = (size_t)T * B * N * 4;
  if (overlap(X, xb, H, xb)) return PRNN_STATUS_BAD_PARAM;
  if (h0 != nullptr && overlap(h0, (size_t)B * N * 4, H, xb)) return PRNN_STATUS_BAD_PARAM;
  return PRNN_STATUS_SUCCESS;
}

StepArgs base_args(prnnContext* h, int N, int B, int T, const float* X, const float* h0, float* H,
                   const Plan& p, int Npad) {
  StepArgs a;
  std::memset(&a, 0, sizeof(a));
  a.X = X;
  a.h0 = h0;
  a.H = H;
  a.ring = h->d_ring;
  a.relay = h->d_ring + 2ull * B * Npad;
  a.relay_slice = p.relay_slice;
  a.status = h->d_status;
  a.status_host = h->h_status_dev;
  a.N = N;
  a.B = B;
  a.T = T;
  a.Npad = Npad;
  a.G = p.G;
  a.base_rows = p.base_rows;
  a.extra_rows = p.extra_rows;
  a.chunks = p.chunks;
  a.spr = p.spr;
  a.lds_stride = p.lds_stride;
  a.xcds_per_row = p.xcds_per_row > 1 ? p.xcds_per_row : 0;
  a.part_rows = p.part_rows;
  a.ring_bytes = static_cast<uint32_t>(2ull * B * Npad * 4);
  a.x_bytes = static_cast<uint32_t>((size_t)T * B * N * 4);
  return a;
}

// One line per launch on stderr when the handle logs (PRNN_LOG).
void log_plan(const prnnContext* h, const char* what, int N, int B, int T, const prnnPlanInfo_t& info) {
  if (!h->log) return;
  static const char* maths[] = {"auto", "exact", "split", "half"};
  std::fprintf(stderr,
               "prnn: %s N=%d B=%d T=%d layout=%s xcds/row=%d grid=%d waves/wg=%d rows/wave=%d instance=(%d,%d) "
               "lds=%d math=%s first_step=%llu\n",
               what, N, B, T, info.layout == PRNN_LAYOUT_TEAM ? "team" : "spread", info.xcds_per_row, info.grid,
               info.waves_per_wg,
               info.rows_per_wave, info.rmax, info.chunks, info.lds_bytes,
               info.math >= 0 && info.math <= 3 ? maths[info.math] : "?", (unsigned long long)info.first_step);
}

// A persistent kernel's launch, cooperative or plain (prnn_set_launch).  A
// plain one is refused (hipErrorCooperativeLaunchTooLarge, as the
// cooperative launch reports it) unless the whole grid fits the device at
// once.
hipError_t launch_persistent(prnnContext* h, const void* fn, int grid, int block, void** args, int lds,
                             hipStream_t stream) {
  // an LDS size the device does not take: NOT_SUPPORTED, as before any launch
  if (lds > 65536 && hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds) != hipSuccess)
    return hipErrorInvalidConfiguration;
  if (h->launch_kind != PRNN_LAUNCH_PLAIN)
    return hipLaunchCooperativeKernel(fn, dim3(grid), dim3(block), args, static_cast<unsigned>(lds), stream);
  int per_cu = -1;
  for (int i = 0; i < h->nfits; ++i)
    if (h->fits[i].fn == fn && h->fits[i].block == block && h->fits[i].lds == lds) per_cu = h->fits[i].per_cu;
  if (per_cu < 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, block, static_cast<size_t>(lds)) != hipSuccess)
      return hipErrorInvalidValue;
    if (h->nfits < static_cast<int>(sizeof(h->fits) / sizeof(h->fits[0]))) h->fits[h->nfits++] = {fn, block, lds, per_cu};
  }
  if ((long long)per_cu * h->num_cu < grid) return hipErrorCooperativeLaunchTooLarge;
  return hipLaunchKernel(fn, dim3(grid), dim3(block), args, static_cast<size_t>(lds), stream);
}

prnnStatus_t launch(prnnContext* h, const Plan& p, StepArgs& a, int T, hipStream_t stream) {
  a.step0 = static_cast<uint32_t>(h->step);
  a.deadline = static_cast<uint64_t>(h->watchdog_us) * 100ull;  // 100 MHz constant clock
  a.skip_wg = h->skip_wg;
  a.skip_step = h->skip_step;
  a.jitter_seed = h->jitter_seed;
  a.jitter_span = h->jitter_span;
  a.trace = nullptr;
  if (h->trace) {
    // records of workgroups without a batch row of their own stay zero
    prnn::launch_fill(reinterpret_cast<uint32_t*>(h->d_trace), (size_t)p.grid * p.waves * prnn::kTraceWords * 2, 0u,
                      stream);
    a.trace = h->d_trace;
  }
  void* args[] = {&a};
  hipError_t e = launch_persistent(h, p.k->fn, p.grid, p.block, args, p.lds_bytes, stream);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return hip_status(e);
  }
  prnnPlanInfo_t& info = h->last_plan;
  info.layout = p.layout;
  info.grid = p.grid;
  info.waves_per_wg = p.waves;
  info.rows_per_wave = p.max_rows;
  info.rmax = p.k->rmax;
  info.chunks = p.k->cap;
  info.lds_bytes = p.lds_bytes;
  info.relay_slice = p.relay_slice;
  info.math = p.math;
  info.xcds_per_row = p.layout == PRNN_LAYOUT_TEAM ? p.xcds_per_row : 0;
  info.first_step = h->step;
  log_plan(h, p.what, a.N, a.B, T, info);
  h->have_plan = true;
  h->trace_records = h->trace ? p.grid * p.waves : 0;
  h->step += static_cast<uint64_t>(T);
  if (p.layout == PRNN_LAYOUT_SPREAD && p.relay_slice > 0) h->relay_next_step = h->step;
  h->skip_wg = -1;
  h->skip_step = -1;
  return PRNN_STATUS_SUCCESS;
}

// The relay and team exchanges rely on workgroup i of a launch running on
// XCD (i + c) % 8 for one constant c.  Checked once per handle, for
// cooperative and for plain launches.
bool check_placement(int num_cu, bool cooperative) {
  const int grid = num_cu;
  void* p = nullptr;
  if (grid < 8 || hipMalloc(&p, grid * 4) != hipSuccess) return false;
  uint32_t* d = static_cast<uint32_t*>(p);
  void* args[] = {&d};
  const hipError_t e =
      cooperative ? hipLaunchCooperativeKernel(prnn::kPlacementKernel, dim3(grid), dim3(64), args, 0, nullptr)
                  : hipLaunchKernel(prnn::kPlacementKernel, dim3(grid), dim3(64), args, 0, nullptr);
  bool ok = e == hipSuccess && hipDeviceSynchronize() == hipSuccess;
  uint32_t* host = new (std::nothrow) uint32_t[grid];
  ok = ok && host != nullptr && hipMemcpy(host, d, grid * 4, hipMemcpyDeviceToHost) == hipSuccess;
  if (ok) {
    const uint32_t c = host[0] % 8u;
    for (int i = 0; i < grid && ok; ++i) ok = host[i] < 8u && (host[i] + 8u - (uint32_t)i % 8u) % 8u == c;
  }
  delete[] host;
  (void)hipGetLastError();
  (void)hipFree(p);
  return ok;
}

// Argument checks and launch plan of a dense forward call.  *empty: T == 0
// (nothing to do).  Nothing is enqueued.
prnnStatus_t prepare_dense(prnnContext* h, int N, int B, int T, prnnDataType_t w_type, const void* W,
                           const float* X, const float* h0, float* H, Plan* p, bool* empty) {
  prnnStatus_t st = check_common(h, N, B, T, X, h0, H, empty);
  if (st != PRNN_STATUS_SUCCESS) return st;
  if (w_type != PRNN_DATA_FLOAT && w_type != PRNN_DATA_HALF) return PRNN_STATUS_BAD_PARAM;
  if (*empty) return PRNN_STATUS_SUCCESS;
  if (W == nullptr) return PRNN_STATUS_BAD_PARAM;
  if (!aligned(W, w_type == PRNN_DATA_FLOAT ? 4 : 2)) return PRNN_STATUS_BAD_PARAM;
  const size_t wb = (size_t)N * N * (w_type == PRNN_DATA_FLOAT ? 4 : 2);
  if (overlap(W, wb, H, (size_t)T * B * N * 4)) return PRNN_STATUS_BAD_PARAM;
  if ((size_t)T * B * N * 4 > 0xFFFFFFF0ull) return PRNN_STATUS_NOT_SUPPORTED;
  const int wt = w_type == PRNN_DATA_FLOAT ? prnn::kF32 : prnn::kF16;
  if (!plan(h, kDense, N, B, 0, wt, p)) return PRNN_STATUS_NOT_SUPPORTED;
  return PRNN_STATUS_SUCCESS;
}

prnnStatus_t run_dense(prnnContext* h, const Plan& p, int N, int B, int T, const void* W, const float* X,
                       const float* h0, float* H, hipStream_t stream) {
  const int Npad = (N + 3) & ~3;
  prnnStatus_t st = ensure_ring(h, p, B, Npad, stream);
  if (st != PRNN_STATUS_SUCCESS) return st;
  StepArgs a = base_args(h, N, B, T, X, h0, H, p, Npad);
  a.W = W;
  a.w_vec = aligned(W, 16) ? 1 : 0;  // W needs only element alignment; vector loads where it allows them
  return launch(h, p, a, T, stream);
}

prnnStatus_t prepare_sparse(prnnContext* h, int N, int B, int T, int K, const int16_t* col, prnnDataType_t val_type,
                            const void* val, const float* X, const float* h0, float* H, Plan* p, bool* empty) {
  prnnStatus_t st = check_common(h, N, B, T, X, h0, H, empty);
  if (st != PRNN_STATUS_SUCCESS) return st;
  if (val_type != PRNN_DATA_FLOAT && val_type != PRNN_DATA_HALF) return PRNN_STATUS_BAD_PARAM;
  if (K < 1 || K > N || N > 32767) return PRNN_STATUS_BAD_PARAM;
  if (*empty) return PRNN_STATUS_SUCCESS;
  if (col == nullptr || val == nullptr) return PRNN_STATUS_BAD_PARAM;
  if (!aligned(col, 2) || !aligned(val, val_type == PRNN_DATA_FLOAT ? 4 : 2)) return PRNN_STATUS_BAD_PARAM;
  const size_t hb = (size_t)T * B * N * 4;
  if (overlap(col, (size_t)N * K * 2, H, hb) ||
      overlap(val, (size_t)N * K * (val_type == PRNN_DATA_FLOAT ? 4 : 2), H, hb))
    return PRNN_STATUS_BAD_PARAM;
  if (hb > 0xFFFFFFF0ull) return PRNN_STATUS_NOT_SUPPORTED;
  const int wt = val_type == PRNN_DATA_FLOAT ? prnn::kF32 : prnn::kF16;
  if (!plan(h, kSparse, N, B, K, wt, p)) return PRNN_STATUS_NOT_SUPPORTED;
  return PRNN_STATUS_SUCCESS;
}

prnnStatus_t run_sparse(prnnContext* h, const Plan& p, int N, int B, int T, int K, const int16_t* col,
                        const void* val, const float* X, const float* h0, float* H, hipStream_t stream) {
  const int Npad = (N + 3) & ~3;
  prnnStatus_t st = ensure_ring(h, p, B, Npad, stream);
  if (st != PRNN_STATUS_SUCCESS) return st;
  StepArgs a = base_args(h, N, B, T, X, h0, H, p, Npad);
  a.W = col;
  a.V = val;
  a.K = K;
  return launch(h, p, a, T, stream);
}

// The handle's row order buffer for sparse rows of unequal length (grown as
// needed; never while the stream is being captured).
prnnStatus_t ensure_sorted(prnnContext* h, int N, hipStream_t stream) {
  if ((size_t)N <= h->sorted_cap) return PRNN_STATUS_SUCCESS;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cs) != hipSuccess) return PRNN_STATUS_INTERNAL_ERROR;
  if (cs != hipStreamCaptureStatusNone) return PRNN_STATUS_NOT_SUPPORTED;
  if (h->d_sorted != nullptr) {
    if (hipDeviceSynchronize() != hipSuccess) return PRNN_STATUS_INTERNAL_ERROR;
    (void)hipFree(h->d_sorted);
    h->d_sorted = nullptr;
    h->sorted_cap = 0;
  }
  void* mem = nullptr;
  if (hipMalloc(&mem, (size_t)N * 4) != hipSuccess) return PRNN_STATUS_ALLOC_FAILED;
  h->d_sorted = static_cast<int32_t*>(mem);
  h->sorted_cap = (size_t)N;
  return PRNN_STATUS_SUCCESS;
}

prnnStatus_t run_sparse_rows(prnnContext* h, const Plan& p, int N, int B, int T, int K, const int16_t* col,
                             const void* val, const int32_t* row_len, const float* X, const float* h0, float* H,
                             hipStream_t stream) {
  prnnStatus_t st = ensure_sorted(h, N, stream);
  if (st != PRNN_STATUS_SUCCESS) return st;
  const int Npad = (N + 3) & ~3;
  st = ensure_ring(h, p, B, Npad, stream);
  if (st != PRNN_STATUS_SUCCESS) return st;
  // each XCD's part ordered on its own on two XCDs per batch row
  prnn::launch_sort_rows(row_len, N, K, p.xcds_per_row > 1 ? p.part_rows : N, h->d_sorted, stream);
  if (hipGetLastError() != hipSuccess) return PRNN_STATUS_INTERNAL_ERROR;
  StepArgs a = base_args(h, N, B, T, X, h0, H, p, Npad);
  a.W = col;
  a.V = val;
  a.K = K;
  a.row_len = row_len;
  a.sorted = h->d_sorted;
  return launch(h, p, a, T, stream);
}

// Argument checks of the input projection; fills the kernel arguments.
prnnStatus_t prepare_project(prnnContext* h, int M, int N, int I, prnnDataType_t x_type, const void* x,
                             prnnDataType_t u_type, const void* U, const float* bias, float* X, prnn::ProjArgs* a,
                             bool* vec) {
  if (h == nullptr || M < 0 || N < 1 || I < 1) return PRNN_STATUS_BAD_PARAM;
  if (x_type != PRNN_DATA_FLOAT && x_type != PRNN_DATA_HALF) return PRNN_STATUS_BAD_PARAM;
  if (u_type != PRNN_DATA_FLOAT && u_type != PRNN_DATA_HALF) return PRNN_STATUS_BAD_PARAM;
  if (u_type != PRNN_DATA_HALF) return PRNN_STATUS_NOT_SUPPORTED;
  if (M == 0) return PRNN_STATUS_SUCCESS;
  if (x == nullptr || U == nullptr || X == nullptr) return PRNN_STATUS_BAD_PARAM;
  const size_t xe = x_type == PRNN_DATA_FLOAT ? 4 : 2;
  if (!aligned(x, xe) || !aligned(U, 2) || !aligned(X, 4) || (bias != nullptr && !aligned(bias, 4)))
    return PRNN_STATUS_BAD_PARAM;
  const size_t xb = (size_t)M * I * xe, ub = (size_t)N * I * 2, ob = (size_t)M * N * 4;
  if (overlap(X, ob, x, xb) || overlap(X, ob, U, ub) || (bias != nullptr && overlap(X, ob, bias, (size_t)N * 4)))
    return PRNN_STATUS_BAD_PARAM;
  const long long tiles = (long long)((M + 63) / 64) * ((N + 63) / 64);  // at most 64 x 64 tiles of X
  if (xb > 0xFFFFFF00ull || ub > 0xFFFFFF00ull || tiles > (1ll << 28)) return PRNN_STATUS_NOT_SUPPORTED;
  a->x = x;
  a->U = U;
  a->bias = bias;
  a->X = X;
  a->status = h->d_status;
  a->status_host = h->h_status_dev;
  a->M = M;
  a->N = N;
  a->I = I;
  a->x_bytes = static_cast<uint32_t>(xb);
  a->u_bytes = static_cast<uint32_t>(ub);
  a->tiles_n = 0;  // the tiling is chosen at launch (launch_project)
  a->tiles = 0;
  a->per_xcd = 0;
  *vec = I % 8 == 0 && aligned(x, 16) && aligned(U, 16);
  return PRNN_STATUS_SUCCESS;
}

// The projection of a layer call into its workspace Xbuf ([T][B][N]): besides
// the projection's own checks, Xbuf must not overlap h0 or the recurrent
// weights (the projection writes it before the recurrence reads them).
prnnStatus_t prepare_layer_projection(prnnContext* h, int N, int I, int B, int T, prnnDataType_t x_type,
                                      const void* x, prnnDataType_t u_type, const void* U, const float* bias,
                                      float* Xbuf, const float* h0, const void* w0, size_t w0_bytes,
                                      const void* w1, size_t w1_bytes, prnn::ProjArgs* a, bool* vec) {
  if (I < 1) return PRNN_STATUS_BAD_PARAM;
  const long long M = (long long)T * B;
  if (M > 0x7fffffffll) return PRNN_STATUS_NOT_SUPPORTED;
  const size_t ob = (size_t)M * N * 4;
  if ((h0 != nullptr && overlap(Xbuf, ob, h0, (size_t)B * N * 4)) || overlap(Xbuf, ob, w0, w0_bytes) ||
      (w1 != nullptr && overlap(Xbuf, ob, w1, w1_bytes)))
    return PRNN_STATUS_BAD_PARAM;
  return prepare_project(h, static_cast<int>(M), N, I, x_type, x, u_type, U, bias, Xbuf, a, vec);
}

}  // namespace

prnnStatus_t prnn::forward_dense_on(const DeviceFacts& dev, uint32_t* ring, uint32_t* status, int N, int B, int T,
                                    prnnDataType_t w_type, const void* W, const float* X, const float* h0, float* H,
                                    hipStream_t stream) {
  // A context on the stack (nothing allocated): default options, the team
  // layout only (its exchange memory is what `ring` holds), no host mirror.
  prnnContext c;
  c.num_cu = dev.num_cu;
  c.lds_per_block = dev.lds_per_block;
  c.coop_placement = dev.placement_round_robin;
  c.plain_placement = dev.plain_placement;
  c.launch_kind = dev.plain_placement ? PRNN_LAUNCH_PLAIN : PRNN_LAUNCH_COOPERATIVE;
  c.placement_round_robin = dev.plain_placement || dev.placement_round_robin;
  c.layout = PRNN_LAYOUT_TEAM;
  c.d_ring = ring;
  c.d_status = status;
  Plan p;
  bool empty = false;
  prnnStatus_t st = prepare_dense(&c, N, B, T, w_type, W, X, h0, H, &p, &empty);
  if (st != PRNN_STATUS_SUCCESS || empty) return st;
  const int Npad = (N + 3) & ~3;
  // every call starts from a reset ring (step 0) and a clear status word;
  // `ring` holds [8][2][Npad] words and, for a split plan, as many again
  prnn::launch_fill(status, 1, 0u, stream);
  prnn::launch_team_fill(ring, Npad, kRingResetWord, stream);
  if (p.xcds_per_row > 1) prnn::launch_fill(ring + 16ull * Npad, 16ull * Npad, kRingResetWord, stream);
  if (hipGetLastError() != hipSuccess) return PRNN_STATUS_INTERNAL_ERROR;
  StepArgs a = base_args(&c, N, B, T, X, h0, H, p, Npad);
  a.W = W;
  a.w_vec = aligned(W, 16) ? 1 : 0;
  return launch(&c, p, a, T, stream);
}

extern "C" {

const char* prnn_status_string(prnnStatus_t s) {
  switch (s) {
    case PRNN_STATUS_SUCCESS: return "PRNN_STATUS_SUCCESS";
    case PRNN_STATUS_BAD_PARAM: return "PRNN_STATUS_BAD_PARAM";
    case PRNN_STATUS_NOT_SUPPORTED: return "PRNN_STATUS_NOT_SUPPORTED";
    case PRNN_STATUS_ALLOC_FAILED: return "PRNN_STATUS_ALLOC_FAILED";
    case PRNN_STATUS_EXECUTION_FAILED: return "PRNN_STATUS_EXECUTION_FAILED";
    case PRNN_STATUS_INTERNAL_ERROR: return "PRNN_STATUS_INTERNAL_ERROR";
    case PRNN_STATUS_MAX_ENUM: break;
  }
  return "PRNN_STATUS_UNKNOWN";
}

prnnStatus_t prnn_create(prnnHandle_t* handle) {
  if (handle == nullptr) return PRNN_STATUS_BAD_PARAM;
  *handle = nullptr;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return PRNN_STATUS_INTERNAL_ERROR;
  hipDeviceProp_t props;
  if (hipGetDeviceProperties(&props, dev) != hipSuccess) return PRNN_STATUS_INTERNAL_ERROR;
  if (std::strncmp(props.gcnArchName, "gfx950", 6) != 0) return PRNN_STATUS_NOT_SUPPORTED;
  if (!props.cooperativeLaunch) return PRNN_STATUS_NOT_SUPPORTED;
  prnnContext* h = new (std::nothrow) prnnContext();
  if (h == nullptr) return PRNN_STATUS_ALLOC_FAILED;
  h->device = dev;
  h->num_cu = props.multiProcessorCount;
  h->lds_per_block = props.sharedMemPerBlock;
  void* p = nullptr;
  if (hipMalloc(&p, 256) != hipSuccess) {
    delete h;
    return PRNN_STATUS_ALLOC_FAILED;
  }
  h->d_status = static_cast<uint32_t*>(p);
  void* hp = nullptr;
  if (hipHostMalloc(&hp, 64, hipHostMallocDefault) != hipSuccess) {
    (void)hipGetLastError();
    (void)hipFree(p);
    delete h;
    return PRNN_STATUS_ALLOC_FAILED;
  }
  h->h_status = static_cast<volatile uint32_t*>(hp);
  for (int i = 0; i < 16; ++i) h->h_status[i] = 0u;
  void* hd = nullptr;
  prnn::launch_fill(h->d_status, 64, 0u, nullptr);
  if (hipHostGetDevicePointer(&hd, hp, 0) != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
    (void)hipGetLastError();
    (void)hipHostFree(hp);
    (void)hipFree(p);
    delete h;
    return PRNN_STATUS_INTERNAL_ERROR;
  }
  h->h_status_dev = static_cast<uint32_t*>(hd);
  // Plain launches where their workgroups are dealt as the layouts assume:
  // they start 10-20 us sooner after the previous kernel than cooperative ones.
  h->coop_placement = check_placement(h->num_cu, true);
  h->plain_placement = check_placement(h->num_cu, false);
  h->launch_kind = h->plain_placement ? PRNN_LAUNCH_PLAIN : PRNN_LAUNCH_COOPERATIVE;
  h->placement_round_robin = h->plain_placement || h->coop_placement;  // the chosen kind's
  const char* log = std::getenv("PRNN_LOG");
  h->log = log != nullptr && log[0] != '\0' && std::strcmp(log, "0") != 0;
  if (h->log)
    std::fprintf(stderr,
                 "prnn: handle on device %d, %d compute units, %zu bytes of LDS per workgroup, team layout %s, "
                 "%s launches\n",
                 h->device, h->num_cu, (size_t)h->lds_per_block, h->placement_round_robin ? "available" : "unavailable",
                 h->launch_kind == PRNN_LAUNCH_PLAIN ? "plain" : "cooperative");
  *handle = h;
  return PRNN_STATUS_SUCCESS;
}

prnnStatus_t prnn_destroy(prnnHandle_t h) {
  if (h == nullptr) return PRNN_STATUS_SUCCESS;
  prnnStatus_t st = PRNN_STATUS_SUCCESS;
  if (hipDeviceSynchronize() != hipSuccess) st = PRNN_STATUS_INTERNAL_ERROR;
  if (h->h_status != nullptr && take_failure(h)) st = PRNN_STATUS_EXECUTION_FAILED;
  if (h->d_ring != nullptr) (void)hipFree(h->d_ring);
  if (h->d_trace != nullptr) (void)hipFree(h->d_trace);
  if (h->d_sorted != nullptr) (void)hipFree(h->d_sorted);
  if (h->d_status != nullptr) (void)hipFree(h->d_status);
  if (h->h_status != nullptr) (void)hipHostFree(const_cast<uint32_t*>(h->h_status));
  delete h;
  return st;
}

prnnStatus_t prnn_set_trace(prnnHandle_t h, int enable) {
  if (h == nullptr) return PRNN_STATUS_BAD_PARAM;
  if (enable != 0 && h->d_trace == nullptr) {
    void* p = nullptr;
    // up to one workgroup of up to 16 waves per compute unit
    if (hipMalloc(&p, (size_t)h->num_cu * 16 * prnn::kTraceWords * sizeof(uint64_t)) != hipSuccess) {
      (void)hipGetLastError();
      return PRNN_STATUS_ALLOC_FAILED;
    }
    h->d_trace = static_cast<uint64_t*>(p);
  }
  h->trace = enable != 0;
  return PRNN_STATUS_SUCCESS;
}

prnnStatus_t prnn_get_trace(prnnHandle_t h, uint64_t* out, size_t capacity, int* records, hipStream_t stream) {
  if (h == nullptr || records == nullptr) return PRNN_STATUS_BAD_PARAM;
  *records = h->trace_records;
  if (h->trace_records == 0) return PRNN_STATUS_BAD_PARAM;
  const size_t words = (size_t)h->trace_records * prnn::kTraceWords;
  if (out == nullptr || capacity < words) return PRNN_STATUS_BAD_PARAM;
  if (hipStreamSynchronize(stream) != hipSuccess) return PRNN_STATUS_INTERNAL_ERROR;
  if (hipMemcpy(out, h->d_trace, words * sizeof(uint64_t), hipMemcpyDeviceToHost) != hipSuccess)
    return PRNN_STATUS_INTERNAL_ERROR;
  return PRNN_STATUS_SUCCESS;
}

prnnStatus_t prnn_set_grid(prnnHandle_t h, int workgroups) {
  if (h == nullptr || workgroups < 0) return PRNN_STATUS_BAD_PARAM;
  h->forced_grid = workgroups;
  return PRNN_STATUS_SUCCESS;
}

prnnStatus_t prnn_set_team_waves(prnnHandle_t h, int waves) {
  if (h == nullptr || (waves != 0 && waves != 8 && waves != 12 && waves != 16)) return PRNN_STATUS_BAD_PARAM;
  h->team_waves = waves;
  return PRNN_STATUS_SUCCESS;
}

prnnStatus_t prnn_set_xcds_per_row(prnnHandle_t h, int xcds) {
  if (h == nullptr || (xcds != 0 && xcds != 1 && xcds != 2 && xcds != 4)) return PRNN_STATUS_BAD_PARAM;
  h->xcds_per_row = xcds;
  return PRNN_STATUS_SUCCESS;
}

prnnStatus_t prnn_set_exchange(prnnHandle_t h, prnnExchange_t mode) {
  if (h == nullptr) return PRNN_STATUS_BAD_PARAM;
  if (mode != PRNN_EXCHANGE_AUTO && mode != PRNN_EXCHANGE_DIRECT && mode != PRNN_EXCHANGE_RELAY)
    return PRNN_STATUS_BAD_PARAM;
  h->exchange = mode;
  return PRNN_STATUS_SUCCESS;
}

prnnStatus_t prnn_set_layout(prnnHandle_t h, prnnLayout_t layout) {
  if (h == nullptr) return PRNN_STATUS_BAD_PARAM;
  if (layout != PRNN_LAYOUT_AUTO && layout != PRNN_LAYOUT_SPREAD && layout != PRNN_LAYOUT_TEAM)
    return PRNN_STATUS_BAD_PARAM;
  h->layout = layout;
  return PRNN_STATUS_SUCCESS;
}

prnnStatus_t prnn_set_math(prnnHandle_t h, prnnMath_t mode) {
  if (h == nullptr) return PRNN_STATUS_BAD_PARAM;
  if (mode != PRNN_MATH_AUTO && mode != PRNN_MATH_EXACT && mode != PRNN_MATH_SPLIT && mode != PRNN_MATH_HALF)
    return PRNN_STATUS_BAD_PARAM;
  h->math = mode;
  return PRNN_STATUS_SUCCESS;
}

prnnStatus_t prnn_set_watchdog_us(prnnHandle_t h, uint32_t us) {
  if (h == nullptr || us == 0) return PRNN_STATUS_BAD_PARAM;
  h->watchdog_us = us;
  return PRNN_STATUS_SUCCESS;
}

prnnStatus_t prnn_get_last_plan(prnnHandle_t h, prnnPlanInfo_t* info) {
  if (h == nullptr || info == nullptr || !h->have_plan) return PRNN_STATUS_BAD_PARAM;
  *info = h->last_plan;
  return PRNN_STATUS_SUCCESS;
}

prnnStatus_t prnn_debug_skip_publish(prnnHandle_t h, int wg, int step) {
  if (h == nullptr) return PRNN_STATUS_BAD_PARAM;
  h->skip_wg = wg < 0 ? -1 : wg;
  h->skip_step = wg < 0 ? -1 : step;
  return PRNN_STATUS_SUCCESS;
}

prnnStatus_t prnn_debug_jitter(prnnHandle_t h, uint32_t seed, int span) {
  if (h == nullptr || span < 0 || span > PRNN_DEBUG_JITTER_MAX) return PRNN_STATUS_BAD_PARAM;
  h->jitter_seed = seed;
  h->jitter_span = static_cast<uint32_t>(span);
  return PRNN_STATUS_SUCCESS;
}

prnnStatus_t prnn_synchronize(prnnHandle_t h, hipStream_t stream) {
  if (h == nullptr) return PRNN_STATUS_BAD_PARAM;
  if (hipStreamSynchronize(stream) != hipSuccess) return PRNN_STATUS_INTERNAL_ERROR;
  return take_failure(h) ? PRNN_STATUS_EXECUTION_FAILED : PRNN_STATUS_SUCCESS;
}

prnnStatus_t prnn_forward_dense(prnnHandle_t h, int N, int B, int T, prnnDataType_t w_type, const void* W,
                                const float* X, const float* h0, float* H, hipStream_t stream) {
  if (h != nullptr && take_failure(h)) return PRNN_STATUS_EXECUTION_FAILED;
  Plan p;
  bool empty = false;
  prnnStatus_t st = prepare_dense(h, N, B, T, w_type, W, X, h0, H, &p, &empty);
  if (st != PRNN_STATUS_SUCCESS || empty) return st;
  return run_dense(h, p, N, B, T, W, X, h0, H, stream);
}

prnnStatus_t prnn_forward_sparse(prnnHandle_t h, int N, int B, int T, int K, const int16_t* col,
                                 prnnDataType_t val_type, const void* val, const float* X, const float* h0,
                                 float* H, hipStream_t stream) {
  if (h != nullptr && take_failure(h)) return PRNN_STATUS_EXECUTION_FAILED;
  Plan p;
  bool empty = false;
  prnnStatus_t st = prepare_sparse(h, N, B, T, K, col, val_type, val, X, h0, H, &p, &empty);
  if (st != PRNN_STATUS_SUCCESS || empty) return st;
  return run_sparse(h, p, N, B, T, K, col, val, X, h0, H, stream);
}

prnnStatus_t prnn_forward_sparse_rows(prnnHandle_t h, int N, int B, int T, int K, const int16_t* col,
                                      prnnDataType_t val_type, const void* val, const int32_t* row_len,
                                      const float* X, const float* h0, float* H, hipStream_t stream) {
  if (h != nullptr && take_failure(h)) return PRNN_STATUS_EXECUTION_FAILED;
  bool empty = false;
  prnnStatus_t st = check_common(h, N, B, T, X, h0, H, &empty);
  if (st != PRNN_STATUS_SUCCESS) return st;
  if (val_type != PRNN_DATA_FLOAT && val_type != PRNN_DATA_HALF) return PRNN_STATUS_BAD_PARAM;
  if (K < 1 || K > N || N > 32767) return PRNN_STATUS_BAD_PARAM;
  if (empty) return PRNN_STATUS_SUCCESS;
  if (col == nullptr || val == nullptr || row_len == nullptr) return PRNN_STATUS_BAD_PARAM;
  if (!aligned(col, 2) || !aligned(val, val_type == PRNN_DATA_FLOAT ? 4 : 2) || !aligned(row_len, 4))
    return PRNN_STATUS_BAD_PARAM;
  const size_t hb = (size_t)T * B * N * 4;
  if (overlap(col, (size_t)N * K * 2, H, hb) ||
      overlap(val, (size_t)N * K * (val_type == PRNN_DATA_FLOAT ? 4 : 2), H, hb) || overlap(row_len, (size_t)N * 4, H, hb))
    return PRNN_STATUS_BAD_PARAM;
  if (hb > 0xFFFFFFF0ull) return PRNN_STATUS_NOT_SUPPORTED;
  if (val_type != PRNN_DATA_HALF || K > prnn::kSparseRowsMaxK) return PRNN_STATUS_NOT_SUPPORTED;
  Plan p;
  if (!plan(h, kSparseRows, N, B, K, prnn::kF16, &p)) return PRNN_STATUS_NOT_SUPPORTED;
  return run_sparse_rows(h, p, N, B, T, K, col, val, row_len, X, h0, H, stream);
}

prnnStatus_t prnn_project(prnnHandle_t h, int M, int N, int I, prnnDataType_t x_type, const void* x,
                          prnnDataType_t u_type, const void* U, const float* bias, float* X, hipStream_t stream) {
  if (h != nullptr && take_failure(h)) return PRNN_STATUS_EXECUTION_FAILED;
  prnn::ProjArgs a;
  bool vec = false;
  prnnStatus_t st = prepare_project(h, M, N, I, x_type, x, u_type, U, bias, X, &a, &vec);
  if (st != PRNN_STATUS_SUCCESS || M == 0) return st;
  st = clear_reported_status(h, stream);
  if (st != PRNN_STATUS_SUCCESS) return st;
  return hip_status(prnn::launch_project(a, x_type == PRNN_DATA_FLOAT, vec, stream));
}

prnnStatus_t prnn_forward_layer_dense(prnnHandle_t h, int N, int I, int B, int T, prnnDataType_t x_type,
                                      const void* x, prnnDataType_t u_type, const void* U, const float* bias,
                                      prnnDataType_t w_type, const void* W, const float* h0, float* Xbuf, float* H,
                                      hipStream_t stream) {
  if (h != nullptr && take_failure(h)) return PRNN_STATUS_EXECUTION_FAILED;
  Plan p;
  bool empty = false;
  prnnStatus_t st = prepare_dense(h, N, B, T, w_type, W, Xbuf, h0, H, &p, &empty);
  if (st != PRNN_STATUS_SUCCESS || empty) return st;
  prnn::ProjArgs a;
  bool vec = false;
  st = prepare_layer_projection(h, N, I, B, T, x_type, x, u_type, U, bias, Xbuf, h0, W,
                                (size_t)N * N * (w_type == PRNN_DATA_FLOAT ? 4 : 2), nullptr, 0, &a, &vec);
  if (st != PRNN_STATUS_SUCCESS) return st;
  st = clear_reported_status(h, stream);
  if (st != PRNN_STATUS_SUCCESS) return st;
  st = hip_status(prnn::launch_project(a, x_type == PRNN_DATA_FLOAT, vec, stream));
  if (st != PRNN_STATUS_SUCCESS) return st;
  return run_dense(h, p, N, B, T, W, Xbuf, h0, H, stream);
}

prnnStatus_t prnn_forward_layer_sparse(prnnHandle_t h, int N, int I, int B, int T, int K, prnnDataType_t x_type,
                                       const void* x, prnnDataType_t u_type, const void* U, const float* bias,
                                       const int16_t* col, prnnDataType_t val_type, const void* val,
                                       const float* h0, float* Xbuf, float* H, hipStream_t stream) {
  if (h != nullptr && take_failure(h)) return PRNN_STATUS_EXECUTION_FAILED;
  Plan p;
  bool empty = false;
  prnnStatus_t st = prepare_sparse(h, N, B, T, K, col, val_type, val, Xbuf, h0, H, &p, &empty);
  if (st != PRNN_STATUS_SUCCESS || empty) return st;
  prnn::ProjArgs a;
  bool vec = false;
  st = prepare_layer_projection(h, N, I, B, T, x_type, x, u_type, U, bias, Xbuf, h0, col, (size_t)N * K * 2, val,
                                (size_t)N * K * (val_type == PRNN_DATA_FLOAT ? 4 : 2), &a, &vec);
  if (st != PRNN_STATUS_SUCCESS) return st;
  st = clear_reported_status(h, stream);
  if (st != PRNN_STATUS_SUCCESS) return st;
  st = hip_status(prnn::launch_project(a, x_type == PRNN_DATA_FLOAT, vec, stream));
  if (st != PRNN_STATUS_SUCCESS) return st;
  return run_sparse(h, p, N, B, T, K, col, val, Xbuf, h0, H, stream);
}

prnnStatus_t prnn_forward_stack_dense(prnnHandle_t h, int L, int N, int I, int B, int T, prnnDataType_t x_type,
                                      const void* x, const void* const* U, const float* const* bias,
                                      const void* const* W, const float* const* h0, float* Xbuf, float* const* H,
                                      hipStream_t stream) {
  if (h == nullptr || L < 1 || N < 1 || I < 1 || B < 1 || B > 8 || T < 0) return PRNN_STATUS_BAD_PARAM;
  if (take_failure(h)) return PRNN_STATUS_EXECUTION_FAILED;
  if (x_type != PRNN_DATA_FLOAT && x_type != PRNN_DATA_HALF) return PRNN_STATUS_BAD_PARAM;
  if (L > prnn::kMaxStack || L * B > 8) return PRNN_STATUS_NOT_SUPPORTED;
  if (T == 0) return PRNN_STATUS_SUCCESS;
  if (U == nullptr || W == nullptr || H == nullptr || x == nullptr || Xbuf == nullptr) return PRNN_STATUS_BAD_PARAM;
  const size_t seq = (size_t)T * B * N * 4;
  if (seq > 0xFFFFFFF0ull) return PRNN_STATUS_NOT_SUPPORTED;
  if (!aligned(Xbuf, 4)) return PRNN_STATUS_BAD_PARAM;
  for (int l = 0; l < L; ++l) {
    const float* hl = h0 != nullptr ? h0[l] : nullptr;
    const float* bl = bias != nullptr ? bias[l] : nullptr;
    if (U[l] == nullptr || W[l] == nullptr || H[l] == nullptr) return PRNN_STATUS_BAD_PARAM;
    if (!aligned(U[l], 16) || !aligned(W[l], 16) || !aligned(H[l], 16) || (hl != nullptr && !aligned(hl, 4)) ||
        (bl != nullptr && !aligned(bl, 4)))
      return PRNN_STATUS_BAD_PARAM;
    // H[l] is written while every weight, bias, h0, the workspace and the
    // other outputs are read: none of them may overlap it.
    if (overlap(H[l], seq, Xbuf, seq)) return PRNN_STATUS_BAD_PARAM;
    for (int m = 0; m < L; ++m) {
      const float* hm = h0 != nullptr ? h0[m] : nullptr;
      const float* bm = bias != nullptr ? bias[m] : nullptr;
      const size_t ub = (size_t)N * (m == 0 ? I : N) * 2;
      if ((m != l && overlap(H[l], seq, H[m], seq)) || overlap(H[l], seq, W[m], (size_t)N * N * 2) ||
          overlap(H[l], seq, U[m], ub) || (hm != nullptr && overlap(H[l], seq, hm, (size_t)B * N * 4)) ||
          (bm != nullptr && overlap(H[l], seq, bm, (size_t)N * 4)))
        return PRNN_STATUS_BAD_PARAM;
    }
  }
  // The workspace is written (layer 0's projection) before the weights, biases
  // and initial states are read.
  for (int m = 0; m < L; ++m) {
    const float* hm = h0 != nullptr ? h0[m] : nullptr;
    const float* bm = bias != nullptr ? bias[m] : nullptr;
    if (overlap(Xbuf, seq, W[m], (size_t)N * N * 2) || overlap(Xbuf, seq, U[m], (size_t)N * (m == 0 ? I : N) * 2) ||
        (hm != nullptr && overlap(Xbuf, seq, hm, (size_t)B * N * 4)) ||
        (bm != nullptr && overlap(Xbuf, seq, bm, (size_t)N * 4)))
      return PRNN_STATUS_BAD_PARAM;
  }
  // Plan: the team grid; each wave keeps its rows of [U_l | W_l].
  if (!h->placement_round_robin || h->num_cu < 8) return PRNN_STATUS_NOT_SUPPORTED;
  int P = h->forced_grid > 0 ? h->forced_grid / 8 : std::min(kTeamMaxWgPerXcd, h->num_cu / 8);
  if (h->forced_grid > 0 && h->forced_grid % 8 != 0) return PRNN_STATUS_NOT_SUPPORTED;
  P = std::min(P, (N + 7) / 8);
  if (P < 1 || 8 * P > h->num_cu) return PRNN_STATUS_NOT_SUPPORTED;
  Plan p;
  p.layout = PRNN_LAYOUT_TEAM;
  p.G = P;
  p.grid = 8 * P;
  p.waves = 8;
  p.block = 512;
  const int Q = 8 * P;
  p.base_rows = N / Q;
  p.extra_rows = N % Q;
  p.max_rows = (N + Q - 1) / Q;
  p.chunks = (N + 255) / 256;
  const prnn::KernelEntry* kb = pick(prnn::kStackBlockedKernels, p.max_rows, p.chunks);
  const prnn::KernelEntry* kf = pick(prnn::kStackFusedKernels, p.max_rows, p.chunks);
  const int lds_b = kb != nullptr ? 2 * 256 * kb->cap * 4 : 0;  // [2 steps][chunks x 256]
  const int lds_f = kf != nullptr ? 2 * 2 * 256 * kf->cap * 4 : 0;  // [2 steps][input, state][chunks x 256]
  if (kb != nullptr && (size_t)lds_b + 256 > h->lds_per_block) kb = nullptr;
  if (kf != nullptr && (size_t)lds_f + 256 > h->lds_per_block) kf = nullptr;
  int mode = h->stack_mode;
  if (mode == PRNN_STACK_AUTO) mode = kb != nullptr ? PRNN_STACK_BLOCKED : PRNN_STACK_LAYERS;
  if ((mode == PRNN_STACK_BLOCKED && kb == nullptr) || (mode == PRNN_STACK_FUSED && kf == nullptr))
    return PRNN_STATUS_NOT_SUPPORTED;
  if (mode == PRNN_STACK_LAYERS) {
    // The layers one after another, each a projection and a recurrence.
    // Every layer's recurrence must have a plan.
    Plan lp;
    if (!plan(h, kDense, N, B, 0, prnn::kF16, &lp)) return PRNN_STATUS_NOT_SUPPORTED;
    for (int l = 0; l < L; ++l) {
      prnnStatus_t st = prnn_forward_layer_dense(h, N, l == 0 ? I : N, B, T, l == 0 ? x_type : PRNN_DATA_FLOAT,
                                                 l == 0 ? x : H[l - 1], PRNN_DATA_HALF, U[l],
                                                 bias != nullptr ? bias[l] : nullptr, PRNN_DATA_HALF, W[l],
                                                 h0 != nullptr ? h0[l] : nullptr, Xbuf, H[l], stream);
      if (st != PRNN_STATUS_SUCCESS) return st;
    }
    return PRNN_STATUS_SUCCESS;
  }
  p.k = mode == PRNN_STACK_BLOCKED ? kb : kf;
  // Blocked launches compute their input products in the launch (in the LDS
  // the recurrence's rows use afterwards).
  p.lds_bytes = mode == PRNN_STACK_BLOCKED ? std::max(lds_b, prnn::kStackProjLds) : lds_f;
  if ((size_t)p.lds_bytes + 256 > h->lds_per_block) return PRNN_STATUS_NOT_SUPPORTED;
  // Layer 0's input projection (x, U[0], bias[0] and the workspace), checked
  // before anything is enqueued; the fused mode runs it into the workspace
  // first.
  prnn::ProjArgs pa;
  bool vec = false;
  prnnStatus_t st = prepare_layer_projection(h, N, I, B, T, x_type, x, PRNN_DATA_HALF, U[0],
                                             bias != nullptr ? bias[0] : nullptr, Xbuf,
                                             h0 != nullptr ? h0[0] : nullptr, W[0], (size_t)N * N * 2, nullptr, 0,
                                             &pa, &vec);
  if (st != PRNN_STATUS_SUCCESS) return st;
  const int Npad = (N + 3) & ~3;
  st = ensure_ring(h, p, B, Npad, stream);
  if (st != PRNN_STATUS_SUCCESS) return st;
  if (mode == PRNN_STACK_FUSED) {
    st = hip_status(prnn::launch_project(pa, x_type == PRNN_DATA_FLOAT, vec, stream));
    if (st != PRNN_STATUS_SUCCESS) return st;
  }

  prnn::StackArgs a;
  std::memset(&a, 0, sizeof(a));
  for (int l = 0; l < L; ++l) {
    a.W[l] = W[l];
    a.U[l] = U[l];
    a.bias[l] = bias != nullptr ? bias[l] : nullptr;
  }
  a.ring = h->d_ring;
  a.status = h->d_status;
  a.status_host = h->h_status_dev;
  a.L = L;
  a.N = N;
  a.B = B;
  a.Npad = Npad;
  a.chunks = p.chunks;
  a.base_rows = p.base_rows;
  a.extra_rows = p.extra_rows;
  a.deadline = static_cast<uint64_t>(h->watchdog_us) * 100ull;
  a.jitter_seed = h->jitter_seed;
  a.jitter_span = h->jitter_span;
  auto launch_stack = [&](int Tlaunch) -> prnnStatus_t {
    a.T = Tlaunch;
    a.step0 = static_cast<uint32_t>(h->step);
    a.x_bytes = static_cast<uint32_t>((size_t)Tlaunch * B * N * 4);
    void* args[] = {&a};
    hipError_t e = launch_persistent(h, p.k->fn, p.grid, p.block, args, p.lds_bytes, stream);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return hip_status(e);
    }
    h->step += static_cast<uint64_t>(Tlaunch);
    return PRNN_STATUS_SUCCESS;
  };

  if (mode == PRNN_STACK_FUSED) {
    for (int l = 0; l + 1 < L; ++l)  // "not written yet" marks for the layers that feed another
      prnn::launch_fill(reinterpret_cast<uint32_t*>(H[l]), (size_t)T * B * N, 0xFFFFFFFFu, stream);
    for (int l = 0; l < L; ++l) {
      a.h0[l] = h0 != nullptr ? h0[l] : nullptr;
      a.H[l] = H[l];
      a.Tl[l] = T;
    }
    a.X[0] = Xbuf;
    st = launch_stack(T);
  } else {
    // Blocks of about 64 steps; launch i runs layer l on block i - l.  The
    // launch first writes each layer's input product for its block (from x
    // for layer 0, from H[l - 1]'s block, finished by the launch before, for
    // the others) into that block of H[l]; the recurrence reads it there and
    // overwrites it with the outputs.  The workspace is not used.
    const int nb = std::max(1, (T + 32) / 64);
    const int tau = (T + nb - 1) / nb;
    const size_t blk = (size_t)tau * B * N;  // floats per full block
    const size_t xe = x_type == PRNN_DATA_FLOAT ? 4 : 2;
    for (int i = 0; i < nb + L - 1 && st == PRNN_STATUS_SUCCESS; ++i) {
      int Tlaunch = 0;
      for (int l = 0; l < L; ++l) {
        const int k = i - l;
        const int len = (k >= 0 && k < nb) ? std::min(tau, T - k * tau) : 0;
        a.Tl[l] = std::max(len, 0);
        a.P[l] = nullptr;
        if (a.Tl[l] == 0) continue;
        Tlaunch = std::max(Tlaunch, a.Tl[l]);
        a.H[l] = H[l] + (size_t)k * blk;
        a.X[l] = a.H[l];
        a.h0[l] = k == 0 ? (h0 != nullptr ? h0[l] : nullptr) : H[l] + (size_t)k * blk - (size_t)B * N;
        if (l == 0) {
          a.P[0] = static_cast<const char*>(x) + (size_t)k * tau * B * I * xe;
          a.p_cols[0] = I;
          a.p_f32[0] = x_type == PRNN_DATA_FLOAT ? 1 : 0;
          a.p_vec[0] = vec ? 1 : 0;  // I % 8 == 0, x and U[0] 16-byte aligned: so is every block
        } else {
          a.P[l] = H[l - 1] + (size_t)k * blk;
          a.p_cols[l] = N;
          a.p_f32[l] = 1;
          a.p_vec[l] = N % 8 == 0 ? 1 : 0;  // H[l - 1] and U[l] are 16-byte aligned
        }
      }
      if (Tlaunch > 0) st = launch_stack(Tlaunch);
    }
  }
  if (st != PRNN_STATUS_SUCCESS) return st;
  prnnPlanInfo_t& info = h->last_plan;
  info.layout = p.layout;
  info.grid = p.grid;
  info.waves_per_wg = p.waves;
  info.rows_per_wave = p.max_rows;
  info.rmax = p.k->rmax;
  info.chunks = p.k->cap;
  info.lds_bytes = p.lds_bytes;
  info.relay_slice = 0;
  info.math = PRNN_MATH_EXACT;
  info.first_step = h->step;
  log_plan(h, "stack", N, B, T, info);
  h->have_plan = true;
  h->trace_records = 0;
  return PRNN_STATUS_SUCCESS;
}

prnnStatus_t prnn_forward_stack_sparse(prnnHandle_t h, int L, int N, int I, int B, int T, int K, prnnDataType_t x_type,
                                       const void* x, const void* const* U, const float* const* bias,
                                       const int16_t* const* col, prnnDataType_t val_type, const void* const* val,
                                       const float* const* h0, float* Xbuf, float* const* H, hipStream_t stream) {
  if (h == nullptr || L < 1 || N < 1 || I < 1 || B < 1 || B > 8 || T < 0) return PRNN_STATUS_BAD_PARAM;
  if (take_failure(h)) return PRNN_STATUS_EXECUTION_FAILED;
  if (x_type != PRNN_DATA_FLOAT && x_type != PRNN_DATA_HALF) return PRNN_STATUS_BAD_PARAM;
  if (val_type != PRNN_DATA_FLOAT && val_type != PRNN_DATA_HALF) return PRNN_STATUS_BAD_PARAM;
  if (K < 1 || K > N || N > 32767) return PRNN_STATUS_BAD_PARAM;
  if (T == 0) return PRNN_STATUS_SUCCESS;
  if (U == nullptr || col == nullptr || val == nullptr || H == nullptr || x == nullptr || Xbuf == nullptr)
    return PRNN_STATUS_BAD_PARAM;
  const size_t seq = (size_t)T * B * N * 4;
  if (seq > 0xFFFFFFF0ull) return PRNN_STATUS_NOT_SUPPORTED;
  if (!aligned(Xbuf, 4)) return PRNN_STATUS_BAD_PARAM;
  const size_t vb = (size_t)N * K * (val_type == PRNN_DATA_FLOAT ? 4 : 2), cb = (size_t)N * K * 2;
  // Every pointer and overlap is checked before anything is enqueued: H[l]
  // is written while every layer's weights, biases and initial states, the
  // workspace and the other outputs are read; the workspace is written
  // before all of those are read.
  for (int l = 0; l < L; ++l) {
    const float* hl = h0 != nullptr ? h0[l] : nullptr;
    const float* bl = bias != nullptr ? bias[l] : nullptr;
    if (U[l] == nullptr || col[l] == nullptr || val[l] == nullptr || H[l] == nullptr) return PRNN_STATUS_BAD_PARAM;
    if (!aligned(U[l], 2) || !aligned(col[l], 2) || !aligned(val[l], val_type == PRNN_DATA_FLOAT ? 4 : 2) ||
        !aligned(H[l], 4) || (hl != nullptr && !aligned(hl, 4)) || (bl != nullptr && !aligned(bl, 4)))
      return PRNN_STATUS_BAD_PARAM;
    if (overlap(H[l], seq, Xbuf, seq)) return PRNN_STATUS_BAD_PARAM;
    for (int m = 0; m < L; ++m) {
      const float* hm = h0 != nullptr ? h0[m] : nullptr;
      const float* bm = bias != nullptr ? bias[m] : nullptr;
      const size_t ub = (size_t)N * (m == 0 ? I : N) * 2;
      if ((m != l && overlap(H[l], seq, H[m], seq)) || overlap(H[l], seq, col[m], cb) || overlap(H[l], seq, val[m], vb) ||
          overlap(H[l], seq, U[m], ub) || (hm != nullptr && overlap(H[l], seq, hm, (size_t)B * N * 4)) ||
          (bm != nullptr && overlap(H[l], seq, bm, (size_t)N * 4)))
        return PRNN_STATUS_BAD_PARAM;
    }
  }
  for (int m = 0; m < L; ++m) {
    const float* hm = h0 != nullptr ? h0[m] : nullptr;
    const float* bm = bias != nullptr ? bias[m] : nullptr;
    if (overlap(Xbuf, seq, col[m], cb) || overlap(Xbuf, seq, val[m], vb) ||
        overlap(Xbuf, seq, U[m], (size_t)N * (m == 0 ? I : N) * 2) ||
        (hm != nullptr && overlap(Xbuf, seq, hm, (size_t)B * N * 4)) || (bm != nullptr && overlap(Xbuf, seq, bm, (size_t)N * 4)))
      return PRNN_STATUS_BAD_PARAM;
  }
  // Every layer's recurrence and layer 0's projection must have a plan.
  Plan lp;
  if (!plan(h, kSparse, N, B, K, val_type == PRNN_DATA_FLOAT ? prnn::kF32 : prnn::kF16, &lp))
    return PRNN_STATUS_NOT_SUPPORTED;
  prnn::ProjArgs pa;
  bool vec = false;
  prnnStatus_t st = prepare_layer_projection(h, N, I, B, T, x_type, x, PRNN_DATA_HALF, U[0],
                                             bias != nullptr ? bias[0] : nullptr, Xbuf,
                                             h0 != nullptr ? h0[0] : nullptr, col[0], cb, val[0], vb, &pa, &vec);
  if (st != PRNN_STATUS_SUCCESS) return st;
  // One layer after another (the sparse layers keep their pairs in registers
  // in the team layout; the layers do not run as a wavefront).
  for (int l = 0; l < L; ++l) {
    st = prnn_forward_layer_sparse(h, N, l == 0 ? I : N, B, T, K, l == 0 ? x_type : PRNN_DATA_FLOAT,
                                   l == 0 ? x : H[l - 1], PRNN_DATA_HALF, U[l], bias != nullptr ? bias[l] : nullptr,
                                   col[l], val_type, val[l], h0 != nullptr ? h0[l] : nullptr, Xbuf, H[l], stream);
    if (st != PRNN_STATUS_SUCCESS) return st;
  }
  return PRNN_STATUS_SUCCESS;
}

prnnStatus_t prnn_set_launch(prnnHandle_t h, prnnLaunch_t kind) {
  if (h == nullptr || (kind != PRNN_LAUNCH_COOPERATIVE && kind != PRNN_LAUNCH_PLAIN)) return PRNN_STATUS_BAD_PARAM;
  h->launch_kind = kind;
  h->placement_round_robin = kind == PRNN_LAUNCH_PLAIN ? h->plain_placement : h->coop_placement;
  return PRNN_STATUS_SUCCESS;
}

prnnStatus_t prnn_set_stack_mode(prnnHandle_t h, prnnStackMode_t mode) {
  if (h == nullptr) return PRNN_STATUS_BAD_PARAM;
  if (mode != PRNN_STACK_AUTO && mode != PRNN_STACK_BLOCKED && mode != PRNN_STACK_FUSED && mode != PRNN_STACK_LAYERS)
    return PRNN_STATUS_BAD_PARAM;
  h->stack_mode = mode;
  return PRNN_STATUS_SUCCESS;
}

prnnStatus_t prnn_sync_floor(prnnHandle_t h, int N, int B, int T, float* H, hipStream_t stream) {
  if (h == nullptr || N < 1 || B < 1 || B > 8 || T < 0) return PRNN_STATUS_BAD_PARAM;
  if (take_failure(h)) return PRNN_STATUS_EXECUTION_FAILED;
  if (T == 0) return PRNN_STATUS_SUCCESS;
  if (H == nullptr || !aligned(H, 4)) return PRNN_STATUS_BAD_PARAM;
  if ((size_t)T * B * N * 4 > 0xFFFFFFF0ull) return PRNN_STATUS_NOT_SUPPORTED;
  Plan p;
  if (!plan(h, kFloor, N, B, 0, prnn::kF16, &p)) return PRNN_STATUS_NOT_SUPPORTED;
  static KernelEntry floor_team = {0, 64, 1 << 30, nullptr};
  static KernelEntry floor_team_trace = {0, 64, 1 << 30, nullptr};
  static KernelEntry floor_team16 = {0, 64, 1 << 30, nullptr, 16};
  static KernelEntry floor_team16_trace = {0, 64, 1 << 30, nullptr, 16};
  static KernelEntry floor_team12 = {0, 64, 1 << 30, nullptr, 12};
  static KernelEntry floor_team12_trace = {0, 64, 1 << 30, nullptr, 12};
  p.what = "floor";
  if (p.layout == PRNN_LAYOUT_TEAM) {
    floor_team.fn = prnn::kFloorTeamKernel;
    floor_team_trace.fn = prnn::kFloorTeamTraceKernel;
    floor_team16.fn = prnn::kFloorTeamKernel16;
    floor_team16_trace.fn = prnn::kFloorTeamTraceKernel16;
    floor_team12.fn = prnn::kFloorTeamKernel12;
    floor_team12_trace.fn = prnn::kFloorTeamTraceKernel12;
    static KernelEntry floor_split = {0, 64, 1 << 30, nullptr};
    static KernelEntry floor_split12 = {0, 64, 1 << 30, nullptr, 12};
    floor_split.fn = prnn::kFloorSplitKernel;
    floor_split12.fn = prnn::kFloorSplitKernel12;
    if (p.xcds_per_row > 1)
      p.k = p.waves == 12 ? &floor_split12 : &floor_split;  // no trace instance: a traced split layer is not planned either
    else if (p.waves == 16)
      p.k = h->trace ? &floor_team16_trace : &floor_team16;
    else if (p.waves == 12)
      p.k = h->trace ? &floor_team12_trace : &floor_team12;
    else
      p.k = h->trace ? &floor_team_trace : &floor_team;
  }
  const int Npad = (N + 3) & ~3;
  prnnStatus_t st = ensure_ring(h, p, B, Npad, stream);
  if (st != PRNN_STATUS_SUCCESS) return st;
  StepArgs a = base_args(h, N, B, T, nullptr, nullptr, H, p, Npad);
  return launch(h, p, a, T, stream);
}

}  // extern "C"
