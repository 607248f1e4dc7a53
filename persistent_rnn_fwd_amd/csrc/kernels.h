// Kernel arguments and launch tables shared by the host library and the
// kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace prnn {

// Arguments of every persistent launch (passed by value).
struct StepArgs {
  const void* W;        // dense: W [N][N]; sparse: col int16 [N][K]
  const void* V;        // sparse: val [N][K]; dense: unused
  const float* X;       // [T][B][N]
  const float* h0;      // [B][N] or nullptr (zeros)
  float* H;             // [T][B][N]
  uint32_t* ring;       // spread layout: [2][B][Npad] tagged words; team layout: [8][2][Npad]
  uint32_t* relay;      // [8][2][B][Npad]: one copy of the ring per XCD (relay mode)
  uint32_t* status;     // device status word (0 = ok)
  uint32_t* status_host;  // host-visible mirror of failures (pinned host memory), or nullptr
  int N, B, T, K, Npad;
  int lds_stride;       // sparse: words per LDS row of h, multiple of 4, >= N + 1
  int G;                // workgroups per batch group
  int base_rows;        // rows per workgroup (team layout: per wave): base_rows, +1 for the first extra_rows
  int extra_rows;
  int chunks;           // 256-column chunks of a row: ceil(N / 256)
  int spr;              // sparse: 64-pair slots per row, ceil(K / 64)
  int relay_slice;      // words of a row each workgroup relays (0 = direct mode)
  int w_vec;            // dense: W is 16-byte aligned, so rows of N % 4 == 0 (MFMA: N % 8 == 0) load as vectors
  int xcds_per_row;     // split team layout: XCDs per batch row (2 or 4; 0 otherwise)
  const int32_t* row_len;  // sparse rows of unequal length: pairs of each row ([N], clamped to [0, K])
  const int32_t* sorted;   // ... and the rows by slot count, most first ([N], sort_rows_kernel)
  int part_rows;        // split team layout: rows per part, a multiple of 256
  uint32_t step0;       // ring step counter at t = 0
  uint32_t ring_bytes;
  uint32_t x_bytes;     // bytes of X (= bytes of H)
  uint64_t deadline;    // bound on one wait, in ticks of the 100 MHz clock
  int skip_wg, skip_step;  // test-only publish skip (skip_wg < 0: off)
  uint32_t jitter_seed, jitter_span;  // test-only publish delay (span 0: off)
  uint64_t* trace;      // trace instances: kTraceWords per wave, [grid][8 waves][kTraceWords]
};

// Per-wave phase record written by the trace instances of the team kernels:
// shader-clock cycles spent in staging (poll + LDS write), at the workgroup
// barrier, in the LDS reads and multiply-adds, in the cross-lane reduction
// and in the epilogue, then the whole time loop in cycles and in ticks of the
// 100 MHz clock, and the number of steps.
constexpr int kTraceWords = 8;
enum TraceWord { kTrStage = 0, kTrBarrier, kTrCompute, kTrReduce, kTrEpilogue, kTrLoopCycles, kTrLoopTicks, kTrSteps };

enum WType { kF32 = 0, kF16 = 1 };

struct KernelEntry {
  int wtype;   // WType
  int rmax;    // compiled row capacity per workgroup
  int cap;     // dense: compiled chunk capacity J; sparse: slots per row SPR
  const void* fn;
  int waves = 8;  // team layout: waves per workgroup the instance is compiled for
};

// Instance tables (each terminated by fn == nullptr).
extern const KernelEntry kDenseF16Kernels[];
extern const KernelEntry kDenseF32Kernels[];
extern const KernelEntry kSparseF16Kernels[];
extern const KernelEntry kSparseF32Kernels[];
extern const KernelEntry kFloorKernels[];   // wtype unused, rmax = 64 rows max
extern const KernelEntry kDenseTeamF16Kernels[];   // team layout: rmax = rows per wave
extern const KernelEntry kDenseTeamF32Kernels[];
extern const KernelEntry kSparseTeamF16Kernels[];
extern const KernelEntry kSparseTeamF32Kernels[];
// Team layout with 16-wave workgroups (4 waves per SIMD), for sparse fp16
// layers whose rows would exceed 16 per wave at 8 waves per workgroup.
extern const KernelEntry kSparseTeamF16Kernels16[];
extern const KernelEntry kSparseTeamF16Kernels12[];   // 12-wave workgroups (3 waves per SIMD)
extern const KernelEntry kSparseTeamF16TraceKernels16[];
// Words between the two LDS rows of h in the sparse team kernels: at least
// N + 1 for every layer an instance of rw rows per wave and `waves` waves per
// workgroup serves (N <= rw x 32 waves per team), a multiple of 4.
constexpr int sparse_team_stride(int rw, int waves) { return rw * 32 * waves + 4; }
// Sparse fp16 rows of unequal length (team layout; 8- and 12-wave workgroups;
// and on two XCDs per batch row, team_split.hip).
extern const KernelEntry kSparseRowsF16Kernels[];
extern const KernelEntry kSparseRowsF16Kernels12[];
extern const KernelEntry kSparseRowsSplitF16Kernels[];
constexpr int kSparseRowsMaxK = 1024;  // longest row: 16 slots of 64 pairs
// Orders the rows of a sparse layer of unequal rows by slot count (most
// first; equal counts in row order) into sorted[N], each segment of `seg`
// rows on its own (seg = n: the whole layer; the part size on two XCDs per
// batch row).  One workgroup per segment.
void launch_sort_rows(const int32_t* row_len, int n, int k, int seg, int32_t* sorted, hipStream_t stream);

// Fills n words with v (grid-stride).
void launch_fill(uint32_t* p, size_t n, uint32_t v, hipStream_t stream);

// One workgroup per entry: out[i] = the XCD (XCC_ID) that ran workgroup i.
extern const void* kPlacementKernel;

// Team layout: the protocol-only kernel, and the ring reset in which every XCD
// fills its own [2][npad] region of the [8][2][npad] ring.
extern const void* kFloorTeamKernel;
// Dense fp16 team layout on the matrix cores (rmax = rows per workgroup,
// cap = 8 chunks of 256 columns, one per wave).
extern const KernelEntry kDenseTeamMfmaKernels[];
extern const KernelEntry kDenseTeamMfmaTraceKernels[];
// Dense fp16 layers split over 2 or 4 XCDs per batch row (team_split.hip):
// rmax = rows per wave, cap = 256-column chunks of the row.  The ring is the
// team ring [8][2][Npad] followed by a shared ring [8][2][Npad].
extern const KernelEntry kDenseSplitF16Kernels[];
extern const void* kFloorSplitKernel;    // the split layout's floor (rows per wave <= 64)
extern const void* kFloorSplitKernel12;  // ... with 12-wave workgroups
// Sparse fp16 layers on 2 XCDs per batch row: rmax = rows per wave, cap =
// 64-pair slots, waves = waves per workgroup (8 or 12).
extern const KernelEntry kSparseSplitF16Kernels[];
// Dense fp16 team layout with h_{t-1} rounded to fp16 (rmax = rows per wave,
// cap = 256-column chunks).
extern const KernelEntry kDenseTeamHalfKernels[];
extern const KernelEntry kDenseTeamHalfTraceKernels[];
// Trace instances (team layout only): the same kernels with phase timing.
extern const KernelEntry kDenseTeamF16TraceKernels[];
extern const KernelEntry kDenseTeamF32TraceKernels[];
extern const KernelEntry kSparseTeamF16TraceKernels[];
extern const KernelEntry kSparseTeamF32TraceKernels[];
extern const void* kFloorTeamTraceKernel;
extern const void* kFloorTeamKernel16;       // the floor with 16-wave workgroups
extern const void* kFloorTeamTraceKernel16;
extern const void* kFloorTeamKernel12;       // ... and with 12-wave workgroups
extern const void* kFloorTeamTraceKernel12;
void launch_team_fill(uint32_t* ring, int npad, uint32_t v, hipStream_t stream);

// A stack of dense fp16 layers as one wavefront (stack.hip).  Team x serves
// layer x / B, batch row x % B (L B <= 8); the team regions are the team
// layout's ring.
constexpr int kMaxStack = 8;
struct StackArgs {
  const void* W[kMaxStack];      // fp16 [N][N] recurrent weights
  const void* U[kMaxStack];      // fp16 [N][p_cols] input weights (fused: layers >= 1 only)
  const float* bias[kMaxStack];  // [N] or nullptr (fused: layers >= 1; layer 0's is in X0)
  const float* h0[kMaxStack];    // [B][N] or nullptr (zeros)
  float* H[kMaxStack];           // [Tl][B][N] outputs (fused: H[0 .. L-2] filled with 0xFFFFFFFF first)
  const float* X[kMaxStack];     // [Tl][B][N] pre-activations (fused: layer 0 only; may alias H[l])
  int Tl[kMaxStack];             // steps of layer l in this launch (<= T; 0: idle)
  // Blocked mode: layer l's input for this launch's block ([Tl][B][p_cols],
  // fp32 or fp16), whose product with U[l] plus bias[l] the launch writes
  // into H[l] before the recurrence reads it there; nullptr: X[l] already
  // holds the pre-activations.
  const void* P[kMaxStack];
  int p_cols[kMaxStack];         // I for layer 0, N above
  int p_f32[kMaxStack];          // 1: fp32 input (split into two fp16 terms), 0: fp16
  int p_vec[kMaxStack];          // 1: 16-byte loads (p_cols % 8 == 0, P and U 16-byte aligned)
  uint32_t* ring;                // [8][2][Npad]
  uint32_t* status;
  uint32_t* status_host;         // host-visible mirror of failures, or nullptr
  int L, N, B, T, Npad, chunks, base_rows, extra_rows;
  uint32_t step0;
  uint32_t x_bytes;              // bytes of one [T][B][N] sequence (T = the launch's steps)
  uint64_t deadline;
  uint32_t jitter_seed, jitter_span;  // test-only publish delay (span 0: off)
};
// (rmax = rows per wave, cap = chunks of each part)
// Dynamic LDS a blocked launch needs for its in-launch input product (the
// 64 x 64 tiles' staging; the recurrence's rows reuse it afterwards).
constexpr int kStackProjLds = 73728;
extern const KernelEntry kStackFusedKernels[];
extern const KernelEntry kStackBlockedKernels[];

// Input projection X[m][n] = bias[n] + sum_i U[n][i] x[m][i] (project.hip).
struct ProjArgs {
  const void* x;      // [M][I], fp32 or fp16
  const void* U;      // [N][I] fp16
  const float* bias;  // [N] or nullptr
  float* X;           // [M][N]
  uint32_t* status;   // kStatusRange if an fp32 x exceeds the fp16 range of its split
  uint32_t* status_host;  // host-visible mirror of failures, or nullptr
  int M, N, I;
  uint32_t x_bytes, u_bytes;
  int tiles_n;        // column tiles of X (set by launch_project)
  int tiles;          // all tiles
  int per_xcd;        // workgroups per XCD (grid = 8 per_xcd workgroups)
  int xcd_rows;       // the 8 XCDs as an xcd_rows x (8 / xcd_rows) grid over the tiles
  int xcd_tile_rows;  // tile rows per XCD row of that grid
  int xcd_tile_cols;  // tile columns per XCD column of that grid
};
// vec: I % 8 == 0 and x, U 16-byte aligned.
hipError_t launch_project(const ProjArgs& a, bool x_f32, bool vec, hipStream_t stream);

}  // namespace prnn
