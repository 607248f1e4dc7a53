// fp32 instances of the team-layout kernels (rows per wave, chunks / pair slots).
#include "team_kernel.h"

namespace prnn {

const KernelEntry kDenseTeamF32Kernels[] = {
    // (rows per wave, 256-column chunks)
    PRNN_DENSE_TEAM(float, kF32, 1, 1), PRNN_DENSE_TEAM(float, kF32, 2, 1), PRNN_DENSE_TEAM(float, kF32, 4, 1),
    PRNN_DENSE_TEAM(float, kF32, 7, 1), PRNN_DENSE_TEAM(float, kF32, 8, 1), PRNN_DENSE_TEAM(float, kF32, 2, 2),
    PRNN_DENSE_TEAM(float, kF32, 4, 2), PRNN_DENSE_TEAM(float, kF32, 8, 2), PRNN_DENSE_TEAM(float, kF32, 4, 4),
    PRNN_DENSE_TEAM(float, kF32, 5, 5), PRNN_DENSE_TEAM(float, kF32, 4, 7), PRNN_DENSE_TEAM(float, kF32, 7, 7),
    {0, 0, 0, nullptr},
};

const KernelEntry kSparseTeamF32Kernels[] = {
    // (rows per wave, 64-pair slots per row)
    PRNN_SPARSE_TEAM(float, kF32, 1, 1), PRNN_SPARSE_TEAM(float, kF32, 2, 1), PRNN_SPARSE_TEAM(float, kF32, 4, 1),
    PRNN_SPARSE_TEAM(float, kF32, 8, 1), PRNN_SPARSE_TEAM(float, kF32, 2, 2), PRNN_SPARSE_TEAM(float, kF32, 4, 2),
    PRNN_SPARSE_TEAM(float, kF32, 8, 2), PRNN_SPARSE_TEAM(float, kF32, 16, 1),
    {0, 0, 0, nullptr},
};

// The team layout's exchange and step protocol without weights or arithmetic
// (WAVES = waves per workgroup, as the layer it is the floor of).
template <bool TRACE, int WAVES = kTeamWaves>
__global__ void __launch_bounds__(64 * WAVES) floor_team_kernel(StepArgs a) {
  extern __shared__ __attribute__((aligned(16))) float lds[];  // float4-staged rows
  __shared__ int abort_flag;
  const TeamPos p = team_pos<WAVES>(a);
  if (threadIdx.x == 0) abort_flag = __builtin_nontemporal_load(a.status) != 0u;
  __syncthreads();
  if (abort_flag) return;
  const int N = a.N;
  const __amdgpu_buffer_rsrc_t region = team_region(a);
  if (!p.primary) {
    team_stamp_tail(a, p, region);
    return;
  }
  PhaseClock<TRACE> clk;
  clk.start();
  for (int t = 0; t < a.T; ++t) {
    const uint32_t S = a.step0 + (uint32_t)t;
    float* hrow = lds + (t & 1) * a.Npad;
    bool ok = true;
    if (t > 0) {
      const uint32_t prev = S - 1u;
      uint32_t unused = 0;
      ok = team_stage<WAVES>(region, prev & 1u, a.Npad, N, a.chunks, p.wave, p.lane, tag_bit(prev), a.deadline, hrow,
                             unused);
    }
    if (!ok && p.lane == 0) {
      abort_flag = 1;
      report_failure(a.status, a.status_host, kStatusTimeout);
    }
    clk.mark(kTrStage);
    __syncthreads();
    clk.mark(kTrBarrier);
    int aborted_now = abort_flag;  // read with the row and tested before the stores, as in the kernels
    const float seen = t > 0 ? hrow[p.lane] : 0.f;
    clk.mark(kTrCompute);
    asm volatile("" : "+v"(aborted_now) : "v"(seen));
    if (aborted_now) return;
    if (p.lane < p.nr) {
      const uint32_t hb = relu_bits((float)(t + 1) + seen * 0.f);
      const int row = p.r0 + p.lane;
      __builtin_amdgcn_raw_buffer_store_b32(hb | tag_bit(S), region, ((S & 1u) * a.Npad + row) * 4u, 0, kPlain);
      a.H[((size_t)t * a.B + p.b) * N + row] = __uint_as_float(hb);
    }
    clk.mark(kTrEpilogue);
  }
  if (TRACE) clk.finish(trace_record<WAVES>(a, p), a.T);
}

// Resets the team ring: every XCD fills its own region (so its L2 never holds
// an older copy of it).  Launched with a multiple of 8 workgroups.
__global__ void team_fill_kernel(uint32_t* ring, int npad, uint32_t v) {
  const uint32_t xcc = __builtin_amdgcn_s_getreg((20) | (31 << 11)) & 7u;  // HW_REG_XCC_ID
  uint32_t* region = ring + (size_t)xcc * 2 * npad;
  const int per_xcd = gridDim.x / 8;
  for (int i = (blockIdx.x >> 3) * blockDim.x + threadIdx.x; i < 2 * npad; i += per_xcd * blockDim.x)
    region[i] = v;
}

const void* kFloorTeamKernel = reinterpret_cast<const void*>(&floor_team_kernel<false>);
const void* kFloorTeamTraceKernel = reinterpret_cast<const void*>(&floor_team_kernel<true>);
const void* kFloorTeamKernel16 = reinterpret_cast<const void*>(&floor_team_kernel<false, 16>);
const void* kFloorTeamKernel12 = reinterpret_cast<const void*>(&floor_team_kernel<false, 12>);
const void* kFloorTeamTraceKernel12 = reinterpret_cast<const void*>(&floor_team_kernel<true, 12>);
const void* kFloorTeamTraceKernel16 = reinterpret_cast<const void*>(&floor_team_kernel<true, 16>);

// Trace instances (the N = 256 fp32 layer).
const KernelEntry kDenseTeamF32TraceKernels[] = {
    PRNN_DENSE_TEAM_TRACE(float, kF32, 1, 1),
    {0, 0, 0, nullptr},
};
const KernelEntry kSparseTeamF32TraceKernels[] = {
    {0, 0, 0, nullptr},
};

void launch_team_fill(uint32_t* ring, int npad, uint32_t v, hipStream_t stream) {
  hipLaunchKernelGGL(team_fill_kernel, dim3(64), dim3(256), 0, stream, ring, npad, v);
}

}  // namespace prnn
