// fp32-weight instances of the dense persistent kernel, the sync-floor
// kernel and the fill kernel.
#include "dense_kernel.h"

namespace prnn {

const KernelEntry kDenseF32Kernels[] = {
    // (rows, chunks); weights take rows * chunks * 4 VGPRs
    PRNN_DENSE(float, kF32, 1, 1), PRNN_DENSE(float, kF32, 1, 2), PRNN_DENSE(float, kF32, 1, 4),
    PRNN_DENSE(float, kF32, 1, 8), PRNN_DENSE(float, kF32, 1, 12), PRNN_DENSE(float, kF32, 1, 16),
    PRNN_DENSE(float, kF32, 2, 1), PRNN_DENSE(float, kF32, 2, 2), PRNN_DENSE(float, kF32, 2, 4),
    PRNN_DENSE(float, kF32, 2, 8), PRNN_DENSE(float, kF32, 2, 12), PRNN_DENSE(float, kF32, 2, 16),
    PRNN_DENSE(float, kF32, 4, 1), PRNN_DENSE(float, kF32, 4, 2), PRNN_DENSE(float, kF32, 4, 4),
    PRNN_DENSE(float, kF32, 4, 8), PRNN_DENSE(float, kF32, 8, 1), PRNN_DENSE(float, kF32, 8, 2),
    PRNN_DENSE(float, kF32, 8, 4), PRNN_DENSE(float, kF32, 16, 1), PRNN_DENSE(float, kF32, 16, 2),
    PRNN_DENSE(float, kF32, 32, 1),
    {0, 0, 0, nullptr},
};

const KernelEntry kFloorKernels[] = {
    PRNN_FLOOR(1), PRNN_FLOOR(2), PRNN_FLOOR(4), PRNN_FLOOR(8), PRNN_FLOOR(12), PRNN_FLOOR(16), PRNN_FLOOR(24),
    {0, 0, 0, nullptr},
};

__global__ void fill_kernel(uint32_t* p, size_t n, uint32_t v) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = v;
}

__global__ void placement_kernel(uint32_t* out) {
  if (threadIdx.x == 0) out[blockIdx.x] = __builtin_amdgcn_s_getreg((20) | (31 << 11)) & 0xFu;  // HW_REG_XCC_ID
}

const void* kPlacementKernel = reinterpret_cast<const void*>(&placement_kernel);

void launch_fill(uint32_t* p, size_t n, uint32_t v, hipStream_t stream) {
  if (n == 0) return;
  size_t blocks = (n + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(fill_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, n, v);
}

}  // namespace prnn
