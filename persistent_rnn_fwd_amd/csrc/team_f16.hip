// fp16 instances of the team-layout kernels (rows per wave, chunks / pair slots).
#include "team_kernel.h"
#include "team_mfma.h"

namespace prnn {

const KernelEntry kDenseTeamF16Kernels[] = {
    // (rows per wave, 256-column chunks).  Widened fp16 (fp32 registers, 4 per
    // weight quad) where rows * chunks <= 50; 8 x 8 and 9 x 9 with 4 rows and
    // 1 row widened (what 196 weight registers hold); packed fp16 elsewhere.
    PRNN_DENSE_TEAM_WIDE(1, 1), PRNN_DENSE_TEAM_WIDE(2, 1), PRNN_DENSE_TEAM_WIDE(4, 1),
    PRNN_DENSE_TEAM_WIDE(8, 1), PRNN_DENSE_TEAM_WIDE(1, 2), PRNN_DENSE_TEAM_WIDE(2, 2),
    PRNN_DENSE_TEAM_WIDE(4, 2), PRNN_DENSE_TEAM_WIDE(8, 2), PRNN_DENSE_TEAM_WIDE(2, 4),
    PRNN_DENSE_TEAM_WIDE(4, 4), PRNN_DENSE_TEAM_WIDE(8, 4), PRNN_DENSE_TEAM_WIDE(4, 5),
    PRNN_DENSE_TEAM_WIDE(5, 5), PRNN_DENSE_TEAM_WIDE(6, 5), PRNN_DENSE_TEAM_WIDE(7, 7),
    PRNN_DENSE_TEAM(_Float16, kF16, 8, 5), PRNN_DENSE_TEAM(_Float16, kF16, 8, 7), PRNN_DENSE_TEAM(_Float16, kF16, 6, 8),
    PRNN_DENSE_TEAM_WIDE(8, 8), PRNN_DENSE_TEAM_WIDE(9, 9), PRNN_DENSE_TEAM(_Float16, kF16, 10, 10),
    {0, 0, 0, nullptr},
};

const KernelEntry kSparseTeamF16Kernels[] = {
    // (rows per wave, 64-pair slots per row)
    PRNN_SPARSE_TEAM(_Float16, kF16, 1, 1), PRNN_SPARSE_TEAM(_Float16, kF16, 2, 1), PRNN_SPARSE_TEAM(_Float16, kF16, 4, 1),
    PRNN_SPARSE_TEAM(_Float16, kF16, 8, 1), PRNN_SPARSE_TEAM(_Float16, kF16, 1, 2), PRNN_SPARSE_TEAM(_Float16, kF16, 2, 2),
    PRNN_SPARSE_TEAM(_Float16, kF16, 4, 2), PRNN_SPARSE_TEAM(_Float16, kF16, 8, 2), PRNN_SPARSE_TEAM(_Float16, kF16, 4, 3),
    PRNN_SPARSE_TEAM(_Float16, kF16, 5, 2), PRNN_SPARSE_TEAM(_Float16, kF16, 7, 1), PRNN_SPARSE_TEAM(_Float16, kF16, 7, 3),
    PRNN_SPARSE_TEAM(_Float16, kF16, 8, 3), PRNN_SPARSE_TEAM(_Float16, kF16, 16, 1), PRNN_SPARSE_TEAM(_Float16, kF16, 23, 1),
    PRNN_SPARSE_TEAM(_Float16, kF16, 24, 1), PRNN_SPARSE_TEAM(_Float16, kF16, 32, 1),
    // 2304-neuron layers at 10 % / 25 % (padded unbalanced rows up to 1024 pairs); 5760 at 5 %
    PRNN_SPARSE_TEAM(_Float16, kF16, 9, 4), PRNN_SPARSE_TEAM(_Float16, kF16, 9, 9), PRNN_SPARSE_TEAM(_Float16, kF16, 9, 10),
    PRNN_SPARSE_TEAM(_Float16, kF16, 23, 5),
    {0, 0, 0, nullptr},
};

// 16-wave workgroups (at most 128 VGPRs): rows of one 64-pair slot, 12 rows per
// wave for the 1 % layer at N = 5760, up to 16.  Wider rows (5 % at N = 5760:
// 12 rows x 5 slots) spill at 128 VGPRs and keep 8-wave workgroups.
const KernelEntry kSparseTeamF16Kernels16[] = {
    PRNN_SPARSE_TEAM16(_Float16, kF16, 12, 1), PRNN_SPARSE_TEAM16(_Float16, kF16, 16, 1),
    {0, 0, 0, nullptr},
};
// 12-wave workgroups (3 waves per SIMD, at most 168 VGPRs): the large layers,
// 15 rows per wave at N = 5760 (5 %: 5 slots), 6 at N = 2304, and up to 11
// rows of 1 or 2 slots (N up to 4224 on 256 workgroups).
const KernelEntry kSparseTeamF16Kernels12[] = {
    PRNN_SPARSE_TEAM12(_Float16, kF16, 15, 5), PRNN_SPARSE_TEAM12(_Float16, kF16, 6, 4),
    PRNN_SPARSE_TEAM12(_Float16, kF16, 6, 9), PRNN_SPARSE_TEAM12(_Float16, kF16, 6, 10),
    PRNN_SPARSE_TEAM12(_Float16, kF16, 11, 1), PRNN_SPARSE_TEAM12(_Float16, kF16, 11, 2),
    {0, 0, 0, nullptr},
};
const KernelEntry kSparseTeamF16TraceKernels16[] = {
    PRNN_SPARSE_TEAM16_TRACE(_Float16, kF16, 12, 1),
    {0, 0, 0, nullptr},
};

// Trace instances: the shapes of the configured layers (N = 1152 and 1792
// dense; 10 % and 1 % sparse at N = 1152, 1792 and 5760).
const KernelEntry kDenseTeamF16TraceKernels[] = {
    PRNN_DENSE_TEAM_WIDE_TRACE(5, 5), PRNN_DENSE_TEAM_WIDE_TRACE(7, 7),
    {0, 0, 0, nullptr},
};
const KernelEntry kSparseTeamF16TraceKernels[] = {
    PRNN_SPARSE_TEAM_TRACE(_Float16, kF16, 5, 2), PRNN_SPARSE_TEAM_TRACE(_Float16, kF16, 7, 1),
    PRNN_SPARSE_TEAM_TRACE(_Float16, kF16, 7, 3), PRNN_SPARSE_TEAM_TRACE(_Float16, kF16, 23, 1),
    {0, 0, 0, nullptr},
};

// Matrix-core dense instances: 16, 32, 48, 64 rows per workgroup.
const KernelEntry kDenseTeamMfmaKernels[] = {
    PRNN_DENSE_TEAM_MFMA(1), PRNN_DENSE_TEAM_MFMA(2), PRNN_DENSE_TEAM_MFMA(3), PRNN_DENSE_TEAM_MFMA(4),
    {0, 0, 0, nullptr},
};
const KernelEntry kDenseTeamMfmaTraceKernels[] = {
    PRNN_DENSE_TEAM_MFMA_TRACE(3), PRNN_DENSE_TEAM_MFMA_TRACE(4),
    {0, 0, 0, nullptr},
};

}  // namespace prnn
