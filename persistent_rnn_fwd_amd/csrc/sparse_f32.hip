// fp32-value instances of the sparse persistent kernel.
#include "sparse_kernel.h"

namespace prnn {

const KernelEntry kSparseF32Kernels[] = {
    // (rows, 64-pair slots per row); two VGPRs per slot
    PRNN_SPARSE(float, kF32, 1, 1), PRNN_SPARSE(float, kF32, 1, 2), PRNN_SPARSE(float, kF32, 1, 4),
    PRNN_SPARSE(float, kF32, 1, 8), PRNN_SPARSE(float, kF32, 1, 16), PRNN_SPARSE(float, kF32, 2, 1),
    PRNN_SPARSE(float, kF32, 2, 2), PRNN_SPARSE(float, kF32, 2, 4), PRNN_SPARSE(float, kF32, 2, 8),
    PRNN_SPARSE(float, kF32, 2, 16), PRNN_SPARSE(float, kF32, 4, 1), PRNN_SPARSE(float, kF32, 4, 2),
    PRNN_SPARSE(float, kF32, 4, 4), PRNN_SPARSE(float, kF32, 4, 8), PRNN_SPARSE(float, kF32, 8, 1),
    PRNN_SPARSE(float, kF32, 8, 2), PRNN_SPARSE(float, kF32, 8, 4), PRNN_SPARSE(float, kF32, 16, 1),
    PRNN_SPARSE(float, kF32, 16, 2), PRNN_SPARSE(float, kF32, 32, 1),
    {0, 0, 0, nullptr},
};

}  // namespace prnn
