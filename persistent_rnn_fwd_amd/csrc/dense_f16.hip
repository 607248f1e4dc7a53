// fp16-weight instances of the dense persistent kernel: power-of-two row and
// chunk capacities for any shape, plus exact fits for N = 1152 and N = 1792.
#include "dense_kernel.h"

namespace prnn {

const KernelEntry kDenseF16Kernels[] = {
    // (rows, chunks); weights take rows * chunks * 2 VGPRs
    PRNN_DENSE(_Float16, kF16, 1, 1), PRNN_DENSE(_Float16, kF16, 1, 2), PRNN_DENSE(_Float16, kF16, 1, 4),
    PRNN_DENSE(_Float16, kF16, 1, 8), PRNN_DENSE(_Float16, kF16, 1, 12), PRNN_DENSE(_Float16, kF16, 1, 16),
    PRNN_DENSE(_Float16, kF16, 2, 1), PRNN_DENSE(_Float16, kF16, 2, 2), PRNN_DENSE(_Float16, kF16, 2, 4),
    PRNN_DENSE(_Float16, kF16, 2, 8), PRNN_DENSE(_Float16, kF16, 2, 12), PRNN_DENSE(_Float16, kF16, 2, 16),
    PRNN_DENSE(_Float16, kF16, 4, 1), PRNN_DENSE(_Float16, kF16, 4, 2), PRNN_DENSE(_Float16, kF16, 4, 4),
    PRNN_DENSE(_Float16, kF16, 4, 8), PRNN_DENSE(_Float16, kF16, 4, 12), PRNN_DENSE(_Float16, kF16, 4, 16),
    PRNN_DENSE(_Float16, kF16, 8, 1), PRNN_DENSE(_Float16, kF16, 8, 2), PRNN_DENSE(_Float16, kF16, 8, 4),
    PRNN_DENSE(_Float16, kF16, 8, 8), PRNN_DENSE(_Float16, kF16, 16, 1), PRNN_DENSE(_Float16, kF16, 16, 2),
    PRNN_DENSE(_Float16, kF16, 16, 4), PRNN_DENSE(_Float16, kF16, 32, 1), PRNN_DENSE(_Float16, kF16, 32, 2),
    PRNN_DENSE(_Float16, kF16, 5, 5), PRNN_DENSE(_Float16, kF16, 6, 5), PRNN_DENSE(_Float16, kF16, 9, 5),
    PRNN_DENSE(_Float16, kF16, 7, 7),
    {0, 0, 0, nullptr},
};

}  // namespace prnn
