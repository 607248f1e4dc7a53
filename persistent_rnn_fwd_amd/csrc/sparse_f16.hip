// fp16-value instances of the sparse persistent kernel: power-of-two row and
// slot capacities for any shape, plus exact fits for the 1152, 1792 and
// 5760-neuron layers.
#include "sparse_kernel.h"

namespace prnn {

const KernelEntry kSparseF16Kernels[] = {
    // (rows, 64-pair slots per row); one VGPR per slot
    PRNN_SPARSE(_Float16, kF16, 1, 1), PRNN_SPARSE(_Float16, kF16, 1, 2), PRNN_SPARSE(_Float16, kF16, 1, 4),
    PRNN_SPARSE(_Float16, kF16, 1, 8), PRNN_SPARSE(_Float16, kF16, 1, 16), PRNN_SPARSE(_Float16, kF16, 2, 1),
    PRNN_SPARSE(_Float16, kF16, 2, 2), PRNN_SPARSE(_Float16, kF16, 2, 4), PRNN_SPARSE(_Float16, kF16, 2, 8),
    PRNN_SPARSE(_Float16, kF16, 2, 16), PRNN_SPARSE(_Float16, kF16, 4, 1), PRNN_SPARSE(_Float16, kF16, 4, 2),
    PRNN_SPARSE(_Float16, kF16, 4, 4), PRNN_SPARSE(_Float16, kF16, 4, 8), PRNN_SPARSE(_Float16, kF16, 4, 16),
    PRNN_SPARSE(_Float16, kF16, 8, 1), PRNN_SPARSE(_Float16, kF16, 8, 2), PRNN_SPARSE(_Float16, kF16, 8, 4),
    PRNN_SPARSE(_Float16, kF16, 8, 8), PRNN_SPARSE(_Float16, kF16, 16, 1), PRNN_SPARSE(_Float16, kF16, 16, 2),
    PRNN_SPARSE(_Float16, kF16, 16, 4), PRNN_SPARSE(_Float16, kF16, 32, 1), PRNN_SPARSE(_Float16, kF16, 32, 2),
    PRNN_SPARSE(_Float16, kF16, 5, 2), PRNN_SPARSE(_Float16, kF16, 6, 2), PRNN_SPARSE(_Float16, kF16, 7, 1),
    PRNN_SPARSE(_Float16, kF16, 7, 3), PRNN_SPARSE(_Float16, kF16, 23, 1), PRNN_SPARSE(_Float16, kF16, 24, 1),
    {0, 0, 0, nullptr},
};

}  // namespace prnn
