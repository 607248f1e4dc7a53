// Half-h instances of the dense fp16 team kernel (PRNN_MATH_HALF): packed fp16
// weights, h_{t-1} staged as fp16, two products per v_dot2_f32_f16.
#include "team_kernel.h"

namespace prnn {

const KernelEntry kDenseTeamHalfKernels[] = {
    // (rows per wave, 256-column chunks): the shapes of the fp16 table, up to
    // 10 x 10 (N = 2560, 245 VGPRs)
    PRNN_DENSE_TEAM_HALF(1, 1), PRNN_DENSE_TEAM_HALF(2, 1), PRNN_DENSE_TEAM_HALF(4, 1), PRNN_DENSE_TEAM_HALF(8, 1),
    PRNN_DENSE_TEAM_HALF(1, 2), PRNN_DENSE_TEAM_HALF(2, 2), PRNN_DENSE_TEAM_HALF(4, 2), PRNN_DENSE_TEAM_HALF(8, 2),
    PRNN_DENSE_TEAM_HALF(2, 4), PRNN_DENSE_TEAM_HALF(4, 4), PRNN_DENSE_TEAM_HALF(8, 4), PRNN_DENSE_TEAM_HALF(4, 5),
    PRNN_DENSE_TEAM_HALF(5, 5), PRNN_DENSE_TEAM_HALF(6, 5), PRNN_DENSE_TEAM_HALF(8, 5), PRNN_DENSE_TEAM_HALF(7, 7),
    PRNN_DENSE_TEAM_HALF(8, 7), PRNN_DENSE_TEAM_HALF(6, 8), PRNN_DENSE_TEAM_HALF(8, 8), PRNN_DENSE_TEAM_HALF(9, 9),
    PRNN_DENSE_TEAM_HALF(10, 10),
    {0, 0, 0, nullptr},
};

// Trace instances: the configured dense layers (N = 1152 and 1792).
const KernelEntry kDenseTeamHalfTraceKernels[] = {
    PRNN_DENSE_TEAM_HALF_TRACE(5, 5), PRNN_DENSE_TEAM_HALF_TRACE(7, 7),
    {0, 0, 0, nullptr},
};

}  // namespace prnn
