// The wide-stream forward with a residual added in the combine
// (kModeForwardRes), in a translation unit of its own: the kernels of
// moe_kernels.hip then form the same code object as without it.
#define MOE_RES_WIDE_TU
#include "moe_kernels.hip"
