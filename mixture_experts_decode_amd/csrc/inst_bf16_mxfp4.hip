// Kernel variants for bf16 activations with mxfp4 routed experts.
#include "moe_kernels.hpp"
#include "moe_launch.hpp"
MOE_INSTANTIATE(BF16, MXFP4, bf16_mxfp4)
