// Kernel variants for f32 activations with mxfp4 routed experts.
#include "moe_kernels.hpp"
#include "moe_launch.hpp"
MOE_INSTANTIATE(F32, MXFP4, f32_mxfp4)
