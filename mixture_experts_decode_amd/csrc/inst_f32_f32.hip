// Kernel variants for f32 activations with f32 routed experts.
#include "moe_kernels.hpp"
#include "moe_launch.hpp"
MOE_INSTANTIATE(F32, F32, f32_f32)
