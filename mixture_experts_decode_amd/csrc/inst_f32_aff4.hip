// Kernel variants for f32 activations with aff4 routed experts.
#include "moe_kernels.hpp"
#include "moe_launch.hpp"
MOE_INSTANTIATE(F32, AFF4, f32_aff4)
