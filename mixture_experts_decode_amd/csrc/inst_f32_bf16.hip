// Kernel variants for f32 activations with bf16 routed experts.
#include "moe_kernels.hpp"
#include "moe_launch.hpp"
MOE_INSTANTIATE(F32, BF16, f32_bf16)
