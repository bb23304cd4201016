// Kernel variants for bf16 activations with f32 routed experts.
#include "moe_kernels.hpp"
#include "moe_launch.hpp"
MOE_INSTANTIATE(BF16, F32, bf16_f32)
