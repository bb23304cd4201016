// Kernel variants for bf16 activations with bf16 routed experts.
#include "moe_kernels.hpp"
#include "moe_launch.hpp"
MOE_INSTANTIATE(BF16, BF16, bf16_bf16)
