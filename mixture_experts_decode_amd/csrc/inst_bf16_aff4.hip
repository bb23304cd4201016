// Kernel variants for bf16 activations with aff4 routed experts.
#include "moe_kernels.hpp"
#include "moe_launch.hpp"
MOE_INSTANTIATE(BF16, AFF4, bf16_aff4)
