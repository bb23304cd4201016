// Kernel variants for f32 activations with fp8 routed experts (m <= 32).
#include "moe_kernels.hpp"
#include "moe_launch.hpp"

namespace moe {
namespace {
constexpr int ACTT = F32, EFT = FP8;
const Variant kV[] = { MOE_V(1,1, 32), MOE_V(1,1, 64), MOE_V(2,2, 32), MOE_V(2,2, 64) };
const GateUpVariant kG[] = { MOE_G(1,1), MOE_G(2,2) };
}  // namespace
MOE_TABLE(f32_fp8)
}  // namespace moe
