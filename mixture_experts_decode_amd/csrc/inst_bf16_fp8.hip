// Kernel variants for bf16 activations with fp8 routed experts.
#include "moe_kernels.hpp"
#include "moe_launch.hpp"

namespace moe {
namespace {
constexpr int ACTT = BF16, EFT = FP8;
const Variant kV[] = { MOE_V(1,1, 32), MOE_V(1,1, 64), MOE_V(2,4, 32), MOE_V(2,4, 64), MOE_V(2,8, 32), MOE_V(2,8, 64), MOE_V(4,8, 32), MOE_V(4,8, 64) };
const GateUpVariant kG[] = { MOE_G(1,1), MOE_G(2,4), MOE_G(2,8), MOE_G(4,8) };
}  // namespace
MOE_TABLE_GROUPED(bf16_fp8)
}  // namespace moe
