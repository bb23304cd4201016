// Kernel variants for bf16 activations with f32 routed experts.
#include "moe_kernels.hpp"
#include "moe_launch.hpp"

namespace moe {
namespace {
constexpr int ACTT = BF16, EFT = F32;
const Variant kV[] = { MOE_V(1,1, 16), MOE_V(1,1, 64), MOE_V(2,4, 16), MOE_V(2,4, 64), MOE_V(2,8, 16), MOE_V(2,8, 64), MOE_V(4,8, 16), MOE_V(4,8, 64), MOE_VN(16, 4), MOE_VN(64, 4) };
const GateUpVariant kG[] = { MOE_G(1,1), MOE_G(2,4), MOE_G(2,8), MOE_G(4,8) };
}  // namespace
MOE_TABLE(bf16_f32)
}  // namespace moe
