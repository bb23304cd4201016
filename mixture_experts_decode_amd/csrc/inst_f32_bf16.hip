// Kernel variants for f32 activations with bf16 routed experts.
#include "moe_kernels.hpp"
#include "moe_launch.hpp"

namespace moe {
namespace {
constexpr int ACTT = F32, EFT = BF16;
const Variant kV[] = { MOE_V(1,1, 32), MOE_V(1,1, 64), MOE_V(2,2, 32), MOE_V(2,2, 64), MOE_VN(32, 4), MOE_VN(64, 4) };
const GateUpVariant kG[] = { MOE_G(1,1), MOE_G(2,2) };
}  // namespace
MOE_TABLE(f32_bf16)
}  // namespace moe
