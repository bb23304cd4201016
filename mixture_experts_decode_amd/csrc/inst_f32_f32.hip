// Kernel variants for f32 activations with f32 routed experts.
#include "moe_kernels.hpp"
#include "moe_launch.hpp"

namespace moe {
namespace {
constexpr int ACTT = F32, EFT = F32;
const Variant kV[] = { MOE_V(1,1, 16), MOE_V(1,1, 64), MOE_V(2,2, 16), MOE_V(2,2, 64), MOE_VN(16, 4), MOE_VN(64, 4) };
const GateUpVariant kG[] = { MOE_G(1,1), MOE_G(2,2) };
}  // namespace
MOE_TABLE(f32_f32)
}  // namespace moe
