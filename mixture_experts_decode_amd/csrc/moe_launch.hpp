// moe_launch.hpp -- launchers of the kernel variants (one translation unit
// per activation/expert format pair instantiates its variants).
#pragma once
#include <hip/hip_runtime.h>

namespace moe {

struct Args;

// (CR, CS): input vectors per pass for routed and shared rows.  Kept to the
// pairs the host's variant choice can produce.
#define MOE_PASS_VARIANTS(X) X(1, 1) X(2, 2) X(2, 4) X(2, 8) X(4, 8) X(8, 8)

hipError_t launch_route(int act, const Args &a, int blocks, hipStream_t st);
hipError_t launch_clear_sync(unsigned *sync, int n, hipStream_t st);

#define MOE_DECLARE_FMT(NAME)                                                              \
  hipError_t launch_gate_up_##NAME(int cr, int cs, const Args &a, int blocks, hipStream_t st); \
  hipError_t launch_down_blend_##NAME(int cr, int cs, int lpr, const Args &a, int blocks,     \
                                      hipStream_t st);
MOE_DECLARE_FMT(f32_f32)
MOE_DECLARE_FMT(f32_bf16)
MOE_DECLARE_FMT(f32_aff4)
MOE_DECLARE_FMT(f32_mxfp4)
MOE_DECLARE_FMT(bf16_f32)
MOE_DECLARE_FMT(bf16_bf16)
MOE_DECLARE_FMT(bf16_aff4)
MOE_DECLARE_FMT(bf16_mxfp4)
#undef MOE_DECLARE_FMT

}  // namespace moe

// Body of one instantiation unit: ACT_ and EF_ are format enums of moe; the
// case macros below see them as the constants ACTT and EFT.
#define MOE_INSTANTIATE(ACT_, EF_, NAME)                                                     \
  namespace moe {                                                                            \
  hipError_t launch_gate_up_##NAME(int cr, int cs, const Args &a, int blocks, hipStream_t st) { \
    constexpr int EFT = EF_, ACTT = ACT_;                                                    \
    bool done = false;                                                                       \
    MOE_PASS_VARIANTS(MOE_GU_CASE)                                                           \
    if (!done) return hipErrorInvalidValue;                                                  \
    return hipGetLastError();                                                                \
  }                                                                                          \
  hipError_t launch_down_blend_##NAME(int cr, int cs, int lpr, const Args &a, int blocks,       \
                                      hipStream_t st) {                                      \
    constexpr int EFT = EF_, ACTT = ACT_;                                                    \
    bool done = false;                                                                       \
    MOE_PASS_VARIANTS(MOE_DB_CASE)                                                           \
    if (!done) return hipErrorInvalidValue;                                                  \
    return hipGetLastError();                                                                \
  }                                                                                          \
  }

#define MOE_GU_CASE(CR_, CS_)                                                                 \
  if (!done && cr == CR_ && cs == CS_) {                                                     \
    hipLaunchKernelGGL((gate_up_kernel<EFT, ACTT, CR_, CS_>), dim3(blocks), dim3(GEMV_THREADS), \
                       0, st, a);                                                            \
    done = true;                                                                             \
  }

#define MOE_DB_CASE(CR_, CS_)                                                                 \
  if (!done && cr == CR_ && cs == CS_) {                                                     \
    if (lpr == 16)                                                                           \
      hipLaunchKernelGGL((down_blend_kernel<EFT, ACTT, CR_, CS_, 16>), dim3(blocks),         \
                         dim3(GEMV_THREADS), 0, st, a);                                      \
    else if (lpr == 32)                                                                      \
      hipLaunchKernelGGL((down_blend_kernel<EFT, ACTT, CR_, CS_, 32>), dim3(blocks),         \
                         dim3(GEMV_THREADS), 0, st, a);                                      \
    else                                                                                     \
      hipLaunchKernelGGL((down_blend_kernel<EFT, ACTT, CR_, CS_, 64>), dim3(blocks),         \
                         dim3(GEMV_THREADS), 0, st, a);                                      \
    done = true;                                                                             \
  }
