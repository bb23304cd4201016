// Route kernel variants and the workspace completion-word reset.
#include "moe_kernels.hpp"
#include "moe_launch.hpp"

namespace moe {

__global__ void clear_sync_kernel(unsigned *sync, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) sync[i] = 0u;
}

template <int ACT, int CS>
static void route_launch(const Args &a, int blocks, hipStream_t st) {
  hipLaunchKernelGGL((route_kernel<ACT, CS>), dim3(blocks), dim3(THREADS), 0, st, a);
}

// cs: shared-expert rows per pass, one of the values the host's pass
// variants use (1, 2, 4, 8).
hipError_t launch_route(int act, int cs, const Args &a, int blocks, hipStream_t st) {
  if (act == F32) {
    if (cs == 1) route_launch<F32, 1>(a, blocks, st);
    else if (cs == 2) route_launch<F32, 2>(a, blocks, st);
    else return hipErrorInvalidValue;
  } else {
    if (cs == 1) route_launch<BF16, 1>(a, blocks, st);
    else if (cs == 4) route_launch<BF16, 4>(a, blocks, st);
    else if (cs == 8) route_launch<BF16, 8>(a, blocks, st);
    else return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_clear_sync(unsigned *sync, int n, hipStream_t st) {
  hipLaunchKernelGGL(clear_sync_kernel, dim3(1), dim3(256), 0, st, sync, n);
  return hipGetLastError();
}

}  // namespace moe
