// Route kernel variants and the workspace counter reset.
#include "moe_kernels.hpp"
#include "moe_launch.hpp"

namespace moe {

__global__ void clear_sync_kernel(unsigned *sync, int n) {
  if ((int)threadIdx.x < n) sync[threadIdx.x] = 0u;
}

hipError_t launch_route(int act, const Args &a, int blocks, hipStream_t st) {
  if (act == F32)
    hipLaunchKernelGGL((route_kernel<F32>), dim3(blocks), dim3(ROUTE_THREADS), 0, st, a);
  else
    hipLaunchKernelGGL((route_kernel<BF16>), dim3(blocks), dim3(ROUTE_THREADS), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_clear_sync(unsigned *sync, int n, hipStream_t st) {
  hipLaunchKernelGGL(clear_sync_kernel, dim3(1), dim3(64), 0, st, sync, n);
  return hipGetLastError();
}

}  // namespace moe
