// Route kernel variants and the workspace completion-word reset.
#include "moe_kernels.hpp"
#include "moe_launch.hpp"

namespace moe {

__global__ void clear_sync_kernel(unsigned *sync, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) sync[i] = 0u;
}

template <int ACT, int CS, int RT = ROUTE_THREADS>
static hipError_t route_launch(const Args &a, int blocks, hipStream_t st, hipEvent_t t0, hipEvent_t t1) {
  return launch_timed(route_kernel<ACT, CS, RT>, blocks, RT, st, t0, t1, a);
}

// cs: shared-expert rows per pass, one of the values the host's pass
// variants use (1, 2, 4, 8).  wide: 1024-thread workgroups (bf16
// activations; the shared expert on the matrix cores, or none).
hipError_t launch_route(int act, int cs, const Args &a, int blocks, hipStream_t st, hipEvent_t t0, hipEvent_t t1,
                        bool wide) {
  if (wide) {
    // Only shared experts on the matrix cores, or none, run there.
    if (act == BF16 && (a.shared_mfma || a.n_shared_gu == 0))
      return route_launch<BF16, 1, ROUTE_THREADS_WIDE>(a, blocks, st, t0, t1);
    return hipErrorInvalidValue;
  }
  if (act == F32) {
    if (cs == 1) return route_launch<F32, 1>(a, blocks, st, t0, t1);
    if (cs == 2) return route_launch<F32, 2>(a, blocks, st, t0, t1);
  } else {
    if (cs == 1) return route_launch<BF16, 1>(a, blocks, st, t0, t1);
    if (cs == 4) return route_launch<BF16, 4>(a, blocks, st, t0, t1);
    if (cs == 8) return route_launch<BF16, 8>(a, blocks, st, t0, t1);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_route_tile(int act, const Args &a, int blocks, hipStream_t st, hipEvent_t t0) {
  if (act == F32) return launch_timed(route_tile_kernel<F32>, blocks, ROUTE_THREADS, st, t0, nullptr, a);
  return launch_timed(route_tile_kernel<BF16>, blocks, ROUTE_THREADS, st, t0, nullptr, a);
}

hipError_t launch_pre_norm(int act, const Args &a, const void *x, const void *w, const void *wr, float eps,
                           void *xe, void *xrn, hipStream_t st, hipEvent_t t0) {
  if (act == F32) return launch_timed(pre_norm_kernel<F32>, a.m, 256, st, t0, nullptr, a, x, w, wr, eps, xe, xrn);
  return launch_timed(pre_norm_kernel<BF16>, a.m, 256, st, t0, nullptr, a, x, w, wr, eps, xe, xrn);
}

hipError_t launch_topk_sort(const Args &a, int blocks, hipStream_t st, hipEvent_t t0, hipEvent_t t1) {
  return launch_timed(topk_sort_kernel<BF16>, blocks, ROUTE_THREADS, st, t0, t1, a);
}

hipError_t launch_blend_grouped(const Args &a, int blocks, hipStream_t st, hipEvent_t t0, hipEvent_t t1) {
  return launch_timed(blend_grouped_kernel<BF16>, blocks, 256, st, t0, t1, a);
}

hipError_t launch_clear_sync(unsigned *sync, int n, hipStream_t st) {
  hipLaunchKernelGGL(clear_sync_kernel, dim3(1), dim3(256), 0, st, sync, n);
  return hipGetLastError();
}

}  // namespace moe

// ------------------------------------------------------ measurement utilities
//
// Plain streaming kernels with the same 16-byte-per-lane access pattern as
// the layer's kernels: the known-size references for the HBM byte counters
// and for the achievable read bandwidth.

namespace moe {

__global__ __launch_bounds__(256) void bench_copy_kernel(const u32x4 *src, u32x4 *dst, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

__global__ __launch_bounds__(256) void bench_read_kernel(const u32x4 *src, size_t n, unsigned *sink) {
  constexpr int U = 8;
  uint32_t acc = 0;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + (U - 1) * stride < n; i += U * stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;  // keeps the loads alive; practically never stores
}

hipError_t launch_bench_copy(const void *src, void *dst, size_t bytes, hipStream_t st) {
  const size_t n = bytes / 16;
  hipLaunchKernelGGL(bench_copy_kernel, dim3(4096), dim3(256), 0, st, reinterpret_cast<const u32x4 *>(src),
                     reinterpret_cast<u32x4 *>(dst), n);
  return hipGetLastError();
}

hipError_t launch_bench_read(const void *src, size_t bytes, unsigned *sink, hipStream_t st) {
  const size_t n = bytes / 16;
  hipLaunchKernelGGL(bench_read_kernel, dim3(4096), dim3(256), 0, st, reinterpret_cast<const u32x4 *>(src), n, sink);
  return hipGetLastError();
}

}  // namespace moe
