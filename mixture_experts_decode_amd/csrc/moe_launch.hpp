// moe_launch.hpp -- per-format tables of the instantiated kernel variants.
//
// Each inst_<act>_<expert>.hip translation unit instantiates the variants
// its format pair needs and exposes them through a FormatKernels table; the
// host picks a (CR, CS, LPR) present in the table.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

namespace moe {

struct Args;

// start/stop: events that take the kernel's own start and end timestamps
// (hipExtLaunchKernelGGL), or null.
typedef hipError_t (*launch_fn)(const Args &a, int blocks, hipStream_t st, hipEvent_t start, hipEvent_t stop);

// Launches kernel K with the layer's block size, timed when start/stop are given.
template <typename K, typename... P>
inline hipError_t launch_timed(K kernel, int blocks, int threads, hipStream_t st, hipEvent_t start, hipEvent_t stop,
                               P... p) {
  if (start || stop)
    hipExtLaunchKernelGGL(kernel, dim3(blocks), dim3(threads), 0, st, start, stop, 0u, p...);
  else
    hipLaunchKernelGGL(kernel, dim3(blocks), dim3(threads), 0, st, p...);
  return hipGetLastError();
}

// (CR, CS): input vectors per pass for routed and shared rows; LPR: lanes
// per down row.
struct Variant {
  int cr, cs, lpr;
  int narrow;             // the m = 1 down of few sub-units per tile: its tile height (rows on 4 waves); 0 if not
  int rd, down_threads;   // down rows per wave sub-unit, threads per down workgroup
  launch_fn down_blend;   // third launch
};
struct GateUpVariant {
  int cr, cs;
  launch_fn gate_up;      // second launch
  launch_fn gate_up_shd;  // the same, also running the shared expert's down on the matrix cores (m <= 16)
  launch_fn gate_up_shd2; // the same for m <= 32
};
struct FormatKernels {
  const Variant *v;
  int nv;
  const GateUpVariant *g;
  int ng;
  launch_fn gate_up_grouped;   // m > 32 (matrix cores), or null where not served
  launch_fn down_grouped;      // down rows of at most 2048
  launch_fn down_grouped_long; // longer down rows
  int gu_grouped_rows;         // intermediate rows per grouped gate/up item
};

// First launch: router items plus the shared expert's gate/up items.
hipError_t launch_route(int act, int cs, const Args &a, int blocks, hipStream_t st, hipEvent_t start,
                        hipEvent_t stop, bool wide);
hipError_t launch_clear_sync(unsigned *sync, int n, hipStream_t st);
// The grouped path's router: units of RT_E router rows x 8 input rows.
hipError_t launch_route_tile(int act, const Args &a, int blocks, hipStream_t st, hipEvent_t start);
// The pre-norms of the m raw rows x (one workgroup per row): with weight w
// into xe (the experts' input) and with weight wr into xrn (the router's);
// a null weight skips its output.  With the router pre-norm and a gated
// shared expert, also the gate's logit of the raw row.
hipError_t launch_pre_norm(int act, const Args &a, const void *x, const void *w, const void *wr, float eps,
                           void *xe, void *xrn, hipStream_t st, hipEvent_t start);
// Grouped path (m > 32): top-k with the sort, and the blend.
hipError_t launch_topk_sort(const Args &a, int blocks, hipStream_t st, hipEvent_t start, hipEvent_t stop);
hipError_t launch_blend_grouped(const Args &a, int blocks, hipStream_t st, hipEvent_t start, hipEvent_t stop);
hipError_t launch_bench_copy(const void *src, void *dst, size_t bytes, hipStream_t st);
hipError_t launch_bench_read(const void *src, size_t bytes, unsigned *sink, hipStream_t st);

const FormatKernels &kernels_f32_f32();
const FormatKernels &kernels_f32_bf16();
const FormatKernels &kernels_f32_aff4();
const FormatKernels &kernels_f32_mxfp4();
const FormatKernels &kernels_bf16_f32();
const FormatKernels &kernels_bf16_bf16();
const FormatKernels &kernels_bf16_aff4();
const FormatKernels &kernels_bf16_mxfp4();
const FormatKernels &kernels_f32_nvfp4();
const FormatKernels &kernels_bf16_nvfp4();
const FormatKernels &kernels_f32_fp8();
const FormatKernels &kernels_bf16_fp8();

#ifdef MOE_KERNELS_HPP_INCLUDED
template <int EF, int ACT, int CR, int CS, int LPR, int NW>
hipError_t launch_down_blend_t(const Args &a, int blocks, hipStream_t st, hipEvent_t start, hipEvent_t stop) {
  return launch_timed(down_blend_kernel<EF, ACT, CR, CS, LPR, NW>, blocks, down_threads<EF, CS, LPR, NW>(), st,
                      start, stop, a);
}
template <int EF>
hipError_t launch_gate_up_grouped_t(const Args &a, int blocks, hipStream_t st, hipEvent_t start, hipEvent_t stop) {
  return launch_timed(gate_up_grouped_kernel<EF>, blocks, 64 * gu_grouped_waves<EF>(), st, start, stop, a);
}
template <int EF, bool WIDE>
hipError_t launch_down_grouped_t(const Args &a, int blocks, hipStream_t st, hipEvent_t start, hipEvent_t stop) {
  return launch_timed(down_grouped_kernel<EF, WIDE>, blocks, down_grouped_threads<EF, WIDE>(), st, start, stop, a);
}
template <int EF, int ACT, int CR, int CS, int SHD>
hipError_t launch_gate_up_t(const Args &a, int blocks, hipStream_t st, hipEvent_t start, hipEvent_t stop) {
  return launch_timed(gate_up_kernel<EF, ACT, CR, CS, SHD>, blocks, THREADS, st, start, stop, a);
}
// The variant with the shared expert's down items exists for bf16
// activations only (the matrix-core path).
template <int EF, int ACT, int CR, int CS, int NCT>
constexpr launch_fn gate_up_shd_fn() {
  if constexpr (ACT == BF16) return &launch_gate_up_t<EF, ACT, CR, CS, NCT>;
  else return nullptr;
}
#endif

}  // namespace moe

// Inside an inst_*.hip unit, with constexpr int EFT and ACTT in scope.
#define MOE_V(CR, CS, LPR) { CR, CS, LPR, 0, down_rd<EFT, CS, 0>(), down_threads<EFT, CS, LPR, 0>(), \
                            &launch_down_blend_t<EFT, ACTT, CR, CS, LPR, 0> }
// The narrow m = 1 down (f32 and bf16 experts), tiles of RD rows.
#define MOE_VN(LPR, RD) { 1, 1, LPR, RD, down_rd<EFT, 1, RD>(), down_threads<EFT, 1, LPR, RD>(), \
                          &launch_down_blend_t<EFT, ACTT, 1, 1, LPR, RD> }
#define MOE_G(CR, CS) { CR, CS, &launch_gate_up_t<EFT, ACTT, CR, CS, 0>, gate_up_shd_fn<EFT, ACTT, CR, CS, 1>(), \
                        gate_up_shd_fn<EFT, ACTT, CR, CS, 2>() }
#define MOE_TABLE(NAME)                                                            \
  const FormatKernels &kernels_##NAME() {                                          \
    static const FormatKernels k{kV, (int)(sizeof kV / sizeof kV[0]), kG,         \
                                 (int)(sizeof kG / sizeof kG[0]), nullptr, nullptr, nullptr, 0}; \
    return k;                                                                      \
  }
// The same with the grouped (m > 32) kernels of the unit's expert format.
#define MOE_TABLE_GROUPED(NAME)                                                    \
  const FormatKernels &kernels_##NAME() {                                          \
    static const FormatKernels k{kV, (int)(sizeof kV / sizeof kV[0]), kG,         \
                                 (int)(sizeof kG / sizeof kG[0]),                  \
                                 &launch_gate_up_grouped_t<EFT>, &launch_down_grouped_t<EFT, true>, \
                                 &launch_down_grouped_t<EFT, false>, 16 * gate_up_grouped_tiles<EFT>()}; \
    return k;                                                                      \
  }
