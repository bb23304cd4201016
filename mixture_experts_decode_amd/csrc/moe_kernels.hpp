// moe_kernels.hpp -- gfx950 device code of the decode MoE layer.
//
// The layer is cut into work items, each run by one 256-thread workgroup:
//   router items       4 router rows each (fp64 accumulation); the last one
//                      to finish scores, selects top-k, computes the routing
//                      weights and counting-sorts the (row, slot) pairs by
//                      expert in LDS ("route tail").
//   shared gate/up     the shared expert's gate/up rows (all m rows of x).
//   routed gate/up     (active-expert slot, row block): streams the slot's
//                      gate and up rows once for all of its pairs,
//                      dequantised in registers, writes silu(g)*v per pair.
//   down tiles         a tile of output columns: the down rows of every
//                      active expert and of the shared expert for the tile,
//                      y per pair in LDS, then the slot-order blend.
// They run as three ordinary kernels on the caller's stream, the kernel
// boundaries ordering them: route_kernel (router items, then the route tail
// in the last one to finish, beside the shared expert's gate/up items),
// gate_up_kernel (routed gate/up items) and down_blend_kernel (down tiles).
// fused_kernel, which would run all items in one persistent launch with
// bounded waits between them, is kept in source but not launched (see it).
//
// Pages: metrale "forward_bf16_grouped_decode.rs" (the five steps and their
// buffers), mlxcel "perf(moe): wire lfm2 to the fused decode-MoE kernel"
// (sigmoid routing with expert_bias, norm_topk_prob, routed_scaling_factor),
// iron "refactor(gemm): split the gemv_q8 grab-bag by family" (biased
// selection, unbiased weight), frink "routed_weight_site.rs" (weight on the
// input vs the output, raw-logit top-k), metrale "helpers_a.rs" (packed
// [N, K/2] weights, [N, K/group] scales, E8M0 block 32).
#pragma once
#define MOE_KERNELS_HPP_INCLUDED 1
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

enum : int { F32 = 0, BF16 = 1, AFF4 = 2, MXFP4 = 3 };
enum : int { ROUTE_SOFTMAX = 0, ROUTE_SIGMOID_BIAS = 1, ROUTE_SIGMOID_LOGIT = 2 };
enum : unsigned { NORM_TOPK = 1u, WEIGHT_BEFORE = 2u, SHARED = 4u, SHARED_GATED = 8u, OUT_F32 = 16u };

constexpr int WAVE = 64;
constexpr int THREADS = 256;            // every kernel: 4 waves per workgroup
constexpr int WPB = THREADS / WAVE;
constexpr int MAX_ROWS = 32;
constexpr int MAX_TOPK = 16;
constexpr int MAX_EXPERTS = 256;
constexpr int MAX_PAIRS = MAX_ROWS * MAX_TOPK;
constexpr int DOWN_RD = 8;              // down rows per wave sub-unit
constexpr int MAX_DOWN_TILE = 2 * DOWN_RD;

// Completion words in the workspace (zero between calls).  Word i lives at
// sync[i * SYNC_STRIDE]: one 128-byte line each, so pollers of one word do
// not contend with the atomics on another.
enum : int {
  SYNC_NEXT = 0,      // next work item to claim (fused)
  SYNC_ROUTER = 1,    // router items finished (ticket)
  SYNC_READY = 2,     // routing published (fused)
  SYNC_EXIT = 3,      // workgroups that left the item loop (fused)
  SYNC_SHARED = 4,    // shared gate/up items finished (fused)
  SYNC_ERR = 5,       // a bounded wait expired: stays set until re-initialised
  SYNC_SLOT0 = 16,    // gate/up items finished, per active slot
  SYNC_STRIDE = 32,
  SYNC_WORDS = (SYNC_SLOT0 + 256) * SYNC_STRIDE
};

// Rows of intermediate per gate/up wave: 2 for 16-byte-per-8-or-4 element
// formats, 4 for the 4-bit ones (their rows are 4x shorter).
template <int WF> constexpr int gate_up_ni() { return WF >= AFF4 ? 4 : 2; }

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Everything a forward's kernels read or write (kernel argument, by value).
struct Args {
  int H, E, K, I, Is, m, te, cap, act_fmt, expert_fmt, routing;
  unsigned flags;
  float rsf;
  // work items
  int n_router, n_shared_gu, gu_items_per_slot, n_routed_gu, n_down, n_items, down_dq;
  const void *x;
  void *out;
  int32_t *idx_out;
  float *w_out;
  const void *router;
  const float *ebias;
  const uint64_t *gw, *uw, *dw, *gs, *us, *ds, *gb, *ub, *db;
  const void *sgw, *suw, *sdw, *sgv;
  double *logits;          // [m, E+1]
  int32_t *topk_idx;       // [te]
  float *topk_w;           // [te]
  float *row_gate;         // [m]
  int32_t *sorted_pair;    // [te]
  int32_t *offsets;        // [E+1]
  int32_t *pair_to_perm;   // [te]
  int32_t *active;         // [cap]
  int32_t *active_count;   // [1]
  float *act;              // [te, I]
  float *sact;             // [m, Is]
  unsigned *sync;          // [SYNC_WORDS]
};

// ---------------------------------------------------------------- helpers

__device__ __forceinline__ u32x4 ld_stream16(const void *p) {
  // Expert weights are read once per call: keep them out of the caches.
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}
__device__ __forceinline__ u32x4 ld16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }
__device__ __forceinline__ u32x2 ld8(const void *p) { return *reinterpret_cast<const u32x2 *>(p); }

__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// acc + a.lo*b.lo + a.hi*b.hi with bf16 pairs a, b (v_dot2c_f32_bf16).
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), acc, false);
}

// float -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// OCP MX E8M0 scale 2^(e-127) as float (e = 0 is the subnormal 2^-127).
__device__ __forceinline__ float e8m0_to_f32(uint32_t e) {
  return __uint_as_float(e == 0 ? 0x00400000u : (e == 255 ? 0x7FC00000u : e << 23));
}

__device__ __forceinline__ float silu_mul(float g, float v) {
  return g / (1.0f + __expf(-g)) * v;
}

__device__ __forceinline__ double sigmoid_d(double v) { return 1.0 / (1.0 + exp(-v)); }

// ------------------------------------------------ cross-lane reductions
//
// DPP moves inside 16-lane rows (no LDS round trip), then readlane of the
// four row totals.  Every order is fixed, and pairs are combined
// symmetrically (a+b in one lane, b+a in its partner), so all lanes of a
// group hold bitwise the same total.

constexpr int DPP_XOR1 = 0xB1;          // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4E;          // quad_perm [2,3,0,1]
constexpr int DPP_HALF_MIRROR = 0x141;  // lane i <- 7-i within 8 lanes
constexpr int DPP_MIRROR = 0x140;       // lane i <- 15-i within 16 lanes

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const unsigned long long b = (unsigned long long)__double_as_longlong(v);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(unsigned)b, CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(unsigned)(b >> 32), CTRL, 0xF, 0xF, false);
  return __longlong_as_double((long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo));
}
__device__ __forceinline__ float readlane_f32(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
__device__ __forceinline__ double readlane_f64(double v, int l) {
  const unsigned long long b = (unsigned long long)__double_as_longlong(v);
  const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)b, l);
  const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)(b >> 32), l);
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

__device__ __forceinline__ float row16_sum(float v) {
  v = v + dpp_f32<DPP_XOR1>(v);
  v = v + dpp_f32<DPP_XOR2>(v);
  v = v + dpp_f32<DPP_HALF_MIRROR>(v);
  return v + dpp_f32<DPP_MIRROR>(v);
}

// Total over each group of LPR consecutive lanes (16, 32 or 64); every lane
// gets its own group's total.
template <int LPR>
__device__ __forceinline__ float group_total(float v) {
  v = row16_sum(v);
  if constexpr (LPR == 16) {
    return v;
  } else {
    const float r0 = readlane_f32(v, 0), r1 = readlane_f32(v, 16);
    const float r2 = readlane_f32(v, 32), r3 = readlane_f32(v, 48);
    if constexpr (LPR == 32) return (threadIdx.x & 32) ? (r2 + r3) : (r0 + r1);
    return (r0 + r1) + (r2 + r3);
  }
}

__device__ __forceinline__ double wave_sum_f64(double v) {
  v = v + dpp_f64<DPP_XOR1>(v);
  v = v + dpp_f64<DPP_XOR2>(v);
  v = v + dpp_f64<DPP_HALF_MIRROR>(v);
  v = v + dpp_f64<DPP_MIRROR>(v);
  return (readlane_f64(v, 0) + readlane_f64(v, 16)) + (readlane_f64(v, 32) + readlane_f64(v, 48));
}

// Wave maximum (NaN-ignoring, like fmax).
__device__ __forceinline__ double wave_max_f64(double v) {
  v = fmax(v, dpp_f64<DPP_XOR1>(v));
  v = fmax(v, dpp_f64<DPP_XOR2>(v));
  v = fmax(v, dpp_f64<DPP_HALF_MIRROR>(v));
  v = fmax(v, dpp_f64<DPP_MIRROR>(v));
  return fmax(fmax(readlane_f64(v, 0), readlane_f64(v, 16)),
              fmax(readlane_f64(v, 32), readlane_f64(v, 48)));
}

// ------------------------------------------------ completion words
//
// A producer publishes with a release fence at agent scope (its stores are
// written back past the XCD's L2) and then an atomic add; a consumer polls
// with relaxed agent-scope atomic loads and then takes an acquire fence.
// Every wait is bounded: on expiry it sets SYNC_ERR and reports failure, and
// the caller then skips the work that depended on it, so a broken counter
// can give a wrong answer (flagged) but never a hang or a wild access.

// Longest a wait may last: 200 ms of the 100 MHz constant clock.  A whole
// forward of the largest layer takes about a millisecond.
constexpr uint64_t WAIT_TICKS = 20000000ull;

__device__ __forceinline__ unsigned *word(unsigned *sync, int i) { return sync + i * SYNC_STRIDE; }

__device__ __forceinline__ unsigned load_word(const unsigned *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void release_agent() { __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent"); }
__device__ __forceinline__ void acquire_agent() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }

// One thread polls until word i >= target.  Every 16th poll is an atomic RMW
// that leaves the value unchanged (it always reads the coherent value), and
// the wait gives up after WAIT_TICKS of wall time or once another wait has
// given up.
__device__ __noinline__ bool poll_geq(unsigned *sync, int i, unsigned target) {
  unsigned *p = word(sync, i);
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  for (unsigned it = 1;; ++it) {
    const unsigned v = (it & 15u) ? load_word(p) : atomicOr(p, 0u);
    if (v >= target) return true;
    if ((it & 15u) == 0u) {
      if (atomicOr(word(sync, SYNC_ERR), 0u) != 0u) return false;
      if (__builtin_amdgcn_s_memrealtime() - t0 > WAIT_TICKS) {
        atomicOr(word(sync, SYNC_ERR), 1u);
        return false;
      }
    }
    __builtin_amdgcn_s_sleep(8);
  }
}

// Whole workgroup waits (thread 0 polls); acquire for every thread.
__device__ __forceinline__ bool wg_wait(unsigned *sync, int i, unsigned target) {
  __shared__ int s_ok;
  if (threadIdx.x == 0) s_ok = poll_geq(sync, i, target) ? 1 : 0;
  __syncthreads();
  const bool ok = s_ok != 0;
  acquire_agent();
  __syncthreads();
  return ok;
}

// One wave waits (its lane 0 polls); acquire for the wave.
__device__ __forceinline__ bool wave_wait(unsigned *sync, int i, unsigned target) {
  int ok = 0;
  if ((threadIdx.x & 63) == 0) ok = poll_geq(sync, i, target) ? 1 : 0;
  ok = __builtin_amdgcn_readfirstlane(ok);
  acquire_agent();
  return ok != 0;
}

// Every thread's stores are written back (its own release), the barrier
// orders them before thread 0's increment, which is itself a release.
__device__ __forceinline__ void wg_signal(unsigned *sync, int i) {
  release_agent();
  __syncthreads();
  if (threadIdx.x == 0)
    __hip_atomic_fetch_add(word(sync, i), 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

// --------------------------------------------------- per-format chunk math
//
// A chunk is 16 bytes of one weight row: 4 f32, 8 bf16 or 32 packed 4-bit
// codes.  Lane `li` of a row group handles chunks li, li+LPR, ...  XF is the
// storage format of the vector the row is dotted with (F32 or BF16).

template <int WF> struct Fmt;
template <> struct Fmt<F32> { static constexpr int EPC = 4; };
template <> struct Fmt<BF16> { static constexpr int EPC = 8; };
template <> struct Fmt<AFF4> { static constexpr int EPC = 32; };
template <> struct Fmt<MXFP4> { static constexpr int EPC = 32; };

// One weight row: data, and for 4-bit formats its scale (and bias) row.
template <int WF> struct Row {
  const char *w;
  const void *s;
  const void *b;
};

// Weight chunk plus its per-chunk dequant constants.
template <int WF> struct WChunk {
  u32x4 q;
  float s, b;
};

template <int WF>
__device__ __forceinline__ WChunk<WF> load_wchunk(const Row<WF> &r, int ch) {
  WChunk<WF> c;
  c.q = ld_stream16(r.w + (size_t)ch * 16);
  if constexpr (WF == AFF4) {
    // One bf16 scale and bias per 64 elements = per 2 chunks.
    c.s = bf16_to_f32(reinterpret_cast<const uint16_t *>(r.s)[ch >> 1]);
    c.b = bf16_to_f32(reinterpret_cast<const uint16_t *>(r.b)[ch >> 1]);
  } else if constexpr (WF == MXFP4) {
    c.s = e8m0_to_f32(reinterpret_cast<const uint8_t *>(r.s)[ch]);
    c.b = 0.f;
  } else {
    c.s = c.b = 0.f;
  }
  return c;
}

// The x elements matching one weight chunk, in the form the dot needs.
template <int WF, int XF> struct XChunk;

// bf16 weights . bf16 x: raw bf16 pairs, v_dot2.
template <> struct XChunk<BF16, BF16> {
  uint32_t d[4];
  __device__ __forceinline__ void load(const char *xrow, int ch) {
    u32x4 v = ld16(xrow + (size_t)ch * 16);
    d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
  }
  __device__ __forceinline__ float dot(const WChunk<BF16> &w, float acc) const {
    acc = dot2(w.q.x, d[0], acc);
    acc = dot2(w.q.y, d[1], acc);
    acc = dot2(w.q.z, d[2], acc);
    return dot2(w.q.w, d[3], acc);
  }
};

// bf16 weights . f32 x.
template <> struct XChunk<BF16, F32> {
  float f[8];
  __device__ __forceinline__ void load(const char *xrow, int ch) {
    u32x4 a = ld16(xrow + (size_t)ch * 32), b = ld16(xrow + (size_t)ch * 32 + 16);
    f[0] = __uint_as_float(a.x); f[1] = __uint_as_float(a.y);
    f[2] = __uint_as_float(a.z); f[3] = __uint_as_float(a.w);
    f[4] = __uint_as_float(b.x); f[5] = __uint_as_float(b.y);
    f[6] = __uint_as_float(b.z); f[7] = __uint_as_float(b.w);
  }
  __device__ __forceinline__ float dot(const WChunk<BF16> &w, float acc) const {
    const uint32_t q[4] = {w.q.x, w.q.y, w.q.z, w.q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc = __builtin_fmaf(bf_lo(q[i]), f[2 * i], acc);
      acc = __builtin_fmaf(bf_hi(q[i]), f[2 * i + 1], acc);
    }
    return acc;
  }
};

// f32 weights . f32 x.
template <> struct XChunk<F32, F32> {
  float f[4];
  __device__ __forceinline__ void load(const char *xrow, int ch) {
    u32x4 a = ld16(xrow + (size_t)ch * 16);
    f[0] = __uint_as_float(a.x); f[1] = __uint_as_float(a.y);
    f[2] = __uint_as_float(a.z); f[3] = __uint_as_float(a.w);
  }
  __device__ __forceinline__ float dot(const WChunk<F32> &w, float acc) const {
    acc = __builtin_fmaf(__uint_as_float(w.q.x), f[0], acc);
    acc = __builtin_fmaf(__uint_as_float(w.q.y), f[1], acc);
    acc = __builtin_fmaf(__uint_as_float(w.q.z), f[2], acc);
    return __builtin_fmaf(__uint_as_float(w.q.w), f[3], acc);
  }
};

// f32 weights . bf16 x.
template <> struct XChunk<F32, BF16> {
  float f[4];
  __device__ __forceinline__ void load(const char *xrow, int ch) {
    u32x2 a = ld8(xrow + (size_t)ch * 8);
    f[0] = bf_lo(a.x); f[1] = bf_hi(a.x); f[2] = bf_lo(a.y); f[3] = bf_hi(a.y);
  }
  __device__ __forceinline__ float dot(const WChunk<F32> &w, float acc) const {
    acc = __builtin_fmaf(__uint_as_float(w.q.x), f[0], acc);
    acc = __builtin_fmaf(__uint_as_float(w.q.y), f[1], acc);
    acc = __builtin_fmaf(__uint_as_float(w.q.z), f[2], acc);
    return __builtin_fmaf(__uint_as_float(w.q.w), f[3], acc);
  }
};

// aff4 weights . bf16 x.  A code dword holds elements e0..e7 (nibble i at
// bits 4i).  OR-ing a nibble into the mantissa of bf16 128.0 (0x4300) gives
// 128 + q exactly, so (u >> 4t) & 0x000F000F | 0x43004300 is the bf16 pair
// (128 + q_t, 128 + q_{t+4}); x is re-paired to (x_t, x_{t+4}) to match.
//   sum q x = sum (128+q) x - 128 sum x, and w = s q + b, so the chunk adds
//   s * D + (b - 128 s) * X  with D = sum (128+q) x, X = sum x.
template <> struct XChunk<AFF4, BF16> {
  uint32_t d[16];
  float xs;
  __device__ __forceinline__ void load(const char *xrow, int ch) {
    const char *p = xrow + (size_t)ch * 64;
    float s = 0.f;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      u32x4 r = ld16(p + 16 * g);  // (x0,x1) (x2,x3) (x4,x5) (x6,x7)
      d[4 * g + 0] = (r.x & 0xFFFFu) | (r.z << 16);
      d[4 * g + 1] = (r.x >> 16) | (r.z & 0xFFFF0000u);
      d[4 * g + 2] = (r.y & 0xFFFFu) | (r.w << 16);
      d[4 * g + 3] = (r.y >> 16) | (r.w & 0xFFFF0000u);
      s = dot2(r.x, 0x3F803F80u, s);
      s = dot2(r.y, 0x3F803F80u, s);
      s = dot2(r.z, 0x3F803F80u, s);
      s = dot2(r.w, 0x3F803F80u, s);
    }
    xs = s;
  }
  __device__ __forceinline__ float dot(const WChunk<AFF4> &w, float acc) const {
    const uint32_t q[4] = {w.q.x, w.q.y, w.q.z, w.q.w};
    float D = 0.f;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        uint32_t n = ((q[g] >> (4 * t)) & 0x000F000Fu) | 0x43004300u;
        D = dot2(n, d[4 * g + t], D);
      }
    }
    acc = __builtin_fmaf(w.s, D, acc);
    return __builtin_fmaf(__builtin_fmaf(-128.0f, w.s, w.b), xs, acc);
  }
};

// aff4 weights . f32 x.
template <> struct XChunk<AFF4, F32> {
  float f[32];
  float xs;
  __device__ __forceinline__ void load(const char *xrow, int ch) {
    const char *p = xrow + (size_t)ch * 128;
    float s = 0.f;
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      u32x4 r = ld16(p + 16 * g);
      f[4 * g + 0] = __uint_as_float(r.x); f[4 * g + 1] = __uint_as_float(r.y);
      f[4 * g + 2] = __uint_as_float(r.z); f[4 * g + 3] = __uint_as_float(r.w);
    }
#pragma unroll
    for (int i = 0; i < 32; ++i) s += f[i];
    xs = s;
  }
  __device__ __forceinline__ float dot(const WChunk<AFF4> &w, float acc) const {
    const uint32_t q[4] = {w.q.x, w.q.y, w.q.z, w.q.w};
    float D = 0.f;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      uint32_t lo = q[g] & 0x0F0F0F0Fu, hi = (q[g] >> 4) & 0x0F0F0F0Fu;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        D = __builtin_fmaf((float)((lo >> (8 * b)) & 0xFFu), f[8 * g + 2 * b], D);
        D = __builtin_fmaf((float)((hi >> (8 * b)) & 0xFFu), f[8 * g + 2 * b + 1], D);
      }
    }
    acc = __builtin_fmaf(w.s, D, acc);
    return __builtin_fmaf(w.b, xs, acc);
  }
};

// mxfp4 weights . bf16 x: v_cvt_scalef32_pk_bf16_fp4 turns byte t of a code
// dword (elements 2t, 2t+1, low nibble first) into an exact bf16 pair that
// lines up with the raw x pair; the E8M0 scale multiplies the chunk sum.
template <> struct XChunk<MXFP4, BF16> {
  uint32_t d[16];
  __device__ __forceinline__ void load(const char *xrow, int ch) {
    const char *p = xrow + (size_t)ch * 64;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      u32x4 r = ld16(p + 16 * g);
      d[4 * g + 0] = r.x; d[4 * g + 1] = r.y; d[4 * g + 2] = r.z; d[4 * g + 3] = r.w;
    }
  }
  __device__ __forceinline__ float dot(const WChunk<MXFP4> &w, float acc) const {
    const uint32_t q[4] = {w.q.x, w.q.y, w.q.z, w.q.w};
    float S = 0.f;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      S = dot2(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q[g], 1.0f, 0)), d[4 * g + 0], S);
      S = dot2(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q[g], 1.0f, 1)), d[4 * g + 1], S);
      S = dot2(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q[g], 1.0f, 2)), d[4 * g + 2], S);
      S = dot2(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q[g], 1.0f, 3)), d[4 * g + 3], S);
    }
    return __builtin_fmaf(S, w.s, acc);
  }
};

// mxfp4 weights . f32 x.
template <> struct XChunk<MXFP4, F32> {
  float f[32];
  __device__ __forceinline__ void load(const char *xrow, int ch) {
    const char *p = xrow + (size_t)ch * 128;
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      u32x4 r = ld16(p + 16 * g);
      f[4 * g + 0] = __uint_as_float(r.x); f[4 * g + 1] = __uint_as_float(r.y);
      f[4 * g + 2] = __uint_as_float(r.z); f[4 * g + 3] = __uint_as_float(r.w);
    }
  }
  __device__ __forceinline__ float dot(const WChunk<MXFP4> &w, float acc) const {
    const uint32_t q[4] = {w.q.x, w.q.y, w.q.z, w.q.w};
    float S = 0.f;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        f32x2 v;
        if (t == 0) v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q[g], 1.0f, 0);
        if (t == 1) v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q[g], 1.0f, 1);
        if (t == 2) v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q[g], 1.0f, 2);
        if (t == 3) v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q[g], 1.0f, 3);
        S = __builtin_fmaf(v.x, f[8 * g + 2 * t], S);
        S = __builtin_fmaf(v.y, f[8 * g + 2 * t + 1], S);
      }
    }
    return __builtin_fmaf(S, w.s, acc);
  }
};


// ------------------------------------------------------ wave row x vector
//
// RG weight rows per lane group (each K = nchunks chunks long) against C
// vectors (xrow[c]).  The wave is split into 64/LPR lane groups; the caller
// passes in `rows` the RG rows of the calling lane's group.  Lane li of a
// group takes chunks li, li + LPR, ...; the loads of U chunk steps are issued
// together before any of them is used.  On return acc[t][c] holds, in every
// lane of the group, the full dot product of rows[t] with vector c.  The
// per-(row, vector) arithmetic does not depend on C, U or the other rows, so
// results are the same for every m.
template <int WF, int XF, int RG, int C, int LPR, int U>
__device__ __forceinline__ void wave_rows_dot(const Row<WF> (&rows)[RG], const char *const (&xrow)[C],
                                              int nchunks, float (&acc)[RG][C]) {
  const int li = threadIdx.x % LPR;
#pragma unroll
  for (int t = 0; t < RG; ++t)
#pragma unroll
    for (int c = 0; c < C; ++c) acc[t][c] = 0.f;
  for (int base = 0; base < nchunks; base += LPR * U) {
    WChunk<WF> w[U][RG];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int ch = base + li + u * LPR;
      if (ch < nchunks) {
#pragma unroll
        for (int t = 0; t < RG; ++t) w[u][t] = load_wchunk<WF>(rows[t], ch);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int ch = base + li + u * LPR;
      if (ch < nchunks) {
#pragma unroll
        for (int c = 0; c < C; ++c) {
          XChunk<WF, XF> xc;
          xc.load(xrow[c], ch);
#pragma unroll
          for (int t = 0; t < RG; ++t) acc[t][c] = xc.dot(w[u][t], acc[t][c]);
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < RG; ++t)
#pragma unroll
    for (int c = 0; c < C; ++c) acc[t][c] = group_total<LPR>(acc[t][c]);
}

// Chunk steps issued together: about 16 loads of 16 bytes per lane.
template <int RG> constexpr int unroll_for() { return RG >= 8 ? 2 : 4; }

template <int WF>
__device__ __forceinline__ size_t row_bytes(int K) {
  return (size_t)K * (WF == F32 ? 4 : WF == BF16 ? 2 : 1) / (WF >= AFF4 ? 2 : 1);
}

template <int WF>
__device__ __forceinline__ Row<WF> make_row(const void *w, const void *s, const void *b, int K, int n) {
  Row<WF> r;
  r.w = reinterpret_cast<const char *>(w) + (size_t)n * row_bytes<WF>(K);
  if constexpr (WF == AFF4) {
    r.s = reinterpret_cast<const uint16_t *>(s) + (size_t)n * (K / 64);
    r.b = reinterpret_cast<const uint16_t *>(b) + (size_t)n * (K / 64);
  } else if constexpr (WF == MXFP4) {
    r.s = reinterpret_cast<const uint8_t *>(s) + (size_t)n * (K / 32);
    r.b = nullptr;
  } else {
    r.s = r.b = nullptr;
  }
  return r;
}

__device__ __forceinline__ size_t act_bytes(int fmt) { return fmt == F32 ? 4 : 2; }

__device__ __forceinline__ const void *tbl(const uint64_t *t, int e) {
  return t ? reinterpret_cast<const void *>(t[e]) : nullptr;
}

// Routing results read back from the workspace, clamped so that even a
// corrupted workspace cannot send an access out of bounds.
__device__ __forceinline__ int active_slots(const Args &a) {
  const int n = a.active_count[0];
  return n < 0 ? 0 : (n > a.cap ? a.cap : n);
}
__device__ __forceinline__ int clamp_i(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

// ------------------------------------------------------------------ router
//
// Wave w of router item `item` computes router row e = 4*item + w (row E is
// the shared expert's gate vector w_g): logits[r, e] = sum_h x[r,h] W[e,h],
// every product and sum in double, for all m rows.
template <int ACT>
__device__ __forceinline__ void router_rows(const Args &a, int item) {
  constexpr int EPC = ACT == F32 ? 4 : 8;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int e = item * WPB + wave;
  const int nrows = a.E + ((a.flags & SHARED_GATED) ? 1 : 0);
  if (e >= nrows) return;
  const int nchunks = a.H / EPC;
  const size_t xstride = (size_t)a.H * act_bytes(ACT);
  const char *wrow = e < a.E ? reinterpret_cast<const char *>(a.router) + (size_t)e * xstride
                             : reinterpret_cast<const char *>(a.sgv);
  const char *x = reinterpret_cast<const char *>(a.x);
  const int LD = a.E + 1;
  for (int r0 = 0; r0 < a.m; r0 += 8) {
    double acc[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) acc[r] = 0.0;
    for (int ch = lane; ch < nchunks; ch += WAVE) {
      float w[EPC];
      const u32x4 q = ld16(wrow + (size_t)ch * 16);
      if constexpr (ACT == F32) {
        w[0] = __uint_as_float(q.x); w[1] = __uint_as_float(q.y);
        w[2] = __uint_as_float(q.z); w[3] = __uint_as_float(q.w);
      } else {
        w[0] = bf_lo(q.x); w[1] = bf_hi(q.x); w[2] = bf_lo(q.y); w[3] = bf_hi(q.y);
        w[4] = bf_lo(q.z); w[5] = bf_hi(q.z); w[6] = bf_lo(q.w); w[7] = bf_hi(q.w);
      }
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        if (r0 + r < a.m) {
          const u32x4 v = ld16(x + (size_t)(r0 + r) * xstride + (size_t)ch * 16);
          float xv[EPC];
          if constexpr (ACT == F32) {
            xv[0] = __uint_as_float(v.x); xv[1] = __uint_as_float(v.y);
            xv[2] = __uint_as_float(v.z); xv[3] = __uint_as_float(v.w);
          } else {
            xv[0] = bf_lo(v.x); xv[1] = bf_hi(v.x); xv[2] = bf_lo(v.y); xv[3] = bf_hi(v.y);
            xv[4] = bf_lo(v.z); xv[5] = bf_hi(v.z); xv[6] = bf_lo(v.w); xv[7] = bf_hi(v.w);
          }
#pragma unroll
          for (int i = 0; i < EPC; ++i) acc[r] = __builtin_fma((double)w[i], (double)xv[i], acc[r]);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      if (r0 + r < a.m) {
        const double t = wave_sum_f64(acc[r]);
        if (lane == 0) a.logits[(size_t)(r0 + r) * LD + e] = t;
      }
    }
  }
}

// Block-wide exclusive scan of one int per thread.
__device__ __forceinline__ int block_excl_scan(int v, int *s_wave, int *total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int d = 1; d < WAVE; d <<= 1) {
    const int o = __shfl_up(incl, d, WAVE);
    if (lane >= d) incl += o;
  }
  if (lane == WAVE - 1) s_wave[wave] = incl;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < WPB; ++w) {
    if (w < wave) base += s_wave[w];
    tot += s_wave[w];
  }
  __syncthreads();
  *total = tot;
  return base + incl - v;
}

// The route tail, run by one whole workgroup once every logit is written:
// per row (one wave per row) the top-k by key (ties to the lower index) and
// the weights, then the stable counting sort of the m*k pairs by expert.
__device__ __forceinline__ void route_tail(const Args &a) {
  constexpr int T = MAX_EXPERTS / WAVE;
  __shared__ int s_idx[MAX_PAIRS];
  __shared__ unsigned s_mask[MAX_EXPERTS];
  __shared__ int s_off[MAX_EXPERTS + 1];
  __shared__ int s_wave[WPB];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int E = a.E, k = a.K, m = a.m, LD = E + 1;
  const bool norm = (a.flags & NORM_TOPK) != 0;

  for (int r = wave; r < m; r += WPB) {
    const double *lr = a.logits + (size_t)r * LD;
    double lg[T], key[T];
    bool taken[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int e = lane + WAVE * t;
      taken[t] = e >= E;
      lg[t] = e < E ? lr[e] : 0.0;
      key[t] = lg[t];
      if (a.routing == ROUTE_SIGMOID_BIAS && e < E) key[t] = sigmoid_d(lg[t]) + (double)a.ebias[e];
    }
    // Slot j's expert and logit end up in lane j.
    int my_e = 0;
    double my_l = 0.0, lmax = 0.0;
    for (int j = 0; j < k; ++j) {
      double mk = -__builtin_inf();
#pragma unroll
      for (int t = 0; t < T; ++t)
        if (!taken[t]) mk = fmax(mk, key[t]);
      mk = wave_max_f64(mk);
      // Lowest index holding the maximum (ballots are wave-uniform).
      int win = -1;
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const unsigned long long b = __builtin_amdgcn_ballot_w64(!taken[t] && key[t] == mk);
        if (win < 0 && b) win = t * WAVE + __builtin_ctzll(b);
      }
      if (win < 0) {  // only NaN keys left: lowest index not yet taken
#pragma unroll
        for (int t = 0; t < T; ++t) {
          const unsigned long long b = __builtin_amdgcn_ballot_w64(!taken[t]);
          if (win < 0 && b) win = t * WAVE + __builtin_ctzll(b);
        }
      }
      win = __builtin_amdgcn_readfirstlane(win);
      const int wt = win >> 6, wl = win & 63;
      double lw = 0.0;
#pragma unroll
      for (int t = 0; t < T; ++t) {
        if (t == wt) {
          lw = lg[t];
          if (lane == wl) taken[t] = true;
        }
      }
      lw = readlane_f64(lw, wl);
      if (j == 0) lmax = lw;
      if (lane == j) {
        my_e = win;
        my_l = lw;
      }
    }
    // Weights, slot j in lane j (double).
    const bool mine = lane < k;
    double w;
    if (a.routing == ROUTE_SOFTMAX) {
      // softmax over all experts; with norm_topk_prob the full denominator
      // cancels and only the selected terms remain.
      const double num = mine ? exp(my_l - lmax) : 0.0;
      double den;
      if (norm) {
        den = wave_sum_f64(num);
      } else {
        double s = 0.0;
#pragma unroll
        for (int t = 0; t < T; ++t)
          if (lane + WAVE * t < E) s += exp(lg[t] - lmax);
        den = wave_sum_f64(s);
      }
      w = num / den;
    } else {
      w = mine ? sigmoid_d(my_l) : 0.0;   // unbiased: the bias only selects
      if (norm) w = w / wave_sum_f64(w);
    }
    if (mine) {
      const float wf = (float)(w * (double)a.rsf);
      const int p = r * k + lane;
      s_idx[p] = my_e;
      a.topk_idx[p] = my_e;
      a.topk_w[p] = wf;
      if (a.idx_out) a.idx_out[p] = my_e;
      if (a.w_out) a.w_out[p] = wf;
    }
    if (lane == 0 && (a.flags & SHARED_GATED)) a.row_gate[r] = (float)sigmoid_d(lr[E]);
  }
  __syncthreads();

  // Counting sort of the te = m*k pairs by expert, stable in pair order.  A
  // row selects an expert at most once, so bit r of s_mask[e] says whether row
  // r chose e; a pair's rank inside its expert is the number of earlier rows
  // that chose the same expert.
  const int te = m * k, tid = threadIdx.x;
  for (int e = tid; e < E; e += THREADS) s_mask[e] = 0u;
  __syncthreads();
  for (int p = tid; p < te; p += THREADS) atomicOr(&s_mask[s_idx[p]], 1u << (p / k));
  __syncthreads();
  const int cnt = tid < E ? __popc(s_mask[tid]) : 0;
  int total;
  const int excl = block_excl_scan(cnt, s_wave, &total);
  int nact;
  const int aexcl = block_excl_scan(cnt > 0 ? 1 : 0, s_wave, &nact);
  if (tid < E) {
    s_off[tid] = excl;
    a.offsets[tid] = excl;
    if (cnt > 0) a.active[aexcl] = tid;
  }
  if (tid == 0) {
    s_off[E] = total;
    a.offsets[E] = total;
    a.active_count[0] = nact;
  }
  __syncthreads();
  for (int p = tid; p < te; p += THREADS) {
    const int e = s_idx[p], r = p / k;
    const int pos = s_off[e] + __popc(s_mask[e] & ((1u << r) - 1u));
    a.sorted_pair[pos] = p;
    a.pair_to_perm[p] = pos;
  }
}

// One router item; the workgroup that finishes last runs the route tail.
// FUSED: the tail then publishes SYNC_READY.
template <int ACT, bool FUSED>
__device__ __forceinline__ void router_item(const Args &a, int item) {
  __shared__ unsigned s_ticket;
  router_rows<ACT>(a, item);
  release_agent();
  __syncthreads();
  if (threadIdx.x == 0)
    s_ticket = __hip_atomic_fetch_add(word(a.sync, SYNC_ROUTER), 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (s_ticket != (unsigned)(a.n_router - 1)) return;
  acquire_agent();
  route_tail(a);
  if (threadIdx.x == 0) *word(a.sync, SYNC_ROUTER) = 0u;  // every ticket is taken
  if constexpr (FUSED) wg_signal(a.sync, SYNC_READY);
}

// ---------------------------------------------------------------- gate/up
//
// One wave: intermediate rows [i0, i0 + NI) of one expert (gate and up), for
// the pairs p = pair(0..np-1) in passes of C; writes silu(g) * v.

template <int EF, int ACT, int C, int NI>
__device__ __forceinline__ void gate_up_rows(const Args &a, const void *gw, const void *uw,
                                             const void *gs, const void *us, const void *gb,
                                             const void *ub, int N, int i0, int off, int np,
                                             bool routed, float *dst, int ld) {
  constexpr int RG = 2 * NI;
  const int H = a.H, k = a.K;
  const size_t xstride = (size_t)H * act_bytes(ACT);
  const char *x = reinterpret_cast<const char *>(a.x);
  Row<EF> rows[RG];
#pragma unroll
  for (int t = 0; t < NI; ++t) {
    const int i = min(i0 + t, N - 1);
    rows[t] = make_row<EF>(gw, gs, gb, H, i);
    rows[NI + t] = make_row<EF>(uw, us, ub, H, i);
  }
  for (int c0 = 0; c0 < np; c0 += C) {
    const int nc = min(C, np - c0);
    const char *xrow[C];
    int pair[C];
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int q = c0 + min(c, nc - 1);
      pair[c] = routed ? clamp_i(a.sorted_pair[off + q], 0, a.te - 1) : q;
      xrow[c] = x + (size_t)(routed ? pair[c] / k : q) * xstride;
    }
    float acc[RG][C];
    wave_rows_dot<EF, ACT, RG, C, WAVE, unroll_for<RG>()>(rows, xrow, H / Fmt<EF>::EPC, acc);
    if ((threadIdx.x & 63) == 0) {
#pragma unroll
      for (int c = 0; c < C; ++c) {
        if (c < nc) {
          const bool scale = routed && (a.flags & WEIGHT_BEFORE);
          const float w = scale ? a.topk_w[pair[c]] : 1.0f;
#pragma unroll
          for (int t = 0; t < NI; ++t) {
            if (i0 + t < N) {
              float g = acc[t][c], v = acc[NI + t][c];
              if (scale) {  // W(w x) = w (W x): scale both pre-activations
                g *= w;
                v *= w;
              }
              dst[(size_t)(off + c0 + c) * ld + i0 + t] = silu_mul(g, v);
            }
          }
        }
      }
    }
  }
}

// Routed gate/up item: slot s = it / items_per_slot, its waves take row
// groups (it % items_per_slot) * 4 + wave.
template <int EF, int ACT, int C, bool FUSED>
__device__ __forceinline__ void routed_gu_item(const Args &a, int it) {
  constexpr int NI = gate_up_ni<EF>();
  const int s = it / a.gu_items_per_slot, b = it - s * a.gu_items_per_slot;
  if constexpr (FUSED) {
    if (!wg_wait(a.sync, SYNC_READY, 1u)) return;
  }
  if (s >= active_slots(a)) return;
  const int e = clamp_i(a.active[s], 0, a.E - 1);
  const int off = clamp_i(a.offsets[e], 0, a.te);
  const int np = clamp_i(a.offsets[e + 1], off, a.te) - off;
  const int i0 = (b * WPB + (threadIdx.x >> 6)) * NI;
  if (i0 < a.I)
    gate_up_rows<EF, ACT, C, NI>(a, tbl(a.gw, e), tbl(a.uw, e), tbl(a.gs, e), tbl(a.us, e),
                                 tbl(a.gb, e), tbl(a.ub, e), a.I, i0, off, np, true, a.act, a.I);
  if constexpr (FUSED) wg_signal(a.sync, SYNC_SLOT0 + s);
}

// Shared-expert gate/up item (act-format weights, unscaled rows of x).
template <int ACT, int C, bool FUSED>
__device__ __forceinline__ void shared_gu_item(const Args &a, int it) {
  constexpr int NI = gate_up_ni<ACT>();
  const int i0 = (it * WPB + (threadIdx.x >> 6)) * NI;
  if (i0 < a.Is)
    gate_up_rows<ACT, ACT, C, NI>(a, a.sgw, a.suw, nullptr, nullptr, nullptr, nullptr, a.Is, i0, 0,
                                  a.m, false, a.sact, a.Is);
  if constexpr (FUSED) wg_signal(a.sync, SYNC_SHARED);
}

// --------------------------------------------------------- down + blend
//
// Down tile `tile`: output columns [h0, h0 + HT), HT = DOWN_RD * down_dq.
// Sub-unit (u, q) is unit u (an active slot, or the shared expert last) and
// row block q; waves take sub-units round-robin, y per pair goes to LDS, then
//   out[r, h] = sum_j c_rj y[perm(r, j), h] + gamma_r ys[r, h]
// in slot order.
template <int EF, int ACT, int CR, int CS, int LPR, bool FUSED>
__device__ __forceinline__ void down_item(const Args &a, int tile) {
  constexpr int GR = WAVE / LPR;                 // routed rows in parallel per wave
  constexpr int RGR = DOWN_RD / GR;              // routed rows per lane group
  static_assert(DOWN_RD % GR == 0, "down rows must split over lane groups");
  __shared__ float y_lds[MAX_PAIRS * MAX_DOWN_TILE];
  __shared__ float ys_lds[MAX_ROWS * MAX_DOWN_TILE];
  __shared__ int s_fail;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int H = a.H, I = a.I, Is = a.Is, m = a.m;
  const int DQ = a.down_dq, HT = DOWN_RD * DQ, h0 = tile * HT;
  if constexpr (FUSED) {
    if (!wg_wait(a.sync, SYNC_READY, 1u)) return;
  }
  if (threadIdx.x == 0) s_fail = 0;
  __syncthreads();
  const int nact = active_slots(a);
  const bool shared = (a.flags & SHARED) != 0;
  const int units = nact + (shared ? 1 : 0);

  for (int su = wave; su < units * DQ; su += WPB) {
    const int u = su / DQ, q = su - u * DQ;
    const int hb = h0 + q * DOWN_RD;             // first column of this row block
    if (u < nact) {
      if constexpr (FUSED) {
        if (!wave_wait(a.sync, SYNC_SLOT0 + u, (unsigned)a.gu_items_per_slot)) {
          if (lane == 0) s_fail = 1;
          continue;
        }
      }
      const int e = clamp_i(a.active[u], 0, a.E - 1);
      const int off = clamp_i(a.offsets[e], 0, a.te);
      const int np = clamp_i(a.offsets[e + 1], off, a.te) - off;
      const void *dw = tbl(a.dw, e), *ds = tbl(a.ds, e), *db = tbl(a.db, e);
      const int grp = lane / LPR;
      Row<EF> rows[RGR];
#pragma unroll
      for (int t = 0; t < RGR; ++t) rows[t] = make_row<EF>(dw, ds, db, I, min(hb + grp + GR * t, H - 1));
      for (int c0 = 0; c0 < np; c0 += CR) {
        const int nc = min(CR, np - c0);
        const char *xrow[CR];
#pragma unroll
        for (int c = 0; c < CR; ++c)
          xrow[c] = reinterpret_cast<const char *>(a.act + (size_t)(off + c0 + min(c, nc - 1)) * I);
        float acc[RGR][CR];
        wave_rows_dot<EF, F32, RGR, CR, LPR, unroll_for<RGR>()>(rows, xrow, I / Fmt<EF>::EPC, acc);
        if (lane % LPR == 0) {
#pragma unroll
          for (int t = 0; t < RGR; ++t)
#pragma unroll
            for (int c = 0; c < CR; ++c)
              if (c < nc) y_lds[(off + c0 + c) * HT + q * DOWN_RD + grp + GR * t] = acc[t][c];
        }
      }
    } else {
      if constexpr (FUSED) {
        if (!wave_wait(a.sync, SYNC_SHARED, (unsigned)a.n_shared_gu)) {
          if (lane == 0) s_fail = 1;
          continue;
        }
      }
      Row<ACT> rows[DOWN_RD];
#pragma unroll
      for (int t = 0; t < DOWN_RD; ++t) rows[t] = make_row<ACT>(a.sdw, nullptr, nullptr, Is, min(hb + t, H - 1));
      for (int c0 = 0; c0 < m; c0 += CS) {
        const int nc = min(CS, m - c0);
        const char *xrow[CS];
#pragma unroll
        for (int c = 0; c < CS; ++c)
          xrow[c] = reinterpret_cast<const char *>(a.sact + (size_t)(c0 + min(c, nc - 1)) * Is);
        float acc[DOWN_RD][CS];
        wave_rows_dot<ACT, F32, DOWN_RD, CS, WAVE, unroll_for<DOWN_RD>()>(rows, xrow, Is / Fmt<ACT>::EPC, acc);
        if (lane == 0) {
#pragma unroll
          for (int t = 0; t < DOWN_RD; ++t)
#pragma unroll
            for (int c = 0; c < CS; ++c)
              if (c < nc) ys_lds[(c0 + c) * HT + q * DOWN_RD + t] = acc[t][c];
        }
      }
    }
  }
  __syncthreads();

  if (s_fail == 0) {
    const bool before = (a.flags & WEIGHT_BEFORE) != 0;
    const bool gated = (a.flags & SHARED_GATED) != 0;
    const bool out_f32 = (a.flags & OUT_F32) != 0 || ACT == F32;
    const int k = a.K;
    for (int t = threadIdx.x; t < m * HT; t += THREADS) {
      const int r = t / HT, hl = t - r * HT, h = h0 + hl;
      if (h >= H) continue;
      float o = 0.f;
      for (int j = 0; j < k; ++j) {
        const int p = r * k + j;
        const float c = before ? 1.0f : a.topk_w[p];
        o = __builtin_fmaf(c, y_lds[clamp_i(a.pair_to_perm[p], 0, a.te - 1) * HT + hl], o);
      }
      if (shared) o = __builtin_fmaf(gated ? a.row_gate[r] : 1.0f, ys_lds[r * HT + hl], o);
      if (out_f32)
        reinterpret_cast<float *>(a.out)[(size_t)r * H + h] = o;
      else
        reinterpret_cast<uint16_t *>(a.out)[(size_t)r * H + h] = f32_to_bf16(o);
    }
  }
  __syncthreads();  // LDS is reused by the next item
}

// ------------------------------------------------------------------ kernels

// The whole layer in one persistent launch (items claimed in queue order).
// NOT LAUNCHED: on MI355X its first launch did not finish (twice, the second
// time with every wait bounded in wall-clock time); the cause is not yet
// identified, so the host refuses this arrangement and nothing instantiates
// it.
template <int EF, int ACT, int CR, int CS, int LPR>
__global__ __launch_bounds__(THREADS) void fused_kernel(Args a) {
  __shared__ int s_item;
  for (;;) {
    if (threadIdx.x == 0) s_item = (int)atomicAdd(word(a.sync, SYNC_NEXT), 1u);
    __syncthreads();
    int item = s_item;
    __syncthreads();
    if (item >= a.n_items) break;
    if (item < a.n_router) {
      router_item<ACT, true>(a, item);
      continue;
    }
    item -= a.n_router;
    if (item < a.n_shared_gu) {
      shared_gu_item<ACT, CS, true>(a, item);
      continue;
    }
    item -= a.n_shared_gu;
    if (item < a.n_routed_gu) {
      routed_gu_item<EF, ACT, CR, true>(a, item);
      continue;
    }
    item -= a.n_routed_gu;
    down_item<EF, ACT, CR, CS, LPR, true>(a, item);
  }
  // The last workgroup out resets the completion words for the next call
  // (SYNC_ERR stays as it is).
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned done =
        __hip_atomic_fetch_add(word(a.sync, SYNC_EXIT), 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    if (done == gridDim.x - 1) {
      *word(a.sync, SYNC_NEXT) = 0u;
      *word(a.sync, SYNC_ROUTER) = 0u;
      *word(a.sync, SYNC_READY) = 0u;
      *word(a.sync, SYNC_EXIT) = 0u;
      *word(a.sync, SYNC_SHARED) = 0u;
      for (int s = 0; s < a.cap; ++s) *word(a.sync, SYNC_SLOT0 + s) = 0u;
      release_agent();
    }
  }
}

// The items as three ordinary kernels.  The shared expert's gate/up does not
// depend on routing, so its items run beside the router items in the first
// launch.
template <int ACT, int CS>
__global__ __launch_bounds__(THREADS) void route_kernel(Args a) {
  const int item = blockIdx.x;
  if (item < a.n_router)
    router_item<ACT, false>(a, item);
  else
    shared_gu_item<ACT, CS, false>(a, item - a.n_router);
}

template <int EF, int ACT, int CR, int CS>
__global__ __launch_bounds__(THREADS) void gate_up_kernel(Args a) {
  routed_gu_item<EF, ACT, CR, false>(a, blockIdx.x);
}

template <int EF, int ACT, int CR, int CS, int LPR>
__global__ __launch_bounds__(THREADS) void down_blend_kernel(Args a) {
  down_item<EF, ACT, CR, CS, LPR, false>(a, blockIdx.x);
}

}  // namespace moe
