// moe_kernels.hpp -- gfx950 device code of the decode MoE layer.
//
// Three kernels per forward, on the caller's stream:
//   route_kernel      router GEMV (fp64 accumulation) spread over many waves;
//                     the last workgroup to finish scores, selects top-k,
//                     computes the routing weights and counting-sorts the
//                     (row, slot) pairs by expert in LDS.
//   gate_up_kernel    one wave per (active expert, group of intermediate
//                     rows): streams the gate and up rows of the expert once
//                     for all of its pairs, dequantises in registers, writes
//                     silu(g)*v per pair.  The shared expert's gate/up rows
//                     are extra waves of the same launch.
//   down_blend_kernel one workgroup per tile of output columns: streams the
//                     down rows of every active expert (and the shared
//                     expert) for the tile, keeps y per pair in LDS and
//                     blends the slots in slot order.
//
// Pages: metrale "forward_bf16_grouped_decode.rs" (the five steps and their
// buffers), mlxcel "perf(moe): wire lfm2 to the fused decode-MoE kernel"
// (sigmoid routing with expert_bias, norm_topk_prob, routed_scaling_factor),
// iron "refactor(gemm): split the gemv_q8 grab-bag by family" (biased
// selection, unbiased weight), frink "routed_weight_site.rs" (weight on the
// input vs the output, raw-logit top-k), metrale "helpers_a.rs" (packed
// [N, K/2] weights, [N, K/group] scales, E8M0 block 32).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

enum : int { F32 = 0, BF16 = 1, AFF4 = 2, MXFP4 = 3 };
enum : int { ROUTE_SOFTMAX = 0, ROUTE_SIGMOID_BIAS = 1, ROUTE_SIGMOID_LOGIT = 2 };
enum : unsigned { NORM_TOPK = 1u, WEIGHT_BEFORE = 2u, SHARED = 4u, SHARED_GATED = 8u, OUT_F32 = 16u };

constexpr int WAVE = 64;
constexpr int MAX_ROWS = 32;
constexpr int MAX_TOPK = 16;
constexpr int MAX_EXPERTS = 256;
constexpr int MAX_PAIRS = MAX_ROWS * MAX_TOPK;
constexpr int ROUTE_THREADS = 512;      // 8 waves
constexpr int GEMV_THREADS = 256;       // 4 waves
constexpr int GATE_UP_ROWS = 8;         // weight rows per wave in gate_up: 4 gate + 4 up
constexpr int DOWN_TILE = 8;            // output columns per down_blend workgroup

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Everything a forward's kernels read or write (kernel argument, by value).
struct Args {
  int H, E, K, I, Is, m, te, cap, act_fmt, expert_fmt, routing;
  unsigned flags;
  float rsf;
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
  unsigned *sync;          // [16]
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

template <typename T>
__device__ __forceinline__ T xor_shfl(T v, int mask) {
  return __shfl_xor(v, mask, WAVE);
}

// Sum over the `width` consecutive lanes of a group; every lane of the group
// gets the total.  Fixed butterfly order: deterministic.
template <int WIDTH>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int mask = 1; mask < WIDTH; mask <<= 1) v += xor_shfl(v, mask);
  return v;
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
// RW weight rows (each K = nchunks chunks long) against C vectors
// (xrow[c]).  The wave is split into G = 64/LPR lane groups; group g takes
// rows g, g + G, ... of the RW, and the caller passes in `rows` only the
// RW/G rows of the calling lane's group (rows[t] = row g + G*t), so no array
// is indexed by a lane-dependent value.  Lane li of a group takes chunks li,
// li + LPR, ...  On return acc[t][c] holds, in every lane of the group, the
// full dot product of row g + G*t with vector c.  The per-(row, vector)
// arithmetic does not depend on C or on the other rows, so results are the
// same for every m.
template <int WF, int XF, int RW, int C, int LPR>
__device__ __forceinline__ void wave_rows_dot(const Row<WF> (&rows)[RW / (WAVE / LPR)],
                                              const char *const (&xrow)[C], int nchunks, int lane,
                                              float (&acc)[RW / (WAVE / LPR)][C]) {
  constexpr int G = WAVE / LPR;
  constexpr int RG = RW / G;
  static_assert(RW % G == 0, "rows must split evenly over lane groups");
  const int li = lane % LPR;
#pragma unroll
  for (int t = 0; t < RG; ++t)
#pragma unroll
    for (int c = 0; c < C; ++c) acc[t][c] = 0.f;
  for (int ch = li; ch < nchunks; ch += LPR) {
    WChunk<WF> w[RG];
#pragma unroll
    for (int t = 0; t < RG; ++t) w[t] = load_wchunk<WF>(rows[t], ch);
#pragma unroll
    for (int c = 0; c < C; ++c) {
      XChunk<WF, XF> xc;
      xc.load(xrow[c], ch);
#pragma unroll
      for (int t = 0; t < RG; ++t) acc[t][c] = xc.dot(w[t], acc[t][c]);
    }
  }
#pragma unroll
  for (int t = 0; t < RG; ++t)
#pragma unroll
    for (int c = 0; c < C; ++c) acc[t][c] = group_sum<LPR>(acc[t][c]);
}

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

// ----------------------------------------------------------- route kernel

__device__ __forceinline__ double sigmoid_d(double v) { return 1.0 / (1.0 + exp(-v)); }

// Block-wide exclusive scan of one int per thread (ROUTE_THREADS threads).
__device__ __forceinline__ int block_excl_scan(int v, int *s_wave, int *total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int d = 1; d < WAVE; d <<= 1) {
    int o = __shfl_up(incl, d, WAVE);
    if (lane >= d) incl += o;
  }
  if (lane == WAVE - 1) s_wave[wave] = incl;
  __syncthreads();
  int base = 0, tot = 0;
  for (int w = 0; w < ROUTE_THREADS / WAVE; ++w) {
    if (w < wave) base += s_wave[w];
    tot += s_wave[w];
  }
  __syncthreads();
  *total = tot;
  return base + incl - v;
}

template <int ACT>
__global__ __launch_bounds__(ROUTE_THREADS) void route_kernel(Args a) {
  constexpr int NW = ROUTE_THREADS / WAVE;
  constexpr int EPC = ACT == F32 ? 4 : 8;        // x / router elements per 16-byte chunk
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int H = a.H, E = a.E, m = a.m, LD = E + 1;
  const int nrows = E + ((a.flags & SHARED_GATED) ? 1 : 0);
  const int nchunks = H / EPC;
  const size_t xstride = (size_t)H * act_bytes(ACT);

  // ---- router GEMV: one router row per wave, fp64 accumulation ---------
  const int e = blockIdx.x * NW + wave;
  if (e < nrows) {
    const char *wrow = e < E ? reinterpret_cast<const char *>(a.router) + (size_t)e * xstride
                             : reinterpret_cast<const char *>(a.sgv);
    for (int r0 = 0; r0 < m; r0 += 8) {
      double acc[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) acc[r] = 0.0;
      for (int ch = lane; ch < nchunks; ch += WAVE) {
        float w[EPC];
        u32x4 q = ld16(wrow + (size_t)ch * 16);
        if constexpr (ACT == F32) {
          w[0] = __uint_as_float(q.x); w[1] = __uint_as_float(q.y);
          w[2] = __uint_as_float(q.z); w[3] = __uint_as_float(q.w);
        } else {
          w[0] = bf_lo(q.x); w[1] = bf_hi(q.x); w[2] = bf_lo(q.y); w[3] = bf_hi(q.y);
          w[4] = bf_lo(q.z); w[5] = bf_hi(q.z); w[6] = bf_lo(q.w); w[7] = bf_hi(q.w);
        }
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          if (r0 + r < m) {
            u32x4 v = ld16(reinterpret_cast<const char *>(a.x) + (size_t)(r0 + r) * xstride + (size_t)ch * 16);
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
        double v = acc[r];
#pragma unroll
        for (int mask = 1; mask < WAVE; mask <<= 1) v += xor_shfl(v, mask);
        if (lane == 0 && r0 + r < m) a.logits[(size_t)(r0 + r) * LD + e] = v;
      }
    }
  }

  // ---- the last workgroup to finish does top-k and the sort -----------
  __shared__ unsigned s_ticket;
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) s_ticket = atomicAdd(&a.sync[0], 1u);
  __syncthreads();
  if (s_ticket != gridDim.x - 1) return;
  __threadfence();

  __shared__ int s_idx[MAX_PAIRS];
  __shared__ float s_w[MAX_PAIRS];
  __shared__ unsigned s_mask[MAX_EXPERTS];
  __shared__ int s_off[MAX_EXPERTS + 1];
  __shared__ int s_wave[NW];
  const int k = a.K;

  // Top-k per row: one wave per row.  Lane l holds experts l, l+64, ...
  for (int r = wave; r < m; r += NW) {
    const double *lr = a.logits + (size_t)r * LD;
    double lg[MAX_EXPERTS / WAVE], key[MAX_EXPERTS / WAVE];
    bool taken[MAX_EXPERTS / WAVE];
#pragma unroll
    for (int t = 0; t < MAX_EXPERTS / WAVE; ++t) {
      const int ee = lane + WAVE * t;
      taken[t] = ee >= E;
      lg[t] = ee < E ? lr[ee] : 0.0;
      key[t] = lg[t];
      if (a.routing == ROUTE_SIGMOID_BIAS && ee < E) key[t] = sigmoid_d(lg[t]) + (double)a.ebias[ee];
    }
    double sel_l[MAX_TOPK];
    int sel_e[MAX_TOPK];
    for (int j = 0; j < k; ++j) {
      // lane-local best (ties to the lower index, i.e. lower t)
      double bk = 0.0;
      int be = -1;
#pragma unroll
      for (int t = 0; t < MAX_EXPERTS / WAVE; ++t)
        if (!taken[t] && (be < 0 || key[t] > bk)) { bk = key[t]; be = lane + WAVE * t; }
#pragma unroll
      for (int mask = 1; mask < WAVE; mask <<= 1) {
        double ok = xor_shfl(bk, mask);
        int oe = xor_shfl(be, mask);
        bool better = oe >= 0 && (be < 0 || ok > bk || (ok == bk && oe < be));
        if (better) { bk = ok; be = oe; }
      }
      // Lane 0's winner for everyone (the butterfly already agrees unless a
      // key is NaN; this keeps a row's experts distinct even then).
      be = __shfl(be, 0, WAVE);
      // Owner marks it taken; everyone learns its logit.
      const int owner = be & 63, tt = be >> 6;
      double lsel = 0.0;
#pragma unroll
      for (int t = 0; t < MAX_EXPERTS / WAVE; ++t)
        if (t == tt) lsel = lg[t];
      lsel = __shfl(lsel, owner, WAVE);
      if (lane == owner) {
#pragma unroll
        for (int t = 0; t < MAX_EXPERTS / WAVE; ++t)
          if (t == tt) taken[t] = true;
      }
      sel_e[j] = be;
      sel_l[j] = lsel;
    }
    // Weights (double), then float.
    double den_all = 0.0;
    if (a.routing == ROUTE_SOFTMAX && !(a.flags & NORM_TOPK)) {
      const double lmax = sel_l[0];
      double s = 0.0;
#pragma unroll
      for (int t = 0; t < MAX_EXPERTS / WAVE; ++t)
        if (lane + WAVE * t < E) s += exp(lg[t] - lmax);
#pragma unroll
      for (int mask = 1; mask < WAVE; mask <<= 1) s += xor_shfl(s, mask);
      den_all = s;
    }
    if (lane == 0) {
      double w[MAX_TOPK];
      if (a.routing == ROUTE_SOFTMAX) {
        const double lmax = sel_l[0];
        double s = 0.0;
        for (int j = 0; j < k; ++j) { w[j] = exp(sel_l[j] - lmax); s += w[j]; }
        const double den = (a.flags & NORM_TOPK) ? s : den_all;
        for (int j = 0; j < k; ++j) w[j] = w[j] / den;
      } else {
        double s = 0.0;
        for (int j = 0; j < k; ++j) { w[j] = sigmoid_d(sel_l[j]); s += w[j]; }
        if (a.flags & NORM_TOPK)
          for (int j = 0; j < k; ++j) w[j] = w[j] / s;
      }
      for (int j = 0; j < k; ++j) {
        const float wf = (float)(w[j] * (double)a.rsf);
        const int p = r * k + j;
        s_idx[p] = sel_e[j];
        s_w[p] = wf;
        a.topk_idx[p] = sel_e[j];
        a.topk_w[p] = wf;
        if (a.idx_out) a.idx_out[p] = sel_e[j];
        if (a.w_out) a.w_out[p] = wf;
      }
      if (a.flags & SHARED_GATED) a.row_gate[r] = (float)sigmoid_d(lr[E]);
    }
  }
  __syncthreads();

  // Counting sort of the te = m*k pairs by expert, stable in pair order.
  // A row selects an expert at most once, so bit r of s_mask[e] says whether
  // row r chose e; a pair's rank inside its expert is the number of earlier
  // rows that chose the same expert.
  const int te = m * k, tid = threadIdx.x;
  for (int ee = tid; ee < E; ee += ROUTE_THREADS) s_mask[ee] = 0u;
  __syncthreads();
  for (int p = tid; p < te; p += ROUTE_THREADS) atomicOr(&s_mask[s_idx[p]], 1u << (p / k));
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
  for (int p = tid; p < te; p += ROUTE_THREADS) {
    const int ee = s_idx[p], r = p / k;
    const int pos = s_off[ee] + __popc(s_mask[ee] & ((1u << r) - 1u));
    a.sorted_pair[pos] = p;
    a.pair_to_perm[p] = pos;
  }
  if (tid == 0) a.sync[0] = 0u;  // ready for the next call
}

// -------------------------------------------------------- gate/up kernel
//
// Waves [0, cap*gpe): routed expert slot s = wave / gpe (skipped if s is not
// an active slot), intermediate rows [(wave % gpe) * 4, +4).  Waves after
// that: the shared expert's rows, for all m rows of x.
template <int EF, int ACT, int CR, int CS>
__global__ __launch_bounds__(GEMV_THREADS) void gate_up_kernel(Args a) {
  constexpr int NI = GATE_UP_ROWS / 2;
  const int lane = threadIdx.x & 63;
  const int gwave = blockIdx.x * (GEMV_THREADS / WAVE) + (threadIdx.x >> 6);
  const int H = a.H, I = a.I, k = a.K;
  const size_t xstride = (size_t)H * act_bytes(ACT);
  const char *x = reinterpret_cast<const char *>(a.x);
  const int gpe = (I + NI - 1) / NI;
  const int routed_waves = a.cap * gpe;

  if (gwave < routed_waves) {
    const int s = gwave / gpe, i0 = (gwave - s * gpe) * NI;
    if (s >= a.active_count[0]) return;
    const int e = a.active[s];
    const int off = a.offsets[e], np = a.offsets[e + 1] - off;
    const void *gw = reinterpret_cast<const void *>(a.gw[e]);
    const void *uw = reinterpret_cast<const void *>(a.uw[e]);
    const void *gs = a.gs ? reinterpret_cast<const void *>(a.gs[e]) : nullptr;
    const void *us = a.us ? reinterpret_cast<const void *>(a.us[e]) : nullptr;
    const void *gb = a.gb ? reinterpret_cast<const void *>(a.gb[e]) : nullptr;
    const void *ub = a.ub ? reinterpret_cast<const void *>(a.ub[e]) : nullptr;
    Row<EF> rows[GATE_UP_ROWS];
#pragma unroll
    for (int t = 0; t < NI; ++t) {
      const int i = min(i0 + t, I - 1);
      rows[t] = make_row<EF>(gw, gs, gb, H, i);
      rows[NI + t] = make_row<EF>(uw, us, ub, H, i);
    }
    for (int c0 = 0; c0 < np; c0 += CR) {
      const int nc = min(CR, np - c0);
      const char *xrow[CR];
      int pair[CR];
#pragma unroll
      for (int c = 0; c < CR; ++c) {
        pair[c] = a.sorted_pair[off + c0 + min(c, nc - 1)];
        xrow[c] = x + (size_t)(pair[c] / k) * xstride;
      }
      float acc[GATE_UP_ROWS][CR];
      wave_rows_dot<EF, ACT, GATE_UP_ROWS, CR, WAVE>(rows, xrow, H / Fmt<EF>::EPC, lane, acc);
      if (lane == 0) {
#pragma unroll
        for (int c = 0; c < CR; ++c) {
          if (c < nc) {
            const float w = (a.flags & WEIGHT_BEFORE) ? a.topk_w[pair[c]] : 1.0f;
#pragma unroll
            for (int t = 0; t < NI; ++t) {
              if (i0 + t < I) {
                float g = acc[t][c], v = acc[NI + t][c];
                if (a.flags & WEIGHT_BEFORE) { g *= w; v *= w; }
                a.act[(size_t)(off + c0 + c) * I + i0 + t] = silu_mul(g, v);
              }
            }
          }
        }
      }
    }
    return;
  }

  // Shared expert (act format weights, unscaled rows).
  const int Is = a.Is;
  const int i0 = (gwave - routed_waves) * NI;
  if (!(a.flags & SHARED) || i0 >= Is) return;
  Row<ACT> rows[GATE_UP_ROWS];
#pragma unroll
  for (int t = 0; t < NI; ++t) {
    const int i = min(i0 + t, Is - 1);
    rows[t] = make_row<ACT>(a.sgw, nullptr, nullptr, H, i);
    rows[NI + t] = make_row<ACT>(a.suw, nullptr, nullptr, H, i);
  }
  for (int c0 = 0; c0 < a.m; c0 += CS) {
    const int nc = min(CS, a.m - c0);
    const char *xrow[CS];
#pragma unroll
    for (int c = 0; c < CS; ++c) xrow[c] = x + (size_t)(c0 + min(c, nc - 1)) * xstride;
    float acc[GATE_UP_ROWS][CS];
    wave_rows_dot<ACT, ACT, GATE_UP_ROWS, CS, WAVE>(rows, xrow, H / Fmt<ACT>::EPC, lane, acc);
    if (lane == 0) {
#pragma unroll
      for (int c = 0; c < CS; ++c)
        if (c < nc)
#pragma unroll
          for (int t = 0; t < NI; ++t)
            if (i0 + t < Is)
              a.sact[(size_t)(c0 + c) * Is + i0 + t] = silu_mul(acc[t][c], acc[NI + t][c]);
    }
  }
}

// ----------------------------------------------------- down+blend kernel
//
// Workgroup b owns output columns [b*DOWN_TILE, +DOWN_TILE).  Its waves take
// work units round-robin: unit u < active_count is active expert slot u (its
// down rows for the tile, for all of its pairs); unit active_count is the
// shared expert.  y per pair and ys per row land in LDS; then the threads
// blend  out[r, h] = sum_j c_rj y[perm(r, j), h] + gamma_r ys[r, h]  in slot
// order.
template <int EF, int ACT, int CR, int CS, int LPR>
__global__ __launch_bounds__(GEMV_THREADS) void down_blend_kernel(Args a) {
  constexpr int HT = DOWN_TILE;
  constexpr int GR = WAVE / LPR;        // lane groups (rows in parallel) for routed rows
  constexpr int GS = 1;                 // shared rows use full-wave groups
  __shared__ float y_lds[MAX_PAIRS * HT];
  __shared__ float ys_lds[MAX_ROWS * HT];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int H = a.H, I = a.I, k = a.K, m = a.m;
  const int h0 = blockIdx.x * HT;
  const int nact = a.active_count[0];
  const bool shared = (a.flags & SHARED) != 0;
  const int units = nact + (shared ? 1 : 0);

  for (int u = wave; u < units; u += GEMV_THREADS / WAVE) {
    if (u < nact) {
      const int e = a.active[u];
      const int off = a.offsets[e], np = a.offsets[e + 1] - off;
      const void *dw = reinterpret_cast<const void *>(a.dw[e]);
      const void *ds = a.ds ? reinterpret_cast<const void *>(a.ds[e]) : nullptr;
      const void *db = a.db ? reinterpret_cast<const void *>(a.db[e]) : nullptr;
      Row<EF> rows[HT / GR];
      const int grp = lane / LPR;
#pragma unroll
      for (int t = 0; t < HT / GR; ++t)
        rows[t] = make_row<EF>(dw, ds, db, I, min(h0 + grp + GR * t, H - 1));
      for (int c0 = 0; c0 < np; c0 += CR) {
        const int nc = min(CR, np - c0);
        const char *xrow[CR];
#pragma unroll
        for (int c = 0; c < CR; ++c)
          xrow[c] = reinterpret_cast<const char *>(a.act + (size_t)(off + c0 + min(c, nc - 1)) * I);
        float acc[HT / GR][CR];
        wave_rows_dot<EF, F32, HT, CR, LPR>(rows, xrow, I / Fmt<EF>::EPC, lane, acc);
        if (lane % LPR == 0) {
          const int g = lane / LPR;
#pragma unroll
          for (int t = 0; t < HT / GR; ++t)
#pragma unroll
            for (int c = 0; c < CR; ++c)
              if (c < nc) y_lds[(off + c0 + c) * HT + g + GR * t] = acc[t][c];
        }
      }
    } else {
      const int Is = a.Is;
      Row<ACT> rows[HT];
#pragma unroll
      for (int t = 0; t < HT; ++t) rows[t] = make_row<ACT>(a.sdw, nullptr, nullptr, Is, min(h0 + t, H - 1));
      for (int c0 = 0; c0 < m; c0 += CS) {
        const int nc = min(CS, m - c0);
        const char *xrow[CS];
#pragma unroll
        for (int c = 0; c < CS; ++c)
          xrow[c] = reinterpret_cast<const char *>(a.sact + (size_t)(c0 + min(c, nc - 1)) * Is);
        float acc[HT / GS][CS];
        wave_rows_dot<ACT, F32, HT, CS, WAVE>(rows, xrow, Is / Fmt<ACT>::EPC, lane, acc);
        if (lane == 0) {
#pragma unroll
          for (int t = 0; t < HT; ++t)
#pragma unroll
            for (int c = 0; c < CS; ++c)
              if (c < nc) ys_lds[(c0 + c) * HT + t] = acc[t][c];
        }
      }
    }
  }
  __syncthreads();

  const bool before = (a.flags & WEIGHT_BEFORE) != 0;
  const bool gated = (a.flags & SHARED_GATED) != 0;
  const bool out_f32 = (a.flags & OUT_F32) != 0 || ACT == F32;
  for (int t = threadIdx.x; t < m * HT; t += GEMV_THREADS) {
    const int r = t / HT, hl = t - r * HT, h = h0 + hl;
    if (h >= H) continue;
    float o = 0.f;
    for (int j = 0; j < k; ++j) {
      const int p = r * k + j;
      const float c = before ? 1.0f : a.topk_w[p];
      o = __builtin_fmaf(c, y_lds[a.pair_to_perm[p] * HT + hl], o);
    }
    if (shared) o = __builtin_fmaf(gated ? a.row_gate[r] : 1.0f, ys_lds[r * HT + hl], o);
    if (out_f32)
      reinterpret_cast<float *>(a.out)[(size_t)r * H + h] = o;
    else
      reinterpret_cast<uint16_t *>(a.out)[(size_t)r * H + h] = f32_to_bf16(o);
  }
}

}  // namespace moe
