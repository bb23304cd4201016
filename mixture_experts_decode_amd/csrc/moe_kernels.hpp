// moe_kernels.hpp -- gfx950 device code of the decode MoE layer.
//
// The layer runs as three kernels on the caller's stream, each made of
// 256-thread work items:
//   route_kernel     router units (router row x block of 8 input rows, fp64
//                    accumulation) writing the logits, and -- since it needs
//                    no routing -- the shared expert's gate/up rows.
//   gate_up_kernel   every workgroup rebuilds the routing from the logits in
//                    LDS (top-k per row, weights, stable counting sort by
//                    expert; block 0 publishes it), then streams the gate and
//                    up rows of its (active-expert slot, row block) once for
//                    all of the slot's pairs, dequantised in registers, and
//                    writes silu(g)*v per pair.
//   down_blend_kernel  a tile of output columns: the down rows of every
//                    active expert and of the shared expert for the tile, y
//                    per pair in LDS, then the slot-order blend.
// No workgroup ever waits for another; the kernel boundaries order the steps.
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

#include <type_traits>

namespace moe {

enum : int { F32 = 0, BF16 = 1, AFF4 = 2, MXFP4 = 3, NVFP4 = 4, FP8 = 5 };
// x format of the down projection's input for 4-bit experts: f32, each row
// stored sub-step-major (element i of the row at ((i % 32) / 8) * (I / 4) +
// (i / 32) * 8 + i % 8), so that in sub-step g adjacent lanes (adjacent
// 32-element chunks) read adjacent 32-byte blocks.
enum : int { F32P = 16 };
// F32I: an f32 vector stored, 4 bytes per element, as the bf16 pair the
// matrix-core products take -- the value's high half (its top 16 bits) in
// the low 16 bits, the bf16 rounding of the rest in the high 16 -- written
// once where the vector is produced; readers unpack pairs instead of
// splitting every value in every item.
enum : int { F32I = 17 };
// The packed 4-bit formats (two codes per byte, per-row block scales).
constexpr bool is_fp4(int f) { return f == AFF4 || f == MXFP4 || f == NVFP4; }
// Formats whose chunks carry dequant constants beside the codes.
constexpr bool is_quant(int f) { return is_fp4(f) || f == FP8; }
enum : int { ROUTE_SOFTMAX = 0, ROUTE_SIGMOID_BIAS = 1, ROUTE_SIGMOID_LOGIT = 2, ROUTE_SQRTSOFTPLUS = 3 };
enum : unsigned { NORM_TOPK = 1u, WEIGHT_BEFORE = 2u, SHARED = 4u, SHARED_GATED = 8u, OUT_F32 = 16u, GEGLU = 32u,
                  PRE_NORM = 64u, ROUTER_NORM = 128u };

constexpr int WAVE = 64;
constexpr int THREADS = 256;            // route and gate/up: 4 waves per workgroup
constexpr int WPB = THREADS / WAVE;
constexpr int DOWN_THREADS = 512;       // down + blend of the widest passes: 8 waves
constexpr int DOWN_WPB = DOWN_THREADS / WAVE;
// Down + blend workgroup of the variant with passes of up to CS vectors: 12
// waves (a tile's sub-units run in fewer rounds: -9 to -16 % on the down at
// m = 2-4) where the registers fit three waves per SIMD, else 8 (the
// eight-vector variants spill, and so would aff4's four-vector one: +9 %).
constexpr int DOWN_RD = 8;              // down rows per wave sub-unit
constexpr int MAX_DOWN_TILE = 2 * DOWN_RD;
// One vector per pass (m = 1): 8 waves; for f32 and bf16 experts held to 128
// registers, so that two workgroups share a CU.  The 4-bit formats'
// expansion does not fit 128 without spilling; their m = 1 grids have at
// most 256 tiles at the workloads' shapes.
// NW ("narrow", m = 1 with f32 or bf16 experts and at most 4 sub-units per
// tile, e.g. one expert with its rows in 4 parts of K): tiles of 4 rows on 4
// waves, each wave's sub-unit (4 rows, one part of K) issued as one batch of
// loads.  Against 8-row sub-units in two batches on 8 waves (320 tiles) a
// probe of the 5120 x 8192 bf16 down streamed 17.2 us instead of 24.0 (a
// plain read of the same bytes: 15.9 us); with 8 experts per row it was
// slower (two rounds of sub-units per wave), so the host takes it only for
// few sub-units.
// The 4-vector variants with 64 lanes per row for f32 and bf16 experts, and
// with 16 lanes per row or 64 for the fp4 formats, run 12 waves only with a
// smaller register budget for the row loop (below 104 they spilled); the
// fp4 formats with 64 lanes keep 8 waves.
template <int EF, int CS, int NW> constexpr int down_rd() { return NW ? NW : DOWN_RD; }
template <int EF, int CS, int LPR, int NW = 0> constexpr int down_threads() {
  return NW ? 256 : CS == 1 || CS >= 8 || EF == AFF4 || (EF >= MXFP4 && LPR == WAVE) ? DOWN_THREADS : 768;
}
template <int EF, int CS, int NW> constexpr int down_min_waves() { return CS == 1 && EF <= BF16 ? 4 : 1; }
// VGPRs the down's row-by-vector loop may plan for (wave_rows_dot's budget).
template <int EF, int CS, int NW> constexpr int down_vgpr_budget() {
  return NW ? (NW == 4 ? 96 : 100) : CS == 1 && EF <= BF16 ? 88 : CS == 4 ? 104 : 128;
}
constexpr int ROUTE_THREADS = 512;      // route launch: 8 waves
constexpr int ROUTE_THREADS_WIDE = 1024; // route launch of a narrow matrix-core shared expert: 16 waves
constexpr int ROUTE_WPB = ROUTE_THREADS / WAVE;
constexpr int RSPLIT = 4;               // waves per router row (its H is split in 4)
constexpr int ROUTE_UNITS_PER_WG = ROUTE_WPB / RSPLIT;
constexpr int MAX_ROWS = 32;
constexpr int CU_COUNT = 256;            // compute units of an MI355X (dispatch-slot heuristics)
constexpr int MAX_TOPK = 16;
constexpr int MAX_EXPERTS = 256;
constexpr int MAX_PAIRS = MAX_ROWS * MAX_TOPK;
constexpr int MAX_SD_PARTS = 16;        // parts of Is the matrix-core shared down splits into, at most

// Reserved words in the workspace (zeroed by moe_decode_workspace_init).
// Word 0 counts the router workgroups that have stored their logits; the
// last one resets it, and so does the next launch of the forward, so it is
// zero between calls whatever a call found there.  Nothing ever waits on it.
constexpr int SYNC_WORDS = 512;
constexpr int SYNC_ROUTER_TICKET = 0;
constexpr int SYNC_TOPK_TICKET = 1;     // grouped path: top-k workgroups (reset by the last arrival)
constexpr int SYNC_PUBLISHED = 2;       // the tag of the call whose routing the records hold
// Grouped path (33 <= m <= MAX_ROWS_G): one routing per row on one wave,
// then the experts' products on the matrix cores, G_COLS pairs per pass.
constexpr int MAX_ROWS_G = 256;
constexpr int G_THREADS = 512;
constexpr int G_WPB = G_THREADS / WAVE;
constexpr int G_NCT = 2;                // column tiles of 16 pairs per pass
constexpr int G_COLS = 16 * G_NCT;
constexpr int G_MU = 2;                 // k steps of 32 per staged batch (registers: two workgroups per CU)

// Rows of intermediate per gate/up wave: 2 for 16-byte-per-8-or-4 element
// formats; 4 for the 4-bit and fp8 ones (their rows are 4x and 2x shorter) with one vector
// per pass.  4-bit passes of several vectors take 2 rows: the registers then
// allow four waves per SIMD, which hide the weights' latency behind each
// other's dequantisation better than twice the rows per wave does.
template <int WF, int CR = 1> constexpr int gate_up_ni() { return is_quant(WF) && CR == 1 ? 4 : 2; }
// Register budget of a gate/up wave's row loop: fp8 rows with one vector
// take one chunk step of 8 rows (two steps spill beside the routing's state);
// with several vectors, 64 registers leave room for four or five waves per
// SIMD instead of two or three (the fp8 layer: -6 to -12 % at m = 2-16).
template <int WF, int CR> constexpr int gate_up_vb() { return WF == FP8 ? (CR == 1 ? 96 : 64) : 128; }

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// Per active slot: what the gate/up and down launches need to start
// streaming, in one 128-byte record (the routing publishes it).
struct alignas(128) SlotRec {
  int32_t e, off, np, tag;       // tag: Args::tag of the forward that wrote it
  uint64_t gw, uw, gs, us, gb, ub, dw, ds, db;
  uint64_t pad2[5];
};
static_assert(sizeof(SlotRec) == 128, "slot records are 128 bytes");

// Everything a forward's kernels read or write (kernel argument, by value).
struct Args {
  int H, E, K, I, Is, m, te, cap, act_fmt, expert_fmt, routing;
  unsigned flags;
  float rsf;
  // work items
  int n_router, n_router_wg, n_shared_gu, gu_items_per_slot, n_routed_gu, n_down, down_dq;
  int route_in_gu;         // 1: every gate/up workgroup routes; 0: the last router workgroup does
  int shared_mfma;         // shared expert on the matrix cores (bf16 activations, H and Is multiples of 32)
  int sact_pairs;          // matrix-core shared activations stored as F32I pairs (bf16 experts), else f32
  int n_shared_dn;         // shared down items in the gate/up launch (matrix-core path)
  int sd_parts;            // parts of Is the shared down items split (partials in sy[part])
  int down_parts;          // parts of I each routed down row is split into (partials added in the blend)
  int max_rows;
  int tag;                 // this call's slot-record tag (odd; a hash of its tables, x, workspace and m)
  const void *x;           // the experts' input (the row, or its pre-expert norm)
  const void *xr;          // the router's input (the row, or its router pre-norm)
  void *out;
  int32_t *idx_out;
  float *w_out;
  const void *router;
  const float *ebias;
  const uint64_t *gw, *uw, *dw, *gs, *us, *ds, *gb, *ub, *db;
  const float *gs2, *us2, *ds2;   // nvfp4: [E] second-level scale per projection
  const void *sgw, *suw, *sdw, *sgv;
  double *logits;          // [m, E+1]
  double *scores;          // [m, E]: sqrt-softplus scores of the logits (that routing only)
  int32_t *topk_idx;       // [te]
  float *topk_w;           // [te]
  float *row_gate;         // [m]
  int32_t *sorted_pair;    // [te]
  int32_t *offsets;        // [E+1]
  int32_t *pair_to_perm;   // [te]
  int32_t *active;         // [cap]
  int32_t *active_count;   // [1]
  SlotRec *slots;          // [cap]
  float *act;              // [te, I]
  float *sact;             // [m, Is]
  float *sy;               // [m, H]: shared-expert output (matrix-core path)
  float *y;                // [te, H]: grouped path, routed down output per pair in sorted order
  unsigned *sync;          // [SYNC_WORDS]
};

// ---------------------------------------------------------------- helpers

__device__ __forceinline__ u32x4 ld_stream16(const void *p) {
  // Expert weights are read once per call: keep them out of the caches.
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}
__device__ __forceinline__ u32x4 ld16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }
__device__ __forceinline__ u32x2 ld8(const void *p) { return *reinterpret_cast<const u32x2 *>(p); }

// Device-coherent (agent-scope) accesses: they bypass the per-XCD caches'
// non-coherent state, for data one workgroup hands to another in a launch.
__device__ __forceinline__ void store_coherent(double *p, double v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ double load_coherent(const double *p) {
  return __hip_atomic_load(const_cast<double *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

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

// GeGLU's activation, the exact GELU g * Phi(g), Phi(g) = 1 - erfc(z) / 2
// for g >= 0 and erfc(z) / 2 below, z = |g| / sqrt 2.  erfc from Abramowitz
// and Stegun 7.1.26 (absolute error at most 1.5e-7; no cancellation for
// negative g): erfc(z) = t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) e^(-z^2),
// t = 1 / (1 + p z).
__device__ __forceinline__ float gelu_mul(float g, float v) {
  const float z = __builtin_fabsf(g) * 0.70710678118654752f;
  const float t = 1.0f / __builtin_fmaf(0.3275911f, z, 1.0f);
  float q = __builtin_fmaf(1.061405429f, t, -1.453152027f);
  q = __builtin_fmaf(q, t, 1.421413741f);
  q = __builtin_fmaf(q, t, -0.284496736f);
  q = __builtin_fmaf(q, t, 0.254829592f);
  const float half_erfc = 0.5f * q * t * __expf(-z * z);
  const float phi = g >= 0.f ? 1.0f - half_erfc : half_erfc;
  return g * phi * v;
}

// The experts' activation: silu(g) * v, or gelu(g) * v with GEGLU.
__device__ __forceinline__ float act_mul(unsigned flags, float g, float v) {
  return (flags & GEGLU) ? gelu_mul(g, v) : silu_mul(g, v);
}

__device__ __forceinline__ double sigmoid_d(double v) { return 1.0 / (1.0 + exp(-v)); }

// The sqrt-softplus router score sqrt(log(1 + e^v)), with log(1 + e^v) taken
// as v + log(1 + e^-v) above 0 (no overflow).
__device__ __forceinline__ double sqrtsoftplus_d(double v) {
  return sqrt(v > 0.0 ? v + log1p(exp(-v)) : log1p(exp(v)));
}

// Whether the routing reads the expert bias: sigmoid+bias always,
// sqrt-softplus when one is given.
__device__ __forceinline__ bool routing_biased(int routing, const float *ebias) {
  return routing == ROUTE_SIGMOID_BIAS || (routing == ROUTE_SQRTSOFTPLUS && ebias != nullptr);
}

// Selection key of logit l (sc: its sqrt-softplus score, b: its bias):
// sigmoid(l) + b (sigmoid+bias), sc + b (sqrt-softplus with a bias), else the
// logit itself (softmax, raw-logit, and sqrt-softplus without a bias, whose
// strictly increasing score orders the experts as the logits do).
template <bool BIASED>
__device__ __forceinline__ double select_key_d(int routing, double l, double sc, double b) {
  if constexpr (BIASED) return routing == ROUTE_SIGMOID_BIAS ? sigmoid_d(l) + b : sc + b;
  return l;
}

// Router rows of the route launch: the experts, and the shared-expert gate
// vector w_g as row E -- unless the router reads a pre-normed row, when the
// pre-norm launch (which reads the raw row) takes the gate instead.
__device__ __forceinline__ int router_rows(const Args &a) {
  return a.E + ((a.flags & SHARED_GATED) && !(a.flags & ROUTER_NORM) ? 1 : 0);
}

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
__device__ __forceinline__ unsigned long long readlane_u64(unsigned long long v, int l) {
  const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)v, l);
  const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)(v >> 32), l);
  return ((unsigned long long)hi << 32) | lo;
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

// Exclusive prefix sum over the wave's lanes of v (0 <= v < 2^BITS), from
// one ballot per bit plane and the count of set lanes below this one.  The
// wave total goes to *total.
template <int BITS>
__device__ __forceinline__ int wave_excl_scan(unsigned v, int *total) {
  int pre = 0, tot = 0;
#pragma unroll
  for (int b = 0; b < BITS; ++b) {
    const unsigned long long m = __builtin_amdgcn_ballot_w64((v >> b) & 1u);
    const int below = (int)__builtin_amdgcn_mbcnt_hi((unsigned)(m >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)m, 0u));
    pre += below << b;
    tot += __builtin_popcountll(m) << b;
  }
  *total = tot;
  return pre;
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


// --------------------------------------------------- per-format chunk math
//
// A chunk is 16 bytes of one weight row: 4 f32, 8 bf16 or 32 packed 4-bit
// codes.  Lane `li` of a row group handles chunks li, li+LPR, ...  XF is the
// storage format of the vector the row is dotted with (F32 or BF16).
//
// A chunk is consumed in SUB sub-steps.  Sub-step g needs only the x
// elements it covers (8 of them for the 4-bit formats, whose chunk spans 32),
// loaded from cache right before use, so the registers x takes stay small
// whatever the number of vectors in a pass.

template <int WF> struct Fmt;
template <> struct Fmt<F32> { static constexpr int EPC = 4; };
template <> struct Fmt<BF16> { static constexpr int EPC = 8; };
template <> struct Fmt<AFF4> { static constexpr int EPC = 32; };
template <> struct Fmt<MXFP4> { static constexpr int EPC = 32; };
template <> struct Fmt<NVFP4> { static constexpr int EPC = 32; };
template <> struct Fmt<FP8> { static constexpr int EPC = 16; };

// One weight row, addressed through buffer resources: the matrix's data
// resource (and, for the 4-bit formats, its scale and bias resources) and the
// row's byte offset in the data.  A 4-bit row of K codes is K/2 bytes and its
// scale row K/32 bytes (aff4: K/64 bf16; mxfp4: K/32 E8M0), so the scale
// row's offset is off / 16 for both; the nvfp4 scale row is K/16 E4M3 bytes,
// at off / 8.
template <int WF> struct Row {
  __amdgpu_buffer_rsrc_t w, s, b;
  int off;
};
// fp8: one fp32 scale per 128 x 128 block; soff is the byte offset of the
// row's block row in the [N / 128, K / 128] scale array.
template <> struct Row<FP8> {
  __amdgpu_buffer_rsrc_t w, s, b;
  int off, soff;
};

// Weight chunk plus the raw bits of its dequant constants (converted where
// they are used, so that no load has to complete before the compute starts).
template <int WF> struct WChunk {
  u32x4 q;
  uint32_t s, b;
};

// VGPRs one loaded chunk holds.
template <int WF> constexpr int wchunk_regs() { return WF == AFF4 ? 6 : WF >= MXFP4 ? 5 : 4; }

constexpr int BUF_NT = 2;        // cache policy: nontemporal (weights are read once per call)

// UNI: the row is the same for the whole wave, its offset goes in the
// scalar offset operand; else it is added to the lane's offset.
template <int WF, bool UNI>
__device__ __forceinline__ WChunk<WF> load_wchunk(const Row<WF> &r, int ch) {
  WChunk<WF> c;
  const int vo = UNI ? 0 : r.off, so = UNI ? r.off : 0;
  c.q = __builtin_amdgcn_raw_buffer_load_b128(r.w, vo + ch * 16, so, BUF_NT);
  if constexpr (WF == AFF4) {
    // One bf16 scale and bias per 64 elements = per 2 chunks.
    c.s = __builtin_amdgcn_raw_buffer_load_b16(r.s, vo / 16 + (ch >> 1) * 2, so / 16, 0);
    c.b = __builtin_amdgcn_raw_buffer_load_b16(r.b, vo / 16 + (ch >> 1) * 2, so / 16, 0);
  } else if constexpr (WF == MXFP4) {
    c.s = __builtin_amdgcn_raw_buffer_load_b8(r.s, vo / 16 + ch, so / 16, 0);
    c.b = 0u;
  } else if constexpr (WF == NVFP4) {
    // The two E4M3 block scales of the chunk (elements 0..15, then 16..31).
    c.s = __builtin_amdgcn_raw_buffer_load_b16(r.s, vo / 8 + ch * 2, so / 8, 0);
    c.b = 0u;
  } else if constexpr (WF == FP8) {
    // The fp32 scale of the chunk's 128-column block (chunks of 16 codes).
    const int svo = UNI ? 0 : r.soff, sso = UNI ? r.soff : 0;
    c.s = __builtin_amdgcn_raw_buffer_load_b32(r.s, svo + (ch >> 3) * 4, sso, 0);
    c.b = 0u;
  } else {
    c.s = c.b = 0u;
  }
  return c;
}

// XOps<WF, XF>: the arithmetic of one chunk against one vector.
//   SUB, XS        sub-steps per chunk; x registers of one sub-step
//   X              x values of one sub-step: X::fetch(xrow, ch, g)
//   xsum(x, s)     running sum of the vector over the chunk (aff4 only)
//   step(w, x, g, p)  adds sub-step g to the chunk partial p
//   finish(w, p, xs, acc)  folds the chunk partial into the row total
// For the 8- and 4-element formats the partial is the row total itself.
template <int WF, int XF> struct XOps;

// bf16 weights . bf16 x: raw bf16 pairs, v_dot2.
template <> struct XOps<BF16, BF16> {
  static constexpr int SUB = 1, XS = 4;
  struct X {
    u32x4 d;
    __device__ __forceinline__ void fetch(const char *xrow, int ch, int, int) { d = ld16(xrow + (size_t)ch * 16); }
  };
  static __device__ __forceinline__ float xsum(const X &, float s) { return s; }
  static __device__ __forceinline__ float start(float acc) { return acc; }
  static __device__ __forceinline__ float step(const WChunk<BF16> &w, const X &x, int, float p) {
    p = dot2(w.q.x, x.d.x, p);
    p = dot2(w.q.y, x.d.y, p);
    p = dot2(w.q.z, x.d.z, p);
    return dot2(w.q.w, x.d.w, p);
  }
  static __device__ __forceinline__ float finish(const WChunk<BF16> &, float p, float, float) { return p; }
};

// bf16 weights . f32 x.
template <> struct XOps<BF16, F32> {
  static constexpr int SUB = 1, XS = 8;
  struct X {
    u32x4 a, b;
    __device__ __forceinline__ void fetch(const char *xrow, int ch, int, int) {
      a = ld16(xrow + (size_t)ch * 32);
      b = ld16(xrow + (size_t)ch * 32 + 16);
    }
  };
  static __device__ __forceinline__ float xsum(const X &, float s) { return s; }
  static __device__ __forceinline__ float start(float acc) { return acc; }
  static __device__ __forceinline__ float step(const WChunk<BF16> &w, const X &x, int, float p) {
    p = __builtin_fmaf(bf_lo(w.q.x), __uint_as_float(x.a.x), p);
    p = __builtin_fmaf(bf_hi(w.q.x), __uint_as_float(x.a.y), p);
    p = __builtin_fmaf(bf_lo(w.q.y), __uint_as_float(x.a.z), p);
    p = __builtin_fmaf(bf_hi(w.q.y), __uint_as_float(x.a.w), p);
    p = __builtin_fmaf(bf_lo(w.q.z), __uint_as_float(x.b.x), p);
    p = __builtin_fmaf(bf_hi(w.q.z), __uint_as_float(x.b.y), p);
    p = __builtin_fmaf(bf_lo(w.q.w), __uint_as_float(x.b.z), p);
    return __builtin_fmaf(bf_hi(w.q.w), __uint_as_float(x.b.w), p);
  }
  static __device__ __forceinline__ float finish(const WChunk<BF16> &, float p, float, float) { return p; }
};

// f32 weights . f32 x.
template <> struct XOps<F32, F32> {
  static constexpr int SUB = 1, XS = 4;
  struct X {
    u32x4 a;
    __device__ __forceinline__ void fetch(const char *xrow, int ch, int, int) { a = ld16(xrow + (size_t)ch * 16); }
  };
  static __device__ __forceinline__ float xsum(const X &, float s) { return s; }
  static __device__ __forceinline__ float start(float acc) { return acc; }
  static __device__ __forceinline__ float step(const WChunk<F32> &w, const X &x, int, float p) {
    p = __builtin_fmaf(__uint_as_float(w.q.x), __uint_as_float(x.a.x), p);
    p = __builtin_fmaf(__uint_as_float(w.q.y), __uint_as_float(x.a.y), p);
    p = __builtin_fmaf(__uint_as_float(w.q.z), __uint_as_float(x.a.z), p);
    return __builtin_fmaf(__uint_as_float(w.q.w), __uint_as_float(x.a.w), p);
  }
  static __device__ __forceinline__ float finish(const WChunk<F32> &, float p, float, float) { return p; }
};

// f32 weights . bf16 x.
template <> struct XOps<F32, BF16> {
  static constexpr int SUB = 1, XS = 2;
  struct X {
    u32x2 raw;
    __device__ __forceinline__ void fetch(const char *xrow, int ch, int, int) { raw = ld8(xrow + (size_t)ch * 8); }
  };
  static __device__ __forceinline__ float xsum(const X &, float s) { return s; }
  static __device__ __forceinline__ float start(float acc) { return acc; }
  static __device__ __forceinline__ float step(const WChunk<F32> &w, const X &x, int, float p) {
    p = __builtin_fmaf(__uint_as_float(w.q.x), bf_lo(x.raw.x), p);
    p = __builtin_fmaf(__uint_as_float(w.q.y), bf_hi(x.raw.x), p);
    p = __builtin_fmaf(__uint_as_float(w.q.z), bf_lo(x.raw.y), p);
    return __builtin_fmaf(__uint_as_float(w.q.w), bf_hi(x.raw.y), p);
  }
  static __device__ __forceinline__ float finish(const WChunk<F32> &, float p, float, float) { return p; }
};

__device__ __forceinline__ uint32_t code_dword(const u32x4 &q, int g) {
  return g == 0 ? q.x : g == 1 ? q.y : g == 2 ? q.z : q.w;
}

// aff4 weights . bf16 x.  Code dword g holds elements 8g..8g+7 (nibble i at
// bits 4i).  OR-ing a nibble into the mantissa of bf16 128.0 (0x4300) gives
// 128 + q exactly, so (u >> 4t) & 0x000F000F | 0x43004300 is the bf16 pair
// (128 + q_t, 128 + q_{t+4}); x is re-paired to (x_t, x_{t+4}) to match.
//   sum q x = sum (128+q) x - 128 sum x, and w = s q + b, so the chunk adds
//   s * D + (b - 128 s) * X  with D = sum (128+q) x, X = sum x.
template <> struct XOps<AFF4, BF16> {
  static constexpr int SUB = 4, XS = 4;
  struct X {
    uint32_t d[4];   // (x0,x4) (x1,x5) (x2,x6) (x3,x7) of the sub-step
    __device__ __forceinline__ void fetch(const char *xrow, int ch, int g, int) {
      const u32x4 v = ld16(xrow + (size_t)ch * 64 + 16 * g);  // (x0,x1) (x2,x3) (x4,x5) (x6,x7)
      d[0] = (v.x & 0xFFFFu) | (v.z << 16);
      d[1] = (v.x >> 16) | (v.z & 0xFFFF0000u);
      d[2] = (v.y & 0xFFFFu) | (v.w << 16);
      d[3] = (v.y >> 16) | (v.w & 0xFFFF0000u);
    }
  };
  static __device__ __forceinline__ float xsum(const X &x, float s) {
#pragma unroll
    for (int t = 0; t < 4; ++t) s = dot2(x.d[t], 0x3F803F80u, s);
    return s;
  }
  static __device__ __forceinline__ float start(float) { return 0.f; }
  static __device__ __forceinline__ float step(const WChunk<AFF4> &w, const X &x, int g, float D) {
    const uint32_t q = code_dword(w.q, g);
#pragma unroll
    for (int t = 0; t < 4; ++t) D = dot2(((q >> (4 * t)) & 0x000F000Fu) | 0x43004300u, x.d[t], D);
    return D;
  }
  static __device__ __forceinline__ float finish(const WChunk<AFF4> &w, float D, float xs, float acc) {
    const float sc = __uint_as_float(w.s << 16), bi = __uint_as_float(w.b << 16);
    acc = __builtin_fmaf(sc, D, acc);
    return __builtin_fmaf(__builtin_fmaf(-128.0f, sc, bi), xs, acc);
  }
};

// aff4 weights . f32 x: w = s q + b, the chunk adds s * sum q x + b * sum x.
template <> struct XOps<AFF4, F32> {
  static constexpr int SUB = 4, XS = 8;
  struct X {
    u32x4 a, b;      // x 8g .. 8g+7
    __device__ __forceinline__ void fetch(const char *xrow, int ch, int g, int) {
      a = ld16(xrow + (size_t)ch * 128 + 32 * g);
      b = ld16(xrow + (size_t)ch * 128 + 32 * g + 16);
    }
    __device__ __forceinline__ float f(int i) const {
      const u32x4 &v = i < 4 ? a : b;
      const int j = i & 3;
      return __uint_as_float(j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w);
    }
  };
  static __device__ __forceinline__ float xsum(const X &x, float s) {
#pragma unroll
    for (int i = 0; i < 8; ++i) s += x.f(i);
    return s;
  }
  static __device__ __forceinline__ float start(float) { return 0.f; }
  static __device__ __forceinline__ float step(const WChunk<AFF4> &w, const X &x, int g, float D) {
    const uint32_t q = code_dword(w.q, g);
    const uint32_t lo = q & 0x0F0F0F0Fu, hi = (q >> 4) & 0x0F0F0F0Fu;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      D = __builtin_fmaf((float)((lo >> (8 * b)) & 0xFFu), x.f(2 * b), D);
      D = __builtin_fmaf((float)((hi >> (8 * b)) & 0xFFu), x.f(2 * b + 1), D);
    }
    return D;
  }
  static __device__ __forceinline__ float finish(const WChunk<AFF4> &w, float D, float xs, float acc) {
    acc = __builtin_fmaf(__uint_as_float(w.s << 16), D, acc);
    return __builtin_fmaf(__uint_as_float(w.b << 16), xs, acc);
  }
};

// mxfp4 weights . bf16 x: v_cvt_scalef32_pk_bf16_fp4 turns byte t of a code
// dword (elements 2t, 2t+1, low nibble first) into an exact bf16 pair that
// lines up with the raw x pair; the E8M0 scale multiplies the chunk sum.
template <> struct XOps<MXFP4, BF16> {
  static constexpr int SUB = 4, XS = 4;
  struct X {
    u32x4 d;
    __device__ __forceinline__ void fetch(const char *xrow, int ch, int g, int) { d = ld16(xrow + (size_t)ch * 64 + 16 * g); }
  };
  static __device__ __forceinline__ float xsum(const X &, float s) { return s; }
  static __device__ __forceinline__ float start(float) { return 0.f; }
  static __device__ __forceinline__ float step(const WChunk<MXFP4> &w, const X &x, int g, float S) {
    const uint32_t q = code_dword(w.q, g);
    S = dot2(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, 1.0f, 0)), x.d.x, S);
    S = dot2(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, 1.0f, 1)), x.d.y, S);
    S = dot2(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, 1.0f, 2)), x.d.z, S);
    return dot2(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, 1.0f, 3)), x.d.w, S);
  }
  static __device__ __forceinline__ float finish(const WChunk<MXFP4> &w, float S, float, float acc) {
    return __builtin_fmaf(S, e8m0_to_f32(w.s), acc);
  }
};

// mxfp4 weights . f32 x.
template <> struct XOps<MXFP4, F32> {
  static constexpr int SUB = 4, XS = 8;
  struct X {
    u32x4 a, b;
    __device__ __forceinline__ void fetch(const char *xrow, int ch, int g, int) {
      a = ld16(xrow + (size_t)ch * 128 + 32 * g);
      b = ld16(xrow + (size_t)ch * 128 + 32 * g + 16);
    }
  };
  static __device__ __forceinline__ float xsum(const X &, float s) { return s; }
  static __device__ __forceinline__ float start(float) { return 0.f; }
  static __device__ __forceinline__ float step(const WChunk<MXFP4> &w, const X &x, int g, float S) {
    const uint32_t q = code_dword(w.q, g);
    const f32x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 0);
    const f32x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 1);
    const f32x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 2);
    const f32x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 3);
    S = __builtin_fmaf(v0.x, __uint_as_float(x.a.x), S);
    S = __builtin_fmaf(v0.y, __uint_as_float(x.a.y), S);
    S = __builtin_fmaf(v1.x, __uint_as_float(x.a.z), S);
    S = __builtin_fmaf(v1.y, __uint_as_float(x.a.w), S);
    S = __builtin_fmaf(v2.x, __uint_as_float(x.b.x), S);
    S = __builtin_fmaf(v2.y, __uint_as_float(x.b.y), S);
    S = __builtin_fmaf(v3.x, __uint_as_float(x.b.z), S);
    return __builtin_fmaf(v3.y, __uint_as_float(x.b.w), S);
  }
  static __device__ __forceinline__ float finish(const WChunk<MXFP4> &w, float S, float, float acc) {
    return __builtin_fmaf(S, e8m0_to_f32(w.s), acc);
  }
};

// OCP FP8 E4M3 byte (bits 7..0 of b; no NaN allowed) to f32: sign bit 7,
// exponent bits 6..3 with bias 7, mantissa bits 2..0, exponent 0 subnormal
// (mantissa * 2^-9).  A normal value is the f32 with exponent field e + 120
// and the mantissa in its top three bits.
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  const uint32_t em = b & 0x7Fu;
  const float v = em >= 8u ? __uint_as_float((em << 20) + (120u << 23)) : (float)em * 0x1p-9f;
  return (b & 0x80u) ? -v : v;
}

// nvfp4 weights (E2M1 codes, an E4M3 scale per 16 elements) . bf16 x: sub-
// step g is block g of the chunk (code dwords 2g, 2g + 1); its sum is taken
// unscaled, then times the block's scale (low scale byte for block 0).  The
// projection's second-level scale multiplies the row total outside.
template <> struct XOps<NVFP4, BF16> {
  static constexpr int SUB = 2, XS = 8;
  struct X {
    u32x4 a, b;      // x 16g .. 16g+7, 16g+8 .. 16g+15
    __device__ __forceinline__ void fetch(const char *xrow, int ch, int g, int) {
      a = ld16(xrow + (size_t)ch * 64 + 32 * g);
      b = ld16(xrow + (size_t)ch * 64 + 32 * g + 16);
    }
  };
  static __device__ __forceinline__ float xsum(const X &, float s) { return s; }
  static __device__ __forceinline__ float start(float) { return 0.f; }
  template <int SEL> static __device__ __forceinline__ uint32_t pk(uint32_t q) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, 1.0f, SEL));
  }
  static __device__ __forceinline__ float step(const WChunk<NVFP4> &w, const X &x, int g, float S) {
    const uint32_t q0 = code_dword(w.q, 2 * g), q1 = code_dword(w.q, 2 * g + 1);
    float t = dot2(pk<0>(q0), x.a.x, 0.f);
    t = dot2(pk<1>(q0), x.a.y, t);
    t = dot2(pk<2>(q0), x.a.z, t);
    t = dot2(pk<3>(q0), x.a.w, t);
    t = dot2(pk<0>(q1), x.b.x, t);
    t = dot2(pk<1>(q1), x.b.y, t);
    t = dot2(pk<2>(q1), x.b.z, t);
    t = dot2(pk<3>(q1), x.b.w, t);
    return __builtin_fmaf(t, e4m3_to_f32(g == 0 ? (w.s & 0xFFu) : (w.s >> 8) & 0xFFu), S);
  }
  static __device__ __forceinline__ float finish(const WChunk<NVFP4> &, float S, float, float acc) { return acc + S; }
};

// nvfp4 weights . f32 x.
template <> struct XOps<NVFP4, F32> {
  static constexpr int SUB = 4, XS = 8;
  using X = XOps<MXFP4, F32>::X;
  static __device__ __forceinline__ float xsum(const X &, float s) { return s; }
  static __device__ __forceinline__ float start(float) { return 0.f; }
  static __device__ __forceinline__ float step(const WChunk<NVFP4> &w, const X &x, int g, float S) {
    const uint32_t q = code_dword(w.q, g);
    const f32x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 0);
    const f32x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 1);
    const f32x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 2);
    const f32x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 3);
    float t = v0.x * __uint_as_float(x.a.x);
    t = __builtin_fmaf(v0.y, __uint_as_float(x.a.y), t);
    t = __builtin_fmaf(v1.x, __uint_as_float(x.a.z), t);
    t = __builtin_fmaf(v1.y, __uint_as_float(x.a.w), t);
    t = __builtin_fmaf(v2.x, __uint_as_float(x.b.x), t);
    t = __builtin_fmaf(v2.y, __uint_as_float(x.b.y), t);
    t = __builtin_fmaf(v3.x, __uint_as_float(x.b.z), t);
    t = __builtin_fmaf(v3.y, __uint_as_float(x.b.w), t);
    return __builtin_fmaf(t, e4m3_to_f32(g < 2 ? (w.s & 0xFFu) : (w.s >> 8) & 0xFFu), S);
  }
  static __device__ __forceinline__ float finish(const WChunk<NVFP4> &, float S, float, float acc) { return acc + S; }
};

// fp8 weights (OCP E4M3 codes, an fp32 scale per 128 x 128 block) . bf16
// x: v_cvt_scalef32_pk_bf16_fp8 turns half of a code dword (elements 2t,
// 2t + 1 of the dword, low byte first) into an exact bf16 pair that lines up
// with the raw x pair; the chunk's 16 products are summed unscaled, then
// times its block's scale.
template <> struct XOps<FP8, BF16> {
  static constexpr int SUB = 1, XS = 8;
  struct X {
    u32x4 a, b;      // x 0..7, 8..15 of the chunk
    __device__ __forceinline__ void fetch(const char *xrow, int ch, int, int) {
      a = ld16(xrow + (size_t)ch * 32);
      b = ld16(xrow + (size_t)ch * 32 + 16);
    }
  };
  template <bool HI> static __device__ __forceinline__ uint32_t pk(uint32_t q) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q, 1.0f, HI));
  }
  static __device__ __forceinline__ float xsum(const X &, float s) { return s; }
  static __device__ __forceinline__ float start(float acc) { return acc; }
  static __device__ __forceinline__ float step(const WChunk<FP8> &w, const X &x, int, float acc) {
    float t = dot2(pk<false>(w.q.x), x.a.x, 0.f);
    t = dot2(pk<true>(w.q.x), x.a.y, t);
    t = dot2(pk<false>(w.q.y), x.a.z, t);
    t = dot2(pk<true>(w.q.y), x.a.w, t);
    t = dot2(pk<false>(w.q.z), x.b.x, t);
    t = dot2(pk<true>(w.q.z), x.b.y, t);
    t = dot2(pk<false>(w.q.w), x.b.z, t);
    t = dot2(pk<true>(w.q.w), x.b.w, t);
    return __builtin_fmaf(t, __uint_as_float(w.s), acc);
  }
  static __device__ __forceinline__ float finish(const WChunk<FP8> &, float acc, float, float) { return acc; }
};

// fp8 weights . f32 x: sub-step g is code dwords 2g, 2g + 1 (8 elements).
template <> struct XOps<FP8, F32> {
  static constexpr int SUB = 2, XS = 8;
  struct X {
    u32x4 a, b;      // x 8g .. 8g+7
    __device__ __forceinline__ void fetch(const char *xrow, int ch, int g, int) {
      a = ld16(xrow + (size_t)ch * 64 + 32 * g);
      b = ld16(xrow + (size_t)ch * 64 + 32 * g + 16);
    }
  };
  static __device__ __forceinline__ float xsum(const X &, float s) { return s; }
  static __device__ __forceinline__ float start(float) { return 0.f; }
  static __device__ __forceinline__ float step(const WChunk<FP8> &w, const X &x, int g, float S) {
    const uint32_t q0 = code_dword(w.q, 2 * g), q1 = code_dword(w.q, 2 * g + 1);
    const f32x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(q0, 1.0f, false);
    const f32x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(q0, 1.0f, true);
    const f32x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(q1, 1.0f, false);
    const f32x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(q1, 1.0f, true);
    S = __builtin_fmaf(v0.x, __uint_as_float(x.a.x), S);
    S = __builtin_fmaf(v0.y, __uint_as_float(x.a.y), S);
    S = __builtin_fmaf(v1.x, __uint_as_float(x.a.z), S);
    S = __builtin_fmaf(v1.y, __uint_as_float(x.a.w), S);
    S = __builtin_fmaf(v2.x, __uint_as_float(x.b.x), S);
    S = __builtin_fmaf(v2.y, __uint_as_float(x.b.y), S);
    S = __builtin_fmaf(v3.x, __uint_as_float(x.b.z), S);
    return __builtin_fmaf(v3.y, __uint_as_float(x.b.w), S);
  }
  static __device__ __forceinline__ float finish(const WChunk<FP8> &w, float S, float, float acc) {
    return __builtin_fmaf(S, __uint_as_float(w.s), acc);
  }
};

// 4-bit weights . sub-step-major f32 x (the down input): the math of the
// f32 case, sub-step g of chunk ch read at g * gs + ch * 32 bytes.
template <> struct XOps<AFF4, F32P> : XOps<AFF4, F32> {
  struct X : XOps<AFF4, F32>::X {
    __device__ __forceinline__ void fetch(const char *xrow, int ch, int g, int gs) {
      a = ld16(xrow + (size_t)g * gs + (size_t)ch * 32);
      b = ld16(xrow + (size_t)g * gs + (size_t)ch * 32 + 16);
    }
  };
};
template <> struct XOps<MXFP4, F32P> : XOps<MXFP4, F32> {
  struct X : XOps<MXFP4, F32>::X {
    __device__ __forceinline__ void fetch(const char *xrow, int ch, int g, int gs) {
      a = ld16(xrow + (size_t)g * gs + (size_t)ch * 32);
      b = ld16(xrow + (size_t)g * gs + (size_t)ch * 32 + 16);
    }
  };
};
template <> struct XOps<NVFP4, F32P> : XOps<NVFP4, F32> {
  using X = XOps<MXFP4, F32P>::X;
};

// ------------------------------------------------------ wave row x vector
//
// RG weight rows per lane group (each K = nchunks chunks long) against C
// vectors (xrow[c]).  The wave is split into 64/LPR lane groups; the caller
// passes in `rows` the RG rows of the calling lane's group.  Lane li of a
// group takes chunks li, li + LPR, ...; the weight loads of U chunk steps --
// and, for the one-sub-step formats where registers allow, their x loads --
// are issued together before any of them is used.  On return acc[t][c]
// holds, in every lane of the group, the full dot product of rows[t] with
// vector c over chunks [c0, nchunks).  The per-(row, vector) arithmetic does
// not depend on C, U or the other rows, so results are the same for every m.

// Chunk steps issued together: as many as fit, with the RG x C totals and
// the x values in use, in about 128 VGPRs.
// XPF: the x values of a step (all its sub-steps) are requested with its
// weights -- one round trip per step -- when they fit: up to 32 registers
// for one-sub-step formats, up to 64 (one step) for the 4-bit ones.
template <int WF, int XF, int RG, int C, int VB = 128> struct Unroll {
  static constexpr int clampu(int v) { return v < 1 ? 1 : (v > 4 ? 4 : v); }
  static constexpr int W = RG * wchunk_regs<WF>();
  static constexpr int XS = XOps<WF, XF>::XS;
  static constexpr int SUB = XOps<WF, XF>::SUB;
  static constexpr int A = RG * C + 2 * XS;
  // 4-bit rows with 4+ vectors: one step (the expansion temporaries are large).
  static constexpr int U0 = (WF >= AFF4 && C >= 4) ? 1 : clampu((VB - A) / W);
  static constexpr bool XPF = SUB == 1 ? U0 * C * XS <= 32 : C * SUB * XS <= 64;
  static constexpr int U = !XPF ? U0 : SUB == 1 ? clampu((VB - RG * C) / (W + C * XS)) : 1;
};

// Issues the loads of the first chunk step of wave_rows_dot<..., U> over
// chunks [c0, nchunks) into pre (used through PRE below).
template <int WF, int RG, int U, int LPR>
__device__ __forceinline__ void preload_step(const Row<WF> (&rows)[RG], int c0, int nchunks, WChunk<WF> (&pre)[U][RG]) {
  const int li = threadIdx.x % LPR;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int ch = c0 + li + u * LPR;
    if (ch < nchunks) {
#pragma unroll
      for (int t = 0; t < RG; ++t) pre[u][t] = load_wchunk<WF, LPR == WAVE>(rows[t], ch);
    }
  }
}

// PRE: pre holds the first chunk step, requested earlier by preload_step
// with the same U; used when use_pre.
template <int WF, int XF, int RG, int C, int LPR, bool PRE = false, int UP = 1, int VB = 128>
__device__ __forceinline__ void wave_rows_dot(const Row<WF> (&rows)[RG], const char *const (&xrow)[C],
                                              int c0, int nchunks, float (&acc)[RG][C], int gs = 0,
                                              const WChunk<WF> (*pre)[RG] = nullptr, bool use_pre = false) {
  using O = XOps<WF, XF>;
  using X = typename O::X;
  constexpr int U = Unroll<WF, XF, RG, C, VB>::U;
  constexpr bool XPF = Unroll<WF, XF, RG, C, VB>::XPF;
  constexpr int SUB = O::SUB;
  static_assert(!PRE || U == UP, "the preloaded step has this pass's unroll");
  const int li = threadIdx.x % LPR;
#pragma unroll
  for (int t = 0; t < RG; ++t)
#pragma unroll
    for (int c = 0; c < C; ++c) acc[t][c] = 0.f;
  for (int base = c0; base < nchunks; base += LPR * U) {
    WChunk<WF> w[U][RG];
    X xp[XPF ? U : 1][XPF ? C : 1][XPF ? SUB : 1];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int ch = base + li + u * LPR;
      if (ch < nchunks) {
        if (PRE && use_pre && base == c0) {
#pragma unroll
          for (int t = 0; t < RG; ++t) w[u][t] = pre[u][t];
        } else {
#pragma unroll
          for (int t = 0; t < RG; ++t) w[u][t] = load_wchunk<WF, LPR == WAVE>(rows[t], ch);
        }
        if constexpr (XPF) {
#pragma unroll
          for (int c = 0; c < C; ++c)
#pragma unroll
            for (int g = 0; g < SUB; ++g) xp[u][c][g].fetch(xrow[c], ch, g, gs);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int ch = base + li + u * LPR;
      if (ch < nchunks) {
        // Sub-step, then row, then vector: a row's expanded codes serve every
        // vector right away and are dead before the next row's are made.
        float p[RG][C], xs[C];
#pragma unroll
        for (int c = 0; c < C; ++c) {
          xs[c] = 0.f;
#pragma unroll
          for (int t = 0; t < RG; ++t) p[t][c] = O::start(acc[t][c]);
        }
        // Without XPF, x of sub-step g + 1 is requested before sub-step g
        // is computed.
        X xn[C];
        if constexpr (!XPF) {
#pragma unroll
          for (int c = 0; c < C; ++c) xn[c].fetch(xrow[c], ch, 0, gs);
        }
#pragma unroll
        for (int g = 0; g < O::SUB; ++g) {
          X x[C];
#pragma unroll
          for (int c = 0; c < C; ++c) x[c] = XPF ? xp[u][c][XPF ? g : 0] : xn[c];
          if (!XPF && g + 1 < O::SUB) {
#pragma unroll
            for (int c = 0; c < C; ++c) xn[c].fetch(xrow[c], ch, g + 1, gs);
          }
#pragma unroll
          for (int c = 0; c < C; ++c) xs[c] = O::xsum(x[c], xs[c]);
#pragma unroll
          for (int t = 0; t < RG; ++t) {
#pragma unroll
            for (int c = 0; c < C; ++c) p[t][c] = O::step(w[u][t], x[c], g, p[t][c]);
            // 4-bit codes expand to several registers per dword: expand
            // each row's right where it is used, not all rows up front.
            if constexpr (O::SUB > 1) __builtin_amdgcn_sched_barrier(0);
          }
        }
#pragma unroll
        for (int t = 0; t < RG; ++t)
#pragma unroll
          for (int c = 0; c < C; ++c) acc[t][c] = O::finish(w[u][t], p[t][c], xs[c], acc[t][c]);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < RG; ++t)
#pragma unroll
    for (int c = 0; c < C; ++c) acc[t][c] = group_total<LPR>(acc[t][c]);
}

// Calls f(integral_constant<C>, c0) over pairs [0, n) in passes of the
// widest power of two up to CMAX that the pairs left fill, so that no pass
// computes a vector twice.
template <int CMAX, typename F>
__device__ __forceinline__ void for_passes(int n, F &&f) {
  int c0 = 0;
  if constexpr (CMAX >= 8)
    for (; n - c0 >= 8; c0 += 8) f(std::integral_constant<int, 8>(), c0);
  if constexpr (CMAX >= 4)
    for (; n - c0 >= 4; c0 += 4) f(std::integral_constant<int, 4>(), c0);
  if constexpr (CMAX >= 2)
    for (; n - c0 >= 2; c0 += 2) f(std::integral_constant<int, 2>(), c0);
  for (; c0 < n; ++c0) f(std::integral_constant<int, 1>(), c0);
}

template <int WF>
__device__ __forceinline__ int row_bytes(int K) {
  return K * (WF == F32 ? 4 : WF == BF16 ? 2 : 1) / (is_fp4(WF) ? 2 : 1);
}

// Every array a wave reads through a resource is the same for the whole
// wave; the base and size are made wave-uniform here so that the compiler
// keeps the resource in scalar registers (a resource it cannot prove uniform
// costs a loop over lanes around every load).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void *p, int bytes) {
  const uint64_t u = (uint64_t)p;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)u);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(u >> 32));
  void *q = reinterpret_cast<void *>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(q, (short)0, __builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

// The matrix [N, K] at w (scales s, biases b for 4-bit formats): one
// resource per array, bounded to the array's bytes.
template <int WF> struct Mat {
  __amdgpu_buffer_rsrc_t w, s, b;
  int rb;  // bytes per row
};

template <int WF>
__device__ __forceinline__ Mat<WF> make_mat(const void *w, const void *s, const void *b, int N, int K) {
  Mat<WF> m;
  m.rb = row_bytes<WF>(K);
  m.w = buf_rsrc(w, N * m.rb);
  if constexpr (WF == FP8) {
    m.s = buf_rsrc(s, (N + 127) / 128 * (K / 128) * 4);
    m.b = m.s;
  } else if constexpr (is_fp4(WF)) {
    m.s = buf_rsrc(s, N * m.rb / (WF == NVFP4 ? 8 : 16));
    m.b = WF == AFF4 ? buf_rsrc(b, N * m.rb / 16) : m.s;
  } else {
    m.s = m.b = m.w;
  }
  return m;
}

// Row n of the matrix.  UNI: n is the same for the whole wave.
template <int WF, bool UNI>
__device__ __forceinline__ Row<WF> make_row(const Mat<WF> &m, int n) {
  Row<WF> r;
  r.w = m.w;
  r.s = m.s;
  r.b = m.b;
  r.off = n * m.rb;
  if constexpr (UNI) r.off = __builtin_amdgcn_readfirstlane(r.off);
  if constexpr (WF == FP8) {   // K = rb for fp8: (n / 128) block rows of K / 128 scales
    r.soff = (n >> 7) * (m.rb >> 5);
    if constexpr (UNI) r.soff = __builtin_amdgcn_readfirstlane(r.soff);
  }
  return r;
}

// ------------------------------------------------------ matrix-core tiles
//
// v_mfma_f32_16x16x32_bf16 on one wave: A = 16 weight rows x 32 k (lane l
// holds row l % 16 at k (l / 16) * 8 .. + 7), B = 32 k x 16 vectors (lane l
// holds vector l % 16 at the same k), D = 16 x 16 f32 (lane l holds rows
// (l / 16) * 4 + i, i < 4, of vector l % 16).  Rows past N and vectors past
// nv repeat the last one; the callers drop their results.  Every (row,
// vector) total is accumulated in the same order whatever the number of
// vectors, so results do not depend on m.


// 8 f32 values as two bf16 octets: hi = the top 16 bits, lo = the rest
// rounded to bf16; hi + lo carries 16 significant bits, and the products
// with bf16 weights are exact in the f32 accumulator.
__device__ __forceinline__ void split_bf16(const u32x4 &a, const u32x4 &b, bf16x8 &hi, bf16x8 &lo) {
  const uint32_t f[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint32_t h[4], r[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t f0 = f[2 * i], f1 = f[2 * i + 1];
    h[i] = (f0 >> 16) | (f1 & 0xFFFF0000u);
    const float r0 = __uint_as_float(f0) - __uint_as_float(f0 & 0xFFFF0000u);
    const float r1 = __uint_as_float(f1) - __uint_as_float(f1 & 0xFFFF0000u);
    r[i] = (uint32_t)f32_to_bf16(r0) | ((uint32_t)f32_to_bf16(r1) << 16);
  }
  const u32x4 hv = {h[0], h[1], h[2], h[3]}, rv = {r[0], r[1], r[2], r[3]};
  hi = __builtin_bit_cast(bf16x8, hv);
  lo = __builtin_bit_cast(bf16x8, rv);
}

// F32I pairs (hi in the low half, lo in the high half) of 8 elements into
// the hi and lo operands split_bf16 makes from the f32 values.
__device__ __forceinline__ void unpack_bf16(const u32x4 &a, const u32x4 &b, bf16x8 &hi, bf16x8 &lo) {
  const uint32_t p[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint32_t h[4], r[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = __builtin_amdgcn_perm(p[2 * i + 1], p[2 * i], 0x05040100u);
    r[i] = __builtin_amdgcn_perm(p[2 * i + 1], p[2 * i], 0x07060302u);
  }
  const u32x4 hv = {h[0], h[1], h[2], h[3]}, rv = {r[0], r[1], r[2], r[3]};
  hi = __builtin_bit_cast(bf16x8, hv);
  lo = __builtin_bit_cast(bf16x8, rv);
}

// One f32 value as its F32I pair.
__device__ __forceinline__ uint32_t f32i_pair(float v) {
  const uint32_t f = __float_as_uint(v);
  return (f >> 16) | ((uint32_t)f32_to_bf16(v - __uint_as_float(f & 0xFFFF0000u)) << 16);
}

__device__ __forceinline__ f32x4 mfma16(const u32x4 &a, const bf16x8 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), b, c, 0, 0, 0);
}

// One wave: rows [n0, n0 + 16) of NA bf16 matrices [N, K] (rb bytes per row,
// resources A[j]) against vectors 0..nv-1 of X (bf16 or f32 rows of xstride
// bytes) over k in [kb, ke) (multiples of 32), into acc[j][ct] for vectors
// 16 ct .. 16 ct + 15.
//
// The weights go through LDS: a batch of MU k-steps (MF_U by default) is 16
// rows x MU * 64 bytes per matrix, loaded with lane-linear 16-byte loads
// (with MU = 4 each instruction reads 4 rows x 256 contiguous bytes; the MFMA
// lane pattern itself would read 16 rows x 64 bytes per instruction, which
// streams about a quarter slower), written to this wave's own LDS region,
// and read back in the MFMA layout.  The next batch's loads are in flight
// meanwhile.  `stage` is the wave's region, NA * 16 * (MU * 64 + 16) bytes.
constexpr int MF_U = 4;                  // k-steps of 32 per batch
constexpr int MF_ROW = MF_U * 64 + 16;   // bytes per staged row (16 bytes of padding)
constexpr int MF_STAGE = 16 * MF_ROW;    // staged bytes per matrix per wave

// xv[ct]: where this lane's vector of column tile ct (vector 16 ct + l % 16)
// starts, plus the lane's k offset (l / 16) * 8 elements.
template <int XF, int NA, int NCT, int MU = MF_U>
__device__ __forceinline__ void mfma_slice_v(const __amdgpu_buffer_rsrc_t (&A)[NA], int rb, int n0, int N,
                                             const char *const (&xv)[NCT], int kb, int ke, char *stage,
                                             f32x4 (&acc)[NA][NCT]) {
  constexpr int ROW = MU * 64 + 16, STAGE = 16 * ROW;   // staging layout of MU k-steps
  static_assert(MU <= MF_U, "the wave's staging region holds MF_U k-steps");
  constexpr int XB = XF == F32 || XF == F32I ? 4 : 2;
  constexpr int XL = XF == BF16 ? 1 : 2;   // 16-byte x loads per step and column tile
  const int l = threadIdx.x & 63, g = l >> 4, rr = l & 15;
  // Loader: a staged row is MU * 64 bytes, LR = 4 MU lanes of 16 bytes;
  // instruction i brings rows RI i + l / LR (RI = 16 / MU rows per
  // instruction), bytes (l % LR) * 16 .. + 16 of the batch.
  constexpr int LR = 4 * MU, RI = 16 / MU;
  static_assert(MU == 1 || MU == 2 || MU == 4, "16 rows split evenly over the loads");
  // Nontemporal loads bring whole 128-byte lines that are not kept: with
  // 64 bytes per row per batch (MU = 1) the next batch's half would be
  // fetched from HBM again, so those loads keep the default policy.
  constexpr int POL = MU >= 2 ? BUF_NT : 0;
  const int lrow = l / LR, lcol = l % LR;
  int loff[MU];
#pragma unroll
  for (int i = 0; i < MU; ++i) loff[i] = min(n0 + RI * i + lrow, N - 1) * rb + lcol * 16;
#pragma unroll
  for (int j = 0; j < NA; ++j)
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) acc[j][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (kb >= ke) return;
  // Weights and x of the next batch are requested together, one batch ahead.
  u32x4 nxt[NA][MU], nxb[MU][NCT][XL];
  auto fetch = [&](int kq) {
#pragma unroll
    for (int j = 0; j < NA; ++j)
#pragma unroll
      for (int i = 0; i < MU; ++i) nxt[j][i] = __builtin_amdgcn_raw_buffer_load_b128(A[j], loff[i] + kq * 2, 0, POL);
#pragma unroll
    for (int u = 0; u < MU; ++u) {
      const int kk = min(kq + 32 * u, ke - 32);
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int h = 0; h < XL; ++h) nxb[u][ct][h] = ld16(xv[ct] + (size_t)kk * XB + 16 * h);
    }
  };
  fetch(kb);
  for (int k0 = kb; k0 < ke; k0 += 32 * MU) {
    u32x4 cur[NA][MU], bv[MU][NCT][XL];
#pragma unroll
    for (int j = 0; j < NA; ++j)
#pragma unroll
      for (int i = 0; i < MU; ++i) cur[j][i] = nxt[j][i];
#pragma unroll
    for (int u = 0; u < MU; ++u)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int h = 0; h < XL; ++h) bv[u][ct][h] = nxb[u][ct][h];
    const int k1 = k0 + 32 * MU;
    if (k1 < ke) fetch(k1);
#pragma unroll
    for (int j = 0; j < NA; ++j)
#pragma unroll
      for (int i = 0; i < MU; ++i)
        *reinterpret_cast<u32x4 *>(stage + j * STAGE + (RI * i + lrow) * ROW + lcol * 16) = cur[j][i];
    // The region is this wave's alone; its LDS accesses complete in order.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int u = 0; u < MU; ++u) {
      if (k0 + 32 * u < ke) {
        u32x4 av[NA];
#pragma unroll
        for (int j = 0; j < NA; ++j)
          av[j] = *reinterpret_cast<const u32x4 *>(stage + j * STAGE + rr * ROW + u * 64 + g * 16);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          if constexpr (XF == BF16) {
            const bf16x8 bb = __builtin_bit_cast(bf16x8, bv[u][ct][0]);
#pragma unroll
            for (int j = 0; j < NA; ++j) acc[j][ct] = mfma16(av[j], bb, acc[j][ct]);
          } else {
            bf16x8 hi, lo;
            if constexpr (XF == F32I) unpack_bf16(bv[u][ct][0], bv[u][ct][XL - 1], hi, lo);
            else split_bf16(bv[u][ct][0], bv[u][ct][XL - 1], hi, lo);
#pragma unroll
            for (int j = 0; j < NA; ++j) {
              acc[j][ct] = mfma16(av[j], hi, acc[j][ct]);
              acc[j][ct] = mfma16(av[j], lo, acc[j][ct]);
            }
          }
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

// Vectors at x + v * xstride, v < nv (vectors past nv repeat the last one).
template <int XF, int NA, int NCT, int MU = MF_U>
__device__ __forceinline__ void mfma_slice(const __amdgpu_buffer_rsrc_t (&A)[NA], int rb, int n0, int N,
                                           const char *x, size_t xstride, int nv, int kb, int ke,
                                           char *stage, f32x4 (&acc)[NA][NCT]) {
  constexpr int XB = XF == F32 || XF == F32I ? 4 : 2;
  const int l = threadIdx.x & 63, g = l >> 4, rr = l & 15;
  const char *xv[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) xv[ct] = x + (size_t)min(16 * ct + rr, nv - 1) * xstride + (size_t)g * 8 * XB;
  mfma_slice_v<XF, NA, NCT, MU>(A, rb, n0, N, xv, kb, ke, stage, acc);
}

// One vector's product with 16 bf16 rows on the matrix cores (the shared
// down at m = 1), with the weights and the f32 input brought into LDS by the
// loads themselves (buffer loads that write LDS).  The wave owns DMA_NB slots
// of one batch each -- 16 rows x 64 k of weights (2 KB) and the input's 64
// values (256 B) -- and keeps DMA_NB - 1 batches in flight while it consumes
// one: twice the bytes in flight of mfma_slice_v's register prefetch, and no
// register holds a weight in flight.  Chunk c (16 bytes) of row r sits at
// chunk r * 8 + (c ^ (r >> 1)) of the slot, so the operand reads of 16 rows at
// one chunk fall in 16 distinct 16-byte bank groups.  The MFMA sequence --
// k steps in order, the input's high then low bf16 part -- is mfma_slice_v's
// with every column reading the one vector, so the sums are bitwise the same.
constexpr int DMA_NB = 3;
constexpr int DMA_SLOT = 2048 + 256;
struct SharedDnRing {
  float part[WPB][4][WAVE];
  alignas(16) char slot[WPB][DMA_NB * DMA_SLOT];
};

__device__ __forceinline__ void mfma_slice_dma(__amdgpu_buffer_rsrc_t A, int rb, int n0, int N,
                                               __amdgpu_buffer_rsrc_t X, int kb, int ke, char *ring,
                                               f32x4 &acc) {
  typedef __attribute__((address_space(3))) void *lds_ptr;
  const int l = threadIdx.x & 63, g = l >> 4, rr = l & 15;
  acc = f32x4{0.f, 0.f, 0.f, 0.f};
  if (kb >= ke) return;
  const int nb = (ke - kb + 63) / 64;
  // Lane l brings chunk positions l and 64 + l of a batch.
  int voff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int p = 64 * i + l, r = p >> 3, c = (p & 7) ^ (r >> 1);
    voff[i] = min(n0 + r, N - 1) * rb + c * 16;
  }
  // Three loads per batch: two of weights, one of input (lanes 0..15).
  auto issue = [&](int b) {
    char *sl = ring + (b % DMA_NB) * DMA_SLOT;
    const int kq = kb + 64 * b;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(A, (lds_ptr)(sl + 1024 * i), 16, voff[i] + kq * 2, 0, 0, BUF_NT);
    if (l < 16) __builtin_amdgcn_raw_ptr_buffer_load_lds(X, (lds_ptr)(sl + 2048), 16, kq * 4 + l * 16, 0, 0, 0);
  };
  for (int b = 0; b < DMA_NB - 1 && b < nb; ++b) issue(b);
  for (int b = 0; b < nb; ++b) {
    if (b + DMA_NB - 1 < nb) issue(b + DMA_NB - 1);
    // Batch b's loads are done once no more than the later batches' remain
    // outstanding (vector memory loads complete in order for the count).
    const int later = min(nb - 1 - b, DMA_NB - 1);
    if (later >= 2) __builtin_amdgcn_s_waitcnt(0x0F70 | 6);
    else if (later == 1) __builtin_amdgcn_s_waitcnt(0x0F70 | 3);
    else __builtin_amdgcn_s_waitcnt(0x0F70);
    asm volatile("" ::: "memory");
    // The slot is read with LDS loads written out here, each batch's three
    // waited for in the same statement: the compiler would otherwise wait for
    // every load into LDS in flight (it cannot tell the slots apart) before
    // any LDS read, which would leave one batch in flight.
    const unsigned sl = (unsigned)(uintptr_t)(lds_ptr)(ring + (b % DMA_NB) * DMA_SLOT);
    const int k0 = kb + 64 * b;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if (k0 + 32 * u < ke) {
        const int c = 4 * u + g;
        const unsigned pa = sl + (rr * 8 + (c ^ (rr >> 1))) * 16, px = sl + 2048 + (32 * u + 8 * g) * 4;
        u32x4 av, b0, b1;
        asm volatile(
            "ds_read_b128 %0, %3\n\t"
            "ds_read_b128 %1, %4\n\t"
            "ds_read_b128 %2, %4 offset:16\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=v"(av), "=v"(b0), "=v"(b1)
            : "v"(pa), "v"(px)
            : "memory");
        bf16x8 hi, lo;
        unpack_bf16(b0, b1, hi, lo);   // the input is stored as F32I pairs
        acc = mfma16(av, hi, acc);
        acc = mfma16(av, lo, acc);
      }
    }
    asm volatile("" ::: "memory");   // the slot's reads precede its next load
  }
}

// 4-bit weights (MXFP4, NVFP4) on the matrix cores.  The loader brings a
// batch of two k steps of 16 rows as codes -- 8 bytes (16 codes) per lane --
// with their block scales, dequantises them to bf16 and stages them in the
// layout mfma_slice_v reads.  Both decodings are exact in bf16: E2M1 times a
// power of two (E8M0), and E2M1 times E4M3 (at most 6 significant bits).
// The NVFP4 second-level scale is left to the caller.
template <int WF> struct QMat {
  // codes [N, K/2]; scale bytes [N, K/32] (mxfp4) or [N, K/16] (nvfp4), or
  // bf16 scales and biases [N, K/64] (aff4); fp8: codes [N, K], fp32
  // scales [N/128, K/128]
  __amdgpu_buffer_rsrc_t w, s, b;
};

template <int WF>
__device__ __forceinline__ QMat<WF> make_qmat(const void *w, const void *s, const void *b, int N, int K) {
  QMat<WF> m;
  if constexpr (WF == FP8) {
    m.w = buf_rsrc(w, N * K);
    m.s = buf_rsrc(s, (N + 127) / 128 * (K / 128) * 4);
    m.b = m.s;
  } else {
    m.w = buf_rsrc(w, N * (K / 2));
    m.s = buf_rsrc(s, WF == AFF4 ? N * (K / 64) * 2 : N * (K / (WF == NVFP4 ? 16 : 32)));
    m.b = WF == AFF4 ? buf_rsrc(b, N * (K / 64) * 2) : m.s;
  }
  return m;
}

// mfma_slice_v with 4-bit weights A[j] (K = the matrices' row length).
// A batch of two k steps is 16 rows x 64 codes = 512 bytes per matrix: lane
// l loads 8 bytes (16 codes: row l / 4, k step (l / 2) % 2, half l % 2).
template <int WF>
__device__ __forceinline__ void dequant16(const u32x2 &q, uint32_t s, u32x4 (&o)[2]) {
  if constexpr (WF == MXFP4) {
    const float sc = e8m0_to_f32(s & 0xFFu);   // a power of two: the scaled conversion is exact
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      const uint32_t qd = d == 0 ? q.x : q.y;
      o[d] = u32x4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(qd, sc, 0)),
                   __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(qd, sc, 1)),
                   __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(qd, sc, 2)),
                   __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(qd, sc, 3))};
    }
  } else {
    const float sc = e4m3_to_f32(s & 0xFFu);
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      const uint32_t qd = d == 0 ? q.x : q.y;
      uint32_t pr[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const f32x2 v = t == 0 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(qd, 1.0f, 0)
                      : t == 1 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(qd, 1.0f, 1)
                      : t == 2 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(qd, 1.0f, 2)
                               : __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(qd, 1.0f, 3);
        const uint32_t x0 = __float_as_uint(v.x * sc), x1 = __float_as_uint(v.y * sc);
        pr[t] = (x0 >> 16) | (x1 & 0xFFFF0000u);
      }
      o[d] = u32x4{pr[0], pr[1], pr[2], pr[3]};
    }
  }
}

template <int WF, int XF, int NA, int NCT, int MU>
__device__ __forceinline__ void mfma_slice_q(const QMat<WF> (&A)[NA], int K, int n0, int N,
                                             const char *const (&xv)[NCT], int kb, int ke, char *stage,
                                             f32x4 (&acc)[NA][NCT]) {
  constexpr int ROW = MU * 64 + 16, STAGE = 16 * ROW;
  static_assert(MU == 2, "two k steps per batch");
  static_assert(WF == MXFP4 || WF == NVFP4, "4-bit formats");
  constexpr int XB = XF == F32 || XF == F32I ? 4 : 2;
  constexpr int XL = XF == F32 ? 2 : 1;
  const int l = threadIdx.x & 63, g = l >> 4, rr = l & 15;
  const int lr = l >> 2, ks = (l >> 1) & 1, hh = l & 1;
  const int qrow = min(n0 + lr, N - 1);
  const int qoff = qrow * (K / 2) + ks * 16 + hh * 8;
  const int soff = WF == NVFP4 ? qrow * (K / 16) + ks * 2 + hh : qrow * (K / 32) + ks;
#pragma unroll
  for (int j = 0; j < NA; ++j)
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) acc[j][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (kb >= ke) return;
  u32x2 nq[NA];
  u32x4 nxb[MU][NCT][XL];
  uint32_t ns[NA];
  auto fetch = [&](int kq) {
#pragma unroll
    for (int j = 0; j < NA; ++j) {
      nq[j] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(A[j].w, qoff + kq / 2, 0, 0));
      if constexpr (WF == NVFP4)
        ns[j] = __builtin_amdgcn_raw_buffer_load_b8(A[j].s, soff + kq / 16, 0, 0);
      else
        ns[j] = __builtin_amdgcn_raw_buffer_load_b8(A[j].s, soff + kq / 32, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < MU; ++u) {
      const int kk = min(kq + 32 * u, ke - 32);
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int hx = 0; hx < XL; ++hx) nxb[u][ct][hx] = ld16(xv[ct] + (size_t)kk * XB + 16 * hx);
    }
  };
  fetch(kb);
  for (int k0 = kb; k0 < ke; k0 += 32 * MU) {
    u32x2 cq[NA];
    u32x4 bv[MU][NCT][XL];
    uint32_t cs[NA];
#pragma unroll
    for (int j = 0; j < NA; ++j) {
      cq[j] = nq[j];
      cs[j] = ns[j];
    }
#pragma unroll
    for (int u = 0; u < MU; ++u)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int hx = 0; hx < XL; ++hx) bv[u][ct][hx] = nxb[u][ct][hx];
    const int k1 = k0 + 32 * MU;
    if (k1 < ke) fetch(k1);
#pragma unroll
    for (int j = 0; j < NA; ++j) {
      u32x4 o[2];
      dequant16<WF>(cq[j], cs[j], o);
#pragma unroll
      for (int t = 0; t < 2; ++t)
        *reinterpret_cast<u32x4 *>(stage + j * STAGE + lr * ROW + ks * 64 + hh * 32 + 16 * t) = o[t];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int u = 0; u < MU; ++u) {
      if (k0 + 32 * u < ke) {
        u32x4 av[NA];
#pragma unroll
        for (int j = 0; j < NA; ++j)
          av[j] = *reinterpret_cast<const u32x4 *>(stage + j * STAGE + rr * ROW + u * 64 + g * 16);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          if constexpr (XF == BF16) {
            const bf16x8 bb = __builtin_bit_cast(bf16x8, bv[u][ct][0]);
#pragma unroll
            for (int j = 0; j < NA; ++j) acc[j][ct] = mfma16(av[j], bb, acc[j][ct]);
          } else {
            bf16x8 hi, lo;
            if constexpr (XF == F32I) unpack_bf16(bv[u][ct][0], bv[u][ct][XL - 1], hi, lo);
            else split_bf16(bv[u][ct][0], bv[u][ct][XL - 1], hi, lo);
#pragma unroll
            for (int j = 0; j < NA; ++j) {
              acc[j][ct] = mfma16(av[j], hi, acc[j][ct]);
              acc[j][ct] = mfma16(av[j], lo, acc[j][ct]);
            }
          }
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

// The same products with the 4-bit codes loaded straight into the MFMA
// operands (no LDS): a k-sum does not depend on the order of k, so within a
// batch of MU k steps (32 MU elements) lane (row r, group g) takes elements
// [8 MU g, 8 MU (g + 1)) -- 4 MU contiguous code bytes, one load -- and uses
// elements 8 u .. 8 u + 7 of that range as its fragment of k step u; the
// input vectors are read in the same order.  Fragments at or past ke are
// zeroed (k ranges are multiples of 32, batches may run past them).
// xr[ct]: the start of this lane's vector 16 ct + l % 16.
template <int WF, int XF, int NA, int NCT, int MU>
__device__ __forceinline__ void mfma_slice_qd(const QMat<WF> (&A)[NA], int K, int n0, int N,
                                              const char *const (&xr)[NCT], int kb, int ke,
                                              f32x4 (&acc)[NA][NCT]) {
  static_assert(WF == MXFP4 || WF == NVFP4, "4-bit formats with one scale per code block");
  static_assert(MU == 1 || MU == 2 || MU == 4, "a lane's range lies in one scale block");
  constexpr int CB = 4 * MU;                       // code bytes per lane per batch
  constexpr int XB = XF == F32 || XF == F32I ? 4 : 2;
  constexpr int XQ = 8 * MU * XB / 16;             // 16-byte x loads per lane, batch and tile
  const int l = threadIdx.x & 63, g = l >> 4, rr = l & 15;
  const int row = min(n0 + rr, N - 1);
  const int qoff = row * (K / 2) + g * CB;
  const int soff = WF == NVFP4 ? row * (K / 16) + (8 * MU * g) / 16 : row * (K / 32) + (8 * MU * g) / 32;
#pragma unroll
  for (int j = 0; j < NA; ++j)
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) acc[j][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (kb >= ke) return;
  typedef uint32_t cvec __attribute__((ext_vector_type(MU)));
  cvec nq[NA];
  uint32_t ns[NA];
  u32x4 nx[NCT][XQ];
  auto fetch = [&](int kq) {
#pragma unroll
    for (int j = 0; j < NA; ++j) {
      if constexpr (MU == 4) nq[j] = __builtin_bit_cast(cvec, __builtin_amdgcn_raw_buffer_load_b128(A[j].w, qoff + kq / 2, 0, 0));
      else if constexpr (MU == 2) nq[j] = __builtin_bit_cast(cvec, __builtin_amdgcn_raw_buffer_load_b64(A[j].w, qoff + kq / 2, 0, 0));
      else nq[j] = __builtin_bit_cast(cvec, __builtin_amdgcn_raw_buffer_load_b32(A[j].w, qoff + kq / 2, 0, 0));
      if constexpr (WF == NVFP4 && MU == 4) ns[j] = __builtin_amdgcn_raw_buffer_load_b16(A[j].s, soff + kq / 16, 0, 0);
      else if constexpr (WF == NVFP4) ns[j] = __builtin_amdgcn_raw_buffer_load_b8(A[j].s, soff + kq / 16, 0, 0);
      else ns[j] = __builtin_amdgcn_raw_buffer_load_b8(A[j].s, soff + kq / 32, 0, 0);
    }
    // The lane's x range, clamped into the row (zeroed fragments cover the
    // part past ke).
    const int kx = min(kq + 8 * MU * g, K - 8 * MU);
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int h = 0; h < XQ; ++h) nx[ct][h] = ld16(xr[ct] + (size_t)kx * XB + 16 * h);
  };
  fetch(kb);
  for (int k0 = kb; k0 < ke; k0 += 32 * MU) {
    cvec cq[NA];
    uint32_t cs[NA];
    u32x4 cx[NCT][XQ];
#pragma unroll
    for (int j = 0; j < NA; ++j) {
      cq[j] = nq[j];
      cs[j] = ns[j];
    }
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int h = 0; h < XQ; ++h) cx[ct][h] = nx[ct][h];
    if (k0 + 32 * MU < ke) fetch(k0 + 32 * MU);
#pragma unroll
    for (int u = 0; u < MU; ++u) {
      const bool valid = k0 + 8 * MU * g + 8 * u < ke;
      u32x4 av[NA];
#pragma unroll
      for (int j = 0; j < NA; ++j) {
        const uint32_t qd = cq[j][u];
        uint32_t pr[4];
        if constexpr (WF == MXFP4) {
          const float sc = e8m0_to_f32(cs[j] & 0xFFu);
          // The E8M0 scale is a power of two: the scaled conversion is exact.
          pr[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(qd, sc, 0));
          pr[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(qd, sc, 1));
          pr[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(qd, sc, 2));
          pr[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(qd, sc, 3));
#pragma unroll
          for (int t = 0; t < 4; ++t) pr[t] = valid ? pr[t] : 0u;
        } else {
          const float sc = e4m3_to_f32(MU == 4 ? (cs[j] >> (8 * (u >> 1))) & 0xFFu : cs[j] & 0xFFu);
          f32x2 v[4];
          v[0] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(qd, 1.0f, 0);
          v[1] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(qd, 1.0f, 1);
          v[2] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(qd, 1.0f, 2);
          v[3] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(qd, 1.0f, 3);
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            // Exact bf16 products: their low 16 bits are zero.
            const uint32_t a = __float_as_uint(v[t].x * sc), b = __float_as_uint(v[t].y * sc);
            pr[t] = valid ? (a >> 16) | (b & 0xFFFF0000u) : 0u;
          }
        }
        av[j] = u32x4{pr[0], pr[1], pr[2], pr[3]};
      }
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        if constexpr (XF == BF16) {
          const bf16x8 bb = __builtin_bit_cast(bf16x8, cx[ct][u]);
#pragma unroll
          for (int j = 0; j < NA; ++j) acc[j][ct] = mfma16(av[j], bb, acc[j][ct]);
        } else {
          bf16x8 hi, lo;
          if constexpr (XF == F32I) unpack_bf16(cx[ct][2 * u], cx[ct][2 * u + 1], hi, lo);
          else split_bf16(cx[ct][2 * u], cx[ct][2 * u + 1], hi, lo);
#pragma unroll
          for (int j = 0; j < NA; ++j) {
            acc[j][ct] = mfma16(av[j], hi, acc[j][ct]);
            acc[j][ct] = mfma16(av[j], lo, acc[j][ct]);
          }
        }
      }
    }
  }
}

// The k range of wave w when nw waves split K (a multiple of 32) evenly.
__device__ __forceinline__ void k_slice(int K, int w, int nw, int &kb, int &ke) {
  const int steps = K / 32, per = (steps + nw - 1) / nw;
  kb = min(w * per, steps) * 32;
  ke = min((w + 1) * per, steps) * 32;
}

// The same in whole 64-element groups (K a multiple of 64).
__device__ __forceinline__ void k_slice64(int K, int w, int nw, int &kb, int &ke) {
  const int steps = K / 64, per = (steps + nw - 1) / nw;
  kb = min(w * per, steps) * 64;
  ke = min((w + 1) * per, steps) * 64;
}

// The same in whole 128-element blocks (K a multiple of 128).
__device__ __forceinline__ void k_slice128(int K, int w, int nw, int &kb, int &ke) {
  const int steps = K / 128, per = (steps + nw - 1) / nw;
  kb = min(w * per, steps) * 128;
  ke = min((w + 1) * per, steps) * 128;
}

// Lane (l & ~3) + I's value, for every lane l (a broadcast within quads).
template <int I> __device__ __forceinline__ uint32_t quad_bcast(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, I * 0x55, 0xF, 0xF, false);
}

// aff4 on the matrix cores.  A 64-element group's weights are s q + b, so
// its sum over k is s (D - 128 X) + b X, with D the sum of (128 + q) x and X
// the sum of x.  The codes enter the products as the bf16 values 128 + q
// (bits 0x4300 | q, exact), X is a product with an all-ones operand, and
// every product of two bf16 values is exact in the f32 accumulators; no
// weight is rounded.  A batch is one group (k ranges are multiples of 64):
// lane (row l % 16, g = l / 16) takes elements [16 g, 16 g + 16) of it, the
// first 8 in k step 0 and the rest in k step 1 (a sum does not depend on the
// order of k), and the input vectors are read in the same order.  D and X
// start from zero in every group; the lane then adds s D + (b - 128 s) X for
// its accumulator rows 4 g + i, whose scale and bias come from lane
// (l & ~3) + i of its quad, which loaded those of row 4 g + i.
// xr[ct]: the start of this lane's vector 16 ct + l % 16.
template <int XF, int NA, int NCT>
__device__ __forceinline__ void mfma_slice_aff4(const QMat<AFF4> (&A)[NA], int K, int n0, int N,
                                                const char *const (&xr)[NCT], int kb, int ke,
                                                f32x4 (&acc)[NA][NCT]) {
  constexpr int XB = XF == F32 || XF == F32I ? 4 : 2;
  constexpr int XQ = XB;                           // 16-byte x loads per lane, group and tile
  const int l = threadIdx.x & 63, g = l >> 4, rr = l & 15;
  const int qoff = min(n0 + rr, N - 1) * (K / 2) + g * 8;
  const int soff = min(n0 + 4 * g + (l & 3), N - 1) * (K / 64) * 2;
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < NA; ++j)
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) acc[j][ct] = zero;
  if (kb >= ke) return;
  const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  u32x2 nq[NA];
  uint32_t ns[NA], nb[NA];
  u32x4 nx[NCT][XQ];
  auto fetch = [&](int kq) {
#pragma unroll
    for (int j = 0; j < NA; ++j) {
      nq[j] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(A[j].w, qoff + kq / 2, 0, 0));
      ns[j] = __builtin_amdgcn_raw_buffer_load_b16(A[j].s, soff + (kq >> 6) * 2, 0, 0);
      nb[j] = __builtin_amdgcn_raw_buffer_load_b16(A[j].b, soff + (kq >> 6) * 2, 0, 0);
    }
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int h = 0; h < XQ; ++h) nx[ct][h] = ld16(xr[ct] + (size_t)(kq + 16 * g) * XB + 16 * h);
  };
  fetch(kb);
  for (int k0 = kb; k0 < ke; k0 += 64) {
    u32x2 cq[NA];
    uint32_t cs[NA], cb[NA];
    u32x4 cx[NCT][XQ];
#pragma unroll
    for (int j = 0; j < NA; ++j) {
      cq[j] = nq[j];
      cs[j] = ns[j];
      cb[j] = nb[j];
    }
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int h = 0; h < XQ; ++h) cx[ct][h] = nx[ct][h];
    if (k0 + 64 < ke) fetch(k0 + 64);
    f32x4 D[NA][NCT], X[NCT];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      u32x4 av[NA];
#pragma unroll
      for (int j = 0; j < NA; ++j) {
        const uint32_t q = cq[j][u], qs = q >> 4;
        uint32_t pr[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          // byte t of q (low nibble: element 2t) to bits 0..7, byte t of
          // q >> 4 (element 2t + 1) to bits 16..23, zeros elsewhere
          const uint32_t p = __builtin_amdgcn_perm(qs, q, 0x0C000C00u | (uint32_t)((4 + t) << 16) | (uint32_t)t);
          pr[t] = (p & 0x000F000Fu) | 0x43004300u;
        }
        av[j] = u32x4{pr[0], pr[1], pr[2], pr[3]};
      }
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        if constexpr (XF == BF16) {
          const bf16x8 bb = __builtin_bit_cast(bf16x8, cx[ct][u]);
          X[ct] = mfma16(ones, bb, u ? X[ct] : zero);
#pragma unroll
          for (int j = 0; j < NA; ++j) D[j][ct] = mfma16(av[j], bb, u ? D[j][ct] : zero);
        } else {
          bf16x8 hi, lo;
          if constexpr (XF == F32I) unpack_bf16(cx[ct][2 * u], cx[ct][2 * u + 1], hi, lo);
          else split_bf16(cx[ct][2 * u], cx[ct][2 * u + 1], hi, lo);
          X[ct] = mfma16(ones, hi, u ? X[ct] : zero);
          X[ct] = mfma16(ones, lo, X[ct]);
#pragma unroll
          for (int j = 0; j < NA; ++j) {
            D[j][ct] = mfma16(av[j], hi, u ? D[j][ct] : zero);
            D[j][ct] = mfma16(av[j], lo, D[j][ct]);
          }
        }
      }
    }
#pragma unroll
    for (int j = 0; j < NA; ++j) {
      float sc[4], bc[4];
      sc[0] = bf16_to_f32((uint16_t)quad_bcast<0>(cs[j]));
      sc[1] = bf16_to_f32((uint16_t)quad_bcast<1>(cs[j]));
      sc[2] = bf16_to_f32((uint16_t)quad_bcast<2>(cs[j]));
      sc[3] = bf16_to_f32((uint16_t)quad_bcast<3>(cs[j]));
      bc[0] = bf16_to_f32((uint16_t)quad_bcast<0>(cb[j]));
      bc[1] = bf16_to_f32((uint16_t)quad_bcast<1>(cb[j]));
      bc[2] = bf16_to_f32((uint16_t)quad_bcast<2>(cb[j]));
      bc[3] = bf16_to_f32((uint16_t)quad_bcast<3>(cb[j]));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float bp = __builtin_fmaf(-128.0f, sc[i], bc[i]);   // b - 128 s, one rounding
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
          acc[j][ct][i] = __builtin_fmaf(sc[i], D[j][ct][i], __builtin_fmaf(bp, X[ct][i], acc[j][ct][i]));
      }
    }
  }
}

// FP8 (E4M3 codes, one fp32 scale per 128 x 128 block) on the matrix cores.
// Every E4M3 value is exact in bf16, so the codes enter the products as
// bf16 (v_cvt_scalef32_pk_bf16_fp8 with scale 1); a 128-element group's sum
// starts from zero and is then added to the total times the group's scale,
// which the 16 rows of a tile share (tiles start at multiples of 16, blocks
// at multiples of 128, N is a multiple of 128).  A batch is half a group
// (two k steps): lane (row l % 16, g = l / 16) takes elements
// [16 g, 16 g + 16) of it -- 16 contiguous code bytes, one load -- the first
// 8 as its fragment of k step 0 and the rest of k step 1 (a sum does not
// depend on the order of k), and the input vectors are read in the same
// order.  K, kb and ke are multiples of 128.
// xr[ct]: the start of this lane's vector 16 ct + l % 16.
template <int XF, int NA, int NCT>
__device__ __forceinline__ void mfma_slice_f8(const QMat<FP8> (&A)[NA], int K, int n0, int N,
                                              const char *const (&xr)[NCT], int kb, int ke,
                                              f32x4 (&acc)[NA][NCT]) {
  constexpr int XB = XF == F32 || XF == F32I ? 4 : 2;
  constexpr int XQ = XB;                           // 16-byte x loads per lane, batch and tile
  const int l = threadIdx.x & 63, g = l >> 4, rr = l & 15;
  const int qoff = min(n0 + rr, N - 1) * K + g * 16;
  const int srow = __builtin_amdgcn_readfirstlane((min(n0, N - 1) >> 7) * (K >> 7) * 4);   // the tile's scale row
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < NA; ++j)
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) acc[j][ct] = zero;
  if (kb >= ke) return;
  u32x4 nq[NA];
  uint32_t ns[NA];
  u32x4 nx[NCT][XQ];
  auto fetch = [&](int kq) {
#pragma unroll
    for (int j = 0; j < NA; ++j) {
      nq[j] = __builtin_amdgcn_raw_buffer_load_b128(A[j].w, qoff + kq, 0, 0);
      ns[j] = __builtin_amdgcn_raw_buffer_load_b32(A[j].s, 0, srow + (kq >> 7) * 4, 0);
    }
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int h = 0; h < XQ; ++h) nx[ct][h] = ld16(xr[ct] + (size_t)(kq + 16 * g) * XB + 16 * h);
  };
  fetch(kb);
  f32x4 D[NA][NCT];
  for (int k0 = kb; k0 < ke; k0 += 64) {
    u32x4 cq[NA];
    uint32_t cs[NA];
    u32x4 cx[NCT][XQ];
#pragma unroll
    for (int j = 0; j < NA; ++j) {
      cq[j] = nq[j];
      cs[j] = ns[j];
    }
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int h = 0; h < XQ; ++h) cx[ct][h] = nx[ct][h];
    if (k0 + 64 < ke) fetch(k0 + 64);
    const bool first = (k0 & 127) == 0;   // the group's first half
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      u32x4 av[NA];
#pragma unroll
      for (int j = 0; j < NA; ++j) {
        const uint32_t q0 = u ? cq[j].z : cq[j].x, q1 = u ? cq[j].w : cq[j].y;
        av[j] = u32x4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q0, 1.0f, false)),
                      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q0, 1.0f, true)),
                      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q1, 1.0f, false)),
                      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q1, 1.0f, true))};
      }
      const bool fresh = first && u == 0;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        if constexpr (XF == BF16) {
          const bf16x8 bb = __builtin_bit_cast(bf16x8, cx[ct][u]);
#pragma unroll
          for (int j = 0; j < NA; ++j) D[j][ct] = mfma16(av[j], bb, fresh ? zero : D[j][ct]);
        } else {
          bf16x8 hi, lo;
          if constexpr (XF == F32I) unpack_bf16(cx[ct][2 * u], cx[ct][2 * u + 1], hi, lo);
          else split_bf16(cx[ct][2 * u], cx[ct][2 * u + 1], hi, lo);
#pragma unroll
          for (int j = 0; j < NA; ++j) {
            D[j][ct] = mfma16(av[j], hi, fresh ? zero : D[j][ct]);
            D[j][ct] = mfma16(av[j], lo, D[j][ct]);
          }
        }
      }
    }
    if (!first) {   // the group is complete: add it, scaled
#pragma unroll
      for (int j = 0; j < NA; ++j) {
        const float sc = __uint_as_float(cs[j]);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[j][ct][i] = __builtin_fmaf(sc, D[j][ct][i], acc[j][ct][i]);
      }
    }
  }
}

// Partials of the NW waves of one matrix-core item, added in wave order.
// MU: k-steps per staged batch (mfma_slice<..., MU>).
template <int NW, int NA, int MU = MF_U> struct MfmaLDS {
  float part[NW][NA][2][4][WAVE];   // [wave][matrix][column tile][i][lane]
  alignas(16) char stage[NW][NA * 16 * (MU * 64 + 16)];   // each wave's weight staging
};

__device__ __forceinline__ size_t act_bytes(int fmt) { return fmt == F32 ? 4 : 2; }

__device__ __forceinline__ int uniform_i(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ uint64_t uniform_u64(uint64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}

// Entry e (wave-uniform) of a device pointer table, as a wave-uniform pointer.
__device__ __forceinline__ const void *tbl(const uint64_t *t, int e) {
  if (!t) return nullptr;
  const uint64_t v = t[uniform_i(e)];
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
  return reinterpret_cast<const void *>(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ int clamp_i(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

// The routing a forward publishes is used only if the publishing workgroup
// wrote this call's tag (Args::tag: the host's hash of the call's tables,
// input, workspace and row count) into the workspace word SYNC_PUBLISHED
// after the slot records and the active count.  A consumer reads the word
// with the count (one memory round trip) and takes no routed work when it
// differs: records another call left behind are never streamed from.
__device__ __forceinline__ int published_count(const Args &a) {
  const int n = a.active_count[0];
  const unsigned pub = a.sync[SYNC_PUBLISHED];
  return pub == (unsigned)a.tag ? clamp_i(n, 0, a.cap) : 0;
}

// Cross-workgroup hand-off inside one launch.  Every workgroup completes its
// stores and takes a ticket from *ctr; the one that takes ticket n - 1 (every
// other has stored by then) returns true.  Nobody waits.  Every thread of the
// workgroup calls it; tk is a __shared__ word.
//
// FENCES: the workgroups release their stores at agent scope before the
// ticket and the last one acquires after it, which orders them under the
// HIP memory model.  Without: the data handed over must be written and read
// only with agent-scope atomics (device-coherent stores and loads, which
// skip the non-coherent state of the per-XCD L2s); s_waitcnt(0) completes the
// stores, at the device-coherent level, before the ticket's atomic is
// issued, so the last arrival's loads find them.  The route launch takes
// this second form: every router workgroup's release fence writes back its
// XCD's L2, where the launch's shared-expert items keep their output, and
// cost up to 5 us of the route stage (256 experts, 16 rows).
template <bool FENCES>
__device__ __forceinline__ bool last_arrival(unsigned *ctr, unsigned n, unsigned &tk) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    if constexpr (FENCES) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    tk = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if constexpr (FENCES) {
      if (tk == n - 1) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
  }
  __syncthreads();
  return tk == n - 1;
}

// ------------------------------------------------------------------ router
//
// Router unit u = (router row e, block of up to 8 input rows): logits[r, e] =
// sum_h x[r,h] W[e,h], every product and sum in double.  Row E is the shared
// expert's gate vector w_g.  RSPLIT waves share a unit, wave `part` taking the
// part-th quarter of the chunks; each returns its per-row partial totals (in
// every lane), which the caller adds in part order.  The loads of a chunk
// step (the router chunk and all 8 rows' x chunks) are issued before any is
// used, so the rows cost one memory round trip, not eight.
template <int ACT>
__device__ __forceinline__ void router_part(const Args &a, int unit, int part, double (&tot)[8]) {
  constexpr int EPC = ACT == F32 ? 4 : 8;
  constexpr int RU = 1;                      // chunk steps whose loads are in flight together
  const int lane = threadIdx.x & 63;
  const int nrows = router_rows(a);
  const int e = unit % nrows, r0 = (unit / nrows) * 8;
  const int nr = min(8, a.m - r0);           // input rows of this unit
  const int nchunks = a.H / EPC;
  const int c0 = part * nchunks / RSPLIT, c1 = (part + 1) * nchunks / RSPLIT;
  const size_t xstride = (size_t)a.H * act_bytes(ACT);
  const char *wrow = e < a.E ? reinterpret_cast<const char *>(a.router) + (size_t)e * xstride
                             : reinterpret_cast<const char *>(a.sgv);
  const char *x = reinterpret_cast<const char *>(a.xr) + (size_t)r0 * xstride;
  double acc[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) acc[r] = 0.0;
  for (int base = c0; base < c1; base += WAVE * RU) {
    // Every load of the step is issued before any is used.  Rows past nr
    // repeat row nr - 1 (in bounds) and are not accumulated.
    u32x4 q[RU], v[8][RU];
#pragma unroll
    for (int u = 0; u < RU; ++u) {
      const int ch = base + lane + u * WAVE;
      if (ch < c1) q[u] = ld16(wrow + (size_t)ch * 16);
    }
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int rr = min(r, nr - 1);
#pragma unroll
      for (int u = 0; u < RU; ++u) {
        const int ch = base + lane + u * WAVE;
        if (ch < c1) v[r][u] = ld16(x + (size_t)rr * xstride + (size_t)ch * 16);
      }
    }
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      if (r < nr) {
#pragma unroll
        for (int u = 0; u < RU; ++u) {
          const int ch = base + lane + u * WAVE;
          if (ch < c1) {
            float w[EPC], xv[EPC];
            if constexpr (ACT == F32) {
              w[0] = __uint_as_float(q[u].x); w[1] = __uint_as_float(q[u].y);
              w[2] = __uint_as_float(q[u].z); w[3] = __uint_as_float(q[u].w);
              xv[0] = __uint_as_float(v[r][u].x); xv[1] = __uint_as_float(v[r][u].y);
              xv[2] = __uint_as_float(v[r][u].z); xv[3] = __uint_as_float(v[r][u].w);
            } else {
              w[0] = bf_lo(q[u].x); w[1] = bf_hi(q[u].x); w[2] = bf_lo(q[u].y); w[3] = bf_hi(q[u].y);
              w[4] = bf_lo(q[u].z); w[5] = bf_hi(q[u].z); w[6] = bf_lo(q[u].w); w[7] = bf_hi(q[u].w);
              xv[0] = bf_lo(v[r][u].x); xv[1] = bf_hi(v[r][u].x); xv[2] = bf_lo(v[r][u].y); xv[3] = bf_hi(v[r][u].y);
              xv[4] = bf_lo(v[r][u].z); xv[5] = bf_hi(v[r][u].z); xv[6] = bf_lo(v[r][u].w); xv[7] = bf_hi(v[r][u].w);
            }
#pragma unroll
            for (int i = 0; i < EPC; ++i) acc[r] = __builtin_fma((double)w[i], (double)xv[i], acc[r]);
          }
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < 8; ++r) tot[r] = r < nr ? wave_sum_f64(acc[r]) : 0.0;
}

// Router tile for many rows (the grouped path): unit u = (block of RT_E
// router rows, block of up to 8 input rows), so each input chunk serves RT_E
// router rows; otherwise as router_part.  Returns, in lanes 2o and 2o + 1,
// the wave's sum for o = 8 j + r: router row j of the block, input row r (0
// past the last row or router row).
constexpr int RT_E = 4;
template <int ACT>
__device__ __forceinline__ double router_tile(const Args &a, int unit, int part) {
  static_assert(RT_E * 8 == 32, "one sum per lane pair");
  constexpr int EPC = ACT == F32 ? 4 : 8;
  const int lane = threadIdx.x & 63;
  const int nrows = router_rows(a);
  const int nbe = (nrows + RT_E - 1) / RT_E;
  const int eb = unit % nbe, r0 = (unit / nbe) * 8;
  const int nr = min(8, a.m - r0);
  const int nchunks = a.H / EPC;
  const int c0 = part * nchunks / RSPLIT, c1 = (part + 1) * nchunks / RSPLIT;
  const size_t xstride = (size_t)a.H * act_bytes(ACT);
  const char *wrow[RT_E];
#pragma unroll
  for (int j = 0; j < RT_E; ++j) {
    const int e = min(eb * RT_E + j, nrows - 1);
    wrow[j] = e < a.E ? reinterpret_cast<const char *>(a.router) + (size_t)e * xstride
                      : reinterpret_cast<const char *>(a.sgv);
  }
  const char *x = reinterpret_cast<const char *>(a.xr) + (size_t)r0 * xstride;
  double acc[RT_E][8];
#pragma unroll
  for (int j = 0; j < RT_E; ++j)
#pragma unroll
    for (int r = 0; r < 8; ++r) acc[j][r] = 0.0;
  for (int base = c0; base < c1; base += WAVE) {
    const int ch = base + lane;
    if (ch < c1) {
      u32x4 q[RT_E], v[8];
#pragma unroll
      for (int j = 0; j < RT_E; ++j) q[j] = ld16(wrow[j] + (size_t)ch * 16);
#pragma unroll
      for (int r = 0; r < 8; ++r) v[r] = ld16(x + (size_t)min(r, nr - 1) * xstride + (size_t)ch * 16);
#pragma unroll
      for (int i = 0; i < EPC; ++i) {
        double xv[8], wv[RT_E];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const u32x4 &u = v[r];
          const uint32_t d = (ACT == F32) ? (i == 0 ? u.x : i == 1 ? u.y : i == 2 ? u.z : u.w)
                                          : ((i >> 1) == 0 ? u.x : (i >> 1) == 1 ? u.y : (i >> 1) == 2 ? u.z : u.w);
          xv[r] = ACT == F32 ? (double)__uint_as_float(d) : (double)((i & 1) ? bf_hi(d) : bf_lo(d));
        }
#pragma unroll
        for (int j = 0; j < RT_E; ++j) {
          const u32x4 &u = q[j];
          const uint32_t d = (ACT == F32) ? (i == 0 ? u.x : i == 1 ? u.y : i == 2 ? u.z : u.w)
                                          : ((i >> 1) == 0 ? u.x : (i >> 1) == 1 ? u.y : (i >> 1) == 2 ? u.z : u.w);
          wv[j] = ACT == F32 ? (double)__uint_as_float(d) : (double)((i & 1) ? bf_hi(d) : bf_lo(d));
        }
#pragma unroll
        for (int j = 0; j < RT_E; ++j)
#pragma unroll
          for (int r = 0; r < 8; ++r) acc[j][r] = __builtin_fma(wv[j], xv[r], acc[j][r]);
      }
    }
  }
  // The 32 sums over the wave by halving: at each step a lane keeps half of
  // its values, adding the partner's copy of that half, and sends the other
  // half; five steps leave one value per lane (the sum over 32 lanes), and a
  // last exchange adds the pair.  Lane l ends with o = l / 2.
  double v[32];
#pragma unroll
  for (int j = 0; j < RT_E; ++j)
#pragma unroll
    for (int r = 0; r < 8; ++r) v[8 * j + r] = acc[j][r];
#pragma unroll
  for (int st = 0; st < 5; ++st) {
    const int half = 16 >> st, off = 32 >> st;
    const bool up = (lane & off) != 0;
#pragma unroll
    for (int i = 0; i < half; ++i) {
      const double keep = up ? v[half + i] : v[i], send = up ? v[i] : v[half + i];
      v[i] = keep + __shfl_xor(send, off);
    }
  }
  const double t = v[0] + __shfl_xor(v[0], 1);
  const int o = lane >> 1, j = o >> 3, r = o & 7;
  return (r < nr && eb * RT_E + j < nrows) ? t : 0.0;
}

// --------------------------------------------------------- top-k and sort
//
// Routing state of one forward, built in LDS by the router workgroup that
// finishes last, then published to the workspace for the gate/up and down
// launches and the caller.
constexpr int RANK_MAX_CMP = 16;        // rank selection: at most this many comparisons per thread

template <int NCAND, int NPAIRS> struct RankLDS {
  unsigned long long key[NCAND];  // order key of candidate (r, i) at r * E + i
  double lg[NCAND];               // its logit
  int rank[NCAND];
  double sel[NPAIRS];             // logit of the expert in slot p
};

// One wave's scratch for the top-k of one row (row_topk).
struct alignas(16) TopkLDS {
  unsigned long long key[WAVE];   // candidates, then the selection
  int id[WAVE];
  double lg[WAVE];
};

// NPAIRS: the most (row, slot) pairs the routing holds (MAX_TOPK for the
// one-row routing of the m = 1 gate/up).
template <int NCAND, int NWV, int NPAIRS = MAX_PAIRS> struct RouteLDS {
  static constexpr int kCand = NCAND;   // rank selection serves at most NCAND = m * E candidates
  static constexpr int kWaves = NWV;    // waves with a top-k scratch
  union {
    RankLDS<NCAND, NPAIRS> rk;   // rank selection
    TopkLDS tk[NWV];     // or per-wave selection
  };
  int idx[NPAIRS];           // selected expert of pair p = r*k + j
  float w[NPAIRS];           // routing weight of pair p (times rsf)
  unsigned mask[MAX_EXPERTS];  // bit r: row r chose expert e
  int off[MAX_EXPERTS + 1];  // start of each expert's run in `sorted`
  int sorted[NPAIRS];        // pairs sorted by expert, stable
  int active[MAX_EXPERTS];   // experts with a pair, ascending
  int slot_of[MAX_EXPERTS];  // position of an active expert in `active`
  int nact;
  uint64_t one_row[6][MAX_TOPK];  // one row, no publishing: slot u's gate, up, gate/up scales, biases
};

// One row's routing inputs held in LDS: the logits, the sqrt-softplus
// scores and the expert biases, by expert.  The m = 1 gate/up requests them
// before its shared-expert items and routes from here afterwards.
struct RowStash {
  double lg[MAX_EXPERTS];
  double sc[MAX_EXPERTS];
  float b[MAX_EXPERTS];
};

// Requests row 0's logits, scores (sqrt-softplus) and biases (when the
// routing reads them) into st with loads that write LDS directly: lane l of
// a wave writes 16 (4) bytes at the wave's LDS base + 16 l (4 l).  Waves 0, 1
// take the logits of experts 0..127 and 128..255, waves 2, 3 the scores,
// every wave 64 biases.  A pair of doubles ending at E reads logit column E
// (the shared gate's) or, for the scores, 8 bytes of the array's alignment
// padding.  256 threads.
__device__ __forceinline__ void stash_row0(const Args &a, RowStash &st) {
  typedef __attribute__((address_space(3))) void *lds_ptr;
  const int w = uniform_i(threadIdx.x >> 6), lane = threadIdx.x & 63, E = a.E;
  const int half = w & 1, e0 = half * 128 + 2 * lane;
  if (w < 2) {
    if (e0 < E) __builtin_amdgcn_global_load_lds(a.logits + e0, (lds_ptr)(st.lg + half * 128), 16, 0, 0);
  } else if (a.routing == ROUTE_SQRTSOFTPLUS) {
    if (e0 < E) __builtin_amdgcn_global_load_lds(a.scores + e0, (lds_ptr)(st.sc + half * 128), 16, 0, 0);
  }
  if (routing_biased(a.routing, a.ebias)) {
    const int e = w * 64 + lane;
    if (e < E) __builtin_amdgcn_global_load_lds(a.ebias + e, (lds_ptr)(st.b + w * 64), 4, 0, 0);
  }
}

// Order-preserving image of a double as an unsigned 64-bit integer.
__device__ __forceinline__ unsigned long long order_key(double v) {
  const unsigned long long b = (unsigned long long)__double_as_longlong(v);
  return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}

// Routing weight of the slot held by this lane (lanes 0..k-1 hold slots
// 0..k-1; `mine` marks them), in double: softmax over all experts -- with
// norm_topk_prob the full denominator cancels and only the selected terms
// remain -- or the unbiased sigmoid (the bias only selects), then the
// normalisation; the sqrt-softplus router weights by its unbiased score the
// same way (for it my_l holds that score, which the router units computed).
// lr: the row's logits; lmax: slot 0's logit (the row's largest under softmax
// routing).  Every lane of the wave must call it.
template <bool STASH>
__device__ __forceinline__ double row_weights(const Args &a, const double *lr, bool mine, double my_l,
                                              double lmax, const RowStash *st) {
  const int lane = threadIdx.x & 63, E = a.E;
  double w;
  if (a.routing == ROUTE_SOFTMAX) {
    const double num = mine ? exp(my_l - lmax) : 0.0;
    double den;
    if (a.flags & NORM_TOPK) {
      den = wave_sum_f64(num);
    } else {
      // Lane l adds experts l, l + 64, ... (E <= 256), all requested at once.
      double v[MAX_EXPERTS / WAVE];
#pragma unroll
      for (int j = 0; j < MAX_EXPERTS / WAVE; ++j) {
        const int e = min(lane + j * WAVE, E - 1);
        v[j] = STASH ? st->lg[e] : load_coherent(lr + e);
      }
      double s = 0.0;
#pragma unroll
      for (int j = 0; j < MAX_EXPERTS / WAVE; ++j)
        if (lane + j * WAVE < E) s += exp(v[j] - lmax);
      den = wave_sum_f64(s);
    }
    w = num / den;
  } else {
    w = mine ? (a.routing == ROUTE_SQRTSOFTPLUS ? my_l : sigmoid_d(my_l)) : 0.0;
    if (a.flags & NORM_TOPK) w = w / wave_sum_f64(w);
  }
  return w;
}

// Lane l's four candidates of a row (experts l, l + 64, l + 128, l + 192; lr:
// the row's logits): order keys, logits (sqrt-softplus: scores) and indices;
// padding past E gets key 0 (below every real key) and a unique index after
// every real one.  Every load is issued before any is used -- one memory
// round trip; a lane past E loads entry E - 1 and discards it.  Adjacent
// lanes read adjacent entries (coalesced, and free of LDS bank conflicts
// from the stash; 4 entries apart cost 8-way conflicts).
template <bool BIASED, bool STASH>
__device__ __forceinline__ void lane_keys(const Args &a, const double *lr, unsigned long long (&key)[4],
                                          double (&lg)[4], int (&id)[4], const RowStash *st) {
  const int lane = threadIdx.x & 63, E = a.E;
  const bool sqsp = a.routing == ROUTE_SQRTSOFTPLUS;
  const int r = (int)((lr - a.logits) / (E + 1));
  float bias[4] = {0.f, 0.f, 0.f, 0.f};
  double sc[4] = {0.0, 0.0, 0.0, 0.0};
  if constexpr (STASH) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = min(lane + WAVE * i, E - 1);
      lg[i] = st->lg[e];
      if (sqsp) sc[i] = st->sc[e];
      if constexpr (BIASED) bias[i] = st->b[e];
    }
  } else {
    if constexpr (BIASED) {
#pragma unroll
      for (int i = 0; i < 4; ++i) bias[i] = a.ebias[min(lane + WAVE * i, E - 1)];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) lg[i] = load_coherent(lr + min(lane + WAVE * i, E - 1));
    if (sqsp) {
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[i] = load_coherent(a.scores + (size_t)r * E + min(lane + WAVE * i, E - 1));
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + WAVE * i;
    const bool ok = e < E;
    if (!ok) lg[i] = 0.0;
    const double kd = select_key_d<BIASED>(a.routing, lg[i], sc[i], (double)bias[i]);
    key[i] = ok ? order_key(kd) : 0ull;
    id[i] = ok ? e : 0x40000000 + e;   // unique, after every real index
    if (sqsp) lg[i] = sc[i];            // the weights read the score
  }
}

// Top-k of row r by one wave (T: the wave's scratch).  Keys are compared as
// order-preserving 64-bit integers, which is exactly the order of the double
// keys; ties go to the lower index, so (key desc, index asc) is a strict
// order.  Lane l holds experts l + 64 i, i < 4 (E <= 256).  Slot j's expert and
// weight end up in lane j.
//
// Selection by threshold: let T be the k-th best of the lanes' best entries.
// Exactly k lanes have a best entry at least T, so at least k entries are,
// and so is every entry of the top k; the entries at least T -- at most 4k,
// all from those k lanes -- are the candidates, and each candidate's rank
// among them (counted against every other candidate) is its slot.  T is
// first sought on the high key words alone; when several lanes' best high
// words tie at the k-th place, on the full (key, index) order.
template <bool STASH, typename TL>
__device__ __forceinline__ void row_topk(const Args &a, int r, TL &T, int &my_e, double &my_w,
                                         const RowStash *st) {
  const int lane = threadIdx.x & 63, k = a.K;
  const double *lr = a.logits + (size_t)r * (a.E + 1);
  unsigned long long key[4];
  double lg[4];
  int id[4];
  if (routing_biased(a.routing, a.ebias)) lane_keys<true, STASH>(a, lr, key, lg, id, st);
  else lane_keys<false, STASH>(a, lr, key, lg, id, st);
  // One wave: its LDS accesses complete in program order, so no barrier.
  unsigned hk[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) hk[i] = (unsigned)(key[i] >> 32);
  const unsigned myh = max(max(hk[0], hk[1]), max(hk[2], hk[3]));   // the lane's best high word
  // t = the k-th largest of the lanes' best high words, bit by bit from the
  // top: keep a bit when at least k lanes reach the value with it set.  (Two
  // bits per step, three independent ballots each, took more cycles.)
  unsigned t = 0u;
  for (int b = 31; b >= 0; --b) {
    const unsigned c = t | (1u << b);
    if (__builtin_popcountll(__builtin_amdgcn_ballot_w64(myh >= c)) >= k) t = c;
  }
  // Exactly one lane's best has high word t when k lanes reach t and k - 1
  // exceed it.
  const bool unique = __builtin_popcountll(__builtin_amdgcn_ballot_w64(myh >= t)) == k &&
                      __builtin_popcountll(__builtin_amdgcn_ballot_w64(myh > t)) == k - 1;
  bool cand[4];
  if (unique) {
    // A real key's high word is never 0, so padding (key 0) is never a
    // candidate.
#pragma unroll
    for (int i = 0; i < 4; ++i) cand[i] = hk[i] >= t;
  } else {
    // The lane's best entry in the full order, and the lanes that beat it.
    unsigned long long bk = key[0];
    int bi = id[0];
#pragma unroll
    for (int i = 1; i < 4; ++i)
      if (key[i] > bk || (key[i] == bk && id[i] < bi)) {
        bk = key[i];
        bi = id[i];
      }
    T.key[lane] = bk;
    T.id[lane] = bi;
    int gf = 0;
#pragma unroll 2
    for (int j = 0; j < WAVE; ++j) {
      const unsigned long long kj = T.key[j];
      const int ij = T.id[j];
      gf += (kj > bk || (kj == bk && ij < bi)) ? 1 : 0;
    }
    const int tl = (int)__builtin_ctzll(__builtin_amdgcn_ballot_w64(gf == k - 1));   // exactly one lane
    const unsigned long long tk = readlane_u64(bk, tl);
    const int ti = __builtin_amdgcn_readlane(bi, tl);
#pragma unroll
    for (int i = 0; i < 4; ++i) cand[i] = key[i] > tk || (key[i] == tk && id[i] <= ti);
  }
  int n = 0;   // this lane's candidates
#pragma unroll
  for (int i = 0; i < 4; ++i) n += cand[i] ? 1 : 0;
  int nc;
  int q = wave_excl_scan<3>((unsigned)n, &nc);   // nc <= 4k <= 64
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (cand[i]) {
      T.key[q] = key[i];
      T.id[q] = id[i];
      T.lg[q] = lg[i];
      ++q;
    }
  // Lane c takes candidate c and counts the candidates that beat it.
  unsigned long long kc = 0ull;
  int ic = 0;
  double lc = 0.0;
  if (lane < nc) {
    kc = T.key[lane];
    ic = T.id[lane];
    lc = T.lg[lane];
  }
  // The candidates come back from LDS as broadcasts, eight requested at a
  // time (entries past nc are in bounds and not counted), instead of a chain
  // of readlanes.
  int rank = 0;
  for (int j0 = 0; j0 < nc; j0 += 8) {
    unsigned long long kj[8];
    int ij[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      kj[q] = T.key[j0 + q];
      ij[q] = T.id[j0 + q];
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) rank += (j0 + q < nc && (kj[q] > kc || (kj[q] == kc && ij[q] < ic))) ? 1 : 0;
  }
  if (lane < nc && rank < k) {   // slot `rank`
    T.id[rank] = ic;
    T.lg[rank] = lc;
  }
  double my_l = 0.0;
  my_e = 0;
  if (lane < k) {
    my_e = T.id[lane];
    my_l = T.lg[lane];
  }
  my_w = row_weights<STASH>(a, lr, lane < k, my_l, T.lg[0], st);
}

// Every thread of a workgroup of NT threads: routing of all m rows into L,
// published to the workspace (and the caller's idx/w outputs), with one
// SlotRec per active slot.
//
// EARLY_TB: thread e < E requests expert e's table entries at the start,
// together with the logits, and holds them until it writes the slot record
// of an active e (the route kernel, where the records are on the critical
// path); otherwise the records' entries are requested at the end.  With one
// row and nothing to publish, waves 1.. copy every expert's gate/up entries
// into tab ([6][MAX_EXPERTS], LDS) meanwhile, and each active slot's entries
// end up in L.one_row; wave 0, which selects, holds none of them.
// STASH: one row, whose routing inputs are in st (LDS).
template <int NT, bool EARLY_TB, bool STASH = false, typename LDS>
__device__ __forceinline__ void route_all(const Args &a, LDS &L, bool publish, uint64_t (*tab)[MAX_EXPERTS],
                                          const RowStash *st = nullptr) {
  constexpr int NW = NT / WAVE;
  static_assert(NW <= LDS::kWaves, "a top-k scratch per wave");
  static_assert(NW >= 2, "one_row: the waves that select no row copy the tables");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, tid = threadIdx.x;
  // Rows go to waves from vw = 0 on, where wave blockIdx % NW is vw 0: the
  // workgroups sharing a compute unit then select on different SIMDs.
  const int vw = (wave + NW - (int)(blockIdx.x % NW)) % NW;
  const int E = a.E, k = a.K, m = a.m, te = m * k;
  const int nc = m * E;
  const bool one_row = m == 1 && !publish;
  uint64_t tb[9] = {0ull, 0ull, 0ull, 0ull, 0ull, 0ull, 0ull, 0ull, 0ull};
  if (tid < E) {
    L.mask[tid] = 0u;
    if (EARLY_TB && publish) {
      tb[0] = a.gw[tid]; tb[1] = a.uw[tid]; tb[2] = a.dw[tid];
      if (a.gs) { tb[3] = a.gs[tid]; tb[4] = a.us[tid]; tb[5] = a.ds[tid]; }
      if (a.gb) { tb[6] = a.gb[tid]; tb[7] = a.ub[tid]; tb[8] = a.db[tid]; }
    }
  }
  if (one_row && vw > 0) {
    for (int e = (vw - 1) * WAVE + lane; e < E; e += NT - WAVE) {
      const uint64_t g = a.gw[e], u = a.uw[e];
      const uint64_t gs = a.gs ? a.gs[e] : 0ull, us = a.gs ? a.us[e] : 0ull;
      const uint64_t gb = a.gb ? a.gb[e] : 0ull, ub = a.gb ? a.ub[e] : 0ull;
      tab[0][e] = g; tab[1][e] = u; tab[2][e] = gs; tab[3][e] = us; tab[4][e] = gb; tab[5][e] = ub;
    }
  }
  const bool by_rank = nc <= LDS::kCand && nc * E <= NT * RANK_MAX_CMP;
  if (by_rank) {
    // Selection by rank: candidate (r, i) is ranked by the number of the
    // row's keys that beat it (a larger key, or an equal key with a lower
    // index) -- a strict order, so ranks 0..k-1 are the slots in order.  S
    // threads share a candidate's comparisons.
    const bool biased = routing_biased(a.routing, a.ebias);
    const bool sqsp = a.routing == ROUTE_SQRTSOFTPLUS;
    for (int c = tid; c < nc; c += NT) {
      const int r = c / E, i = c - r * E;
      double l, kd, sc = 0.0;
      if constexpr (STASH) {   // one row, from LDS
        l = st->lg[i];
        if (sqsp) sc = st->sc[i];
        kd = biased ? select_key_d<true>(a.routing, l, sc, (double)st->b[i]) : select_key_d<false>(a.routing, l, sc, 0.0);
      } else if (biased) {   // the loads go out together
        const float b = a.ebias[i];
        l = load_coherent(a.logits + (size_t)r * (E + 1) + i);
        if (sqsp) sc = load_coherent(a.scores + (size_t)r * E + i);
        kd = select_key_d<true>(a.routing, l, sc, (double)b);
      } else {
        l = load_coherent(a.logits + (size_t)r * (E + 1) + i);
        if (sqsp) sc = load_coherent(a.scores + (size_t)r * E + i);
        kd = select_key_d<false>(a.routing, l, sc, 0.0);
      }
      L.rk.key[c] = order_key(kd);
      L.rk.lg[c] = sqsp ? sc : l;   // what the weights read
      L.rk.rank[c] = 0;
    }
    __syncthreads();
    int S = 1;
    while (S < 64 && nc * S * 2 <= NT) S *= 2;
    for (int t = tid; t < nc * S; t += NT) {
      const int c = t / S, part = t - c * S;
      const int r = c / E, i = c - r * E;
      // Part `part` takes keys part, part + S, ...: the S threads of a
      // candidate read adjacent words (distinct LDS banks).
      const unsigned long long ki = L.rk.key[c];
      const unsigned long long *kr = L.rk.key + r * E;
      int cnt = 0;
      int j = part;
      for (; j + 7 * S < E; j += 8 * S) {
        unsigned long long kj[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) kj[q] = kr[j + q * S];
#pragma unroll
        for (int q = 0; q < 8; ++q) cnt += (kj[q] > ki || (kj[q] == ki && j + q * S < i)) ? 1 : 0;
      }
      for (; j < E; j += S) {
        const unsigned long long kj = kr[j];
        cnt += (kj > ki || (kj == ki && j < i)) ? 1 : 0;
      }
      if (cnt) atomicAdd(&L.rk.rank[c], cnt);
    }
    __syncthreads();
    for (int c = tid; c < nc; c += NT) {
      const int rank = L.rk.rank[c];
      if (rank < k) {
        const int r = c / E, p = r * k + rank;
        L.idx[p] = c - r * E;
        L.rk.sel[p] = L.rk.lg[c];
      }
    }
    __syncthreads();
  }
  int one_e = 0, one_pos = 0;   // one row: this lane's expert and its slot (lanes < k of vw 0)
  for (int r = vw; r < m; r += NW) {
    int e;
    double w;
    if (by_rank) {
      const bool mine = lane < k;
      e = mine ? L.idx[r * k + lane] : 0;
      const double my_l = mine ? L.rk.sel[r * k + lane] : 0.0;
      w = row_weights<STASH>(a, a.logits + (size_t)r * (E + 1), mine, my_l, L.rk.sel[r * k], st);
    } else {
      row_topk<STASH>(a, r, L.tk[wave], e, w, st);
    }
    if (lane < k) {
      const float wf = (float)(w * (double)a.rsf);
      const int p = r * k + lane;
      L.idx[p] = e;
      L.w[p] = wf;
      if (publish) {
        a.topk_idx[p] = e;
        a.topk_w[p] = wf;
        if (a.idx_out) a.idx_out[p] = e;
        if (a.w_out) a.w_out[p] = wf;
      }
    }
    if (publish && lane == 0 && (a.flags & SHARED_GATED))
      a.row_gate[r] = (float)sigmoid_d(load_coherent(a.logits + (size_t)r * (E + 1) + E));
    if (m == 1 && !publish) {
      // One row (nothing to publish): its k experts are distinct, so slot
      // u of the ascending order holds the expert with u smaller selected
      // experts, and pair j is that slot's only pair.  The selection is read
      // back from LDS as broadcasts (by rank: L.idx; else the wave's top-k
      // scratch, slots 0..k-1), four at a time (past k: in bounds, not
      // counted).
      const int *sel = by_rank ? L.idx + r * k : L.tk[wave].id;
      int pos = 0;
      for (int i0 = 0; i0 < k; i0 += 4) {
        int si[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) si[q] = sel[i0 + q];
#pragma unroll
        for (int q = 0; q < 4; ++q) pos += (i0 + q < k && si[q] < e) ? 1 : 0;
      }
      one_e = e;
      one_pos = pos;
      if (lane < k) {
        L.active[pos] = e;
        L.sorted[pos] = lane;
        L.off[e] = pos;          // np = off[e + 1] - off[e] = 1; a selected e + 1
        L.off[e + 1] = pos + 1;  // writes the same value here
      }
      if (lane == 0) L.nact = k;
    }
  }
  __syncthreads();
  if (one_row) {
    // The selecting wave's lanes j < k hold slot one_pos's expert one_e; the
    // other waves' table copies are complete after the barrier above.
    if (vw == 0 && lane < k) {
#pragma unroll
      for (int j = 0; j < 6; ++j) L.one_row[j][one_pos] = tab[j][clamp_i(one_e, 0, E - 1)];
    }
    __syncthreads();
    return;
  }
  // Stable counting sort by expert (mask zeroed at the start).  A row selects an expert at most once, so
  // bit r of mask[e] says whether row r chose e, and a pair's rank inside its
  // expert is the number of earlier rows that chose the same expert.
  for (int p = tid; p < te; p += NT) atomicOr(&L.mask[L.idx[p]], 1u << (p / k));
  __syncthreads();
  if (wave == 0) {
    // Lane l: experts 4l..4l+3; wave-wide exclusive scans of counts and of
    // "active" flags.
    int cnt[4], act[4], ct = 0, at = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * lane + i;
      cnt[i] = e < E ? __popc(L.mask[e]) : 0;
      act[i] = cnt[i] > 0 ? 1 : 0;
      ct += cnt[i];
      at += act[i];
    }
    int ci, ai;                          // wave totals
    const int cpre = wave_excl_scan<8>((unsigned)ct, &ci);   // ct <= 4 * 32
    const int apre = wave_excl_scan<3>((unsigned)at, &ai);   // at <= 4
    int co = cpre, ao = apre;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * lane + i;
      if (e < E) {
        L.off[e] = co;
        if (publish) a.offsets[e] = co;
        if (act[i]) {
          L.active[ao] = e;
          L.slot_of[e] = ao;
          if (publish) a.active[ao] = e;
        }
      }
      co += cnt[i];
      ao += act[i];
    }
    if (lane == WAVE - 1) {
      L.off[E] = ci;
      L.nact = ai;
      if (publish) {
        a.offsets[E] = ci;
        a.active_count[0] = ai;
      }
    }
  }
  __syncthreads();
  for (int p = tid; p < te; p += NT) {
    const int e = L.idx[p], r = p / k;
    const int pos = L.off[e] + __popc(L.mask[e] & ((1u << r) - 1u));
    L.sorted[pos] = p;
    if (publish) {
      a.sorted_pair[pos] = p;
      a.pair_to_perm[p] = pos;
    }
  }
  if (publish && tid < E && L.mask[tid] != 0u) {
    const int e = tid;
    if (!EARLY_TB) {
      tb[0] = a.gw[e]; tb[1] = a.uw[e]; tb[2] = a.dw[e];
      if (a.gs) { tb[3] = a.gs[e]; tb[4] = a.us[e]; tb[5] = a.ds[e]; }
      if (a.gb) { tb[6] = a.gb[e]; tb[7] = a.ub[e]; tb[8] = a.db[e]; }
    }
    SlotRec rec;
    rec.e = e;
    rec.off = L.off[e];
    rec.np = L.off[e + 1] - L.off[e];
    rec.tag = a.tag;
    rec.gw = tb[0]; rec.uw = tb[1]; rec.dw = tb[2];
    rec.gs = tb[3]; rec.us = tb[4]; rec.ds = tb[5];
    rec.gb = tb[6]; rec.ub = tb[7]; rec.db = tb[8];
#pragma unroll
    for (int i = 0; i < 5; ++i) rec.pad2[i] = 0ull;
    a.slots[L.slot_of[e]] = rec;
  }
  __syncthreads();
  if (publish && tid == 0) a.sync[SYNC_PUBLISHED] = (unsigned)a.tag;   // after the records and the count
}

// ---------------------------------------------------------------- gate/up
//
// One wave: intermediate rows [i0, i0 + NI) of one expert (gate and up), for
// pairs pair[0..np-1] (routed: row = pair / k, routing weight w[pair]) or
// input rows 0..np-1 (shared), in passes of C; writes silu(g) * v at
// dst[(off + c) * ld + i].
template <int EF, int ACT, int CMAX, int NI>
__device__ __forceinline__ void gate_up_rows(const Args &a, const void *gw, const void *uw,
                                             const void *gs, const void *us, const void *gb,
                                             const void *ub, int N, int i0, int off, int np,
                                             const int *pairs, const float *pw, float *dst, int ld,
                                             float s2g = 1.0f, float s2u = 1.0f) {
  constexpr int RG = 2 * NI;
  const int H = a.H, k = a.K;
  const size_t xstride = (size_t)H * act_bytes(ACT);
  const char *x = reinterpret_cast<const char *>(a.x);
  const bool routed = pairs != nullptr;
  const bool scale = routed && (a.flags & WEIGHT_BEFORE);
  const Mat<EF> mg = make_mat<EF>(gw, gs, gb, N, H), mu = make_mat<EF>(uw, us, ub, N, H);
  Row<EF> rows[RG];
#pragma unroll
  for (int t = 0; t < NI; ++t) {
    const int i = min(i0 + t, N - 1);
    rows[t] = make_row<EF, true>(mg, i);
    rows[NI + t] = make_row<EF, true>(mu, i);
  }
  for_passes<CMAX>(np, [&](auto cc, int c0) {
    constexpr int C = decltype(cc)::value;
    const char *xrow[C];
    int pair[C];
#pragma unroll
    for (int c = 0; c < C; ++c) {
      pair[c] = routed ? pairs[c0 + c] : c0 + c;
      xrow[c] = x + (size_t)(routed ? pair[c] / k : c0 + c) * xstride;
    }
    float acc[RG][C];
    wave_rows_dot<EF, ACT, RG, C, WAVE, false, 1, gate_up_vb<EF, CMAX>()>(rows, xrow, 0, H / Fmt<EF>::EPC, acc);
    if ((threadIdx.x & 63) == 0) {
#pragma unroll
      for (int c = 0; c < C; ++c) {
        const float w = scale ? pw[pair[c]] : 1.0f;
#pragma unroll
        for (int t = 0; t < NI; ++t) {
          if (i0 + t < N) {
            float g = acc[t][c], v = acc[NI + t][c];
            if constexpr (EF == NVFP4) {   // the projections' second-level scales
              g *= s2g;
              v *= s2u;
            }
            if (scale) {  // W(w x) = w (W x): scale both pre-activations
              g *= w;
              v *= w;
            }
            const int i = i0 + t;
            // 4-bit experts: the row is stored sub-step-major (F32P).
            const int pos = (is_fp4(EF) && routed) ? ((i & 31) >> 3) * (ld >> 2) + (i >> 5) * 8 + (i & 7) : i;
            dst[(size_t)(off + c0 + c) * ld + pos] = act_mul(a.flags, g, v);
          }
        }
      }
    }
  });
}

// --------------------------------------------------------- down + blend
//
// Down tile `tile`: output columns [h0, h0 + HT), HT = RD * down_dq with RD
// rows per sub-unit (down_rd).
// Sub-unit (u, q) is unit u (an active slot, or the shared expert last) and
// row block q; waves take sub-units round-robin, y per pair goes to LDS, then
//   out[r, h] = sum_j c_rj y[perm(r, j), h] + gamma_r ys[r, h]
// in slot order.
template <int EF, int ACT, int CR, int CS, int LPR, int NW>
__device__ __forceinline__ void down_item(const Args &a, int tile) {
  constexpr int GR = WAVE / LPR;                 // routed rows in parallel per wave
  constexpr int RGR = down_rd<EF, CS, NW>() / GR;     // routed rows per lane group
  constexpr int NWD = down_threads<EF, CS, LPR, NW>() / WAVE; // waves of the workgroup
  constexpr int RD = down_rd<EF, CS, NW>();
  static_assert(RD % GR == 0, "down rows must split over lane groups");
  // One row: at most 4 parts of K times k pairs, one row of the shared expert.
  constexpr bool NARROW = CR == 1 && CS == 1;
  __shared__ float y_lds[(NARROW ? 4 * MAX_TOPK : MAX_PAIRS) * MAX_DOWN_TILE];
  __shared__ float ys_lds[(NARROW ? 1 : MAX_ROWS) * MAX_DOWN_TILE];
  __shared__ float s_c[MAX_PAIRS];               // blend coefficient of pair p
  __shared__ int s_perm[MAX_PAIRS];              // sorted position of pair p
  __shared__ float s_gamma[MAX_ROWS];
  // The narrow tiles' prologue (one row, few sub-units: its latency is the
  // launch's) takes the shared output's parts through LDS.
  constexpr bool LDS_YS = NW > 0;
  __shared__ float ys_parts[LDS_YS ? MAX_SD_PARTS : 1][WAVE];
  const int wave = uniform_i(threadIdx.x >> 6), lane = threadIdx.x & 63, tid = threadIdx.x;
  const int H = a.H, I = a.I, Is = a.Is, m = a.m, te = a.te;
  const int DQ = a.down_dq, HT = RD * DQ, h0 = tile * HT;
  const bool shared = (a.flags & SHARED) != 0;
  const bool sh_mfma = shared && a.shared_mfma;  // shared output already in sy
  const int sh = shared && !sh_mfma ? 1 : 0;     // else the shared expert is unit 0
  const bool before = (a.flags & WEIGHT_BEFORE) != 0;
  const bool gated = (a.flags & SHARED_GATED) != 0;

  // The fields a down sub-unit needs, of the wave's next routed sub-unit.
  struct DownRec {
    int e, off, np;
    uint64_t dw, ds, db;
  };
  auto load_rec = [&](int slot) {
    const SlotRec &r = a.slots[slot];
    DownRec d;
    d.e = r.e; d.off = r.off; d.np = r.np; d.dw = r.dw; d.ds = r.ds; d.db = r.db;
    return d;
  };
  // This wave's first routed record (the record array always has cap
  // entries; a stale one is never used).
  const int slot0 = clamp_i(wave / (DQ * a.down_parts) - sh, 0, a.cap - 1);
  float my_c = 0.f, my_g = 0.f;
  float my_ys = 0.f;                             // wider variants: this thread's shared output for the blend
  int my_perm = 0;                               // clamped where it is used
  DownRec nxt;
  int nact;
  if constexpr (LDS_YS) {
    // One row: every load of the prologue goes out before any is used (one
    // memory round trip, not one per dependent use) -- the record, the
    // published tag and count, the blend operands, and the shared output's
    // parts, which go straight to LDS (lane t of wave 0 writes column t of
    // part q at ys_parts[q][t]) and are added after the streaming.
    nxt = load_rec(slot0);
    const int cnt = a.active_count[0];
    const unsigned pub = a.sync[SYNC_PUBLISHED];
    if (tid < te) {
      my_c = before ? 1.0f : a.topk_w[tid];
      my_perm = a.pair_to_perm[tid];
    }
    if (tid < m) my_g = gated ? a.row_gate[tid] : 1.0f;
    if (sh_mfma && wave == 0 && tid < HT && h0 + tid < H) {
      typedef __attribute__((address_space(3))) void *lds_ptr;
      for (int q = 0; q < a.sd_parts; ++q)
        __builtin_amdgcn_global_load_lds(a.sy + (size_t)q * a.max_rows * H + h0 + tid, (lds_ptr)ys_parts[q], 4, 0, 0);
    }
    // The count and tag are needed before the first sub-unit; holding them
    // here keeps the count's load from sinking behind the tag's comparison.
    asm volatile("" ::"s"(cnt), "s"(pub));
    nact = pub == (unsigned)a.tag ? clamp_i(cnt, 0, a.cap) : 0;
  } else {
    // Blend operands, requested now and used after the streaming.
    if (tid < te) {
      my_c = before ? 1.0f : a.topk_w[tid];
      my_perm = a.pair_to_perm[tid];
    }
    if (tid < m) my_g = gated ? a.row_gate[tid] : 1.0f;
    if (sh_mfma && tid < m * HT) {
      const int r = tid / HT, h = h0 + (tid - r * HT);
      if (h < H)
        for (int q = 0; q < a.sd_parts; ++q) my_ys += a.sy[((size_t)q * a.max_rows + r) * H + h];
    }
    // The record, requested together with the count.
    nxt = load_rec(slot0);
    nact = published_count(a);
  }
  int nxt_slot = slot0;
  const int units = nact + sh;

  // Sub-unit su = (unit, row block q, part pt of the down rows' K); the
  // parts' totals are added in order in the blend.
  const int NP = a.down_parts;
  const int nsu = units * DQ * NP;
  for (int su = wave; su < nsu; su += NWD) {
    const int uq = su / NP, pt = su - uq * NP;
    const int u = uq / DQ, q = uq - u * DQ;
    const int hb = h0 + q * RD;                  // first column of this row block
    if (u >= sh) {
      if (nxt_slot != u - sh) {   // not requested ahead (only when the wave's first sub-unit was shared)
        nxt = load_rec(u - sh);
        nxt_slot = u - sh;
      }
      const DownRec rec = nxt;
      const int su2 = su + NWD;
      if (su2 < nsu) {
        const int s2 = (su2 / NP) / DQ - sh;
        if (s2 >= 0 && s2 != nxt_slot) {
          nxt = load_rec(s2);
          nxt_slot = s2;
        }
      }
      const int nch = I / Fmt<EF>::EPC;
      const int kc0 = pt * nch / NP, kc1 = (pt + 1) * nch / NP;
      const int off = uniform_i(clamp_i(rec.off, 0, te));
      const int np = uniform_i(clamp_i(rec.np, 0, te - off));
      const void *dw = reinterpret_cast<const void *>(rec.dw);
      const void *ds = reinterpret_cast<const void *>(rec.ds);
      const void *db = reinterpret_cast<const void *>(rec.db);
      const int grp = lane / LPR;
      float s2d = 1.0f;   // nvfp4: the down projection's second-level scale
      if constexpr (EF == NVFP4) s2d = a.ds2[uniform_i(clamp_i(rec.e, 0, a.E - 1))];
      const Mat<EF> md = make_mat<EF>(dw, ds, db, H, I);
      Row<EF> rows[RGR];
#pragma unroll
      for (int t = 0; t < RGR; ++t) rows[t] = make_row<EF, LPR == WAVE>(md, min(hb + grp + GR * t, H - 1));
      for_passes<CR>(np, [&](auto cc, int c0) {
        constexpr int C = decltype(cc)::value;
        const char *xrow[C];
#pragma unroll
        for (int c = 0; c < C; ++c) xrow[c] = reinterpret_cast<const char *>(a.act + (size_t)(off + c0 + c) * I);
        float acc[RGR][C];
        wave_rows_dot<EF, (is_fp4(EF) ? F32P : F32), RGR, C, LPR, false, 1, down_vgpr_budget<EF, CS, NW>()>(
            rows, xrow, kc0, kc1, acc, I);
        if (lane % LPR == 0) {
#pragma unroll
          for (int t = 0; t < RGR; ++t)
#pragma unroll
            for (int c = 0; c < C; ++c)
              y_lds[(pt * te + off + c0 + c) * HT + q * RD + grp + GR * t] =
                  EF == NVFP4 ? acc[t][c] * s2d : acc[t][c];
        }
      });
    } else if (pt == 0) {
      const Mat<ACT> ms = make_mat<ACT>(a.sdw, nullptr, nullptr, H, Is);
      Row<ACT> rows[RD];
#pragma unroll
      for (int t = 0; t < RD; ++t) rows[t] = make_row<ACT, true>(ms, min(hb + t, H - 1));
      for_passes<CS>(m, [&](auto cc, int c0) {
        constexpr int C = decltype(cc)::value;
        const char *xrow[C];
#pragma unroll
        for (int c = 0; c < C; ++c) xrow[c] = reinterpret_cast<const char *>(a.sact + (size_t)(c0 + c) * Is);
        float acc[RD][C];
        wave_rows_dot<ACT, F32, RD, C, WAVE, false, 1, down_vgpr_budget<EF, CS, NW>()>(rows, xrow, 0,
                                                                                   Is / Fmt<ACT>::EPC, acc);
        if (lane == 0) {
#pragma unroll
          for (int t = 0; t < RD; ++t)
#pragma unroll
            for (int c = 0; c < C; ++c) ys_lds[(c0 + c) * HT + q * RD + t] = acc[t][c];
        }
      });
    }
  }
  if (tid < te) {
    s_c[tid] = my_c;
    s_perm[tid] = clamp_i(my_perm, 0, te - 1);
  }
  if (tid < m) s_gamma[tid] = my_g;
  if constexpr (LDS_YS) __builtin_amdgcn_s_waitcnt(0);   // the parts' loads have written LDS
  __syncthreads();

  const bool out_f32 = (a.flags & OUT_F32) != 0 || ACT == F32;
  const int k = a.K;
  for (int t = threadIdx.x; t < m * HT; t += down_threads<EF, CS, LPR, NW>()) {
    const int r = t / HT, hl = t - r * HT, h = h0 + hl;
    if (h >= H) continue;
    float o = 0.f;
    for (int j = 0; j < k; ++j) {
      const int p = r * k + j;
      float y = y_lds[s_perm[p] * HT + hl];
      for (int q2 = 1; q2 < NP; ++q2) y += y_lds[(q2 * te + s_perm[p]) * HT + hl];
      o = __builtin_fmaf(s_c[p], y, o);
    }
    if (shared) {
      float ys;
      if (!sh_mfma) {
        ys = ys_lds[r * HT + hl];
      } else if constexpr (LDS_YS) {   // the parts in order, as the other variants add them
        ys = 0.f;
        for (int q = 0; q < a.sd_parts; ++q) ys += ys_parts[q][hl];
      } else {
        ys = my_ys;
      }
      o = __builtin_fmaf(s_gamma[r], ys, o);
    }
    if (out_f32)
      reinterpret_cast<float *>(a.out)[(size_t)r * H + h] = o;
    else
      reinterpret_cast<uint16_t *>(a.out)[(size_t)r * H + h] = f32_to_bf16(o);
  }
}

// Shared expert gate/up on the matrix cores: item = 16 intermediate rows on
// the eight waves wb..wb+7; waves wb..wb+3 take the gate rows and the others
// the up rows, each a quarter of H; writes silu(g) * u to sact.  Every wave
// of the workgroup calls it (one barrier); live: the item exists.
template <int NCT, int WPB = ROUTE_WPB>
__device__ __forceinline__ void shared_gu_mfma(const Args &a, int item, MfmaLDS<WPB, 1> &S, int wb = 0,
                                               bool live = true) {
  static_assert(WPB % 8 == 0, "items of eight waves");
  const int w = uniform_i(threadIdx.x >> 6), wl = w - wb, lane = threadIdx.x & 63;
  const int H = a.H, Is = a.Is, m = a.m, n0 = item * 16;
  if (live) {
    const __amdgpu_buffer_rsrc_t A[1] = {buf_rsrc(wl < 4 ? a.sgw : a.suw, Is * H * 2)};
    int kb, ke;
    k_slice(H, wl & 3, 4, kb, ke);
    f32x4 acc[1][NCT];
    mfma_slice<BF16, 1, NCT>(A, H * 2, n0, Is, reinterpret_cast<const char *>(a.x), (size_t)H * 2, m, kb, ke,
                             S.stage[w], acc);
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) S.part[w][0][ct][i][lane] = acc[0][ct][i];
  }
  __syncthreads();
  // Wave wb + j finishes (column tile j / 4, element i = j % 4).
  const int ct = wl / 4, i = wl % 4;
  if (live && ct < NCT) {
    float gs = 0.f, us = 0.f;
    for (int p = 0; p < 4; ++p) {
      gs += S.part[wb + p][0][ct][i][lane];
      us += S.part[wb + 4 + p][0][ct][i][lane];
    }
    const int row = n0 + (lane >> 4) * 4 + i, v = 16 * ct + (lane & 15);
    // With bf16 experts stored as F32I pairs, the form their matrix-core
    // shared down reads (it then skips the per-item split); else f32.
    if (row < Is && v < m) {
      const float y = act_mul(a.flags, gs, us);
      if (a.sact_pairs) reinterpret_cast<uint32_t *>(a.sact)[(size_t)v * Is + row] = f32i_pair(y);
      else a.sact[(size_t)v * Is + row] = y;
    }
  }
}

// Shared expert down on the matrix cores: item = (16 output columns, part q
// of the a.sd_parts parts of Is); the WPB waves of the workgroup split the
// part, and the part's total goes to sy[q] (the blend adds the parts in
// order).
// XF: how the shared activations are stored (F32I with bf16 experts, F32).
template <int NCT, int MU, int XF>
__device__ __forceinline__ void shared_dn_mfma(const Args &a, int item, MfmaLDS<WPB, 1, MU> &S) {
  const int w = uniform_i(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int H = a.H, Is = a.Is, m = a.m, P = a.sd_parts;
  const int tile = item / P, q = item - tile * P, n0 = tile * 16;
  const __amdgpu_buffer_rsrc_t A[1] = {buf_rsrc(a.sdw, H * Is * 2)};
  int pb, pe, kb, ke;
  k_slice(Is, q, P, pb, pe);
  k_slice(pe - pb, w, WPB, kb, ke);
  f32x4 acc[1][NCT];
  mfma_slice<XF, 1, NCT, MU>(A, Is * 2, n0, H, reinterpret_cast<const char *>(a.sact), (size_t)Is * 4, m,
                         pb + kb, pb + ke, S.stage[w], acc);
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
    for (int i = 0; i < 4; ++i) S.part[w][0][ct][i][lane] = acc[0][ct][i];
  __syncthreads();
  const int i = w;   // WPB == 4: wave w finishes element i = w of every column tile
  float *sy = a.sy + (size_t)q * a.max_rows * H;
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    float y = 0.f;
    for (int p = 0; p < WPB; ++p) y += S.part[p][0][ct][i][lane];
    const int row = n0 + (lane >> 4) * 4 + i, v = 16 * ct + (lane & 15);
    if (row < H && v < m) sy[(size_t)v * H + row] = y;
  }
  __syncthreads();   // S is reused by the workgroup's next item
}

// The same item at m = 1 through mfma_slice_dma (one vector, so one column
// tile); the waves' partials are added in the same order.
__device__ __forceinline__ void shared_dn_ring(const Args &a, int item, SharedDnRing &S) {
  const int w = uniform_i(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int H = a.H, Is = a.Is, P = a.sd_parts;
  const int tile = item / P, q = item - tile * P, n0 = tile * 16;
  const __amdgpu_buffer_rsrc_t A = buf_rsrc(a.sdw, H * Is * 2);
  const __amdgpu_buffer_rsrc_t X = buf_rsrc(a.sact, Is * 4);
  int pb, pe, kb, ke;
  k_slice(Is, q, P, pb, pe);
  k_slice(pe - pb, w, WPB, kb, ke);
  f32x4 acc;
  mfma_slice_dma(A, Is * 2, n0, H, X, pb + kb, pb + ke, S.slot[w], acc);
#pragma unroll
  for (int i = 0; i < 4; ++i) S.part[w][i][lane] = acc[i];
  __syncthreads();
  const int i = w;   // WPB == 4: wave w finishes element i = w
  float y = 0.f;
  for (int p = 0; p < WPB; ++p) y += S.part[p][i][lane];
  const int row = n0 + (lane >> 4) * 4 + i, v = lane & 15;
  if (row < H && v < 1) a.sy[(size_t)q * a.max_rows * H + row] = y;
  __syncthreads();   // S is reused by the workgroup's next item
}

template <int ACT, int NCT, int MU, int EF>
__device__ __forceinline__ void shared_dn_item(const Args &a, int item, MfmaLDS<WPB, 1, MU> &S) {
  // The matrix-core path; the activations are F32I pairs with bf16 experts.
  if constexpr (ACT == BF16 && NCT > 0) shared_dn_mfma<NCT, MU, EF == BF16 ? F32I : F32>(a, item, S);
}

// k-steps per batch of the shared down items in a gate/up variant: 2 where
// that lets the variant reach four waves per SIMD (registers and LDS) -- one
// vector per pass, or 4-bit experts -- else 4, which streams a long shared
// down faster.
template <int EF, int CR> constexpr int shared_dn_mu() { return CR == 1 || EF >= AFF4 ? 2 : 4; }

// ------------------------------------------------------------------ kernels

// gate_up's LDS: the shared down items' staging (variants that run them), or
// -- one row, routing in every workgroup -- the experts' gate/up table
// entries, which are consumed before any item starts.
template <bool MF, int MU> union GateUpLDS {
  MfmaLDS<WPB, 1, MU> mf;
  uint64_t tab[6][MAX_EXPERTS];
};
template <int MU> union GateUpLDS<false, MU> {
  uint64_t tab[6][MAX_EXPERTS];
};

// The routing of one row as the routed items read it: per active slot the
// expert, its pair range and its gate/up table entries, and the pairs and
// weights in sorted order.
struct OneRowRouting {
  int nact;
  int e[MAX_TOPK], off[MAX_TOPK], np[MAX_TOPK], sorted[MAX_TOPK];
  float w[MAX_TOPK];
  uint64_t p[6][MAX_TOPK];
};

// One row with bf16 experts: the shared down items' LDS ring -- their items
// come first -- then the routing's table entries and arrays, which the
// routed items read after it.
union GateUpRingLDS {
  SharedDnRing ring;
  struct {
    uint64_t tab[6][MAX_EXPERTS];
    RouteLDS<256, WPB, MAX_TOPK> L;
  } rt;
};

// Launch 1: router workgroups (ROUTE_UNITS_PER_WG units, RSPLIT waves each),
// then the shared expert's gate/up items -- these need no routing, so they
// stream meanwhile.  Each router workgroup stores its logits and takes a
// ticket; the one that takes the last ticket (every other router workgroup
// has stored and released its logits by then) computes the routing once for
// the whole forward and resets the counter.  No workgroup waits for another.
// Held to 128 registers (two workgroups per CU) but for the 8-vector passes
// of the vector-unit shared gate/up, which spill there.
template <int CS> constexpr int route_min_waves() { return CS >= 8 ? 1 : 4; }
// RT: threads per workgroup.  512 (8 waves, two workgroups per CU); 1024
// (16 waves, one per CU) above 8 rows when the launch fits one round of
// those: the routing's top-k then takes up to 16 rows at once, one per wave,
// and each shared-expert workgroup runs two items of eight waves with the
// same arithmetic.
template <int ACT, int CS, int RT = ROUTE_THREADS>
__global__ __launch_bounds__(RT, route_min_waves<CS>()) void route_kernel(Args a) {
  constexpr int WPB_R = RT / WAVE;
  constexpr int UPW = WPB_R / RSPLIT;   // router units per workgroup
  struct RouterSmem {
    double part[WPB_R][8];
    unsigned ticket;
    RouteLDS<1024, WPB_R> L;
  };
  __shared__ union {
    RouterSmem r;
    MfmaLDS<WPB_R, 1> mf;
  } sm;
  const int item = blockIdx.x, tid = threadIdx.x;
  const int wave = uniform_i(threadIdx.x >> 6);
  if (item < a.n_router_wg) {
    double (&s_part)[WPB_R][8] = sm.r.part;
    unsigned &s_ticket = sm.r.ticket;
    RouteLDS<1024, WPB_R> &L = sm.r.L;
    const int unit = item * UPW + wave / RSPLIT, part = wave % RSPLIT;
    const bool live = unit < a.n_router;
    double tot[8];
    if (live) router_part<ACT>(a, unit, part, tot);
    if ((threadIdx.x & 63) == 0) {
#pragma unroll
      for (int r = 0; r < 8; ++r) s_part[wave][r] = live ? tot[r] : 0.0;
    }
    __syncthreads();
    if (tid < UPW * 8) {
      const int ul = tid / 8, r = tid % 8, u = item * UPW + ul;
      const int nrows = router_rows(a);
      const int e = u % nrows, rr = (u / nrows) * 8 + r;
      if (u < a.n_router && rr < a.m) {
        double t = s_part[ul * RSPLIT][r];
#pragma unroll
        for (int p = 1; p < RSPLIT; ++p) t += s_part[ul * RSPLIT + p][r];
        store_coherent(a.logits + (size_t)rr * (a.E + 1) + e, t);
        if (a.routing == ROUTE_SQRTSOFTPLUS && e < a.E) store_coherent(a.scores + (size_t)rr * a.E + e, sqrtsoftplus_d(t));
      }
    }
    if (a.route_in_gu) return;   // every gate/up workgroup routes from the logits
    // The logits go out through store_coherent and come back through
    // load_coherent (agent-scope atomics): the hand-off without fences.
    if (!last_arrival<false>(a.sync + SYNC_ROUTER_TICKET, (unsigned)a.n_router_wg, s_ticket)) return;
    route_all<RT, true>(a, L, true, nullptr);
    if (tid == 0) a.sync[SYNC_ROUTER_TICKET] = 0u;  // every ticket is taken
    return;
  }
  const int sitem = item - a.n_router_wg;
  if (ACT == BF16 && a.shared_mfma) {
    if constexpr (WPB_R == 8) {
      if (a.m > 16) shared_gu_mfma<2>(a, sitem, sm.mf);
      else shared_gu_mfma<1>(a, sitem, sm.mf);
    } else {
      // Eight waves per item: WPB_R / 8 items per workgroup.
      const int wb = wave / 8 * 8, it = sitem * (WPB_R / 8) + wave / 8;
      const bool live = it < a.n_shared_gu;
      if (a.m > 16) shared_gu_mfma<2, WPB_R>(a, it, sm.mf, wb, live);
      else shared_gu_mfma<1, WPB_R>(a, it, sm.mf, wb, live);
    }
    return;
  }
  constexpr int NI = gate_up_ni<ACT>();
  const int i0 = (sitem * WPB_R + wave) * NI;
  if (i0 < a.Is)
    gate_up_rows<ACT, ACT, CS, NI>(a, a.sgw, a.suw, nullptr, nullptr, nullptr, nullptr, a.Is, i0, 0,
                                   a.m, nullptr, nullptr, a.sact, a.Is);
}

// The router units only, as tiles of RT_E router rows (the grouped path).
template <int ACT>
__global__ __launch_bounds__(ROUTE_THREADS) void route_tile_kernel(Args a) {
  __shared__ double s_part[ROUTE_WPB][RT_E * 8];
  const int item = blockIdx.x, tid = threadIdx.x;
  const int wave = uniform_i(threadIdx.x >> 6);
  const int unit = item * ROUTE_UNITS_PER_WG + wave / RSPLIT, part = wave % RSPLIT;
  const bool live = unit < a.n_router;
  const double tot = live ? router_tile<ACT>(a, unit, part) : 0.0;
  if ((threadIdx.x & 1) == 0) s_part[wave][(threadIdx.x & 63) >> 1] = tot;
  __syncthreads();
  if (tid < ROUTE_UNITS_PER_WG * RT_E * 8) {
    const int ul = tid / (RT_E * 8), o = tid % (RT_E * 8), j = o / 8, r = o % 8;
    const int u = item * ROUTE_UNITS_PER_WG + ul;
    const int nrows = router_rows(a);
    const int nbe = (nrows + RT_E - 1) / RT_E;
    const int e = (u % nbe) * RT_E + j, rr = (u / nbe) * 8 + r;
    if (u < a.n_router && rr < a.m && e < nrows) {
      double t = s_part[ul * RSPLIT][o];
#pragma unroll
      for (int p = 1; p < RSPLIT; ++p) t += s_part[ul * RSPLIT + p][o];
      a.logits[(size_t)rr * (a.E + 1) + e] = t;
      if (a.routing == ROUTE_SQRTSOFTPLUS && e < a.E) a.scores[(size_t)rr * a.E + e] = sqrtsoftplus_d(t);
    }
  }
}


// Launch 2: items blockIdx, blockIdx + gridDim, ... of a list of the routed
// items (active slot s, row block b) of the nact * items_per_slot that exist,
// whose waves take row groups b * 4 + wave of slot s, and of the shared
// expert's down items (SHD > 0).  Either the routing is published (the first
// routed item's slot record is requested together with the active count), or
// -- route_in_gu, chosen for small m where it starts the streaming sooner --
// every workgroup computes it from the logits in LDS and one extra
// workgroup, the last, publishes it; then the shared items come first in the
// list, since they need no routing: a workgroup streams them before it takes
// the routing (-6 % on the gate/up of the weight-before workload at m = 1).
// SHD: 0, or the column tiles (1: m <= 16, 2: m <= 32) of the shared
// expert's down items this variant also runs.
// The variants m = 1 runs (one vector per pass, at most one shared column
// tile) are held to 128 registers, four waves per SIMD: their natural size is
// within a few registers of it.  Argument: CR * 4 + SHD.
// (f32 activations, the latency-bound tiny layer's, spill at 128 and keep
// no bound.)
template <int CRS, bool F32Q = false> constexpr int gate_up_min_waves() {
  return !F32Q && CRS / 4 == 1 && CRS % 4 <= 1 ? 4 : 1;
}
template <int EF, int ACT, int CR, int CS, int SHD>
__global__ __launch_bounds__(THREADS, (gate_up_min_waves<CR * 4 + SHD, ACT == F32>()))
void gate_up_kernel(Args a) {
  constexpr int NI = gate_up_ni<EF, CR>();
  const int ips = a.gu_items_per_slot;
  const int wave = uniform_i(threadIdx.x >> 6);
  constexpr int SDMU = shared_dn_mu<EF, CR>();
  // One vector per pass (CR == 1) is m = 1: the host picks these variants
  // for one row only.
  // At m = 1 the bf16-expert variants stream the shared down items through
  // the LDS ring (the same sums).  (With both paths in one kernel the 4-bit
  // variants spilled; on the 512-wide shared expert of the 4-bit layers,
  // whose waves take two batches each, the ring was 0.4 us slower.)
  constexpr bool RING = CR == 1 && ACT == BF16 && EF == BF16 && SHD == 1;
  __shared__ std::conditional_t<RING, GateUpRingLDS, GateUpLDS<(SHD > 0), SDMU>> G;
  auto shared_item = [&](int it) {
    if constexpr (RING) shared_dn_ring(a, it, G.ring);
    else if constexpr (SHD > 0) shared_dn_item<ACT, SHD, SDMU, EF>(a, it, G.mf);
  };
  // The route launch is over: its ticket word starts the next forward at 0,
  // whatever this forward found in it.
  if (blockIdx.x == 0 && threadIdx.x == 0) a.sync[SYNC_ROUTER_TICKET] = 0u;
  const int S = SHD > 0 ? a.n_shared_dn : 0;   // shared down items
  // Only the one-vector variants (m = 1) carry the routing: the top-k's
  // registers would cost the streaming variants of m > 1 occupancy.
  if constexpr (CR == 1) {
    if (a.route_in_gu) {
      // The last workgroup only publishes the routing; the others stream.
      RouteLDS<256, WPB, MAX_TOPK> *Lp;
      uint64_t (*tab)[MAX_EXPERTS];
      if constexpr (RING) {
        Lp = &G.rt.L;
        tab = G.rt.tab;
      } else {
        __shared__ RouteLDS<256, WPB, MAX_TOPK> L0;
        Lp = &L0;
        tab = G.tab;
      }
      RouteLDS<256, WPB, MAX_TOPK> &L = *Lp;
      __shared__ RowStash ST;
      const int nb = gridDim.x - 1;
      const bool publisher = (int)blockIdx.x == nb;
      // The row's logits (scores, biases) go straight to LDS, requested
      // before the shared-expert items: their round trip overlaps the items'
      // streaming instead of following it, and holds no registers.
      stash_row0(a, ST);
      int it = blockIdx.x;
      // With the ring, the workgroups dispatched second on each CU route
      // before their shared item, the others after: the routing (a few us
      // with no weights streaming) then overlaps the other workgroups of the
      // CU streaming, instead of three of the four routing at once.  Their
      // routing result is copied out of the LDS the ring reuses.
      const bool route_first = RING && (int)blockIdx.x / CU_COUNT == 1;
      if constexpr (SHD > 0) {
        if (!route_first)
          for (; !publisher && it < S; it += nb) shared_item(it);
      }
      __builtin_amdgcn_s_waitcnt(0);   // the stash's loads have written LDS
      __syncthreads();
      route_all<THREADS, false, true>(a, L, publisher, tab, &ST);
      if (publisher) return;
      if constexpr (RING) {
        __shared__ OneRowRouting R1;
        const int tid = threadIdx.x;
        if (tid == 0) R1.nact = L.nact;
        if (tid < a.K) {
          R1.sorted[tid] = L.sorted[tid];
          R1.w[tid] = L.w[tid];
        }
        if (tid < L.nact) {
          const int e = clamp_i(L.active[tid], 0, a.E - 1);
          R1.e[tid] = e;
          R1.off[tid] = L.off[e];
          R1.np[tid] = L.off[e + 1] - L.off[e];
#pragma unroll
          for (int j = 0; j < 6; ++j) R1.p[j][tid] = L.one_row[j][tid];
        }
        __syncthreads();
        if constexpr (SHD > 0) {
          if (route_first)
            for (; it < S; it += nb) shared_item(it);
        }
        const int n = R1.nact * ips;
        for (; it < S + n; it += nb) {
          const int ri = it - S;
          const int s = ri / ips, b = ri - s * ips;
          const int off = uniform_i(R1.off[s]), np = uniform_i(R1.np[s]);
          const int i0 = (b * WPB + wave) * NI;
          if (i0 < a.I) {
            const void *p[6];
#pragma unroll
            for (int j = 0; j < 6; ++j) p[j] = reinterpret_cast<const void *>(uniform_u64(R1.p[j][s]));
            gate_up_rows<EF, ACT, CR, NI>(a, p[0], p[1], p[2], p[3], p[4], p[5], a.I, i0, off, np,
                                          R1.sorted + off, R1.w, a.act, a.I);
          }
        }
        return;
      }
      const int n = L.nact * ips;
      for (; it < S + n; it += nb) {
        const int ri = it - S;
        const int s = ri / ips, b = ri - s * ips;
        const int e = uniform_i(clamp_i(L.active[s], 0, a.E - 1));
        const int off = uniform_i(L.off[e]), np = uniform_i(L.off[e + 1]) - off;
        const int i0 = (b * WPB + wave) * NI;
        if (i0 < a.I) {
          const void *p[6];
          if (a.m == 1) {   // entries requested with the logits
#pragma unroll
            for (int j = 0; j < 6; ++j) p[j] = reinterpret_cast<const void *>(uniform_u64(L.one_row[j][s]));
          } else {
            p[0] = tbl(a.gw, e); p[1] = tbl(a.uw, e); p[2] = tbl(a.gs, e);
            p[3] = tbl(a.us, e); p[4] = tbl(a.gb, e); p[5] = tbl(a.ub, e);
          }
          float s2g = 1.0f, s2u = 1.0f;
          if constexpr (EF == NVFP4) {
            s2g = a.gs2[e];
            s2u = a.us2[e];
          }
          gate_up_rows<EF, ACT, CR, NI>(a, p[0], p[1], p[2], p[3], p[4], p[5], a.I, i0, off, np,
                                        L.sorted + off, L.w, a.act, a.I, s2g, s2u);
        }
      }
      return;
    }
  }
  // With the routing published the list runs routed items first (the larger
  // ones: shared items last balance the workgroups' ends; shared items first
  // made the gate/up 6 % slower at m = 8 and 32 on the weight-before
  // workload).  The first item's record is requested with the active count.
  const SlotRec pre = a.slots[clamp_i((int)blockIdx.x / ips, 0, a.cap - 1)];
  const int nact = published_count(a);
  const int n = nact * ips;
  SlotRec nxt = pre;   // record of the next routed item, requested one item ahead
  for (int ri = blockIdx.x; ri < n + S; ri += gridDim.x) {
    if constexpr (SHD > 0) {
      if (ri >= n) {
        shared_item(ri - n);
        continue;
      }
    }
    const int s = ri / ips, b = ri - s * ips;
    const SlotRec rec = nxt;
    if (ri + (int)gridDim.x < n) nxt = a.slots[(ri + (int)gridDim.x) / ips];
    const int off = uniform_i(clamp_i(rec.off, 0, a.te));
    const int np = uniform_i(clamp_i(rec.np, 0, a.te - off));
    const int i0 = (b * WPB + wave) * NI;
    if (i0 < a.I) {
      float s2g = 1.0f, s2u = 1.0f;
      if constexpr (EF == NVFP4) {
        const int e = uniform_i(clamp_i(rec.e, 0, a.E - 1));
        s2g = a.gs2[e];
        s2u = a.us2[e];
      }
      gate_up_rows<EF, ACT, CR, NI>(a, reinterpret_cast<const void *>(rec.gw), reinterpret_cast<const void *>(rec.uw),
                                    reinterpret_cast<const void *>(rec.gs), reinterpret_cast<const void *>(rec.us),
                                    reinterpret_cast<const void *>(rec.gb), reinterpret_cast<const void *>(rec.ub),
                                    a.I, i0, off, np, a.sorted_pair + off, a.topk_w, a.act, a.I, s2g, s2u);
    }
  }
}

// Launch 3: down tiles with the blend.
template <int EF, int ACT, int CR, int CS, int LPR, int NW>
__global__ __launch_bounds__((down_threads<EF, CS, LPR, NW>()), (down_min_waves<EF, CS, NW>())) void down_blend_kernel(Args a) {
  down_item<EF, ACT, CR, CS, LPR, NW>(a, blockIdx.x);
}


// ================================================== pre-norms
//
// One workgroup per row: the RMS norm x * w / sqrt(mean(x^2) + eps) of the
// raw row, in double (the squares and products of stored values are exact),
// rounded once to the activation format (bf16: to nearest, ties to even, from
// the double) -- with the experts' weight into xe (pre-expert norm) and with
// the router's weight into xrn (router pre-norm).  With the router pre-norm
// and a gated shared expert it also takes the gate's logit x . w_g of the raw
// row (the router units then read the normed row only).

// A double to bf16 bits, rounded to nearest (ties to even) in one step:
// the double's significand is rounded to 8 bits on its bit pattern, which is
// then exact in float.  Finite values in bf16's normal range.
__device__ __forceinline__ uint16_t f64_to_bf16(double v) {
  uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint64_t lsb = (u >> 45) & 1ull;
  u = (u + 0x00000FFFFFFFFFFFull + lsb) & ~0x00001FFFFFFFFFFFull;
  return (uint16_t)(__float_as_uint((float)__longlong_as_double((long long)u)) >> 16);
}

template <int ACT>
__global__ __launch_bounds__(256) void pre_norm_kernel(Args a, const void *x, const void *w, const void *wr,
                                                       float eps, void *xe, void *xrn) {
  constexpr int EPC = ACT == F32 ? 4 : 8;   // elements per 16-byte chunk
  __shared__ double s_part[2][4];
  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int H = a.H, nch = H / EPC;
  const size_t rb = (size_t)H * act_bytes(ACT);
  const char *xrow = reinterpret_cast<const char *>(x) + (size_t)r * rb;
  const bool gate = (a.flags & ROUTER_NORM) && (a.flags & SHARED_GATED);
  auto elems = [&](const u32x4 &q, double (&v)[EPC]) {
    if constexpr (ACT == F32) {
      v[0] = __uint_as_float(q.x); v[1] = __uint_as_float(q.y);
      v[2] = __uint_as_float(q.z); v[3] = __uint_as_float(q.w);
    } else {
      v[0] = bf_lo(q.x); v[1] = bf_hi(q.x); v[2] = bf_lo(q.y); v[3] = bf_hi(q.y);
      v[4] = bf_lo(q.z); v[5] = bf_hi(q.z); v[6] = bf_lo(q.w); v[7] = bf_hi(q.w);
    }
  };
  double ss = 0.0, gd = 0.0;
  for (int c = tid; c < nch; c += 256) {
    double v[EPC];
    elems(ld16(xrow + (size_t)c * 16), v);
#pragma unroll
    for (int i = 0; i < EPC; ++i) ss = __builtin_fma(v[i], v[i], ss);
    if (gate) {
      double g[EPC];
      elems(ld16(reinterpret_cast<const char *>(a.sgv) + (size_t)c * 16), g);
#pragma unroll
      for (int i = 0; i < EPC; ++i) gd = __builtin_fma(v[i], g[i], gd);
    }
  }
  ss = wave_sum_f64(ss);
  gd = wave_sum_f64(gd);
  if (lane == 0) {
    s_part[0][wave] = ss;
    s_part[1][wave] = gd;
  }
  __syncthreads();
  const double tot = (s_part[0][0] + s_part[0][1]) + (s_part[0][2] + s_part[0][3]);
  if (gate && tid == 0)
    store_coherent(a.logits + (size_t)r * (a.E + 1) + a.E, (s_part[1][0] + s_part[1][1]) + (s_part[1][2] + s_part[1][3]));
  const double inv = 1.0 / __builtin_sqrt(tot / (double)H + (double)eps);
  for (int o = 0; o < 2; ++o) {
    const void *nw = o == 0 ? w : wr;
    if (!nw) continue;
    char *orow = reinterpret_cast<char *>(o == 0 ? xe : xrn) + (size_t)r * rb;
    for (int c = tid; c < nch; c += 256) {
      double v[EPC], g[EPC];
      elems(ld16(xrow + (size_t)c * 16), v);
      elems(ld16(reinterpret_cast<const char *>(nw) + (size_t)c * 16), g);
      if constexpr (ACT == F32) {
        u32x4 q;
        q.x = __float_as_uint((float)(v[0] * g[0] * inv));
        q.y = __float_as_uint((float)(v[1] * g[1] * inv));
        q.z = __float_as_uint((float)(v[2] * g[2] * inv));
        q.w = __float_as_uint((float)(v[3] * g[3] * inv));
        *reinterpret_cast<u32x4 *>(orow + (size_t)c * 16) = q;
      } else {
        uint32_t q[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          q[i] = (uint32_t)f64_to_bf16(v[2 * i] * g[2 * i] * inv) |
                 ((uint32_t)f64_to_bf16(v[2 * i + 1] * g[2 * i + 1] * inv) << 16);
        *reinterpret_cast<u32x4 *>(orow + (size_t)c * 16) = u32x4{q[0], q[1], q[2], q[3]};
      }
    }
  }
}

// ================================================== grouped path (m > 32)
//
// For 33..MAX_ROWS_G rows the pairs per active expert are many enough that
// the experts' products are small GEMMs: five launches on the caller's stream.
//   route_kernel         the router units only (the logits)
//   topk_sort_kernel     one row per wave: top-k and weights; the workgroup
//                        that takes the last ticket sorts the pairs by expert
//   gate_up_grouped      item = (active slot, 16 intermediate rows) or a
//                        shared-expert row tile: each wave both matrices over
//                        an eighth of H, on the matrix cores, G_COLS of the
//                        expert's pairs per pass
//   down_grouped         item = (active slot, 16 to 64 output columns) or a
//                        shared tile: the waves split the tiles and K; y per
//                        pair to HBM
//   blend_grouped        out[r] = sum_j c_rj y[perm(r, j)] + gamma_r ys[r]
// The (row, vector) sums are accumulated in an order fixed by the layer's
// shapes, so a row's result does not depend on m within this path.

// Stable counting sort of the te pairs in one workgroup: bit r of
// rows[e][r / 32] is set when row r selected expert e; a pair's position is
// its expert's offset plus the number of earlier rows that selected it.
struct SortLDS {
  uint32_t rows[MAX_EXPERTS][MAX_ROWS_G / 32];
  int off[MAX_EXPERTS + 1];
  int slot[MAX_EXPERTS];
  int wtot[2][ROUTE_WPB];
};

template <int ACT>
__global__ __launch_bounds__(ROUTE_THREADS) void topk_sort_kernel(Args a) {
  __shared__ union {
    TopkLDS tk[ROUTE_WPB];
    SortLDS s;
  } sm;
  __shared__ unsigned s_ticket;
  const int wave = uniform_i(threadIdx.x >> 6), lane = threadIdx.x & 63, tid = threadIdx.x;
  const int E = a.E, k = a.K, m = a.m, te = m * k;
  const int r = (int)blockIdx.x * ROUTE_WPB + wave;
  if (r < m) {
    int e;
    double w;
    row_topk<false>(a, r, sm.tk[wave], e, w, nullptr);
    if (lane < k) {
      const float wf = (float)(w * (double)a.rsf);
      const int p = r * k + lane;
      // The sort below reads the selections of every workgroup: they go
      // through device-coherent stores.
      __hip_atomic_store(a.topk_idx + p, e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      a.topk_w[p] = wf;
      if (a.idx_out) a.idx_out[p] = e;
      if (a.w_out) a.w_out[p] = wf;
    }
    if (lane == 0 && (a.flags & SHARED_GATED))
      a.row_gate[r] = (float)sigmoid_d(load_coherent(a.logits + (size_t)r * (E + 1) + E));
  }
  // Only the workgroup that takes the last ticket goes on (nobody waits).
  if (!last_arrival<true>(a.sync + SYNC_TOPK_TICKET, gridDim.x, s_ticket)) return;
  SortLDS &S = sm.s;
  constexpr int RW = MAX_ROWS_G / 32;
  for (int i = tid; i < MAX_EXPERTS * RW; i += ROUTE_THREADS) (&S.rows[0][0])[i] = 0u;
  __syncthreads();
  for (int p = tid; p < te; p += ROUTE_THREADS) {
    const int e = clamp_i(__hip_atomic_load(a.topk_idx + p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT), 0, E - 1);
    const int rr = p / k;
    atomicOr(&S.rows[e][rr >> 5], 1u << (rr & 31));
  }
  __syncthreads();
  // Exclusive scans over the experts of the pair counts and of the active
  // flags: waves 0..3 take 64 experts each.
  int cnt = 0, pre_c = 0, pre_a = 0;
  if (wave < 4) {
    const int e = wave * WAVE + lane;
    if (e < E) {
#pragma unroll
      for (int j = 0; j < RW; ++j) cnt += __popc(S.rows[e][j]);
    }
    int tc, ta;
    pre_c = wave_excl_scan<9>((unsigned)cnt, &tc);
    pre_a = wave_excl_scan<1>(cnt > 0 ? 1u : 0u, &ta);
    if (lane == 0) {
      S.wtot[0][wave] = tc;
      S.wtot[1][wave] = ta;
    }
  }
  __syncthreads();
  if (wave < 4) {
    const int e = wave * WAVE + lane;
    for (int w2 = 0; w2 < wave; ++w2) {
      pre_c += S.wtot[0][w2];
      pre_a += S.wtot[1][w2];
    }
    if (e < E) {
      S.off[e] = pre_c;
      S.slot[e] = pre_a;
      a.offsets[e] = pre_c;
      if (cnt > 0) {
        // The slot's record: what the gate/up and down items need, in one load.
        a.active[pre_a] = e;
        SlotRec rec;
        rec.e = e;
        rec.off = pre_c;
        rec.np = cnt;
        rec.tag = a.tag;
        rec.gw = a.gw[e]; rec.uw = a.uw[e]; rec.dw = a.dw[e];
        rec.gs = a.gs ? a.gs[e] : 0ull; rec.us = a.gs ? a.us[e] : 0ull; rec.ds = a.gs ? a.ds[e] : 0ull;
        rec.gb = a.gb ? a.gb[e] : 0ull; rec.ub = a.gb ? a.ub[e] : 0ull; rec.db = a.gb ? a.db[e] : 0ull;
#pragma unroll
        for (int i = 0; i < 5; ++i) rec.pad2[i] = 0ull;
        a.slots[pre_a] = rec;
      }
      if (e == E - 1) {
        S.off[E] = pre_c + cnt;
        a.offsets[E] = pre_c + cnt;
        a.active_count[0] = pre_a + (cnt > 0 ? 1 : 0);
      }
    }
  }
  __syncthreads();
  for (int p = tid; p < te; p += ROUTE_THREADS) {
    const int e = clamp_i(__hip_atomic_load(a.topk_idx + p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT), 0, E - 1);
    const int rr = p / k;
    int before = __popc(S.rows[e][rr >> 5] & ((1u << (rr & 31)) - 1u));
    for (int j = 0; j < (rr >> 5); ++j) before += __popc(S.rows[e][j]);
    const int pos = S.off[e] + before;
    a.sorted_pair[pos] = p;
    a.pair_to_perm[p] = pos;
  }
  if (tid == 0) {
    a.sync[SYNC_TOPK_TICKET] = 0u;   // every ticket is taken
    a.sync[SYNC_PUBLISHED] = (unsigned)a.tag;
  }
}

// The expert's pair range and weights of gate/up or down item `item` of a
// routed slot, or of the shared expert past the routed items.
struct GroupedItem {
  bool live, routed;
  int e, off, np, n0;
  const void *gw, *uw, *gs, *us, *dw, *ds, *gb, *ub, *db;   // the routed expert's matrices
};

// Shared-expert items: one per (tile, block of G_COLS rows).  They start at
// the first multiple of 8 at or after the routed items, in groups of 8 tiles:
// the row blocks of one tile take block indices 8 apart, so the round-robin
// dispatch puts them on one XCD one after another and the tile's weights are
// read from HBM once and then from that XCD's L2.
__host__ __device__ constexpr int shared_row_blocks(int m) { return (m + G_COLS - 1) / G_COLS; }
__host__ __device__ constexpr int grouped_shared_base(int nrout) { return (nrout + 7) / 8 * 8; }
__host__ __device__ constexpr int grouped_item_count(int nrout, bool shared, int stiles, int m) {
  return shared ? grouped_shared_base(nrout) + (stiles + 7) / 8 * 8 * shared_row_blocks(m) : nrout;
}

__device__ __forceinline__ GroupedItem grouped_item(const Args &a, int item, int tiles, int stiles) {
  GroupedItem g;
  const int nrout = a.cap * tiles;
  if (item < nrout) {
    const int s = item / tiles;
    const int nact = published_count(a);
    g.live = s < nact;
    g.routed = true;
    const SlotRec &r = a.slots[min(s, a.cap - 1)];   // one record, requested with the count
    g.e = uniform_i(clamp_i(r.e, 0, a.E - 1));
    g.off = uniform_i(clamp_i(r.off, 0, a.te));
    g.np = uniform_i(clamp_i(r.np, 0, a.te - g.off));
    g.gw = reinterpret_cast<const void *>(uniform_u64(r.gw));
    g.uw = reinterpret_cast<const void *>(uniform_u64(r.uw));
    g.gs = reinterpret_cast<const void *>(uniform_u64(r.gs));
    g.us = reinterpret_cast<const void *>(uniform_u64(r.us));
    g.dw = reinterpret_cast<const void *>(uniform_u64(r.dw));
    g.ds = reinterpret_cast<const void *>(uniform_u64(r.ds));
    g.gb = reinterpret_cast<const void *>(uniform_u64(r.gb));
    g.ub = reinterpret_cast<const void *>(uniform_u64(r.ub));
    g.db = reinterpret_cast<const void *>(uniform_u64(r.db));
    g.n0 = (item - s * tiles) * 16;
  } else {
    const int P = shared_row_blocks(a.m), sidx = item - grouped_shared_base(nrout);
    const int grp = sidx / (8 * P), r = sidx - grp * 8 * P;
    const int tile = grp * 8 + (r & 7), blk = r >> 3;
    g.live = (a.flags & SHARED) != 0 && sidx >= 0 && tile < stiles;
    g.routed = false;
    g.e = 0;
    g.off = blk * G_COLS;                       // the block's first row
    g.np = max(0, min(G_COLS, a.m - g.off));
    g.n0 = tile * 16;
    g.gw = g.uw = g.gs = g.us = g.dw = g.ds = g.gb = g.ub = g.db = nullptr;
  }
  return g;
}

// Gate/up: item = 16 GT intermediate rows (GT tiles of 16) of one active
// expert (or of the shared expert); wave w takes both matrices of tile
// w % GT over part w / GT of H, so a pair's input fragment serves the gate
// and the up products; the parts are added in part order.  Writes
// silu(g) * v per pair (act, sorted order) or per row (sact).  (Items of two
// or four tiles were slower for every format.)  A pass of at most 16 pairs
// takes one column tile.
template <int EF> constexpr int gate_up_grouped_tiles() { return 1; }
template <int EF> constexpr int gu_grouped_min_waves() { return EF == AFF4 ? 4 : 1; }
// Waves per item, each a part of H: four for MXFP4 and aff4 experts (a
// 16-row item holds a quarter of bf16's bytes, so longer runs of k per wave
// pay: -3 to -11 %), eight for bf16 and for NVFP4, whose dequantisation
// (a float scale per 16 codes) takes the most work per code (-7 % at 256
// rows against four).
template <int EF> constexpr int gu_grouped_waves() { return EF == BF16 || EF == NVFP4 ? 8 : 4; }
// fp8 items hold half of bf16's bytes: four waves, like the 4-bit ones.
template <int EF>
__global__ __launch_bounds__(64 * gu_grouped_waves<EF>(), gu_grouped_min_waves<EF>()) void gate_up_grouped_kernel(Args a) {
  constexpr int NWG = gu_grouped_waves<EF>();
  static_assert(EF == BF16 || EF == MXFP4 || EF == NVFP4 || EF == AFF4 || EF == FP8, "matrix-core experts");
  constexpr int GT = gate_up_grouped_tiles<EF>(), KP = NWG / GT;
  constexpr int QF = EF == BF16 ? MXFP4 : EF;
  __shared__ MfmaLDS<NWG, 2, G_MU> S;
  const int w = uniform_i(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int H = a.H, k = a.K;
  // The top-k launch is over: its ticket word starts the next forward at 0.
  if (blockIdx.x == 0 && threadIdx.x == 0) a.sync[SYNC_TOPK_TICKET] = 0u;
  const GroupedItem it = grouped_item(a, blockIdx.x, (a.I + 16 * GT - 1) / (16 * GT), (a.Is + 16 * GT - 1) / (16 * GT));
  if (!it.live) return;
  const int N = it.routed ? a.I : a.Is;
  const int r0 = it.n0 * GT;                 // the item's first row
  const int n0 = r0 + 16 * (w % GT);         // this wave's 16 rows
  const void *mg = it.routed ? it.gw : a.sgw;
  const void *mu = it.routed ? it.uw : a.suw;
  // bf16 rows (the shared expert's always): one resource per matrix.
  __amdgpu_buffer_rsrc_t A[2];
  QMat<QF> Q[2];
  const bool quant = EF != BF16 && it.routed;
  if (quant) {
    Q[0] = make_qmat<QF>(mg, it.gs, it.gb, N, H);
    Q[1] = make_qmat<QF>(mu, it.us, it.ub, N, H);
  } else {
    A[0] = buf_rsrc(mg, N * H * 2);
    A[1] = buf_rsrc(mu, N * H * 2);
  }
  float s2g = 1.0f, s2u = 1.0f;   // nvfp4: the projections' second-level scales
  if constexpr (EF == NVFP4) {
    if (it.routed) {
      s2g = a.gs2[it.e];
      s2u = a.us2[it.e];
    }
  }
  int kb, ke;
  if (EF == AFF4 && quant) k_slice64(H, w / GT, KP, kb, ke);   // whole scale groups
  else if (EF == FP8 && quant) k_slice128(H, w / GT, KP, kb, ke);
  else k_slice(H, w / GT, KP, kb, ke);
  const bool before = it.routed && (a.flags & WEIGHT_BEFORE);
  const char *x = reinterpret_cast<const char *>(a.x);
  const int g4 = lane >> 4, rr = lane & 15;
  // One pass over the tile: NCT column tiles of 16 pairs from c0 on.
  auto pass = [&](auto nct, int c0, int nv) {
    constexpr int NCT = decltype(nct)::value;
    const char *xv[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const int v = c0 + min(16 * ct + rr, nv - 1);
      const int row = it.routed ? min(clamp_i(a.sorted_pair[it.off + v], 0, a.te - 1) / k, a.m - 1) : it.off + v;
      xv[ct] = x + (size_t)row * H * 2 + (size_t)g4 * 16;
    }
    f32x4 acc[2][NCT];
    if (quant) {
      if constexpr (QF == AFF4 || QF == FP8) {   // codes straight into the operands, group sums
        const char *xr[NCT];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) xr[ct] = xv[ct] - (size_t)g4 * 16;
        if constexpr (QF == AFF4) mfma_slice_aff4<BF16, 2, NCT>(Q, H, n0, N, xr, kb, ke, acc);
        else mfma_slice_f8<BF16, 2, NCT>(Q, H, n0, N, xr, kb, ke, acc);
      } else {
        mfma_slice_q<QF, BF16, 2, NCT, G_MU>(Q, H, n0, N, xv, kb, ke, S.stage[w], acc);
      }
    } else
      mfma_slice_v<BF16, 2, NCT, G_MU>(A, H * 2, n0, N, xv, kb, ke, S.stage[w], acc);
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) S.part[w][j][ct][i][lane] = acc[j][ct][i];
  };
  for (int c0 = 0; c0 < it.np; c0 += G_COLS) {
    const int nv = min(G_COLS, it.np - c0);
    const int nct = nv > 16 ? 2 : 1;
    if (nct == 2) pass(std::integral_constant<int, 2>(), c0, nv);
    else pass(std::integral_constant<int, 1>(), c0, nv);
    __syncthreads();
    // (tile t, column tile ct, element i) combinations, G_WPB at a time.
    for (int c = w; c < GT * nct * 4; c += NWG) {
      const int t = c / (nct * 4), ct = (c / 4) % nct, i = c % 4;
      float gs = 0.f, us = 0.f;
#pragma unroll
      for (int p = 0; p < KP; ++p) {
        gs += S.part[p * GT + t][0][ct][i][lane];
        us += S.part[p * GT + t][1][ct][i][lane];
      }
      gs *= s2g;
      us *= s2u;
      const int row = r0 + 16 * t + (lane >> 4) * 4 + i, v = 16 * ct + (lane & 15);
      if (row < N && v < nv) {
        if (it.routed) {
          if (before) {   // W(w x) = w (W x)
            const float wt = a.topk_w[clamp_i(a.sorted_pair[it.off + c0 + v], 0, a.te - 1)];
            gs *= wt;
            us *= wt;
          }
          // Stored as F32I pairs, the form the grouped down reads.
          reinterpret_cast<uint32_t *>(a.act)[(size_t)(it.off + c0 + v) * a.I + row] = f32i_pair(act_mul(a.flags, gs, us));
        } else {
          reinterpret_cast<uint32_t *>(a.sact)[(size_t)(it.off + c0 + v) * a.Is + row] = f32i_pair(act_mul(a.flags, gs, us));
        }
      }
    }
    __syncthreads();   // the partials are reused by the next pass
  }
}

// Down: y per pair (sorted order) or ys per row, for one active expert (or
// the shared expert):
//   WIDE (rows of at most 2048): item = G_DT tiles of 16 output columns on
//     two waves (four for aff4), each all the tiles over its part of K, so
//     one input fragment serves G_DT tiles;
//   else: item = G_DTL tiles on eight waves, each both tiles over an eighth
//     of K (a long run of k per wave; two tiles halve the input re-reads
//     from L2 that dominate these rows, four cost a wave per SIMD in LDS).
// The parts of K are added in part order.
constexpr int G_DT = 4;
constexpr int G_DTL = 2;
// Wide items run on two waves (longer runs of k per wave), aff4's on
// four: its products per byte are the most, and four parts of K were
// 21-32 % faster than two.
template <int EF, bool WIDE> constexpr int down_grouped_threads() {
  return WIDE ? (EF == AFF4 ? 256 : 128) : G_THREADS;
}
template <bool WIDE> constexpr int down_grouped_cols() { return WIDE ? 16 * G_DT : 16 * G_DTL; }
template <int EF, bool WIDE>
__global__ __launch_bounds__((down_grouped_threads<EF, WIDE>())) void down_grouped_kernel(Args a) {
  static_assert(EF == BF16 || EF == MXFP4 || EF == NVFP4 || EF == AFF4 || EF == FP8, "matrix-core experts");
  constexpr int QF = EF == BF16 ? MXFP4 : EF;                  // the quantised loader's format
  constexpr int NW = down_grouped_threads<EF, WIDE>() / WAVE;   // waves = parts of K
  constexpr int NA = WIDE ? G_DT : G_DTL;                        // tiles per wave
  // bf16 rows of at most 2048: two k steps per staged batch (longer runs per
  // row beat the wave per SIMD they cost); 4-bit kernels keep one, so their
  // shared-expert items do not set their register count.
  constexpr int MU = WIDE ? (EF == BF16 ? 2 : 1) : G_MU;
  constexpr int COLS = down_grouped_cols<WIDE>();
  __shared__ MfmaLDS<NW, NA, MU> S;
  const int w = uniform_i(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int H = a.H;
  const GroupedItem it = grouped_item(a, blockIdx.x, (H + COLS - 1) / COLS, (H + COLS - 1) / COLS);
  if (!it.live) return;
  const int K = it.routed ? a.I : a.Is;
  const char *mat = reinterpret_cast<const char *>(it.routed ? it.dw : a.sdw);
  const int h0 = it.n0 / 16 * COLS;   // the item's first column
  // One resource per tile, bounded to the tile's rows (a tile past H reads
  // nothing).
  __amdgpu_buffer_rsrc_t A[NA];
  QMat<QF> Q[NA];
  const bool quant = EF != BF16 && it.routed;
  float s2d = 1.0f;   // nvfp4: the down projection's second-level scale
  if (quant) {
    const char *smat = reinterpret_cast<const char *>(it.ds);
    const char *bmat = reinterpret_cast<const char *>(it.db);
    // Scale bytes per row: K/16 (nvfp4), K/32 (mxfp4), K/64 bf16 (aff4);
    // fp8: the tile's 128-row block row of K/128 fp32 scales.
    const int sb = QF == NVFP4 ? K / 16 : QF == AFF4 ? K / 32 : K / 32;
#pragma unroll
    for (int j = 0; j < NA; ++j) {
      const int r0 = h0 + 16 * j, nr = max(0, min(16, H - r0));
      if constexpr (QF == FP8) {
        Q[j].w = buf_rsrc(mat + (size_t)min(r0, H) * K, nr * K);
        Q[j].s = buf_rsrc(smat + (size_t)(min(r0, H - 1) / 128) * (K / 128) * 4, nr > 0 ? (K / 128) * 4 : 0);
        Q[j].b = Q[j].s;
      } else {
        Q[j].w = buf_rsrc(mat + (size_t)min(r0, H) * (K / 2), nr * (K / 2));
        Q[j].s = buf_rsrc(smat + (size_t)min(r0, H) * sb, nr * sb);
        Q[j].b = QF == AFF4 ? buf_rsrc(bmat + (size_t)min(r0, H) * sb, nr * sb) : Q[j].s;
      }
    }
    if constexpr (EF == NVFP4) s2d = a.ds2[it.e];
  } else {
#pragma unroll
    for (int j = 0; j < NA; ++j) {
      const int r0 = h0 + 16 * j;
      A[j] = buf_rsrc(mat + (size_t)min(r0, H) * K * 2, max(0, min(16, H - r0)) * K * 2);
    }
  }
  int kb, ke;
  if (EF == AFF4 && quant) k_slice64(K, w, NW, kb, ke);   // whole scale groups
  else if (EF == FP8 && quant) k_slice128(K, w, NW, kb, ke);
  else k_slice(K, w, NW, kb, ke);
  // The input rows as F32I pairs (written so by the grouped gate/up).
  const char *xb = reinterpret_cast<const char *>((it.routed ? a.act : a.sact) + (size_t)it.off * K);
  float *dst = (it.routed ? a.y : a.sy) + (size_t)it.off * H;
  // One pass: NCT column tiles of 16 pairs from c0 on.
  auto pass = [&](auto nct, int c0, int nv) {
    constexpr int NCT = decltype(nct)::value;
    f32x4 acc[NA][NCT];
    if (quant) {   // 4-bit codes straight into the operands; passes of one column tile
      if constexpr (NCT == 1) {
        const char *xr[1] = {xb + (size_t)(c0 + min(lane & 15, nv - 1)) * K * 4};
        if constexpr (QF == AFF4) mfma_slice_aff4<F32I, NA, 1>(Q, K, 0, 16, xr, kb, ke, acc);
        else if constexpr (QF == FP8) mfma_slice_f8<F32I, NA, 1>(Q, K, 0, 16, xr, kb, ke, acc);
        else mfma_slice_qd<QF, F32I, NA, 1, 2>(Q, K, 0, 16, xr, kb, ke, acc);
      }
    } else {
      mfma_slice<F32I, NA, NCT, MU>(A, K * 2, 0, 16, xb + (size_t)c0 * K * 4, (size_t)K * 4, nv, kb, ke,
                                    S.stage[w], acc);
    }
#pragma unroll
    for (int j = 0; j < NA; ++j)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) S.part[w][j][ct][i][lane] = acc[j][ct][i];
  };
  // 4-bit passes take 16 pairs (one column tile): two tiles' inputs would
  // cost a wave per SIMD in registers.  A pair's sum does not depend on the
  // pass it is in.
  const int step = quant ? 16 : G_COLS;
  for (int c0 = 0; c0 < it.np; c0 += step) {
    const int nv = min(step, it.np - c0);
    const int nct = nv > 16 ? 2 : 1;
    if (nct == 2) pass(std::integral_constant<int, 2>(), c0, nv);
    else pass(std::integral_constant<int, 1>(), c0, nv);
    __syncthreads();
    // (tile t, column tile ct, element i) combinations, NW at a time.
    for (int c = w; c < NA * nct * 4; c += NW) {
      const int t = c / (nct * 4), ct = (c / 4) % nct, i = c % 4;
      float sum = 0.f;
#pragma unroll
      for (int p = 0; p < NW; ++p) sum += S.part[p][t][ct][i][lane];
      const int row = h0 + 16 * t + (lane >> 4) * 4 + i, v = 16 * ct + (lane & 15);
      if (row < H && v < nv) dst[(size_t)(c0 + v) * H + row] = sum * s2d;
    }
    __syncthreads();
  }
}

// Blend: thread = (row r, 4 output columns); slots in order, then the shared
// term.
template <int ACT>
__global__ __launch_bounds__(256) void blend_grouped_kernel(Args a) {
  const int H = a.H, k = a.K, q = H / 4;
  const int t = (int)blockIdx.x * 256 + (int)threadIdx.x;
  const int r = t / q, h = (t - r * q) * 4;
  if (r >= a.m) return;
  const bool before = (a.flags & WEIGHT_BEFORE) != 0;
  float o[4] = {0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < k; ++j) {
    const int p = r * k + j;
    const float c = before ? 1.0f : a.topk_w[p];
    const int pos = clamp_i(a.pair_to_perm[p], 0, a.te - 1);
    const u32x4 y = ld16(a.y + (size_t)pos * H + h);
    o[0] = __builtin_fmaf(c, __uint_as_float(y.x), o[0]);
    o[1] = __builtin_fmaf(c, __uint_as_float(y.y), o[1]);
    o[2] = __builtin_fmaf(c, __uint_as_float(y.z), o[2]);
    o[3] = __builtin_fmaf(c, __uint_as_float(y.w), o[3]);
  }
  if (a.flags & SHARED) {
    const float gm = (a.flags & SHARED_GATED) ? a.row_gate[r] : 1.0f;
    const u32x4 ys = ld16(a.sy + (size_t)r * H + h);
    o[0] = __builtin_fmaf(gm, __uint_as_float(ys.x), o[0]);
    o[1] = __builtin_fmaf(gm, __uint_as_float(ys.y), o[1]);
    o[2] = __builtin_fmaf(gm, __uint_as_float(ys.z), o[2]);
    o[3] = __builtin_fmaf(gm, __uint_as_float(ys.w), o[3]);
  }
  if ((a.flags & OUT_F32) || ACT == F32) {
    *reinterpret_cast<u32x4 *>(reinterpret_cast<float *>(a.out) + (size_t)r * H + h) =
        u32x4{__float_as_uint(o[0]), __float_as_uint(o[1]), __float_as_uint(o[2]), __float_as_uint(o[3])};
  } else {
    *reinterpret_cast<u32x2 *>(reinterpret_cast<uint16_t *>(a.out) + (size_t)r * H + h) =
        u32x2{(uint32_t)f32_to_bf16(o[0]) | ((uint32_t)f32_to_bf16(o[1]) << 16),
              (uint32_t)f32_to_bf16(o[2]) | ((uint32_t)f32_to_bf16(o[3]) << 16)};
  }
}

}  // namespace moe
