/*
 * moe_decode.h -- C ABI of libmoe_decode.so: the fused small-batch decode
 * Mixture-of-Experts layer on one AMD Instinct MI355X (gfx950).
 *
 * One call of moe_decode_forward evaluates, for m = 1..max_rows token rows,
 * the whole decode MoE layer that the metrale page
 * "forward_bf16_grouped_decode.rs" (fn forward_bf16_grouped_decode) lays out
 * as five steps -- the per-row router, the sort of (row, slot) pairs by
 * expert, expert gate+up with SiLU, expert down, and the grouped blend with a
 * gated shared expert -- on the caller's HIP stream, without host
 * synchronisation:
 *
 *   logits[r,e] = sum_h x[r,h] * Wr[e,h]
 *   selection   softmax:        top-k of the logits, weight softmax(l)
 *               sigmoid+bias:   top-k of sigmoid(l)+bias, weight sigmoid(l)
 *                               (mlxcel page "perf(moe): wire lfm2 to the
 *                               fused decode-MoE kernel", Summary; iron page
 *                               "refactor(gemm): split the gemv_q8 grab-bag
 *                               by family", commit message: select by the
 *                               biased score, weight by the unbiased one)
 *               raw-logit:      top-k of the logits, weight sigmoid(l)
 *                               (frink page "routed_weight_site.rs", module doc)
 *               ties go to the lower expert index; slots are ordered by key
 *               descending.  Optional norm_topk_prob (divide by the sum of the
 *               selected weights), then times routed_scaling_factor.
 *   expert      y = Wd * (silu(Wg u) * (Wu u)), u = x (weight on the output)
 *               or u = w x (weight on the input, frink "routed_weight_site.rs",
 *               fn routed_slot)
 *   out[r]      = sum_j c_rj y_rj + gamma_r * shared(x_r), c = w or 1,
 *               gamma = sigmoid(x . w_g) (gated) or 1.
 *
 * m = 1..32 is the fused decode path the page describes (three launches).
 * m = 33..256 (prefill chunks, speculative-decoding verification) takes a
 * grouped path of the same steps whose expert products run on the matrix
 * cores (five launches); it needs bf16 activations, bf16, aff4, mxfp4,
 * nvfp4 or fp8 experts and H, I, Is multiples of 32, which moe_decode_plan checks
 * when max_rows > 32.  Each path gives a row the same bits for every m it
 * serves; the two paths agree within the tolerance of their accumulation
 * orders.
 *
 * Ownership: the caller owns every device buffer (weights, pointer tables,
 * x, out, idx/w outputs, workspace).  A plan owns host memory only; it is
 * immutable after moe_decode_plan and may be shared by threads and streams,
 * with one workspace per concurrently running call.  moe_decode_forward
 * allocates nothing, never synchronises, never reads device memory on the
 * host, and launches only kernels (no memset/memcpy nodes), so it can be
 * captured into a HIP graph.
 *
 * Errors: every entry point returns a moe_status.  On any status other than
 * MOE_OK nothing has been launched (except MOE_EHIP from a launch itself);
 * moe_decode_last_error() then returns a thread-local message.
 */
#ifndef MOE_DECODE_H
#define MOE_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_EINVAL = 1,        /* bad argument: null pointer, m out of range, ... */
  MOE_EUNSUPPORTED = 2,  /* a shape or format combination the kernels do not serve */
  MOE_EWORKSPACE = 3,    /* workspace missing, too small or misaligned */
  MOE_EHIP = 4           /* a HIP call failed; the message holds its error string */
} moe_status;

/* Storage formats.  All arrays are row-major [N, K] with K the reduction
 * dimension (gate/up: N = inter, K = hidden; down: N = hidden, K = inter),
 * as in the metrale page "helpers_a.rs" (packed [N, K/2] weights and
 * [N, K/group] scales; scale block 32 for E8M0).
 *   MOE_F32        float32
 *   MOE_BF16       bfloat16 bit patterns (uint16)
 *   MOE_AFF4_G64   4-bit unsigned codes q, packed [N, K/2] with element 2t in
 *                  the low nibble of byte t; value = scale*q + bias with one
 *                  bf16 scale and one bf16 bias per 64 elements along K
 *                  ([N, K/64] each)
 *   MOE_MXFP4_B32  OCP MX FP4 E2M1 codes, packed like aff4; value =
 *                  E2M1(code) * 2^(e-127) with one E8M0 byte e per 32
 *                  elements along K ([N, K/32]); e = 255 (NaN) is not valid.
 *   MOE_NVFP4_B16  NVFP4 (the same page: scale block 16, plus the per-expert
 *                  second-level scale each projection carries): E2M1 codes
 *                  packed like aff4; value = E2M1(code) * E4M3(s) * s2 with
 *                  one OCP FP8 E4M3 byte s per 16 elements along K ([N, K/16])
 *                  and one float32 s2 per expert projection (the *_scale2
 *                  arrays below); the E4M3 NaN bytes 0x7F / 0xFF are not valid.
 *                  The activations stay in act_fmt (weight-only dequantisation).
 *   MOE_FP8_B128   FP8 experts (metrale "forward_bf16_grouped_decode.rs": the
 *                  grouped decode serves NVFP4, FP8 and BF16 experts; the
 *                  page fixes no layout, this is the library's reading): one
 *                  OCP FP8 E4M3 byte per element, [N, K]; value = E4M3(code)
 *                  * s with one float32 s per 128 x 128 block of the matrix
 *                  ([N/128, K/128], row-major); H and I must be multiples of
 *                  128; the NaN bytes 0x7F / 0xFF are not valid.  Weight-only
 *                  dequantisation like NVFP4. */
typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_AFF4_G64 = 2, MOE_MXFP4_B32 = 3, MOE_NVFP4_B16 = 4,
               MOE_FP8_B128 = 5 } moe_format;

typedef enum {
  MOE_ROUTE_SOFTMAX = 0,        /* select by logit, weight softmax(l) over all E */
  MOE_ROUTE_SIGMOID_BIAS = 1,   /* select by sigmoid(l)+bias, weight sigmoid(l) */
  MOE_ROUTE_SIGMOID_LOGIT = 2,  /* select by logit, weight sigmoid(l) */
  MOE_ROUTE_SQRTSOFTPLUS = 3    /* score s = sqrt(log(1 + e^l)): select by s, or by s + bias when
                                   expert_bias is given; weight s (iron page "refactor(gemm): split
                                   the gemv_q8 grab-bag by family", commit message: router_sqrtsoftplus) */
} moe_routing;

enum {
  MOE_NORM_TOPK = 1,          /* divide the selected weights by their sum */
  MOE_WEIGHT_BEFORE_FFN = 2,  /* the routing weight scales the expert input; output weight 1 */
  MOE_SHARED = 4,             /* add a shared SwiGLU expert on every row (unscaled input) */
  MOE_SHARED_GATED = 8,       /* ... times sigmoid(x . w_g) (requires MOE_SHARED) */
  MOE_OUT_F32 = 16,           /* write out as float32 instead of act_fmt */
  MOE_GEGLU = 32,             /* expert activation gelu(gate) * up (GeGLU, exact GELU
                                 g * Phi(g)) instead of silu(gate) * up, routed and shared;
                                 metrale "helpers_a.rs", set_gelu_activation */
  MOE_PRE_EXPERT_NORM = 64,   /* the experts (routed and shared) read each row RMS-normed,
                                 x * w / sqrt(mean(x^2) + norm_eps) with w = pre_norm_w,
                                 stored in act_fmt (to nearest, ties to even); the router and
                                 the shared-expert gate read the row as it is.  metrale
                                 "helpers_a.rs", set_pre_expert_norm */
  MOE_ROUTER_PRE_NORM = 128   /* the router reads each row RMS-normed with router_norm_w (same
                                 form, norm_eps and rounding as the pre-expert norm); the experts
                                 and the shared-expert gate do not.  metrale
                                 "forward_bf16_grouped_decode.rs" (weights.router_pre_norm) */
};

typedef struct {
  int32_t hidden;        /* H: multiple of 8 (f32/bf16), 64 (aff4), 32 (mxfp4, nvfp4), 128 (fp8) */
  int32_t num_experts;   /* E: 1..256 */
  int32_t top_k;         /* k: 1..min(E, 16) */
  int32_t inter;         /* I: routed expert intermediate size, same multiples as H */
  int32_t shared_inter;  /* Is: shared expert intermediate (multiple of 8), 0 without MOE_SHARED */
  int32_t max_rows;      /* largest m a forward will be given: 1..256 (above 32: see the top) */
  int32_t act_fmt;       /* moe_format of x, out, router, shared expert, w_g: MOE_F32 or MOE_BF16 */
  int32_t expert_fmt;    /* moe_format of the routed experts: any */
  int32_t routing;       /* moe_routing */
  uint32_t flags;        /* MOE_NORM_TOPK | MOE_WEIGHT_BEFORE_FFN | MOE_SHARED | ... */
  float routed_scaling_factor;
  float norm_eps;        /* MOE_PRE_EXPERT_NORM, MOE_ROUTER_PRE_NORM: finite, >= 0; else ignored */
} moe_decode_desc;

/* Device pointers.  The per-expert tables are DEVICE arrays of E uint64
 * device addresses (one per routed expert); each entry must be non-null and
 * 16-byte aligned, which the library documents but does not check. */
typedef struct {
  const void *router_w;        /* [E, H] act_fmt */
  const float *expert_bias;    /* [E] float32; required by MOE_ROUTE_SIGMOID_BIAS, optional with
                                  MOE_ROUTE_SQRTSOFTPLUS, ignored otherwise */
  const uint64_t *gate_w;      /* table: [I, H] (packed [I, H/2] for 4-bit; bytes for fp8) */
  const uint64_t *up_w;        /* table: [I, H] */
  const uint64_t *down_w;      /* table: [H, I] (packed [H, I/2]) */
  const uint64_t *gate_s;      /* table of scales: aff4 bf16 [I, H/64], mxfp4 u8 [I, H/32],
                                  nvfp4 u8 [I, H/16], fp8 float32 [I/128, H/128]; else NULL */
  const uint64_t *up_s;
  const uint64_t *down_s;      /* aff4 bf16 [H, I/64], mxfp4 u8 [H, I/32], nvfp4 u8 [H, I/16],
                                  fp8 float32 [H/128, I/128] */
  const uint64_t *gate_b;      /* table of aff4 biases, bf16 like the scales; else NULL */
  const uint64_t *up_b;
  const uint64_t *down_b;
  const void *sh_gate_w;       /* [Is, H] act_fmt (MOE_SHARED) */
  const void *sh_up_w;         /* [Is, H] act_fmt */
  const void *sh_down_w;       /* [H, Is] act_fmt */
  const void *sh_gate_vec;     /* [H] act_fmt (MOE_SHARED_GATED) */
  const float *gate_scale2;    /* nvfp4: [E] float32 second-level scale of each expert's gate; else ignored */
  const float *up_scale2;      /* nvfp4: [E] float32, up */
  const float *down_scale2;    /* nvfp4: [E] float32, down */
  const void *pre_norm_w;      /* [H] act_fmt (MOE_PRE_EXPERT_NORM), 16-byte aligned */
  const void *router_norm_w;   /* [H] act_fmt (MOE_ROUTER_PRE_NORM), 16-byte aligned */
} moe_decode_weights;

typedef struct moe_decode_plan moe_decode_plan_t;

/* Byte offsets (from the workspace base) of the arrays a forward leaves in
 * the workspace, for inspection.  Sizes are for max_rows rows;
 * te = max_rows * top_k, cap = min(te, E). */
typedef struct {
  size_t logits;          /* double [max_rows, E+1]: router logits; column E = x . w_g */
  size_t scores;          /* double [max_rows, E]: sqrt-softplus scores of the logits
                             (MOE_ROUTE_SQRTSOFTPLUS; a 4-byte placeholder otherwise) */
  size_t topk_idx;        /* int32 [te]: selected experts, row-major [m, k] */
  size_t topk_w;          /* float [te]: routing weights (before placement) */
  size_t row_gate;        /* float [max_rows]: shared-expert gate gamma_r */
  size_t sorted_pair;     /* int32 [te]: pair ids p = r*k + j sorted by expert, stable */
  size_t expert_offsets;  /* int32 [E+1]: start of each expert's run in sorted_pair */
  size_t pair_to_perm;    /* int32 [te]: position of pair p in sorted_pair */
  size_t active_experts;  /* int32 [cap]: experts with at least one pair, ascending */
  size_t active_count;    /* int32 [1] */
  size_t slot_info;       /* [cap] 128-byte records, one per active slot u < active_count:
                             int32 expert, first position in sorted_pair, pair count, and a
                             tag (odd) that hashes the call's tables, x, workspace and m;
                             then the expert's gate_w, up_w, gate_s, up_s, gate_b, up_b,
                             down_w, down_s, down_b entries (uint64), then 40 zero bytes */
  size_t act;             /* float [te, I]: routed SwiGLU activations, sorted order; for 4-bit
                             experts each row is stored sub-step-major: element i at
                             ((i % 32) / 8) * (I / 4) + (i / 32) * 8 + i % 8.  Above 32
                             rows each 4-byte element holds the value as a bf16 pair:
                             its top 16 bits in the low half, the bf16 rounding of the
                             remainder in the high half */
  size_t shared_act;      /* float [max_rows, Is]; as bf16 pairs (like act above 32 rows)
                             above 32 rows, and at every m with bf16 experts and the shared
                             expert on the matrix cores */
  size_t shared_y;        /* float [P, max_rows, H]: shared-expert output in P parts of Is
                             (matrix-core path; P = max(1, min(Is / 2048, 16))) */
  size_t routed_y;        /* float [te, H]: routed expert outputs per pair, sorted order
                             (m > 32 only; a 4-byte placeholder when max_rows <= 32) */
  size_t normed_x;        /* act_fmt [max_rows, H]: the experts' input under
                             MOE_PRE_EXPERT_NORM (a 4-byte placeholder without it) */
  size_t router_x;        /* act_fmt [max_rows, H]: the router's input under
                             MOE_ROUTER_PRE_NORM (a 4-byte placeholder without it) */
  size_t sync;            /* uint32 [512]: reserved words.  Word 0 counts the router
                             workgroups, word 1 the top-k workgroups of the m > 32 path;
                             the last arrival resets each and the forward's next launch
                             resets it again, so a forward leaves them zero whatever it
                             found there.  Word 2 holds the tag of the last call whose
                             routing was published: the launches that read the slot records
                             take routed work only when it is their call's.  The rest stay
                             zero. */
  size_t total;           /* bytes a workspace must have */
} moe_decode_ws_layout;

/* Validate a layer description and build a plan: the predicate of the metrale
 * page "forward_bf16_grouped_decode.rs" (fn bf16_grouped_decode_arena_ok and
 * bf16_grouped_decode_ok: the shape, weight, kernel and arena terms decided
 * before anything runs, the m cap, the arena need of grouped_decode_buffer_need
 * here returned as the workspace size).  MOE_EUNSUPPORTED for shapes or format
 * combinations the kernels do not serve, MOE_EINVAL for malformed fields;
 * *workspace_bytes receives the workspace size (alignment 256 bytes).  The
 * plan is host memory the caller releases with moe_decode_plan_destroy. */
moe_status moe_decode_plan(const moe_decode_desc *desc, moe_decode_plan_t **plan,
                           size_t *workspace_bytes);

void moe_decode_plan_destroy(moe_decode_plan_t *plan);

/* Fill *layout for this plan (host only). */
moe_status moe_decode_workspace_layout(const moe_decode_plan_t *plan,
                                       moe_decode_ws_layout *layout);

/* Prepare a freshly allocated workspace (zeroes its reserved completion words
 * with a kernel on `stream`).  Call once before the first forward on a
 * workspace; forwards leave them zero.  Without it, the first forward on the
 * workspace may route from an incomplete set of logits (its output is then
 * wrong; it reads only in-range memory) and every later forward is correct. */
moe_status moe_decode_workspace_init(const moe_decode_plan_t *plan, void *workspace,
                                     size_t workspace_bytes, void *stream);

/* The layer on m rows: fn forward_bf16_grouped_decode of the metrale page
 * "forward_bf16_grouped_decode.rs" -- the per-row router, the sort of the
 * (row, slot) pairs by expert, gate+up with the activation, down, and the blend
 * with the shared expert, the output landing in rows 0..m of `out`, an error
 * returned with nothing launched when the predicate fails; the routing of the
 * mlxcel page "perf(moe): wire lfm2 to the fused decode-MoE kernel" (Summary)
 * and the weight placement of the frink page "routed_weight_site.rs"
 * (fn routed_slot) as described at the top of this file.
 *   x          device [m, H] act_fmt
 *   out        device [m, H] act_fmt (float32 with MOE_OUT_F32)
 *   idx_out    device int32 [m, k] selected experts, or NULL
 *   w_out      device float [m, k] routing weights, or NULL
 *   workspace  device, >= the plan's size, 256-byte aligned, initialised once
 *   stream     hipStream_t (NULL = the null stream)
 * MOE_EINVAL for m outside 1..max_rows or a missing pointer the flags need,
 * MOE_EWORKSPACE for a missing/small/misaligned workspace; nothing launches
 * on error.  Calls that share a workspace must not overlap. */
moe_status moe_decode_forward(const moe_decode_plan_t *plan, const moe_decode_weights *w,
                              const void *x, int32_t m, void *out, int32_t *idx_out,
                              float *w_out, void *workspace, size_t workspace_bytes,
                              void *stream);

/* The same forward with no workspace argument, for callers that cannot
 * allocate (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): it allocates nothing and uses a library-owned device
 * array of 32 MiB, one per GPU, held until the process ends.  A plan whose
 * workspace (moe_decode_plan's *workspace_bytes) exceeds 32 MiB is rejected
 * with MOE_EWORKSPACE, launching nothing.  Every such call on a GPU shares
 * that GPU's array, which keeps the last call's contents: calls that overlap
 * on one GPU race.  The first call on a GPU also launches a kernel that
 * clears the array's reserved words.  Other arguments and errors as
 * moe_decode_forward. */
moe_status moe_decode_forward_noalloc(const moe_decode_plan_t *plan, const moe_decode_weights *w,
                                      const void *x, int32_t m, void *out, int32_t *idx_out,
                                      float *w_out, void *stream);

/* Number of kernel launches (stages) one forward makes, and the name of
 * stage i ("route", "gate_up", "down_blend", ...). */
int32_t moe_decode_num_stages(const moe_decode_plan_t *plan);
const char *moe_decode_stage_name(const moe_decode_plan_t *plan, int32_t i);

/* As moe_decode_forward, with per-stage timing: stage i is launched with
 * hipExtLaunchKernelGGL so that events[2i] and events[2i+1] (hipEvent_t,
 * created with timing enabled) take that kernel's own start and end
 * timestamps; hipEventElapsedTime(events[2i], events[2i+1]) is then the
 * kernel's duration without launch gaps.  n_events must equal
 * 2 * moe_decode_num_stages(plan); no entry may be NULL.  Not for stream
 * capture (use moe_decode_forward there). */
moe_status moe_decode_forward_timed(const moe_decode_plan_t *plan, const moe_decode_weights *w,
                                    const void *x, int32_t m, void *out, int32_t *idx_out,
                                    float *w_out, void *workspace, size_t workspace_bytes,
                                    void *stream, void *const *events, int32_t n_events);

/* Thread-local message of the last failed call on this thread ("" if none). */
const char *moe_decode_last_error(void);

/* Library version string. */
const char *moe_decode_version(void);

/* Measurement utilities (not part of the layer).  Plain streaming kernels
 * with the layer's 16-byte-per-lane access pattern, used as known-size
 * references for HBM byte counters and for achievable bandwidth.
 *   moe_decode_bench_copy  dst[0..bytes) = src[0..bytes)   (device buffers)
 *   moe_decode_bench_read  reads src[0..bytes) once; sink is a device uint32
 *                          that is (practically) never written
 * bytes must be a multiple of 16 and the buffers 16-byte aligned; launched on
 * `stream`; MOE_EINVAL otherwise. */
moe_status moe_decode_bench_copy(const void *src, void *dst, size_t bytes, void *stream);
moe_status moe_decode_bench_read(const void *src, size_t bytes, uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_DECODE_H */
