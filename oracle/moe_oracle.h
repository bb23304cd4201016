/*
 * moe_oracle.h -- plain, slow, fp64 CPU oracle of the small-batch decode MoE
 * layer.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the CPU
 * baseline leg of the bench call it; the product path never does.
 *
 * It shares no code, header or table with the HIP library.  Every stored
 * value is decoded exactly to double and every sum, exponential and product
 * is taken in double; nothing is blocked, fused or reordered beyond the
 * definition.  Host pointers only.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage formats (numbers chosen independently of the HIP library's). */
enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_AFF4 = 2, ORC_MXFP4 = 3, ORC_NVFP4 = 4, ORC_FP8 = 5 };
/* Routing modes. */
enum { ORC_SOFTMAX = 0, ORC_SIGMOID_BIAS = 1, ORC_SIGMOID_LOGIT = 2, ORC_SQRTSOFTPLUS = 3 };

typedef struct {
  int32_t hidden, num_experts, top_k, inter, shared_inter;
  int32_t act_fmt;      /* ORC_F32 / ORC_BF16: x, router, shared expert, w_g */
  int32_t expert_fmt;   /* ORC_F32 / ORC_BF16 / ORC_AFF4 / ORC_MXFP4 / ORC_NVFP4 / ORC_FP8 */
  int32_t routing;
  int32_t norm_topk, weight_before_ffn, shared, shared_gated;
  double routed_scaling_factor;
  int32_t geglu;        /* expert activation gelu(gate) * up instead of silu(gate) * up */
  int32_t pre_norm;     /* experts read the row RMS-normed with pre_norm_w (router: raw) */
  double norm_eps;
  int32_t router_pre_norm; /* the router reads the row RMS-normed with router_norm_w */
} orc_desc;

typedef struct {
  const void *router;                 /* [E,H] act_fmt */
  const float *expert_bias;           /* [E] or NULL */
  /* Per-expert host pointers, [E] each.  f32/bf16: [N,K]; 4-bit: packed
   * [N,K/2] bytes, low nibble = even element; scale [N,K/G]; aff4 bias
   * [N,K/64] bf16; nvfp4: the "bias" entry points to the projection's one
   * fp32 second-level scale.  fp8: one E4M3 byte per element, [N,K], and
   * one fp32 scale per 128 x 128 block, [ceil(N/128), ceil(K/128)]. */
  const void *const *gate, *const *up, *const *down;
  const void *const *gate_s, *const *up_s, *const *down_s;
  const void *const *gate_b, *const *up_b, *const *down_b;
  const void *sh_gate, *sh_up, *sh_down; /* [Is,H],[Is,H],[H,Is] act_fmt */
  const void *sh_gate_vec;               /* [H] act_fmt */
  const void *pre_norm_w;                /* [H] act_fmt (pre_norm) */
  const void *router_norm_w;             /* [H] act_fmt (router_pre_norm) */
} orc_weights;

/* One OCP FP8 E4M3 byte decoded to double (NaN for the NaN codes). */
double orc_e4m3_value(uint8_t b);
/* Threads the oracle spreads a projection's output neurons over (OpenMP;
 * default 1).  Results are the same for every count. */
void orc_set_threads(int32_t n);
int32_t orc_get_threads(void);

/* v rounded to the activation format (float32, or bf16 to nearest, ties to
 * even, subnormals included), as a double. */
double orc_round_act(int32_t fmt, double v);
/* One stored element decoded to double. */
double orc_decode_act(int32_t fmt, const void *p, int64_t i);
/* Row n of an [N,K] expert projection, decoded to double, out[K]. */
void orc_decode_row(int32_t fmt, const void *w, const void *s, const void *b,
                    int32_t K, int32_t n, double *out);

/* One row's expert input under the pre-expert norm: xe[H] from x[H]. */
void orc_pre_expert_norm(const orc_desc *d, const void *norm_w, const double *x, double *xe);

/* One routed slot's expert input and output weight (weight placement). */
void orc_routed_slot(const double *x, int32_t n, double w, int32_t before_ffn,
                     double *x_out, double *w_out);

/* Router logits of one row: logits[E] (x_row stored in act_fmt, read as it
 * is: the router pre-norm is applied by orc_forward). */
void orc_router_logits(const orc_desc *d, const orc_weights *wt, const void *x_row,
                       double *logits);

/* The sqrt-softplus score sqrt(log(1 + e^l)). */
double orc_sqrtsoftplus(double l);

/* Selection and weights of one row from its logits (expert_bias: [E], or NULL
 * where the routing takes none). idx[k], w[k]; margin =
 * smallest gap between consecutive keys among the top min(k+1,E) keys. */
void orc_select(const orc_desc *d, const float *expert_bias, const double *logits,
                int32_t *idx, double *w, double *margin);

/* Stable counting sort of the m*k (row, slot) pairs by expert. */
void orc_sort_pairs(int32_t m, int32_t k, int32_t E, const int32_t *idx,
                    int32_t *sorted_pair, int32_t *expert_offsets,
                    int32_t *pair_to_perm, int32_t *active_experts,
                    int32_t *active_count);

/* The whole layer on m rows.  x [m,H] act_fmt.  out [m,H] double.  idx/w/
 * logits/margin may be NULL.  Returns 0, or -1 on an invalid descriptor. */
int32_t orc_forward(const orc_desc *d, const orc_weights *wt, const void *x, int32_t m,
                    double *out, int32_t *idx, double *w, double *logits, double *margin);

#ifdef __cplusplus
}
#endif
#endif
