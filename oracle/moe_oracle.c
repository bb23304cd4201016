/*
 * moe_oracle.c -- the oracle: a plain fp64 CPU evaluation of the small-batch
 * decode MoE layer, written from the pages' description of what the layer
 * computes.  TEST INFRASTRUCTURE ONLY (tests, smoke check, CPU baseline).
 *
 * Pages followed (cited by page title and the item on it):
 *  - "forward_bf16_grouped_decode.rs" (metrale): module doc and
 *    fn forward_bf16_grouped_decode -- per-row router, sort of the (row, slot)
 *    pairs by expert, gate+up and SiLU, down, blend with a gated shared
 *    expert; the invariant that a row's result does not depend on m.
 *  - "perf(moe): wire lfm2 to the fused decode-MoE kernel" (mlxcel #309),
 *    Summary -- sigmoid routing with expert_bias selection, norm_topk_prob and
 *    routed_scaling_factor applied to the scores.
 *  - "refactor(gemm): split the gemv_q8 grab-bag by family" (iron #24),
 *    commit message -- the biased router selects by the biased score and
 *    weights by the unbiased one.
 *  - "routed_weight_site.rs" (frink-models): module doc and fn routed_slot --
 *    where the routing weight multiplies a routed expert (input or output);
 *    the raw-logit top-k of the weight-before-FFN model.
 *  - "helpers_a.rs" (metrale): transpose_for_prefill_impl -- the E8M0 scale
 *    block of 32; packed [N, K/2] weights with [N, K/group] scales; the
 *    NVFP4 scale block of 16, and the per-expert second-level scale
 *    (weight_scale_2, the scale2 values) each projection carries.
 *
 * Every stored value is decoded exactly to double; every dot product,
 * exponential, normalisation and sum is taken in double, in the order the
 * definition states.  Readings of points the pages leave open:
 *  - selection ties go to the lower expert index; slots are listed by key
 *    descending, then index ascending;
 *  - the softmax selection key is the logit (softmax is monotone);
 *  - normalisation (sum of the selected weights, no epsilon) comes before
 *    routed_scaling_factor;
 *  - the shared expert reads the unscaled row; its gate is sigmoid(x . w_g);
 *  - the blend sums the slots in slot order, then adds the shared term;
 *  - GeGLU ("helpers_a.rs", set_gelu_activation: the expert activation
 *    kernel becomes gelu_mul) is gelu(gate) * up with the exact GELU,
 *    gelu(v) = v * Phi(v) = v/2 * (1 + erf(v / sqrt 2)); the page names no
 *    approximation.  It applies to the routed and the shared expert alike;
 *  - the pre-expert norm ("helpers_a.rs", set_pre_expert_norm: the router
 *    reads the input as it is, the experts read it normed with the norm
 *    weight) is the RMS norm xe = x * w / sqrt(mean(x^2) + eps) of each row,
 *    stored in the activation format (rounded to nearest, ties to even) as
 *    the experts' input; the routed experts (through the weight placement)
 *    and the shared expert read xe, the router and the shared-expert gate
 *    read x;
 *  - the sqrt-softplus router ("refactor(gemm): split the gemv_q8 grab-bag by
 *    family", commit message: router_sqrtsoftplus among the routers, next to
 *    the biased router that selects by the biased score and weights by the
 *    unbiased one) scores an expert s = sqrt(softplus(l)), softplus(l) =
 *    log(1 + e^l); it selects by s + bias when an expert bias is given, else
 *    by s -- taken as the logit, which s orders the same way -- and weights
 *    a slot by its unbiased s (then norm_topk_prob and routed_scaling_factor
 *    as for the other routers);
 *  - the router pre-norm ("forward_bf16_grouped_decode.rs", the predicate
 *    refuses weights.router_pre_norm: a norm the router's input goes through)
 *    is the RMS norm of each row with its own weight router_norm_w, stored in
 *    the activation format like the pre-expert norm, with the same eps; only
 *    the router's logits read it -- the experts, the shared expert and the
 *    shared-expert gate read the row as it is (or, for the experts and the
 *    shared expert, the pre-expert norm);
 *  - NVFP4 weights are the NVIDIA NVFP4 encoding the page names: E2M1 codes,
 *    one E4M3 block scale per 16 elements along K, times the projection's
 *    fp32 second-level scale; the activations stay in their own format
 *    (weight-only dequantisation; the page's input_scale, which quantises
 *    activations for a 4-bit GEMM, has no part in it);
 *  - FP8 weights ("forward_bf16_grouped_decode.rs": the grouped decode
 *    dispatch serves NVFP4, then FP8, then BF16 experts, the FP8 one in its
 *    own forward_fp8_grouped_decode; the page fixes neither the encoding nor
 *    the scales) are OCP FP8 E4M3 codes, one byte per element in the [N, K]
 *    order of the other formats, with one fp32 scale per 128 x 128 block of
 *    the projection (row-major [ceil(N/128), ceil(K/128)], the last blocks
 *    ragged): the value is E4M3(code) * scale.  E4M3 is the FP8 weight
 *    encoding of block-scaled checkpoints and 128 x 128 their usual block;
 *    the activations stay in their own format (weight-only dequantisation).
 */
#include "moe_oracle.h"

#include <math.h>
#include <omp.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- decode */

static double bf16_value(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

double orc_decode_act(int32_t fmt, const void *p, int64_t i) {
  if (fmt == ORC_F32) return (double)((const float *)p)[i];
  return bf16_value(((const uint16_t *)p)[i]);
}

/* OCP MX E2M1: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0;
 * exponent 0 is subnormal (0 or 0.5). */
static double e2m1_value(unsigned code) {
  double sign = (code & 8u) ? -1.0 : 1.0;
  unsigned ex = (code >> 1) & 3u, man = code & 1u;
  double mag = ex == 0 ? 0.5 * man : ldexp(1.0 + 0.5 * man, (int)ex - 1);
  return sign * mag;
}

/* OCP MX E8M0 scale: 2^(e - 127). */
static double e8m0_value(uint8_t e) { return ldexp(1.0, (int)e - 127); }

/* OCP FP8 E4M3 (the "FN" variant: no infinities): sign bit 7, exponent
 * bits 6..3 (bias 7), mantissa bits 2..0; exponent 0 is subnormal
 * (mantissa/8 * 2^-6); exponent and mantissa all ones is NaN. */
double orc_e4m3_value(uint8_t b) {
  double sign = (b & 0x80u) ? -1.0 : 1.0;
  unsigned ex = (b >> 3) & 15u, man = b & 7u;
  if (ex == 15u && man == 7u) return NAN;
  double mag = ex == 0 ? ldexp((double)man / 8.0, -6) : ldexp(1.0 + (double)man / 8.0, (int)ex - 7);
  return sign * mag;
}

/* The 4-bit code of element k of row n of a packed [N, K/2] array: element
 * 2t in the low nibble of byte t. */
static unsigned nibble(const uint8_t *packed, int32_t K, int32_t n, int32_t k) {
  uint8_t byte = packed[(size_t)n * (K / 2) + k / 2];
  return (k & 1) ? (byte >> 4) : (byte & 15u);
}

void orc_decode_row(int32_t fmt, const void *w, const void *s, const void *b,
                    int32_t K, int32_t n, double *out) {
  for (int32_t k = 0; k < K; ++k) {
    switch (fmt) {
      case ORC_F32:
        out[k] = (double)((const float *)w)[(size_t)n * K + k];
        break;
      case ORC_BF16:
        out[k] = bf16_value(((const uint16_t *)w)[(size_t)n * K + k]);
        break;
      case ORC_AFF4: { /* value = scale * q + bias, one bf16 scale/bias per 64 */
        size_t g = (size_t)n * (K / 64) + k / 64;
        double sc = bf16_value(((const uint16_t *)s)[g]);
        double bi = bf16_value(((const uint16_t *)b)[g]);
        out[k] = sc * (double)nibble((const uint8_t *)w, K, n, k) + bi;
        break;
      }
      case ORC_MXFP4: { /* value = E2M1(code) * 2^(e-127), one E8M0 per 32 */
        size_t g = (size_t)n * (K / 32) + k / 32;
        out[k] = e2m1_value(nibble((const uint8_t *)w, K, n, k)) *
                 e8m0_value(((const uint8_t *)s)[g]);
        break;
      }
      case ORC_NVFP4: { /* value = E2M1(code) * E4M3(s) * s2, one E4M3 per 16 */
        size_t g = (size_t)n * (K / 16) + k / 16;
        out[k] = e2m1_value(nibble((const uint8_t *)w, K, n, k)) *
                 orc_e4m3_value(((const uint8_t *)s)[g]) * (double)*(const float *)b;
        break;
      }
      case ORC_FP8: { /* value = E4M3(code) * scale, one fp32 scale per 128 x 128 */
        size_t g = (size_t)(n / 128) * (size_t)((K + 127) / 128) + (size_t)(k / 128);
        out[k] = orc_e4m3_value(((const uint8_t *)w)[(size_t)n * K + k]) * (double)((const float *)s)[g];
        break;
      }
      default:
        out[k] = NAN;
    }
  }
}

/* A double rounded to the activation format: float32 (to nearest), or bf16
 * to nearest, ties to even.  bf16 keeps float32's exponent range with 8
 * significant bits: the spacing of the values in [2^(e-1), 2^e) is 2^(e-8),
 * and below the smallest normal 2^-126 the subnormals keep the spacing
 * 2^-133 of the lowest binade; a result past the largest finite value
 * (2^128 - 2^120) rounds to infinity. */
double orc_round_act(int32_t fmt, double v) {
  if (fmt == ORC_F32) return (double)(float)v;
  if (v == 0.0 || !isfinite(v)) return v;
  int e;
  frexp(v, &e);                          /* |v| in [2^(e-1), 2^e) */
  if (e < -125) e = -125;                /* subnormal: the spacing of [2^-126, 2^-125) */
  const double quantum = ldexp(1.0, e - 8);
  const double r = nearbyint(v / quantum) * quantum; /* default rounding: to nearest, ties to even */
  return fabs(r) >= ldexp(1.0, 128) ? copysign(INFINITY, v) : r;
}

/* "helpers_a.rs", set_pre_expert_norm: one row's expert input, the RMS norm
 * x * w / sqrt(mean(x^2) + eps) in the activation format.  With the router's
 * weight it is also the router pre-norm. */
void orc_pre_expert_norm(const orc_desc *d, const void *norm_w, const double *x, double *xe) {
  const int32_t H = d->hidden;
  double ss = 0.0;
  for (int32_t h = 0; h < H; ++h) ss += x[h] * x[h];
  const double inv = 1.0 / sqrt(ss / (double)H + d->norm_eps);
  for (int32_t h = 0; h < H; ++h)
    xe[h] = orc_round_act(d->act_fmt, x[h] * orc_decode_act(d->act_fmt, norm_w, h) * inv);
}

/* Threads over output neurons (OpenMP).  Each neuron's dot product is taken
 * by one thread in the order of the definition, so the results do not depend
 * on the thread count; 1 unless orc_set_threads says otherwise. */
static int g_threads = 1;

void orc_set_threads(int32_t n) { g_threads = n < 1 ? 1 : n; }

int32_t orc_get_threads(void) { return g_threads; }

/* ------------------------------------------------------------ small math */

static double dot(const double *a, const double *b, int32_t n) {
  double acc = 0.0;
  for (int32_t i = 0; i < n; ++i) acc += a[i] * b[i];
  return acc;
}

static double sigmoid(double v) { return 1.0 / (1.0 + exp(-v)); }

static double silu(double v) { return v / (1.0 + exp(-v)); }

/* GELU, exact: v * Phi(v) with Phi the standard normal distribution. */
static double gelu(double v) { return 0.5 * v * (1.0 + erf(v / sqrt(2.0))); }

/* ------------------------------------------------------- routing (S1-S3) */

/* "routed_weight_site.rs", fn routed_slot: the slot's input and the weight
 * its output carries -- (x, w) when the weight sits on the output, (w*x, 1)
 * when it sits on the input. */
void orc_routed_slot(const double *x, int32_t n, double w, int32_t before_ffn,
                     double *x_out, double *w_out) {
  if (before_ffn) {
    for (int32_t i = 0; i < n; ++i) x_out[i] = w * x[i];
    *w_out = 1.0;
  } else {
    for (int32_t i = 0; i < n; ++i) x_out[i] = x[i];
    *w_out = w;
  }
}

/* "forward_bf16_grouped_decode.rs": the per-row router GEMV,
 * logits[e] = sum_h x[h] * Wr[e, h], of a decoded row x[H]. */
static void router_logits(const orc_desc *d, const orc_weights *wt, const double *x, double *logits) {
  const int32_t H = d->hidden;
#pragma omp parallel for num_threads(g_threads) schedule(static)
  for (int32_t e = 0; e < d->num_experts; ++e) {
    double acc = 0.0;
    for (int32_t h = 0; h < H; ++h) acc += x[h] * orc_decode_act(d->act_fmt, wt->router, (int64_t)e * H + h);
    logits[e] = acc;
  }
}

void orc_router_logits(const orc_desc *d, const orc_weights *wt, const void *x_row,
                       double *logits) {
  double *x = (double *)malloc(sizeof(double) * (size_t)d->hidden);
  for (int32_t h = 0; h < d->hidden; ++h) x[h] = orc_decode_act(d->act_fmt, x_row, h);
  router_logits(d, wt, x, logits);
  free(x);
}

/* softplus(l) = log(1 + e^l), taken as l + log(1 + e^-l) for l > 0 so that
 * e^l never overflows; the score is its square root. */
double orc_sqrtsoftplus(double l) {
  const double sp = l > 0.0 ? l + log1p(exp(-l)) : log1p(exp(l));
  return sqrt(sp);
}

/* Selection key of expert e.  Softmax: the logit (same order as the
 * probability).  Sigmoid with bias ("wire lfm2" Summary; iron #24 commit:
 * select by the biased score): sigmoid(logit) + bias.  Raw-logit sigmoid
 * ("routed_weight_site.rs" module doc: top-k on the raw logits, a monotone
 * map of the sigmoid): the logit.  Sqrt-softplus: the score plus the bias
 * when one is given; without one, the logit (the score is strictly
 * increasing in it: the same order, with no rounding of the score to tie
 * two different logits). */
static double select_key(const orc_desc *d, const float *bias, const double *l, int32_t e) {
  if (d->routing == ORC_SIGMOID_BIAS) return sigmoid(l[e]) + (double)bias[e];
  if (d->routing == ORC_SQRTSOFTPLUS && bias) return orc_sqrtsoftplus(l[e]) + (double)bias[e];
  return l[e];
}

/* The n largest keys in order: key descending, ties to the lower index. */
static void top_n(const double *key, int32_t E, int32_t n, int32_t *out, unsigned char *taken) {
  memset(taken, 0, (size_t)E);
  for (int32_t j = 0; j < n; ++j) {
    int32_t best = -1;
    for (int32_t e = 0; e < E; ++e)
      if (!taken[e] && (best < 0 || key[e] > key[best])) best = e;
    out[j] = best;
    taken[best] = 1;
  }
}

void orc_select(const orc_desc *d, const float *expert_bias, const double *logits,
                int32_t *idx, double *w, double *margin) {
  const int32_t E = d->num_experts, k = d->top_k;
  double *key = (double *)malloc(sizeof(double) * (size_t)E);
  int32_t *order = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
  unsigned char *taken = (unsigned char *)malloc((size_t)E);
  for (int32_t e = 0; e < E; ++e) key[e] = select_key(d, expert_bias, logits, e);
  const int32_t n = k < E ? k + 1 : E;
  top_n(key, E, n, order, taken);
  for (int32_t j = 0; j < k; ++j) idx[j] = order[j];
  if (margin) {
    double mg = INFINITY;
    for (int32_t j = 0; j + 1 < n; ++j) {
      double gap = key[order[j]] - key[order[j + 1]];
      if (gap < mg) mg = gap;
    }
    *margin = mg;
  }

  if (d->routing == ORC_SOFTMAX) {
    /* p = softmax(logits) over all experts; the slot weight is p of its
     * expert. */
    double lmax = logits[0];
    for (int32_t e = 1; e < E; ++e)
      if (logits[e] > lmax) lmax = logits[e];
    double den = 0.0;
    for (int32_t e = 0; e < E; ++e) den += exp(logits[e] - lmax);
    for (int32_t j = 0; j < k; ++j) w[j] = exp(logits[idx[j]] - lmax) / den;
  } else if (d->routing == ORC_SQRTSOFTPLUS) {
    /* The unbiased score of the selected expert. */
    for (int32_t j = 0; j < k; ++j) w[j] = orc_sqrtsoftplus(logits[idx[j]]);
  } else {
    /* Both sigmoid modes weight by the unbiased sigmoid of the logit. */
    for (int32_t j = 0; j < k; ++j) w[j] = sigmoid(logits[idx[j]]);
  }
  if (d->norm_topk) { /* norm_topk_prob: divide by the selected weights' sum */
    double s = 0.0;
    for (int32_t j = 0; j < k; ++j) s += w[j];
    for (int32_t j = 0; j < k; ++j) w[j] = w[j] / s;
  }
  for (int32_t j = 0; j < k; ++j) w[j] = w[j] * d->routed_scaling_factor;
  free(key);
  free(order);
  free(taken);
}

/* "forward_bf16_grouped_decode.rs", the sort step (moe_fp8_grouped_sort and
 * its outputs: sorted ids, per-expert offsets, the pair -> position map and
 * the list and count of active experts): a stable counting sort of the pairs
 * p = r*k + j by expert. */
void orc_sort_pairs(int32_t m, int32_t k, int32_t E, const int32_t *idx,
                    int32_t *sorted_pair, int32_t *expert_offsets,
                    int32_t *pair_to_perm, int32_t *active_experts,
                    int32_t *active_count) {
  const int32_t te = m * k;
  int32_t *fill = (int32_t *)calloc((size_t)E + 1, sizeof(int32_t));
  for (int32_t e = 0; e <= E; ++e) expert_offsets[e] = 0;
  for (int32_t p = 0; p < te; ++p) expert_offsets[idx[p] + 1] += 1;
  for (int32_t e = 0; e < E; ++e) expert_offsets[e + 1] += expert_offsets[e];
  for (int32_t p = 0; p < te; ++p) {
    int32_t e = idx[p];
    int32_t pos = expert_offsets[e] + fill[e]++;
    sorted_pair[pos] = p;
    pair_to_perm[p] = pos;
  }
  int32_t na = 0;
  for (int32_t e = 0; e < E; ++e)
    if (expert_offsets[e + 1] > expert_offsets[e]) active_experts[na++] = e;
  *active_count = na;
  free(fill);
}

/* ----------------------------------------------------- expert FFN (S4-S5) */

/* One gated expert: y = down( act(gate u) * (up u) ), act = silu, or gelu
 * with geglu (GeGLU).  Each projection is
 * row-major [N, K]; gate/up have (N, K) = (I, H), down (H, I). */
static void swiglu_expert(int32_t fmt, int32_t geglu, const void *gw, const void *gs, const void *gb,
                          const void *uw, const void *us, const void *ub,
                          const void *dw, const void *ds, const void *db,
                          int32_t H, int32_t I, const double *u, double *y, double *act) {
#pragma omp parallel num_threads(g_threads)
  {
    double *row = (double *)malloc(sizeof(double) * (size_t)(H > I ? H : I));
#pragma omp for schedule(static)
    for (int32_t i = 0; i < I; ++i) {
      orc_decode_row(fmt, gw, gs, gb, H, i, row);
      double g = dot(row, u, H);
      orc_decode_row(fmt, uw, us, ub, H, i, row);
      double v = dot(row, u, H);
      act[i] = (geglu ? gelu(g) : silu(g)) * v;
    }
#pragma omp for schedule(static)
    for (int32_t h = 0; h < H; ++h) {
      orc_decode_row(fmt, dw, ds, db, I, h, row);
      y[h] = dot(row, act, I);
    }
    free(row);
  }
}

static const void *tbl(const void *const *t, int32_t e) { return t ? t[e] : NULL; }

static int valid_desc(const orc_desc *d) {
  if (d->hidden <= 0 || d->num_experts <= 0 || d->inter <= 0) return 0;
  if (d->top_k <= 0 || d->top_k > d->num_experts) return 0;
  if (d->act_fmt != ORC_F32 && d->act_fmt != ORC_BF16) return 0;
  if (d->expert_fmt < ORC_F32 || d->expert_fmt > ORC_FP8) return 0;
  if (d->routing < ORC_SOFTMAX || d->routing > ORC_SQRTSOFTPLUS) return 0;
  if (d->expert_fmt == ORC_AFF4 && (d->hidden % 64 || d->inter % 64)) return 0;
  if (d->expert_fmt == ORC_MXFP4 && (d->hidden % 32 || d->inter % 32)) return 0;
  if (d->expert_fmt == ORC_NVFP4 && (d->hidden % 16 || d->inter % 16)) return 0;
  if (d->shared && d->shared_inter <= 0) return 0;
  if ((d->pre_norm || d->router_pre_norm) && !(d->norm_eps >= 0.0)) return 0;
  return 1;
}

int32_t orc_forward(const orc_desc *d, const orc_weights *wt, const void *x, int32_t m,
                    double *out, int32_t *idx, double *w, double *logits, double *margin) {
  if (!valid_desc(d) || m < 0) return -1;
  const int32_t H = d->hidden, E = d->num_experts, k = d->top_k, I = d->inter;
  const int32_t Is = d->shared ? d->shared_inter : 0;
  double *xr = (double *)malloc(sizeof(double) * (size_t)H);
  double *xe = (double *)malloc(sizeof(double) * (size_t)H);   /* the experts' input */
  double *xn = (double *)malloc(sizeof(double) * (size_t)H);   /* the router's input */
  double *u = (double *)malloc(sizeof(double) * (size_t)H);
  double *y = (double *)malloc(sizeof(double) * (size_t)H);
  double *acc = (double *)malloc(sizeof(double) * (size_t)H);
  double *act = (double *)malloc(sizeof(double) * (size_t)(I > Is ? I : Is));
  double *lg = (double *)malloc(sizeof(double) * (size_t)E);
  int32_t *sel = (int32_t *)malloc(sizeof(int32_t) * (size_t)k);
  double *sw = (double *)malloc(sizeof(double) * (size_t)k);

  for (int32_t r = 0; r < m; ++r) {
    /* Each row on its own: the result of a row does not depend on m. */
    const char *xrow = (const char *)x + (size_t)r * H * (d->act_fmt == ORC_F32 ? 4 : 2);
    for (int32_t h = 0; h < H; ++h) xr[h] = orc_decode_act(d->act_fmt, xrow, h);
    if (d->pre_norm)
      orc_pre_expert_norm(d, wt->pre_norm_w, xr, xe);
    else
      for (int32_t h = 0; h < H; ++h) xe[h] = xr[h];
    if (d->router_pre_norm)
      orc_pre_expert_norm(d, wt->router_norm_w, xr, xn);   /* the same RMS norm, the router's weight */
    else
      for (int32_t h = 0; h < H; ++h) xn[h] = xr[h];
    router_logits(d, wt, xn, lg);
    orc_select(d, wt->expert_bias, lg, sel, sw, margin ? &margin[r] : NULL);
    if (idx)
      for (int32_t j = 0; j < k; ++j) idx[(size_t)r * k + j] = sel[j];
    if (w)
      for (int32_t j = 0; j < k; ++j) w[(size_t)r * k + j] = sw[j];
    if (logits)
      for (int32_t e = 0; e < E; ++e) logits[(size_t)r * E + e] = lg[e];

    for (int32_t h = 0; h < H; ++h) acc[h] = 0.0;
    for (int32_t j = 0; j < k; ++j) {
      const int32_t e = sel[j];
      double c;
      orc_routed_slot(xe, H, sw[j], d->weight_before_ffn, u, &c);
      swiglu_expert(d->expert_fmt, d->geglu, wt->gate[e], tbl(wt->gate_s, e), tbl(wt->gate_b, e),
                    wt->up[e], tbl(wt->up_s, e), tbl(wt->up_b, e), wt->down[e],
                    tbl(wt->down_s, e), tbl(wt->down_b, e), H, I, u, y, act);
      for (int32_t h = 0; h < H; ++h) acc[h] += c * y[h];
    }
    if (d->shared) {
      /* Shared expert on the unscaled row, times its gate sigmoid(x . w_g)
       * when gated (the blend of "forward_bf16_grouped_decode.rs" takes the
       * input and the shared-expert gate weight). */
      double gamma = 1.0;
      if (d->shared_gated) {
        double s = 0.0;
        for (int32_t h = 0; h < H; ++h)
          s += xr[h] * orc_decode_act(d->act_fmt, wt->sh_gate_vec, h);
        gamma = sigmoid(s);
      }
      swiglu_expert(d->act_fmt, d->geglu, wt->sh_gate, NULL, NULL, wt->sh_up, NULL, NULL,
                    wt->sh_down, NULL, NULL, H, Is, xe, y, act);
      for (int32_t h = 0; h < H; ++h) acc[h] += gamma * y[h];
    }
    for (int32_t h = 0; h < H; ++h) out[(size_t)r * H + h] = acc[h];
  }
  free(xr); free(xe); free(xn); free(u); free(y); free(acc); free(act); free(lg); free(sel); free(sw);
  return 0;
}
