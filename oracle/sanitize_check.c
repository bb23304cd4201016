/*
 * sanitize_check.c -- drives the oracle under AddressSanitizer and
 * UndefinedBehaviorSanitizer (test infrastructure, CPU only).
 *
 * Built by tests/test_sanitizers.py with moe_oracle.c:
 *   gcc -std=c11 -g -O1 -fsanitize=address,undefined -fno-sanitize-recover=all
 *       -fno-omit-frame-pointer -fopenmp sanitize_check.c moe_oracle.c -lm
 * Every array is allocated at its exact size (no padding), so an access one
 * element past any of them is reported.  It runs every expert format,
 * routing mode and feature flag on small random layers with ragged shapes
 * and the largest k; prints "ok" and exits 0 when nothing was reported.
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "moe_oracle.h"

static unsigned long long g_state = 0x9E3779B97F4A7C15ull;
static unsigned rnd(void) {   /* xorshift64* */
  g_state ^= g_state >> 12;
  g_state ^= g_state << 25;
  g_state ^= g_state >> 27;
  return (unsigned)((g_state * 0x2545F4914F6CDD1Dull) >> 32);
}
static float frnd(float scale) { return scale * ((float)(rnd() & 0xFFFF) / 32768.0f - 1.0f); }

static uint16_t bf16_bits(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

/* An act-format array of n values (f32 or bf16 bits), exactly sized. */
static void *act_array(int32_t fmt, size_t n, float scale) {
  if (fmt == ORC_F32) {
    float *p = malloc(n * sizeof *p);
    for (size_t i = 0; i < n; ++i) p[i] = frnd(scale);
    return p;
  }
  uint16_t *p = malloc(n * sizeof *p);
  for (size_t i = 0; i < n; ++i) p[i] = bf16_bits(frnd(scale));
  return p;
}

/* Byte array of n random bytes; fp8 and nvfp4 scale bytes avoid the E4M3 NaN codes. */
static uint8_t *bytes(size_t n, int e4m3) {
  uint8_t *p = malloc(n);
  for (size_t i = 0; i < n; ++i) {
    p[i] = (uint8_t)rnd();
    if (e4m3 && (p[i] & 0x7Fu) == 0x7Fu) p[i] = 0x38;
  }
  return p;
}

typedef struct {
  void *w, *s, *b;
} proj;

/* One [N, K] projection in format fmt, every array exactly sized. */
static proj make_proj(int32_t fmt, int32_t N, int32_t K) {
  proj p = {NULL, NULL, NULL};
  const size_t nk = (size_t)N * K;
  switch (fmt) {
    case ORC_F32:
    case ORC_BF16:
      p.w = act_array(fmt, nk, 0.1f);
      break;
    case ORC_AFF4: {
      p.w = bytes(nk / 2, 0);
      uint16_t *s = malloc((nk / 64) * sizeof *s), *b = malloc((nk / 64) * sizeof *b);
      for (size_t i = 0; i < nk / 64; ++i) {
        s[i] = bf16_bits(0.01f + 0.01f * (float)(rnd() & 7));
        b[i] = bf16_bits(frnd(0.05f));
      }
      p.s = s;
      p.b = b;
      break;
    }
    case ORC_MXFP4: {
      p.w = bytes(nk / 2, 0);
      uint8_t *s = malloc(nk / 32);
      for (size_t i = 0; i < nk / 32; ++i) s[i] = (uint8_t)(120 + (rnd() & 7));
      p.s = s;
      break;
    }
    case ORC_NVFP4: {
      p.w = bytes(nk / 2, 0);
      p.s = bytes(nk / 16, 1);
      float *s2 = malloc(sizeof *s2);
      *s2 = 0.01f;
      p.b = s2;
      break;
    }
    case ORC_FP8: {
      p.w = bytes(nk, 1);
      const size_t nb = (size_t)((N + 127) / 128) * (size_t)((K + 127) / 128);
      float *s = malloc(nb * sizeof *s);
      for (size_t i = 0; i < nb; ++i) s[i] = 0.001f * (float)(1 + (rnd() & 3));
      p.s = s;
      break;
    }
  }
  return p;
}

static void free_proj(proj p) {
  free(p.w);
  free(p.s);
  free(p.b);
}

static int run_case(int32_t act, int32_t fmt, int32_t routing, int32_t flags_bits, int32_t H, int32_t E,
                    int32_t k, int32_t I, int32_t Is, int32_t m) {
  orc_desc d;
  memset(&d, 0, sizeof d);
  d.hidden = H;
  d.num_experts = E;
  d.top_k = k;
  d.inter = I;
  d.shared_inter = Is;
  d.act_fmt = act;
  d.expert_fmt = fmt;
  d.routing = routing;
  d.norm_topk = flags_bits & 1;
  d.weight_before_ffn = (flags_bits >> 1) & 1;
  d.shared = Is > 0;
  d.shared_gated = Is > 0 && ((flags_bits >> 2) & 1);
  d.routed_scaling_factor = 1.25;
  d.geglu = (flags_bits >> 3) & 1;
  d.pre_norm = (flags_bits >> 4) & 1;
  d.router_pre_norm = (flags_bits >> 5) & 1;
  d.norm_eps = 1e-6;
  const int biased = routing == ORC_SIGMOID_BIAS || (routing == ORC_SQRTSOFTPLUS && ((flags_bits >> 6) & 1));

  orc_weights wt;
  memset(&wt, 0, sizeof wt);
  void *router = act_array(act, (size_t)E * H, 0.1f);
  float *bias = NULL;
  if (biased) {
    bias = malloc((size_t)E * sizeof *bias);
    for (int32_t e = 0; e < E; ++e) bias[e] = frnd(0.1f);
  }
  proj *g = malloc((size_t)E * sizeof *g), *u = malloc((size_t)E * sizeof *u), *dn = malloc((size_t)E * sizeof *dn);
  const void **tg = malloc((size_t)E * sizeof *tg), **tu = malloc((size_t)E * sizeof *tu),
             **td = malloc((size_t)E * sizeof *td);
  const void **tgs = malloc((size_t)E * sizeof *tgs), **tus = malloc((size_t)E * sizeof *tus),
             **tds = malloc((size_t)E * sizeof *tds);
  const void **tgb = malloc((size_t)E * sizeof *tgb), **tub = malloc((size_t)E * sizeof *tub),
             **tdb = malloc((size_t)E * sizeof *tdb);
  for (int32_t e = 0; e < E; ++e) {
    g[e] = make_proj(fmt, I, H);
    u[e] = make_proj(fmt, I, H);
    dn[e] = make_proj(fmt, H, I);
    tg[e] = g[e].w; tu[e] = u[e].w; td[e] = dn[e].w;
    tgs[e] = g[e].s; tus[e] = u[e].s; tds[e] = dn[e].s;
    tgb[e] = g[e].b; tub[e] = u[e].b; tdb[e] = dn[e].b;
  }
  wt.router = router;
  wt.expert_bias = bias;
  wt.gate = tg; wt.up = tu; wt.down = td;
  wt.gate_s = tgs; wt.up_s = tus; wt.down_s = tds;
  wt.gate_b = tgb; wt.up_b = tub; wt.down_b = tdb;
  void *sg = NULL, *su = NULL, *sd = NULL, *sv = NULL, *pn = NULL, *rn = NULL;
  if (Is > 0) {
    sg = act_array(act, (size_t)Is * H, 0.1f);
    su = act_array(act, (size_t)Is * H, 0.1f);
    sd = act_array(act, (size_t)H * Is, 0.1f);
    if (d.shared_gated) sv = act_array(act, (size_t)H, 0.1f);
  }
  if (d.pre_norm) pn = act_array(act, (size_t)H, 1.0f);
  if (d.router_pre_norm) rn = act_array(act, (size_t)H, 1.0f);
  wt.sh_gate = sg; wt.sh_up = su; wt.sh_down = sd; wt.sh_gate_vec = sv;
  wt.pre_norm_w = pn;
  wt.router_norm_w = rn;

  void *x = act_array(act, (size_t)m * H, 1.0f);
  double *out = malloc((size_t)m * H * sizeof *out);
  int32_t *idx = malloc((size_t)m * k * sizeof *idx);
  double *w = malloc((size_t)m * k * sizeof *w);
  double *logits = malloc((size_t)m * (E + 1) * sizeof *logits);
  double *margin = malloc((size_t)m * sizeof *margin);
  int rc = orc_forward(&d, &wt, x, m, out, idx, w, logits, margin);
  int bad = rc != 0;
  for (size_t i = 0; i < (size_t)m * H && !bad; ++i) bad = !isfinite(out[i]);
  /* The sort of the selection, into exactly sized arrays. */
  const int32_t te = m * k, cap = te < E ? te : E;
  int32_t *sp = malloc((size_t)te * sizeof *sp), *off = malloc((size_t)(E + 1) * sizeof *off);
  int32_t *p2p = malloc((size_t)te * sizeof *p2p), *act_e = malloc((size_t)cap * sizeof *act_e), cnt = 0;
  if (!bad) orc_sort_pairs(m, k, E, idx, sp, off, p2p, act_e, &cnt);
  if (!bad) bad = cnt < 1 || cnt > cap;

  free(sp); free(off); free(p2p); free(act_e);
  free(x); free(out); free(idx); free(w); free(logits); free(margin);
  free(sg); free(su); free(sd); free(sv); free(pn); free(rn);
  for (int32_t e = 0; e < E; ++e) {
    free_proj(g[e]);
    free_proj(u[e]);
    free_proj(dn[e]);
  }
  free(g); free(u); free(dn);
  free(tg); free(tu); free(td); free(tgs); free(tus); free(tds); free(tgb); free(tub); free(tdb);
  free(router);
  free(bias);
  if (bad) fprintf(stderr, "case act=%d fmt=%d routing=%d flags=%d failed (rc %d)\n", act, fmt, routing, flags_bits, rc);
  return bad;
}

int main(void) {
  int bad = 0, cases = 0;
  for (int32_t act = ORC_F32; act <= ORC_BF16; ++act)
    for (int32_t fmt = ORC_F32; fmt <= ORC_FP8; ++fmt)
      for (int32_t routing = ORC_SOFTMAX; routing <= ORC_SQRTSOFTPLUS; ++routing) {
        /* Shapes each format accepts; fp8 with ragged 128-blocks. */
        const int32_t H = fmt == ORC_FP8 ? 192 : 128, I = fmt == ORC_FP8 ? 160 : 64;
        const int32_t flags = (int32_t)(rnd() & 127u);
        bad |= run_case(act, fmt, routing, flags, H, 7, 3, I, 32, 3);
        bad |= run_case(act, fmt, routing, flags ^ 127, H, 16, 16, I, 0, 2);   /* k = E = 16 */
        cases += 2;
      }
  orc_set_threads(3);
  bad |= run_case(ORC_BF16, ORC_MXFP4, ORC_SOFTMAX, 0x3F, 128, 9, 4, 64, 64, 5);
  ++cases;
  /* Single values at their edges. */
  for (int b = 0; b < 256; ++b) (void)orc_e4m3_value((uint8_t)b);
  (void)orc_round_act(ORC_BF16, 3.0e38);
  (void)orc_round_act(ORC_BF16, 1e-45);
  (void)orc_sqrtsoftplus(-800.0);
  (void)orc_sqrtsoftplus(800.0);
  if (bad) return 1;
  printf("ok: %d cases\n", cases);
  return 0;
}
