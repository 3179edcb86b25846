/*
 * moe_oracle.c - plain, slow, single-threaded CPU oracle of the MoE decode
 * layer. TEST INFRASTRUCTURE ONLY: only the tests, the smoke check and the
 * benchmark's CPU-baseline leg call it; libmoedecode never does, and the two
 * share no code.
 *
 * The layer's parts are named in the pages (decode = normalisation, matmul,
 * activation, routing: openai-hub.com "Kimi K3 ... 1.68x", section on why
 * decode suits a megakernel; router scores and a shared expert: smzdm.com post,
 * section "what changed", MoE de-duplication item; 16 of 896 experts per
 * token: aiposthub.com article, section on what the K3 decode path changed).
 * The formula and rounding points are the readings recorded in the design doc;
 * every loop below is that definition written out, in double.
 *
 * Build: gcc -O2 -std=c11 -shared -fPIC moe_oracle.c -lm  (no -ffast-math, no threads)
 */
#include "moe_oracle.h"

#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>

#define ORC_EINVAL (-1)
#define ORC_EMISSING (-2)
#define ORC_ENOMEM (-3)

const char *orc_error_string(int code) {
  switch (code) {
    case 0: return "ok";
    case ORC_EINVAL: return "invalid argument";
    case ORC_EMISSING: return "a selected expert has no weights (NULL pointer)";
    case ORC_ENOMEM: return "out of host memory";
    default: return "unknown error";
  }
}

/* ---- number formats ---------------------------------------------------- */

/* bf16: the top 16 bits of an IEEE binary32. */
double orc_bf16_value(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* Round v to binary32 (the C conversion, nearest-even), then to bf16 with
 * round-to-nearest-even on the 16 dropped bits. NaN maps to a quiet NaN. */
uint16_t orc_bf16_round(double v) {
  float f = (float)v;
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  if (isnan(f)) return (uint16_t)(0x7FC0u | ((u >> 16) & 0x8000u));
  uint32_t hi = u >> 16, lo = u & 0xFFFFu;
  if (lo > 0x8000u || (lo == 0x8000u && (hi & 1u))) hi += 1u;  /* carry may reach the exponent: correct */
  return (uint16_t)hi;
}

/* OCP 8-bit E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits; exponent 0
 * is subnormal (m/8 * 2^-6); S.1111.111 is NaN; there is no infinity. */
double orc_e4m3_value(uint8_t code) {
  int s = code >> 7, e = (code >> 3) & 0xF, m = code & 7;
  if (e == 0xF && m == 7) return NAN;
  double mag = (e == 0) ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + (double)m / 8.0, e - 7);
  return s ? -mag : mag;
}

/* element i of an activation buffer (ORC_F32 or ORC_BF16) */
static double act_get(int32_t dtype, const void *p, size_t i) {
  if (dtype == ORC_BF16) return orc_bf16_value(((const uint16_t *)p)[i]);
  return (double)((const float *)p)[i];
}

static void act_put(int32_t dtype, void *p, size_t i, double v) {
  if (dtype == ORC_BF16) ((uint16_t *)p)[i] = orc_bf16_round(v);
  else ((float *)p)[i] = (float)v;
}

/* value of activation v once stored in the activation dtype */
static float act_round(int32_t dtype, double v) {
  if (dtype == ORC_BF16) return (float)orc_bf16_value(orc_bf16_round(v));
  return (float)v;
}

/* weight element (row, col) of a [rows][cols] matrix; fp8 rows share one bf16
 * scale per `group` rows, and e4m3 holds orc_e4m3_value of every code (a
 * lookup table of that function, filled by the caller) */
static double w_get(int32_t dtype, const void *p, const uint16_t *scale, int32_t group, size_t row,
                    size_t cols, size_t col, const double *e4m3) {
  size_t i = row * cols + col;
  switch (dtype) {
    case ORC_F32: return (double)((const float *)p)[i];
    case ORC_BF16: return orc_bf16_value(((const uint16_t *)p)[i]);
    default: return e4m3[((const uint8_t *)p)[i]] * orc_bf16_value(scale[row / (size_t)group]);
  }
}

static int desc_ok(const orc_desc *d) {
  if (!d) return 0;
  if (d->hidden <= 0 || d->num_experts <= 0 || d->top_k <= 0 || d->top_k > d->num_experts) return 0;
  if (d->expert_inter <= 0 || d->shared_inter < 0) return 0;
  if (d->act != ORC_F32 && d->act != ORC_BF16) return 0;
  if (d->router != ORC_F32 && d->router != ORC_BF16) return 0;
  if (d->shared != ORC_F32 && d->shared != ORC_BF16) return 0;
  if (d->expert != ORC_F32 && d->expert != ORC_BF16 && d->expert != ORC_FP8_E4M3) return 0;
  if (d->expert == ORC_FP8_E4M3) {
    if (d->scale_group <= 0) return 0;
    if ((2 * d->expert_inter) % d->scale_group || d->hidden % d->scale_group) return 0;
  }
  return 1;
}

/* ---- RMSNorm ----------------------------------------------------------- */

/* xhat[h] = x[h] / sqrt(mean(x^2) + eps) * gamma[h], rounded to float;
 * xact = xhat stored in the activation dtype (the FFNs' input). */
int orc_rmsnorm(const orc_desc *d, const void *x_t, const void *gamma, float *xhat, float *xact) {
  if (!desc_ok(d) || !x_t || !gamma || !xhat) return ORC_EINVAL;
  const int32_t H = d->hidden;
  double ss = 0.0;
  for (int32_t h = 0; h < H; ++h) {
    double v = act_get(d->act, x_t, (size_t)h);
    ss += v * v;
  }
  const double r = 1.0 / sqrt(ss / (double)H + (double)d->rms_eps);
  for (int32_t h = 0; h < H; ++h) {
    xhat[h] = (float)(act_get(d->act, x_t, (size_t)h) * r * act_get(d->act, gamma, (size_t)h));
    if (xact) xact[h] = act_round(d->act, (double)xhat[h]);
  }
  return 0;
}

/* ---- router ------------------------------------------------------------ */

/* logits[e] = float(sum_h Wr[e][h] * xhat[h]) + bias[e]; the router sees the
 * fp32 normalised input. */
int orc_router_logits(const orc_desc *d, const orc_weights *w, const float *xhat, float *logits) {
  if (!desc_ok(d) || !w || !w->router_w || !xhat || !logits) return ORC_EINVAL;
  const int32_t H = d->hidden, E = d->num_experts;
  for (int32_t e = 0; e < E; ++e) {
    double acc = 0.0;
    for (int32_t h = 0; h < H; ++h)
      acc += w_get(d->router, w->router_w, NULL, 1, (size_t)e, (size_t)H, (size_t)h, NULL) * (double)xhat[h];
    float l = (float)acc;
    if (w->router_bias) l = l + w->router_bias[e];
    logits[e] = l;
  }
  return 0;
}

/* a ranks before b: larger logit first, equal logits by lower index */
static int ranks_before(const float *l, int32_t a, int32_t b) {
  return l[a] > l[b] || (l[a] == l[b] && a < b);
}

/* Weights of a given selection S (k distinct experts, rank order): the
 * softmax over all E logits, restricted to S and renormalised to sum to one,
 * w_i = p_{S_i} / sum_j p_{S_j}. */
int orc_route_weights(const orc_desc *d, const float *logits, const int32_t *idx, float *wts) {
  if (!desc_ok(d) || !logits || !idx || !wts) return ORC_EINVAL;
  const int32_t E = d->num_experts, k = d->top_k;
  for (int32_t i = 0; i < k; ++i) {
    if (idx[i] < 0 || idx[i] >= E) return ORC_EINVAL;
    for (int32_t j = 0; j < i; ++j)
      if (idx[j] == idx[i]) return ORC_EINVAL;
  }
  double *p = (double *)malloc(sizeof(double) * (size_t)E);
  if (!p) return ORC_ENOMEM;
  double lmax = (double)logits[0];
  for (int32_t e = 1; e < E; ++e)
    if ((double)logits[e] > lmax) lmax = (double)logits[e];
  double z = 0.0;
  for (int32_t e = 0; e < E; ++e) { p[e] = exp((double)logits[e] - lmax); z += p[e]; }
  for (int32_t e = 0; e < E; ++e) p[e] /= z;
  double sel = 0.0;
  for (int32_t i = 0; i < k; ++i) sel += p[idx[i]];
  for (int32_t i = 0; i < k; ++i) wts[i] = (float)(p[idx[i]] / sel);
  free(p);
  return 0;
}

/* Top-k by logit (ties: lower index), in rank order, then the weights of that
 * selection (orc_route_weights). */
int orc_route(const orc_desc *d, const float *logits, int32_t *idx, float *wts) {
  if (!desc_ok(d) || !logits || !idx || !wts) return ORC_EINVAL;
  const int32_t E = d->num_experts, k = d->top_k;
  char *taken = (char *)calloc((size_t)E, 1);
  if (!taken) return ORC_ENOMEM;
  for (int32_t i = 0; i < k; ++i) {
    int32_t best = -1;
    for (int32_t e = 0; e < E; ++e)
      if (!taken[e] && (best < 0 || ranks_before(logits, e, best))) best = e;
    taken[best] = 1;
    idx[i] = best;
  }
  free(taken);
  return orc_route_weights(d, logits, idx, wts);
}

/* ---- SwiGLU FFN (routed or shared expert) ------------------------------- */

/* g[j] = float(sum_h Wgu[j][h] xact[h]), u[j] = float(sum_h Wgu[I+j][h] xact[h]),
 * h[j] = act(float(silu(g) * u)), silu(z) = z / (1 + e^-z),
 * d[o] = float(sum_j Wd[o][j] h[j]). h_out [I] and d_out [H] may be NULL. */
int orc_ffn(const orc_desc *dsc, int32_t dtype, int32_t inter, const void *gate_up, const void *down,
            const uint16_t *gate_up_scale, const uint16_t *down_scale, const float *xact,
            float *h_out, float *d_out) {
  if (!desc_ok(dsc) || !gate_up || !down || !xact || inter <= 0) return ORC_EINVAL;
  if (dtype == ORC_FP8_E4M3 && (!gate_up_scale || !down_scale)) return ORC_EINVAL;
  const int32_t H = dsc->hidden, G = dsc->scale_group;
  float *h = (float *)malloc(sizeof(float) * (size_t)inter);
  if (!h) return ORC_ENOMEM;
  double e4m3[256];
  for (int c = 0; c < 256; ++c) e4m3[c] = orc_e4m3_value((uint8_t)c);
  for (int32_t j = 0; j < inter; ++j) {
    double g = 0.0, u = 0.0;
    for (int32_t c = 0; c < H; ++c) {
      g += w_get(dtype, gate_up, gate_up_scale, G, (size_t)j, (size_t)H, (size_t)c, e4m3) * (double)xact[c];
      u += w_get(dtype, gate_up, gate_up_scale, G, (size_t)(inter + j), (size_t)H, (size_t)c, e4m3) * (double)xact[c];
    }
    const double gf = (double)(float)g, uf = (double)(float)u;
    const double silu = gf / (1.0 + exp(-gf));
    h[j] = act_round(dsc->act, (double)(float)(silu * uf));
    if (h_out) h_out[j] = h[j];
  }
  if (d_out) {
    for (int32_t o = 0; o < H; ++o) {
      double acc = 0.0;
      for (int32_t j = 0; j < inter; ++j)
        acc += w_get(dtype, down, down_scale, G, (size_t)o, (size_t)inter, (size_t)j, e4m3) * (double)h[j];
      d_out[o] = (float)acc;
    }
  }
  free(h);
  return 0;
}

/* ---- the layer --------------------------------------------------------- */

/* The rest of a token's layer once its selection (idx, wts) is fixed:
 * y = act(x + shared(xact) + sum_i wts_i expert_{idx_i}(xact)), the routed sum
 * in rank order. */
static int finish_token(const orc_desc *d, const orc_weights *w, const void *x_t, const float *xact,
                        const int32_t *idx, const float *wts, void *y_t) {
  const int32_t H = d->hidden, k = d->top_k;
  float *dv = (float *)malloc(sizeof(float) * (size_t)H);
  double *routed = (double *)calloc((size_t)H, sizeof(double));
  int rc = ORC_ENOMEM;
  if (!dv || !routed) goto done;

  /* routed experts: sum_i w_i * expert_{S_i}(xact), in rank order */
  for (int32_t i = 0; i < k; ++i) {
    const int32_t e = idx[i];
    if (!w->expert_gate_up || !w->expert_down || !w->expert_gate_up[e] || !w->expert_down[e]) {
      rc = ORC_EMISSING;
      goto done;
    }
    const uint16_t *gs = w->expert_gate_up_scale ? w->expert_gate_up_scale[e] : NULL;
    const uint16_t *ds = w->expert_down_scale ? w->expert_down_scale[e] : NULL;
    rc = orc_ffn(d, d->expert, d->expert_inter, w->expert_gate_up[e], w->expert_down[e], gs, ds, xact,
                 NULL, dv);
    if (rc) goto done;
    for (int32_t h = 0; h < H; ++h) routed[h] += (double)wts[i] * (double)dv[h];
  }

  /* shared expert (weight 1) and the residual */
  if (d->shared_inter > 0) {
    if (!w->shared_gate_up || !w->shared_down) { rc = ORC_EINVAL; goto done; }
    rc = orc_ffn(d, d->shared, d->shared_inter, w->shared_gate_up, w->shared_down, NULL, NULL, xact,
                 NULL, dv);
    if (rc) goto done;
  } else {
    for (int32_t h = 0; h < H; ++h) dv[h] = 0.0f;
  }
  for (int32_t h = 0; h < H; ++h) {
    double v = act_get(d->act, x_t, (size_t)h) + (double)dv[h] + routed[h];
    act_put(d->act, y_t, (size_t)h, (double)(float)v);
  }
  rc = 0;
done:
  free(dv); free(routed);
  return rc;
}

/* One token through the layer. With given != 0 the selection is the caller's
 * idx (k distinct experts in rank order) instead of the top-k; its weights are
 * still the restricted softmax of this token's logits. */
static int layer_token(const orc_desc *d, const orc_weights *w, const void *x_t, void *y_t, int32_t *idx,
                       float *wts, float *logits, int given) {
  if (!desc_ok(d) || !w || !x_t || !y_t || !idx || !wts) return ORC_EINVAL;
  const int32_t H = d->hidden, E = d->num_experts;
  float *xhat = (float *)malloc(sizeof(float) * (size_t)H);
  float *xact = (float *)malloc(sizeof(float) * (size_t)H);
  float *lg = (float *)malloc(sizeof(float) * (size_t)E);
  int rc = ORC_ENOMEM;
  if (!xhat || !xact || !lg) goto done;

  rc = orc_rmsnorm(d, x_t, w->rms_gamma, xhat, xact);
  if (rc) goto done;
  rc = orc_router_logits(d, w, xhat, lg);
  if (rc) goto done;
  rc = given ? orc_route_weights(d, lg, idx, wts) : orc_route(d, lg, idx, wts);
  if (rc) goto done;
  if (logits) memcpy(logits, lg, sizeof(float) * (size_t)E);
  rc = finish_token(d, w, x_t, xact, idx, wts, y_t);
done:
  free(xhat); free(xact); free(lg);
  return rc;
}

int orc_layer_token(const orc_desc *d, const orc_weights *w, const void *x_t, void *y_t,
                    int32_t *idx, float *wts, float *logits) {
  return layer_token(d, w, x_t, y_t, idx, wts, logits, 0);
}

int orc_layer_token_given(const orc_desc *d, const orc_weights *w, const void *x_t, const int32_t *idx,
                          void *y_t, float *wts, float *logits) {
  /* with given != 0, idx is only read */
  return layer_token(d, w, x_t, y_t, (int32_t *)idx, wts, logits, 1);
}

static size_t act_bytes(const orc_desc *d) { return d->act == ORC_BF16 ? 2u : 4u; }

int orc_layer(const orc_desc *d, const orc_weights *w, const void *x, int32_t B, void *y,
              int32_t *idx, float *wts, float *logits) {
  if (!desc_ok(d) || B < 0 || (B > 0 && (!x || !y || !idx || !wts))) return ORC_EINVAL;
  const size_t row = (size_t)d->hidden * act_bytes(d);
  for (int32_t t = 0; t < B; ++t) {
    int rc = orc_layer_token(d, w, (const char *)x + (size_t)t * row, (char *)y + (size_t)t * row,
                             idx + (size_t)t * d->top_k, wts + (size_t)t * d->top_k,
                             logits ? logits + (size_t)t * d->num_experts : NULL);
    if (rc) return rc;
  }
  return 0;
}

int orc_stack(const orc_desc *d, const orc_weights *layers, int32_t L, const void *x, int32_t B,
              void *y, int32_t *idx, float *wts, float *logits) {
  if (!desc_ok(d) || !layers || L < 1 || B < 0 || (B > 0 && (!x || !y || !idx || !wts)))
    return ORC_EINVAL;
  const size_t bytes = (size_t)B * (size_t)d->hidden * act_bytes(d);
  void *cur = malloc(bytes ? bytes : 1), *nxt = malloc(bytes ? bytes : 1);
  if (!cur || !nxt) { free(cur); free(nxt); return ORC_ENOMEM; }
  memcpy(cur, x, bytes);
  int rc = 0;
  for (int32_t l = 0; l < L && !rc; ++l) {
    const size_t sel = (size_t)l * (size_t)B * (size_t)d->top_k;
    rc = orc_layer(d, &layers[l], cur, B, nxt, idx + sel, wts + sel,
                   logits ? logits + (size_t)l * (size_t)B * (size_t)d->num_experts : NULL);
    void *t = cur; cur = nxt; nxt = t;
  }
  if (!rc) memcpy(y, cur, bytes);
  free(cur);
  free(nxt);
  return rc;
}
