/*
 * CPU oracle for the transformer decode step -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU baseline leg
 * may load this library.  It shares no code with the GPU engine.  Every
 * routine below is the plain definition of its operation in fp64 with a
 * single sequential accumulation order; OpenMP only splits independent
 * output rows (or heads, or positions) across threads, which leaves every
 * individual sum unchanged.  The readings taken where the pages are silent
 * are listed in oracle.h.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- scalar codecs --------------------------------------------------- */

double orc_bf16_to_double(uint16_t b) {
  /* bf16 is the top half of an IEEE binary32. */
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

uint16_t orc_float_to_bf16(float f) {
  /* Round to nearest, ties to even, on the 16 dropped bits. */
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu) != 0)
    return (uint16_t)((u >> 16) | 0x0040u); /* quiet NaN, sign kept */
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7fffu + lsb;
  return (uint16_t)(u >> 16);
}

double orc_fp8e4m3_to_double(uint8_t c) {
  /* OCP E4M3 ("fn"): 1 sign, 4 exponent (bias 7), 3 mantissa bits; no
   * infinities; S.1111.111 is NaN; exponent 0 is subnormal. */
  int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
  double v;
  if (e == 15 && m == 7)
    return NAN;
  if (e == 0)
    v = ldexp((double)m / 8.0, -6);
  else
    v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return s ? -v : v;
}

uint8_t orc_float_to_fp8e4m3(float x) {
  /* OCP E4M3: magnitudes below 2^-6 are subnormal multiples of 2^-9; above,
   * 3 mantissa bits under exponents -6..8; 448 = 1.75 * 2^8 is the largest
   * finite value (S.1111.111 is NaN). */
  if (isnan(x)) return 0x7F;
  uint8_t s = signbit(x) ? 0x80 : 0x00;
  float a = fabsf(x);
  if (a >= 448.0f) return (uint8_t)(s | 0x7E);
  if (a < 0x1p-6f) {
    /* a * 2^9 is exact; rounding it to an integer (ties to even) gives the
     * subnormal's mantissa, and 8 is the smallest normal, code 0x08 */
    return (uint8_t)(s | (uint8_t)nearbyintf(a * 512.0f));
  }
  int e;
  frexpf(a, &e); /* a = f * 2^e, f in [0.5, 1): a in [2^(e-1), 2^e) */
  int E = e - 1;
  float m = nearbyintf(ldexpf(a, 3 - E)); /* 1.mmm * 8, ties to even: 8..16 */
  if (m == 16.0f) {
    m = 8.0f;
    E += 1;
  }
  if (E > 8 || (E == 8 && m > 14.0f)) return (uint8_t)(s | 0x7E);
  return (uint8_t)(s | (uint8_t)(((E + 7) << 3) | ((int)m - 8)));
}

void orc_quantize_row_fp8(const float *x, int n, uint8_t *codes, float *scale) {
  float amax = 0.0f;
  for (int i = 0; i < n; ++i)
    if (fabsf(x[i]) > amax) amax = fabsf(x[i]);
  float sc = amax > 0.0f ? amax / 448.0f : 1.0f;
  for (int i = 0; i < n; ++i) codes[i] = orc_float_to_fp8e4m3(x[i] / sc);
  *scale = sc;
}

double orc_silu(double z) { return z / (1.0 + exp(-z)); }

/* ---- building blocks --------------------------------------------------- */

void orc_rmsnorm(const double *x, const uint16_t *g, int n, double eps, double *out) {
  double ss = 0.0;
  for (int i = 0; i < n; ++i) ss += x[i] * x[i];
  double r = 1.0 / sqrt(ss / (double)n + eps);
  for (int i = 0; i < n; ++i) out[i] = x[i] * r * orc_bf16_to_double(g[i]);
}

void orc_gemv_bf16(const uint16_t *W, int m, int k, const double *x, double *y) {
#pragma omp parallel for schedule(static)
  for (int i = 0; i < m; ++i) {
    const uint16_t *row = W + (int64_t)i * k;
    double acc = 0.0;
    for (int j = 0; j < k; ++j) acc += orc_bf16_to_double(row[j]) * x[j];
    y[i] = acc;
  }
}

void orc_gemv_fp8(const uint8_t *Q, const uint16_t *scales, int m, int k,
                  const double *x, double *y) {
  int kb = (k + 127) / 128;
#pragma omp parallel for schedule(static)
  for (int i = 0; i < m; ++i) {
    const uint8_t *row = Q + (int64_t)i * k;
    const uint16_t *srow = scales + (int64_t)(i / 128) * kb;
    double acc = 0.0;
    for (int j = 0; j < k; ++j) {
      double w = orc_fp8e4m3_to_double(row[j]) * orc_bf16_to_double(srow[j / 128]);
      acc += w * x[j];
    }
    y[i] = acc;
  }
}

void orc_rope(double *v, int d, int pos, double theta) {
  int half = d / 2;
  for (int i = 0; i < half; ++i) {
    double inv_freq = pow(theta, -2.0 * (double)i / (double)d);
    double ang = (double)pos * inv_freq;
    double c = cos(ang), s = sin(ang);
    double a = v[i], b = v[i + half];
    v[i] = a * c - b * s;
    v[i + half] = b * c + a * s;
  }
}

void orc_softmax(const double *s, int n, double *p) {
  double mx = s[0];
  for (int i = 1; i < n; ++i)
    if (s[i] > mx) mx = s[i];
  double sum = 0.0;
  for (int i = 0; i < n; ++i) {
    p[i] = exp(s[i] - mx);
    sum += p[i];
  }
  for (int i = 0; i < n; ++i) p[i] /= sum;
}

void orc_attend(const double *q, const uint16_t *K, const uint16_t *V, int n_pos,
                int d, double *o) {
  double *s = (double *)malloc(sizeof(double) * (size_t)n_pos);
  double *p = (double *)malloc(sizeof(double) * (size_t)n_pos);
  double scale = 1.0 / sqrt((double)d);
  for (int t = 0; t < n_pos; ++t) {
    double acc = 0.0;
    for (int j = 0; j < d; ++j) acc += q[j] * orc_bf16_to_double(K[(int64_t)t * d + j]);
    s[t] = acc * scale;
  }
  orc_softmax(s, n_pos, p);
  for (int j = 0; j < d; ++j) o[j] = 0.0;
  for (int t = 0; t < n_pos; ++t)
    for (int j = 0; j < d; ++j) o[j] += p[t] * orc_bf16_to_double(V[(int64_t)t * d + j]);
  free(s);
  free(p);
}

void orc_attend_fp8(const double *q, const uint8_t *Kc, const float *Ks, const uint8_t *Vc,
                    const float *Vs, int n_pos, int d, double *o) {
  double *s = (double *)malloc(sizeof(double) * (size_t)n_pos);
  double *p = (double *)malloc(sizeof(double) * (size_t)n_pos);
  double scale = 1.0 / sqrt((double)d);
  for (int t = 0; t < n_pos; ++t) {
    double acc = 0.0;
    for (int j = 0; j < d; ++j)
      acc += q[j] * (orc_fp8e4m3_to_double(Kc[(int64_t)t * d + j]) * (double)Ks[t]);
    s[t] = acc * scale;
  }
  orc_softmax(s, n_pos, p);
  for (int j = 0; j < d; ++j) o[j] = 0.0;
  for (int t = 0; t < n_pos; ++t)
    for (int j = 0; j < d; ++j)
      o[j] += p[t] * (orc_fp8e4m3_to_double(Vc[(int64_t)t * d + j]) * (double)Vs[t]);
  free(s);
  free(p);
}

int orc_argmax(const double *v, int n) {
  int best = 0;
  for (int i = 0; i < n; ++i) {
    if (isnan(v[i])) return -1;
    if (v[i] > v[best]) best = i; /* strict: the lowest index wins ties */
  }
  return best;
}

void orc_topk(const double *p, int n, int k, int32_t *idx) {
  char *taken = (char *)calloc((size_t)n, 1);
  for (int r = 0; r < k; ++r) {
    int best = -1;
    for (int i = 0; i < n; ++i)
      if (!taken[i] && (best < 0 || p[i] > p[best])) best = i;
    taken[best] = 1;
    idx[r] = best;
  }
  free(taken);
}

/* One fp8 SwiGLU expert: Wd (silu(Wg b) * (Wu b)), accumulated as weight * E(b)
 * into acc. */
static void expert_apply(int h, int f, const uint8_t *wg, const uint16_t *sg,
                         const uint8_t *wu, const uint16_t *su, const uint8_t *wd,
                         const uint16_t *sd, const double *b, double weight, double *acc) {
  double *gt = (double *)malloc(sizeof(double) * (size_t)f);
  double *up = (double *)malloc(sizeof(double) * (size_t)f);
  double *y = (double *)malloc(sizeof(double) * (size_t)h);
  orc_gemv_fp8(wg, sg, f, h, b, gt);
  orc_gemv_fp8(wu, su, f, h, b, up);
  for (int i = 0; i < f; ++i) gt[i] = orc_silu(gt[i]) * up[i];
  orc_gemv_fp8(wd, sd, h, f, gt, y);
  for (int i = 0; i < h; ++i) acc[i] += weight * y[i];
  free(gt);
  free(up);
  free(y);
}

void orc_moe_ffn(const orc_config *c, const orc_layer *L, const double *b,
                 double *delta, int32_t *sel_out, double *sel_w_out) {
  int h = c->hidden, f = c->expert_ffn, E = c->n_experts;
  int hb = (h + 127) / 128, fb = (f + 127) / 128;
  int64_t up_sz = (int64_t)f * h;          /* elements of a gate or up matrix */
  int64_t up_sc = (int64_t)fb * hb;        /* its block scales */
  int64_t dn_sc = (int64_t)hb * fb;
  double *r = (double *)malloc(sizeof(double) * (size_t)E);
  double *p = (double *)malloc(sizeof(double) * (size_t)E);
  int32_t sel[64];
  orc_gemv_bf16(L->router, E, h, b, r);
  orc_softmax(r, E, p);
  orc_topk(p, E, c->top_k, sel);
  for (int i = 0; i < h; ++i) delta[i] = 0.0;
  for (int s = 0; s < c->n_shared; ++s)
    expert_apply(h, f, L->s_wg + s * up_sz, L->s_sg + s * up_sc, L->s_wu + s * up_sz,
                 L->s_su + s * up_sc, L->s_wd + s * up_sz, L->s_sd + s * dn_sc, b, 1.0,
                 delta);
  for (int kk = 0; kk < c->top_k; ++kk) {
    int e = sel[kk];
    expert_apply(h, f, L->e_wg + e * up_sz, L->e_sg + e * up_sc, L->e_wu + e * up_sz,
                 L->e_su + e * up_sc, L->e_wd + e * up_sz, L->e_sd + e * dn_sc, b, p[e],
                 delta);
    if (sel_out) sel_out[kk] = e;
    if (sel_w_out) sel_w_out[kk] = p[e];
  }
  free(r);
  free(p);
}

/* ---- whole model ------------------------------------------------------- */

static void dense_ffn(const orc_config *c, const orc_layer *L, const double *b,
                      double *delta) {
  int h = c->hidden, f = c->ffn_dim;
  double *gt = (double *)malloc(sizeof(double) * (size_t)f);
  double *up = (double *)malloc(sizeof(double) * (size_t)f);
  orc_gemv_bf16(L->wg, f, h, b, gt);
  orc_gemv_bf16(L->wu, f, h, b, up);
  for (int i = 0; i < f; ++i) gt[i] = orc_silu(gt[i]) * up[i];
  orc_gemv_bf16(L->wd, h, f, gt, delta);
  free(gt);
  free(up);
}

static void ffn_block(const orc_config *c, const orc_layer *L, double *x) {
  int h = c->hidden;
  double *b = (double *)malloc(sizeof(double) * (size_t)h);
  double *dl = (double *)malloc(sizeof(double) * (size_t)h);
  orc_rmsnorm(x, L->ffn_norm, h, c->rms_eps, b);
  if (c->n_experts > 0)
    orc_moe_ffn(c, L, b, dl, NULL, NULL);
  else
    dense_ffn(c, L, b, dl);
  for (int i = 0; i < h; ++i) x[i] += dl[i];
  free(b);
  free(dl);
}

static int lm_head(const orc_config *c, const orc_weights *w, const double *x,
                   double *logits_out, double *hidden_out) {
  int h = c->hidden, V = c->vocab;
  double *y = (double *)malloc(sizeof(double) * (size_t)h);
  double *lg = (double *)malloc(sizeof(double) * (size_t)V);
  if (hidden_out) memcpy(hidden_out, x, sizeof(double) * (size_t)h);
  orc_rmsnorm(x, w->final_norm, h, c->rms_eps, y);
  orc_gemv_bf16(w->lm_head, V, h, y, lg);
  int tok = orc_argmax(lg, V);
  if (logits_out) memcpy(logits_out, lg, sizeof(double) * (size_t)V);
  free(y);
  free(lg);
  return tok;
}

int orc_decode_step(const orc_config *c, const orc_weights *w, uint16_t *kc,
                    uint16_t *vc, int64_t layer_stride, int token, int pos,
                    double *logits_out, double *hidden_out) {
  orc_kv kv = {kc, vc, NULL, NULL, layer_stride, 0, 0};
  return orc_decode_step_kv(c, w, &kv, token, pos, logits_out, hidden_out);
}

int orc_decode_step_kv(const orc_config *c, const orc_weights *w, const orc_kv *kv, int token,
                       int pos, double *logits_out, double *hidden_out) {
  int h = c->hidden, Hq = c->n_q_heads, Hkv = c->n_kv_heads, d = c->head_dim;
  int64_t layer_stride = kv->layer_stride;
  if (token < 0 || token >= c->vocab || pos < 0 || pos >= c->max_ctx) return -1;
  double *x = (double *)malloc(sizeof(double) * (size_t)h);
  double *a = (double *)malloc(sizeof(double) * (size_t)h);
  double *q = (double *)malloc(sizeof(double) * (size_t)Hq * d);
  double *k = (double *)malloc(sizeof(double) * (size_t)Hkv * d);
  double *v = (double *)malloc(sizeof(double) * (size_t)Hkv * d);
  double *o = (double *)malloc(sizeof(double) * (size_t)Hq * d);
  double *dl = (double *)malloc(sizeof(double) * (size_t)h);
  for (int i = 0; i < h; ++i) x[i] = orc_bf16_to_double(w->embed[(int64_t)token * h + i]);
  for (int l = 0; l < c->n_layers; ++l) {
    const orc_layer *L = &w->layers[l];
    orc_rmsnorm(x, L->attn_norm, h, c->rms_eps, a);
    orc_gemv_bf16(L->wq, Hq * d, h, a, q);
    orc_gemv_bf16(L->wk, Hkv * d, h, a, k);
    orc_gemv_bf16(L->wv, Hkv * d, h, a, v);
    for (int hh = 0; hh < Hq; ++hh) orc_rope(q + hh * d, d, pos, c->rope_theta);
    for (int g = 0; g < Hkv; ++g) orc_rope(k + g * d, d, pos, c->rope_theta);
    if (!kv->fp8) {
      uint16_t *Kl = (uint16_t *)kv->k + (int64_t)l * layer_stride;
      uint16_t *Vl = (uint16_t *)kv->v + (int64_t)l * layer_stride;
      for (int g = 0; g < Hkv; ++g)
        for (int j = 0; j < d; ++j) {
          int64_t off = ((int64_t)g * c->max_ctx + pos) * d + j;
          Kl[off] = orc_float_to_bf16((float)k[g * d + j]);
          Vl[off] = orc_float_to_bf16((float)v[g * d + j]);
        }
#pragma omp parallel for schedule(static)
      for (int hh = 0; hh < Hq; ++hh) {
        int g = (int)(((int64_t)hh * Hkv) / Hq);
        orc_attend(q + hh * d, Kl + (int64_t)g * c->max_ctx * d,
                   Vl + (int64_t)g * c->max_ctx * d, pos + 1, d, o + hh * d);
      }
    } else {
      uint8_t *Kl = (uint8_t *)kv->k + (int64_t)l * layer_stride;
      uint8_t *Vl = (uint8_t *)kv->v + (int64_t)l * layer_stride;
      float *KSl = kv->k_scale + (int64_t)l * kv->scale_layer_stride;
      float *VSl = kv->v_scale + (int64_t)l * kv->scale_layer_stride;
      float *row = (float *)malloc(sizeof(float) * (size_t)d);
      for (int g = 0; g < Hkv; ++g) {
        int64_t r = (int64_t)g * c->max_ctx + pos;
        for (int j = 0; j < d; ++j) row[j] = (float)k[g * d + j];
        orc_quantize_row_fp8(row, d, Kl + r * d, KSl + r);
        for (int j = 0; j < d; ++j) row[j] = (float)v[g * d + j];
        orc_quantize_row_fp8(row, d, Vl + r * d, VSl + r);
      }
      free(row);
#pragma omp parallel for schedule(static)
      for (int hh = 0; hh < Hq; ++hh) {
        int g = (int)(((int64_t)hh * Hkv) / Hq);
        orc_attend_fp8(q + hh * d, Kl + (int64_t)g * c->max_ctx * d, KSl + (int64_t)g * c->max_ctx,
                       Vl + (int64_t)g * c->max_ctx * d, VSl + (int64_t)g * c->max_ctx, pos + 1, d,
                       o + hh * d);
      }
    }
    orc_gemv_bf16(L->wo, h, Hq * d, o, dl);
    for (int i = 0; i < h; ++i) x[i] += dl[i];
    ffn_block(c, L, x);
  }
  int tok = lm_head(c, w, x, logits_out, hidden_out);
  free(x); free(a); free(q); free(k); free(v); free(o); free(dl);
  return tok;
}

int orc_forward_full(const orc_config *c, const orc_weights *w, const int32_t *tokens,
                     int n, double *logits_out, double *hidden_out) {
  int h = c->hidden, Hq = c->n_q_heads, Hkv = c->n_kv_heads, d = c->head_dim;
  int64_t nh = (int64_t)n * h;
  double *X = (double *)malloc(sizeof(double) * (size_t)nh);
  double *A = (double *)malloc(sizeof(double) * (size_t)nh);
  double *Q = (double *)malloc(sizeof(double) * (size_t)n * Hq * d);
  double *Kf = (double *)malloc(sizeof(double) * (size_t)n * Hkv * d);
  double *Vf = (double *)malloc(sizeof(double) * (size_t)n * Hkv * d);
  double *O = (double *)malloc(sizeof(double) * (size_t)n * Hq * d);
  double *D = (double *)malloc(sizeof(double) * (size_t)nh);
  /* K/V of every position for one layer, [Hkv][n][d], rounded as the cache is. */
  uint16_t *Kb = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)n * Hkv * d);
  uint16_t *Vb = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)n * Hkv * d);
  int tok = -1;
  for (int t = 0; t < n; ++t)
    for (int i = 0; i < h; ++i)
      X[(int64_t)t * h + i] = orc_bf16_to_double(w->embed[(int64_t)tokens[t] * h + i]);
  for (int l = 0; l < c->n_layers; ++l) {
    const orc_layer *L = &w->layers[l];
    for (int t = 0; t < n; ++t) {
      double *at = A + (int64_t)t * h;
      orc_rmsnorm(X + (int64_t)t * h, L->attn_norm, h, c->rms_eps, at);
      orc_gemv_bf16(L->wq, Hq * d, h, at, Q + (int64_t)t * Hq * d);
      orc_gemv_bf16(L->wk, Hkv * d, h, at, Kf + (int64_t)t * Hkv * d);
      orc_gemv_bf16(L->wv, Hkv * d, h, at, Vf + (int64_t)t * Hkv * d);
      for (int hh = 0; hh < Hq; ++hh) orc_rope(Q + ((int64_t)t * Hq + hh) * d, d, t, c->rope_theta);
      for (int g = 0; g < Hkv; ++g) orc_rope(Kf + ((int64_t)t * Hkv + g) * d, d, t, c->rope_theta);
      for (int g = 0; g < Hkv; ++g)
        for (int j = 0; j < d; ++j) {
          Kb[((int64_t)g * n + t) * d + j] = orc_float_to_bf16((float)Kf[((int64_t)t * Hkv + g) * d + j]);
          Vb[((int64_t)g * n + t) * d + j] = orc_float_to_bf16((float)Vf[((int64_t)t * Hkv + g) * d + j]);
        }
    }
#pragma omp parallel for collapse(2) schedule(static)
    for (int t = 0; t < n; ++t)
      for (int hh = 0; hh < Hq; ++hh) {
        int g = (int)(((int64_t)hh * Hkv) / Hq);
        orc_attend(Q + ((int64_t)t * Hq + hh) * d, Kb + (int64_t)g * n * d,
                   Vb + (int64_t)g * n * d, t + 1, d, O + ((int64_t)t * Hq + hh) * d);
      }
    for (int t = 0; t < n; ++t) {
      orc_gemv_bf16(L->wo, h, Hq * d, O + (int64_t)t * Hq * d, D + (int64_t)t * h);
      for (int i = 0; i < h; ++i) X[(int64_t)t * h + i] += D[(int64_t)t * h + i];
      ffn_block(c, L, X + (int64_t)t * h);
    }
  }
  for (int t = 0; t < n; ++t)
    tok = lm_head(c, w, X + (int64_t)t * h, logits_out ? logits_out + (int64_t)t * c->vocab : NULL,
                  hidden_out ? hidden_out + (int64_t)t * h : NULL);
  free(X); free(A); free(Q); free(Kf); free(Vf); free(O); free(D); free(Kb); free(Vb);
  return tok;
}

int orc_prefill(const orc_config *c, const orc_weights *w, uint16_t *kc, uint16_t *vc,
                int64_t layer_stride, const int32_t *tokens, int n) {
  int tok = -1;
  for (int t = 0; t < n; ++t)
    tok = orc_decode_step(c, w, kc, vc, layer_stride, tokens[t], t, NULL, NULL);
  return tok;
}

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void orc_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}
