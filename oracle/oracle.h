/*
 * CPU oracle for the batch-1 / micro-batch transformer decode step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link
 * or call this code: only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark use it.  It shares no code, header, table or
 * constant with the GPU engine.
 *
 * What it computes is the plain definition of a pre-norm decoder step, in
 * fp64, with one sequential accumulation order per dot product, a full-row
 * softmax (not an online one) and normalise-then-project.  The operator list
 * (attention QKV, softmax, activation, norm, KV-cache update) is the one the
 * "Persistent execution paradigm" survey page names in its section 1; the
 * fusion of RMSNorm with the following projection is its section 4; routed
 * experts with top-8 selection followed by gate/up projection and SiLU are
 * its section 7.1.  The pages print no formula for any of these, so every
 * formula here is the textbook one, and the readings taken where the pages
 * are silent are listed in the design notes of the repository:
 *   - pre-norm residual blocks, no biases, no embedding scale, final RMSNorm;
 *   - RMSNorm: x_i * g_i / sqrt(mean(x^2) + eps), eps inside the root;
 *   - RoPE rotate-half pairs (i, i + d/2), inv_freq_i = theta^(-2i/d), angle
 *     and cos/sin in fp64, applied to q and k before k enters the cache;
 *   - attention scale 1/sqrt(d), causal over positions 0..p inclusive,
 *     query head h reads KV head floor(h * Hkv / Hq);
 *   - rounding points: weights as given (bf16, or fp8 e4m3 times a bf16
 *     128x128 block scale); K and V rounded to bf16 (round to nearest even)
 *     from an fp32 value when appended (or, with an fp8 cache, quantized per
 *     row: an fp32 scale amax/448 and e4m3 codes of the fp32 quotients, ties
 *     to even, saturating at 448); nothing else is rounded;
 *   - SwiGLU FFN: Wd (silu(Wg b) * (Wu b)), silu(z) = z / (1 + e^-z);
 *   - MoE: softmax over all router logits, the top-k probabilities (ties to
 *     the lower expert id) weight their experts without renormalisation,
 *     the shared expert has weight 1;
 *   - LM head untied from the embedding; greedy argmax, ties to the lowest
 *     token id, NaN is an error (returns -1).
 *
 * Parity pins live in tests/test_oracle_pins.py.
 */
#ifndef PRE_ORACLE_H
#define PRE_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int32_t n_layers, hidden, n_q_heads, n_kv_heads, head_dim, ffn_dim, vocab;
  int32_t max_ctx;
  double rope_theta, rms_eps;
  int32_t n_experts, top_k, n_shared, expert_ffn; /* n_experts == 0: dense */
} orc_config;

/* Host pointers.  bf16 and the fp8 codes are raw bit patterns.  Matrices are
 * [out][in] row-major.  Expert tensors are stacked [E][out][in]; block scales
 * are [E][ceil(out/128)][ceil(in/128)]. */
typedef struct {
  const uint16_t *attn_norm, *wq, *wk, *wv, *wo, *ffn_norm;
  const uint16_t *wg, *wu, *wd;             /* dense FFN */
  const uint16_t *router;                   /* MoE router [E][h] */
  const uint8_t *e_wg, *e_wu, *e_wd;        /* routed experts, fp8 e4m3 */
  const uint16_t *e_sg, *e_su, *e_sd;       /* their block scales, bf16 */
  const uint8_t *s_wg, *s_wu, *s_wd;        /* shared expert, fp8 e4m3 */
  const uint16_t *s_sg, *s_su, *s_sd;
} orc_layer;

typedef struct {
  const uint16_t *embed, *final_norm, *lm_head;
  const orc_layer *layers;
} orc_weights;

/* Scalar codecs. */
double orc_bf16_to_double(uint16_t b);
uint16_t orc_float_to_bf16(float f);
double orc_fp8e4m3_to_double(uint8_t c);
/* fp32 -> OCP E4M3 code: round to nearest, ties to even, magnitudes at or
 * above 448 (the largest finite value) saturate to +-448, NaN -> 0x7F. */
uint8_t orc_float_to_fp8e4m3(float x);
/* One cached K or V row in fp8: scale = amax(|x|) / 448 in fp32 (1 for an
 * all-zero row), codes[j] = e4m3(x[j] / scale) with the fp32 quotient. */
void orc_quantize_row_fp8(const float *x, int n, uint8_t *codes, float *scale);

/* The K/V cache of one sequence: bf16 rows, or fp8 e4m3 codes with one fp32
 * scale per row.  k, v: [n_layers][n_kv_heads][max_ctx][head_dim] (layer
 * distance layer_stride elements); k_scale, v_scale: [n_layers][n_kv_heads]
 * [max_ctx] (layer distance scale_layer_stride) when fp8. */
typedef struct {
  void *k, *v;
  float *k_scale, *v_scale;
  int64_t layer_stride, scale_layer_stride;
  int32_t fp8;
} orc_kv;

/* Building blocks (each a plain definition). */
void orc_rmsnorm(const double *x, const uint16_t *g, int n, double eps, double *out);
void orc_gemv_bf16(const uint16_t *W, int m, int k, const double *x, double *y);
void orc_gemv_fp8(const uint8_t *Q, const uint16_t *scales, int m, int k,
                  const double *x, double *y);
void orc_rope(double *v, int d, int pos, double theta);
void orc_softmax(const double *s, int n, double *p);
void orc_attend(const double *q, const uint16_t *K, const uint16_t *V, int n_pos,
                int d, double *o);
/* The same over fp8 rows: K[t][j] = fp8dec(Kc[t][j]) * Ks[t] (V alike). */
void orc_attend_fp8(const double *q, const uint8_t *Kc, const float *Ks, const uint8_t *Vc,
                    const float *Vs, int n_pos, int d, double *o);
int orc_argmax(const double *v, int n);
void orc_topk(const double *p, int n, int k, int32_t *idx);
double orc_silu(double z);
void orc_moe_ffn(const orc_config *c, const orc_layer *L, const double *b,
                 double *delta, int32_t *sel_out, double *sel_w_out);

/* One decode step of one sequence at position pos (0-based).  The caches are
 * bf16 [n_layers][n_kv_heads][max_ctx][head_dim] with the given distance (in
 * elements) between consecutive layers; positions 0..pos-1 must hold the
 * sequence's K/V, position pos is written here.  logits_out [vocab] and
 * hidden_out [hidden] (the residual stream before the final norm) may be
 * NULL.  Returns the greedy token, or -1 if a logit is NaN. */
int orc_decode_step(const orc_config *c, const orc_weights *w, uint16_t *kc,
                    uint16_t *vc, int64_t layer_stride, int token, int pos,
                    double *logits_out, double *hidden_out);

/* The same step over either cache format (orc_kv): with fp8, the new K and V
 * rows are quantized (orc_quantize_row_fp8 of their fp32 values) when
 * appended, and attention reads the dequantized rows. */
int orc_decode_step_kv(const orc_config *c, const orc_weights *w, const orc_kv *kv, int token,
                       int pos, double *logits_out, double *hidden_out);

/* The same model recomputed from scratch over tokens[0..n): layer by layer
 * over all positions, with its own K/V storage and no cache input.
 * logits_out is [n][vocab] (NULL allowed), hidden_out [n][hidden] (NULL
 * allowed).  Returns the greedy token after the last position. */
int orc_forward_full(const orc_config *c, const orc_weights *w, const int32_t *tokens,
                     int n, double *logits_out, double *hidden_out);

/* Prefill the cache causally from tokens[0..n) (decode steps at positions
 * 0..n-1) and return the greedy token after position n-1. */
int orc_prefill(const orc_config *c, const orc_weights *w, uint16_t *kc, uint16_t *vc,
                int64_t layer_stride, const int32_t *tokens, int n);

/* Number of OpenMP threads the oracle uses, and a way to change it (timing
 * only: every sum is sequential whatever the thread count). */
int orc_num_threads(void);
void orc_set_num_threads(int n);

#ifdef __cplusplus
}
#endif
#endif
