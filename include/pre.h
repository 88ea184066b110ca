/*
 * pre.h -- C ABI of the persistent resident decode engine (MI355X, gfx950).
 *
 * The engine runs a transformer decode step -- RMSNorm, QKV projection with
 * RoPE, KV-cache append, split-KV attention with an online-softmax combine,
 * output projection and residual, RMSNorm, SwiGLU FFN or routed fp8 experts,
 * LM head and greedy argmax -- as ONE resident GPU kernel per call.  Inside
 * it, one workgroup per compute unit walks a task table that was built on
 * the host when the engine was created; tasks are ordered by per-task ready
 * flags in device memory instead of by kernel boundaries, and the greedy
 * token is fed back on the device, so the host launches once per call of
 * pre_engine_decode(n_steps).
 *
 * Sources of the design (the pages this engine follows):
 *  - "Persistent execution paradigm: from kernel boundary elimination to an
 *    ultra-low-latency engine", section 1 (per-token operator list, launch
 *    overhead, private per-XCD L2s), section 4 (cross-operator fusion of
 *    RMSNorm with the projection; static task graph), section 5.1 (task
 *    graph fixed at compile time, dispatched by a per-XCD scheduler),
 *    section 6.2 (a megakernel holding every CU), section 7.1 (top-8 expert
 *    selection fused with gate/up projection and SiLU), section 7.2
 *    (two-level event synchronisation with CDNA cache-scope modifiers);
 *  - the TileRT notes, "persistent engine kernel" (the whole model as one
 *    resident kernel launched once) and "tile pipeline";
 *  - "TileRT speed scaling law", the compile-time tile routing table among
 *    its future directions;
 *  - the SemiAnalysis TileRT digest, its bandwidth-roofline arithmetic
 *    (bytes per token over HBM bandwidth) and its prefill/decode split (a
 *    decode engine that receives a cache filled elsewhere).
 * The pages print no formulas; the arithmetic follows the plain definition
 * of a pre-norm decoder, as the CPU oracle in oracle/ does.
 *
 * Conventions for every call:
 *  - Pointers named d_* and all weight / cache / workspace pointers are
 *    DEVICE pointers owned by the caller; the engine never frees them and
 *    they must outlive the engine.  Pointers named h_* are host pointers.
 *  - Streams are hipStream_t values passed as void* (NULL = the null stream).
 *  - Calls return PRE_OK (0) or a negative PRE_ERR_* code; nothing throws.
 *    Errors detected on the device are latched in the workspace and read
 *    with pre_engine_status after the stream has been synchronised.
 *  - Matrices are [out][in] row-major (each output row contiguous along the
 *    reduction axis), bf16 unless stated.  Every weight pointer must be
 *    16-byte aligned.
 */
#ifndef PRE_H
#define PRE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- error codes ------------------------------------------------------ */
#define PRE_OK 0
#define PRE_ERR_ARG (-1)         /* NULL handle/pointer, n_steps < 0, ...    */
#define PRE_ERR_SHAPE (-2)       /* configuration outside what is supported */
#define PRE_ERR_ALIGN (-3)       /* a weight or buffer not 16-byte aligned   */
#define PRE_ERR_WORKSPACE (-4)   /* workspace too small                       */
#define PRE_ERR_HIP (-5)         /* a HIP runtime call failed                 */
#define PRE_ERR_UNSUPPORTED (-6) /* valid but not built (e.g. batch > 1 MoE)  */
#define PRE_ERR_DEVICE (-7)      /* the device latched an error (see status)  */
#define PRE_ERR_BROKEN (-8)      /* engine poisoned by an earlier device
                                    error; call pre_engine_reset first       */
#define PRE_ERR_CONTEXT (-9)     /* positions + n_steps would pass max_ctx    */

/* Device error kinds in pre_status.error. */
#define PRE_DEV_OK 0
#define PRE_DEV_TIMEOUT 1   /* a dependency wait exceeded the watchdog      */
#define PRE_DEV_BAD_TOKEN 2 /* an input or forced token outside [0, vocab)  */
#define PRE_DEV_NAN 3       /* a NaN logit reached the argmax               */
#define PRE_DEV_PLACEMENT 4 /* a workgroup ran on another XCD than the
                               XCD-local hand-offs assume (see xcd_local)   */

/* ---- model configuration ---------------------------------------------- */
/* Plain data, read once at create.  n_experts == 0 means a dense SwiGLU FFN
 * of width ffn_dim; n_experts > 0 means a routed MoE FFN (router over
 * n_experts, top_k chosen, n_shared always-on experts, each a SwiGLU of width
 * expert_ffn) with expert_dtype 1 = fp8 e4m3 (OCP) codes and one bf16 scale
 * per 128x128 block.  Query head h reads KV head h * n_kv_heads / n_q_heads.
 * RoPE pairs element i with i + head_dim/2 (rotate-half).
 * grid_wgs: workgroups that take part (0 = one per CU, or fewer -- one per
 * 32 KB of a layer's weights, a multiple of 8 -- for small models);
 * wg_threads: threads per workgroup (0 = 512).  attn_splits: KV chunks per KV
 * head and sequence (0 = about one per 128 positions of max_ctx, at most 16
 * and at most the workgroups per KV head).  xcd_local: 0 = hand the q/K/V rows and the
 * attention partials from producer to consumer through the XCD's own L2
 * when every consumer sits on the producer's XCD (8 KV heads, a grid that is
 * a multiple of 8: KV head g's QKV rows, attention chunks and output
 * projection slice all run on XCD g), or, when the grid fits one XCD's CUs
 * (small models; the default grid of a small model is capped at that), run
 * every workgroup on XCD 0 and hand every flag over in its L2; -1 = always
 * hand off at device scope, no placement.  The persistent kernel checks the
 * placement it assumes and latches PRE_DEV_PLACEMENT if the hardware put a
 * workgroup elsewhere. */
typedef struct pre_config {
  int32_t n_layers, hidden, n_q_heads, n_kv_heads, head_dim, ffn_dim, vocab;
  int32_t batch, max_ctx;
  float rope_theta, rms_eps;
  int32_t n_experts, top_k, n_shared, expert_ffn, expert_dtype;
  int32_t grid_wgs, wg_threads, attn_splits;
  int32_t xcd_local;
} pre_config;

/* Per-layer weights (device pointers).  Dense: wg, wu [ffn][hidden], wd
 * [hidden][ffn].  MoE: router [n_experts][hidden] bf16; e_wg, e_wu
 * [n_experts][expert_ffn][hidden] and e_wd [n_experts][hidden][expert_ffn] as
 * fp8 codes (one byte each); e_sg, e_su [n_experts][expert_ffn/128][hidden/128]
 * and e_sd [n_experts][hidden/128][expert_ffn/128] bf16 block scales (ceil
 * division); s_* the same for the n_shared shared experts.  Unused pointers
 * may be NULL. */
typedef struct pre_layer_w {
  const void *attn_norm, *wq, *wk, *wv, *wo, *ffn_norm;
  const void *wg, *wu, *wd;
  const void *router;
  const void *e_wg, *e_wu, *e_wd, *e_sg, *e_su, *e_sd;
  const void *s_wg, *s_wu, *s_wd, *s_sg, *s_su, *s_sd;
} pre_layer_w;

/* embed [vocab][hidden], final_norm [hidden], lm_head [vocab][hidden] (device);
 * layers is a HOST array of n_layers entries, copied at create. */
typedef struct pre_weights {
  const void *embed, *final_norm, *lm_head;
  const pre_layer_w *layers;
} pre_weights;

/* KV cache (device): k and v are bf16 [n_layers][batch][n_kv_heads][max_ctx]
 * [head_dim].  Positions below a sequence's current position must hold its
 * K/V (post-RoPE K); the engine appends at the current position. */
typedef struct pre_kv {
  void *k, *v;
} pre_kv;

/* Optional per-call outputs for checking (device, may be NULL):
 * logits fp32 [n_steps][batch][vocab]; hidden fp32 [n_steps][batch][hidden]
 * = the residual stream after the last layer, before the final RMSNorm. */
typedef struct pre_check {
  float *logits, *hidden;
} pre_check;

/* Latched device status (read after a stream synchronise). */
typedef struct pre_status {
  int32_t error;     /* PRE_DEV_* */
  int32_t step;      /* decode step (within the call) where it happened  */
  int32_t stage;     /* stage instance index in the task table            */
  int32_t slot;      /* ready flag being waited on (timeout)              */
  int32_t wg;        /* workgroup that latched it                         */
  uint32_t observed; /* flag value seen (timeout) / bad token value       */
  uint32_t expected; /* epoch waited for                                  */
  int32_t xcc_mismatch; /* workgroups whose XCD differed from the plan's  */
} pre_status;

typedef struct pre_engine pre_engine;

/* Bytes of device workspace the engine needs for cfg (task table, ready
 * flags, activation slots, attention partials, RoPE table, status).  The
 * caller allocates it (16-byte aligned) and passes it to create. */
int pre_workspace_size(const pre_config *cfg, size_t *bytes);

/* Validate cfg and the pointers, build and check the task table on the
 * host, and upload it, the RoPE cos/sin table and zeroed flags into the
 * workspace on `stream` (asynchronously).  Positions start at 0.  *out is an
 * opaque host handle.  Returns PRE_ERR_SHAPE / PRE_ERR_ALIGN /
 * PRE_ERR_WORKSPACE / PRE_ERR_HIP on failure, leaving *out NULL. */
int pre_engine_create(const pre_config *cfg, const pre_weights *w, const pre_kv *kv,
                      void *d_workspace, size_t ws_bytes, void *stream, pre_engine **out);

/* Set / read the position each sequence decodes at next (host-side state:
 * h_pos[batch]).  A position is also the number of cached tokens. */
int pre_engine_set_positions(pre_engine *e, const int32_t *h_pos);
int pre_engine_get_positions(const pre_engine *e, int32_t *h_pos);

/* Run n_steps decode steps in ONE persistent kernel launch on `stream`
 * (asynchronous).  Step s of sequence b decodes at position pos[b] + s: its
 * input token is d_in_tokens[b] at s = 0 and the previous step's greedy
 * token after that, unless d_forced is non-NULL, in which case it is
 * d_forced[s * batch + b] (teacher forcing; used to fill a cache from a
 * prompt).  d_out_tokens[s * batch + b] receives the greedy token of step s.
 * Advances the host positions by n_steps.  n_steps == 0 returns PRE_OK at
 * once without reading any buffer.  Returns PRE_ERR_CONTEXT if a position
 * would pass max_ctx, PRE_ERR_BROKEN after a latched device error until
 * pre_engine_reset. */
int pre_engine_decode(pre_engine *e, int32_t n_steps, const int32_t *d_in_tokens,
                      const int32_t *d_forced, int32_t *d_out_tokens, const pre_check *chk,
                      void *stream);

/* The same decode as a conventional one-kernel-per-operator launch sequence
 * (seven launches per dense layer, eight per MoE layer, four per step),
 * using the same tile code and the same workspace, so that both paths can be
 * timed through identical calls. */
int pre_baseline_decode(pre_engine *e, int32_t n_steps, const int32_t *d_in_tokens,
                        const int32_t *d_forced, int32_t *d_out_tokens, const pre_check *chk,
                        void *stream);

/* Copy the latched device status to *out (synchronises the engine's
 * create stream).  Returns PRE_OK, or PRE_ERR_DEVICE if an error is latched
 * (the engine is then BROKEN until pre_engine_reset). */
int pre_engine_status(pre_engine *e, pre_status *out);

/* Zero the ready flags, counters and status on `stream` and clear the
 * broken state.  Positions are kept. */
int pre_engine_reset(pre_engine *e, void *stream);

/* Watchdog for dependency waits, in milliseconds (default 2000; the
 * environment variable PRE_WATCHDOG_MS overrides the default). */
int pre_engine_set_watchdog(pre_engine *e, uint32_t ms);

/* Optional per-task timestamps.  d_buf receives, per (step, stage instance,
 * workgroup) executed, 8 uint32: {stage | wg << 16, t_begin, t_wait_end,
 * t_end, m0, m1, m2, m3} in 100 MHz realtime ticks (low 32 bits), where m*
 * are task phase marks (input staged, rows streamed, ...; stale where a task
 * kind sets fewer); records beyond `bytes` are dropped.  NULL disables. */
int pre_engine_set_trace(pre_engine *e, void *d_buf, size_t bytes);

/* Free the host-side state (no device memory is owned). */
int pre_engine_destroy(pre_engine *e);

/* Static description of an error code. */
const char *pre_strerror(int code);

/* ---- introspection (host only, no GPU needed) ------------------------- */
/* Summary of the task table built for cfg: stage instances per step, the
 * workgroups used, ready-flag slots, and the result of the table validator
 * (0 = every check passed, otherwise the number of the first failed check).
 * Also dumps up to max_tasks task records (8 int32 each: op, layer, r0, r1,
 * aux, wait_lo, wait_hi, signal) in table order when h_tasks is non-NULL. */
typedef struct pre_plan_info {
  int32_t n_stage_inst, n_wgs, n_slots, n_tasks, attn_splits, validator;
  int32_t xcd_local;  /* 1: per-KV-head XCD-local hand-offs; 2: every workgroup on one XCD; 0: none */
  int64_t workspace_bytes;
} pre_plan_info;
int pre_plan_describe(const pre_config *cfg, pre_plan_info *out, int32_t *h_tasks,
                      int32_t max_tasks);

/* Run the table validator on a caller-supplied table (n_tasks records of 8
 * int32 in the layout pre_plan_describe dumps).  Returns 0 if it passes, the
 * number of the first failed check otherwise, or a negative PRE_ERR_* code. */
int pre_plan_validate(const pre_config *cfg, const int32_t *h_tasks, int32_t n_tasks);

/* Algorithmic bytes one decode step moves for sequences at the given
 * positions (h_pos[batch]): every weight read once (active experts only),
 * the attended K/V read once, the new K/V written.  For bandwidth figures. */
int64_t pre_step_bytes(const pre_config *cfg, const int32_t *h_pos);

#ifdef __cplusplus
}
#endif
#endif /* PRE_H */
