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
#define PRE_ERR_BUSY (-10)       /* a serving loop holds the engine, or the
                                    request ring has no free slot            */

/* Device error kinds in pre_status.error. */
#define PRE_DEV_OK 0
#define PRE_DEV_TIMEOUT 1   /* a dependency wait exceeded the watchdog      */
#define PRE_DEV_BAD_TOKEN 2 /* an input or forced token outside [0, vocab)  */
#define PRE_DEV_NAN 3       /* a NaN logit reached the argmax               */
#define PRE_DEV_PLACEMENT 4 /* a workgroup ran on another XCD than the
                               XCD-local hand-offs assume (see xcd_local)   */
#define PRE_DEV_CONTEXT 5   /* a sequence's position was negative, or the
                               call's steps would pass max_ctx (slot = the
                               sequence, observed = its position, expected =
                               max_ctx)                                      */

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
 * workgroup elsewhere.
 * chunk (batch-1 dense engines): 0 = none; 2..8 = also build the chunk
 * task set, the micro-batch tiles run over `chunk` consecutive tokens of the
 * engine's one sequence, used by pre_engine_prefill and pre_engine_verify
 * (hidden, ffn_dim and n_q_heads * head_dim multiples of 32; MoE returns
 * PRE_ERR_UNSUPPORTED).
 * kv_dtype: 0 = bf16 K/V cache; 1 = fp8 e4m3 K/V codes with one fp32 scale
 * per cached row (layer, sequence, KV head, position): scale = amax(|row|) /
 * 448 in fp32 (1 for an all-zero row), codes = e4m3 of row / scale (ties to
 * even, saturating at 448); attention reads code x scale.  Batch-1 engines
 * (the decode kernel, its per-operator path and the serving loop); a
 * micro-batch or chunk task set returns PRE_ERR_UNSUPPORTED.  The pages
 * name quantized KV inside a persistent kernel as open work ("Persistent
 * execution paradigm" section 7.5; XL-Persistent-Kernel, future work) but
 * fix no format: this is the reading taken.
 * fold_ffn: 0 = in the decode kernel of a small one-XCD dense engine with
 * a bf16 cache (hidden <= wg_threads; every gate/up task's rows start at a
 * multiple of 8 and number at most 32; every workgroup a QKV producer), each
 * gate/up task also multiplies its slice of the SwiGLU output by the
 * matching columns of Wd and leaves that split-K partial of the down
 * projection; the next layer's QKV stage (or the LM head) adds the partials
 * while it stages its input, so a layer takes one hand-off fewer (the pages'
 * fusion of adjacent operators into one task to remove synchronisation
 * points, "Persistent execution paradigm" sections 4 and 6.1); -1 = never.
 * The per-operator path and the serving loop always run the down stage.
 * fold_attn: 0 = in the decode kernel of a small one-XCD batch-1 engine
 * with a bf16 cache (when the whole context's scores fit the LDS beside the
 * projection's input), every output-projection task computes its KV head's
 * attention over all positions itself, in place of the attention stage and
 * its hand-off (each of the head's workgroups repeats it: the cache is read
 * from the XCD's L2); -1 = never.  The per-operator path and the serving
 * loop always run the attention stage. */
typedef struct pre_config {
  int32_t n_layers, hidden, n_q_heads, n_kv_heads, head_dim, ffn_dim, vocab;
  int32_t batch, max_ctx;
  float rope_theta, rms_eps;
  int32_t n_experts, top_k, n_shared, expert_ffn, expert_dtype;
  int32_t grid_wgs, wg_threads, attn_splits;
  int32_t xcd_local;
  int32_t chunk;
  int32_t kv_dtype;
  int32_t fold_ffn;
  int32_t fold_attn;
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
 * K/V (post-RoPE K); the engine appends at the current position.
 * d_ctx_len (device, int32 [batch], 4-byte aligned, caller-owned, may be
 * NULL): sequence b's current position = the number of its cached tokens.
 * Every decode call reads it on the device at its start and advances it by
 * n_steps on the device at its end, so the host never tracks positions
 * (the pages' split of prefill and decode: a decode engine takes over a
 * cache that another engine filled -- SemiAnalysis TileRT digest, "PD
 * separation").  With NULL the engine keeps its own device array in the
 * workspace, starting at 0.
 * With kv_dtype 1, k and v hold one e4m3 code per element (uint8, same
 * shape) and k_scale, v_scale (device, fp32 [n_layers][batch][n_kv_heads]
 * [max_ctx], caller-owned) the rows' scales; NULL otherwise. */
typedef struct pre_kv {
  void *k, *v;
  int32_t *d_ctx_len;
  float *k_scale, *v_scale;
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
 * caller allocates it (16-byte aligned) and passes it to create, so the
 * caller's framework stays the only device allocator.  Source: the static
 * task graph and its buffers are fixed before the run ("Persistent execution
 * paradigm" sections 4 and 5.1, Fleet's precompiled task graph). */
int pre_workspace_size(const pre_config *cfg, size_t *bytes);

/* Validate cfg and the pointers, build and check the task table on the
 * host, and upload it, the RoPE cos/sin table and zeroed flags into the
 * workspace on `stream` (asynchronously).  Positions come from kv->d_ctx_len
 * (or start at 0).  *out is an opaque host handle.  Returns PRE_ERR_SHAPE /
 * PRE_ERR_ALIGN / PRE_ERR_WORKSPACE / PRE_ERR_HIP on failure, leaving *out
 * NULL.  Sources: the whole model unrolled ahead of time into one resident
 * kernel's work (TileRT notes, "persistent engine kernel"); the task graph
 * fixed at compile time with per-XCD placement ("Persistent execution
 * paradigm" section 5.1; "TileRT speed scaling law", the compile-time tile
 * routing table among its future directions); sampling and other knobs fixed
 * when the engine is built ("Persistent execution paradigm" section 5.1). */
int pre_engine_create(const pre_config *cfg, const pre_weights *w, const pre_kv *kv,
                      void *d_workspace, size_t ws_bytes, void *stream, pre_engine **out);

/* The engine without a caller workspace, for callers that cannot allocate
 * device memory (code under stream capture, tight serving loops, harnesses
 * that forbid allocation).  Same as pre_engine_create, but the workspace is
 * a static device array of the library, PRE_STATIC_WORKSPACE_BYTES per GPU
 * (each GPU the library runs on holds its copy until the process ends).  It
 * allocates no device memory: no hipMalloc/hipFree or allocating library
 * routine is called (host bookkeeping uses the C++ heap).  Configurations
 * whose workspace (pre_workspace_size) exceeds the array return
 * PRE_ERR_WORKSPACE; the batch-1 workloads here need 0.1-22 MB.  The used
 * part of the array is cleared at create.  All engines created this way on
 * one GPU share the array: each create takes it over, and calls on an engine
 * created earlier on that GPU then return PRE_ERR_BROKEN; calls on one GPU
 * that overlap in time race. */
#define PRE_STATIC_WORKSPACE_BYTES (32u << 20)
int pre_engine_create_static(const pre_config *cfg, const pre_weights *w, const pre_kv *kv, void *stream,
                             pre_engine **out);

/* Set / read the position each sequence decodes at next (h_pos[batch],
 * host).  The positions live on the device (kv->d_ctx_len, or the engine's
 * own array); these calls synchronise the device and copy them, and are
 * only needed to move a sequence by hand -- decode, prefill and verify
 * advance them on the device.  A position is also the number of cached
 * tokens.  PRE_ERR_BUSY while a serving loop holds the engine.  Source: a
 * decode engine that takes over a cache filled elsewhere (SemiAnalysis
 * TileRT digest, "PD separation"). */
int pre_engine_set_positions(pre_engine *e, const int32_t *h_pos);
int pre_engine_get_positions(const pre_engine *e, int32_t *h_pos);

/* Run n_steps decode steps in ONE persistent kernel launch on `stream`
 * (asynchronous).  Step s of sequence b decodes at position pos[b] + s, where
 * pos[b] is read from the device positions when the kernel starts: its
 * input token is d_in_tokens[b] at s = 0 and the previous step's greedy
 * token after that, unless d_forced is non-NULL, in which case it is
 * d_forced[s * batch + b] (teacher forcing; used to fill a cache from a
 * prompt).  d_out_tokens[s * batch + b] receives the greedy token of step s.
 * The kernel advances the device positions by n_steps at its end.
 * n_steps == 0 returns PRE_OK at once without reading any buffer.  Returns
 * PRE_ERR_CONTEXT if n_steps exceeds max_ctx; a position that would pass
 * max_ctx is caught on the device (PRE_DEV_CONTEXT, nothing is written).
 * PRE_ERR_BROKEN after a latched device error until pre_engine_reset.
 * Sources: the host launches once and the GPU stays resident for the
 * decode (TileRT notes, "persistent engine kernel"; SemiAnalysis TileRT
 * digest, what TileRT is); tile tasks ordered on the device instead of by
 * kernel boundaries (TileRT notes, "tile pipeline"; "Persistent execution
 * paradigm" sections 1, 4 and 6.2); the per-token operator chain
 * ("Persistent execution paradigm" section 1 and section 4's fused RMSNorm
 * and projection; section 7.1's expert selection fused with gate/up and
 * SiLU). */
int pre_engine_decode(pre_engine *e, int32_t n_steps, const int32_t *d_in_tokens,
                      const int32_t *d_forced, int32_t *d_out_tokens, const pre_check *chk,
                      void *stream);

/* Prefill inside the engine: the n_tokens prompt tokens d_tokens (device)
 * are decoded teacher-forced from the sequence's position, `chunk` tokens per
 * step through the chunk task set -- every weight is read once per chunk,
 * the skinny GEMMs run on the matrix cores, attention is causal inside the
 * chunk -- in ONE launch (the last chunk may be ragged: its padding columns
 * append nothing).  d_out_tokens[i] (device) receives the greedy successor
 * of token i, so d_out_tokens[n_tokens - 1] is the first generated token;
 * chk (optional) receives logits [n_tokens][vocab] and hidden states
 * [n_tokens][hidden].  The position advances by n_tokens on the device.
 * Sources: XL-Persistent-Kernel, the request lifecycle's prefill; the
 * SemiAnalysis TileRT digest, the prefill/decode split.  PRE_ERR_UNSUPPORTED
 * without a chunk task set. */
int pre_engine_prefill(pre_engine *e, int32_t n_tokens, const int32_t *d_tokens, int32_t *d_out_tokens,
                       const pre_check *chk, void *stream);

/* Speculative verify of n_draft draft tokens in one step (n_draft + 1 <=
 * chunk): d_tokens (device) = the current input token, then the drafts, at
 * positions pos .. pos + n_draft.  d_out_tokens[i] receives the greedy
 * successor of tokens 0..i; on the device, the drafts are accepted while
 * each equals the greedy successor of the token before it, *d_accepted
 * (device) receives their number a, the position advances by a + 1 (the
 * current token and the accepted drafts stay in the cache; rows past them
 * are overwritten later), and d_out_tokens[a] is the next input.  The
 * committed tokens are exactly those of plain greedy decoding.  Sources:
 * TileRT notes, v0.1.2-alpha.1 (multi-token prediction in the execution
 * flow); XL-Persistent-Kernel, the lifecycle's draft and verify steps. */
int pre_engine_verify(pre_engine *e, int32_t n_draft, const int32_t *d_tokens, int32_t *d_out_tokens,
                      int32_t *d_accepted, const pre_check *chk, void *stream);

/* The same decode as a conventional one-kernel-per-operator launch sequence
 * (seven launches per dense layer, eight per MoE layer, four per step),
 * using the same tile code and the same workspace, so that both paths can be
 * timed through identical calls.  Source: the launch and boundary cost the
 * resident kernel removes ("Persistent execution paradigm" sections 1 and
 * 6.1: microseconds per launch and hundreds of launches per token);
 * XL-Persistent-Kernel, benchmark modes (a host-driven decode next to the
 * resident one). */
int pre_baseline_decode(pre_engine *e, int32_t n_steps, const int32_t *d_in_tokens,
                        const int32_t *d_forced, int32_t *d_out_tokens, const pre_check *chk,
                        void *stream);

/* Copy the latched device status to *out (synchronises the engine's
 * create stream).  Returns PRE_OK, or PRE_ERR_DEVICE if an error is latched
 * (the engine is then BROKEN until pre_engine_reset).  Source: a persistent
 * kernel has no margin for a fault, one error ends the whole decode, so the
 * device reports where it stopped ("Persistent execution paradigm" section
 * 7.3). */
int pre_engine_status(pre_engine *e, pre_status *out);

/* Zero the ready flags, counters and status on `stream` and clear the
 * broken state.  Positions are kept.  Source: as pre_engine_status
 * ("Persistent execution paradigm" section 7.3). */
int pre_engine_reset(pre_engine *e, void *stream);

/* Watchdog for dependency waits, in milliseconds (default 2000; the
 * environment variable PRE_WATCHDOG_MS overrides the default).  A wait that
 * runs out latches PRE_DEV_TIMEOUT with the flag and epoch, and every
 * workgroup leaves through the abort word.  Source: "Persistent execution
 * paradigm" section 7.3 (a stuck resident kernel must end by itself). */
int pre_engine_set_watchdog(pre_engine *e, uint32_t ms);

/* Optional per-task timestamps.  d_buf receives, per (step, stage instance,
 * workgroup) executed, 8 uint32: {stage | wg << 16, t_begin, t_wait_end,
 * t_end, m0, m1, m2, m3} in 100 MHz realtime ticks (low 32 bits), where m*
 * are task phase marks (input staged, rows streamed, ...; stale where a task
 * kind sets fewer); records beyond `bytes` are dropped.  NULL disables.
 * Source: CU busy and idle gaps as the measure of what a resident kernel
 * recovers ("Persistent execution paradigm" section 6.1; SemiAnalysis TileRT
 * digest, the gap between the bandwidth roofline and the measured rate). */
int pre_engine_set_trace(pre_engine *e, void *d_buf, size_t bytes);

/* Free the host-side state (no device memory is owned: the caller owns the
 * workspace, weights and cache, as pre_engine_create states). */
int pre_engine_destroy(pre_engine *e);

/* ---- the serving loop: one resident launch, requests through a ring ------
 * The resident kernel stays on the GPU between requests and takes them from
 * a ring of descriptors in coherent host memory: the host writes a
 * descriptor and marks it ready, the kernel's scheduler (workgroup 0) polls
 * the ring, claims the oldest ready slot, and every workgroup decodes the
 * request -- its prompt teacher-forced, then greedy tokens fed back on the
 * device until the EOS token or the budget -- while workgroup 0 streams the
 * tokens into the slot.  Each slot moves FREE -> READY (host) -> RUNNING ->
 * DONE (kernel) -> FREE (host).  Sources: "Persistent execution paradigm"
 * section 4 (a resident kernel that polls for work on the device) and
 * section 5.6 (a GPU-resident scheduler over a ring with a per-slot state
 * machine); XL-Persistent-Kernel, the request lifecycle (prompt, decode,
 * stop at EOS or budget) and device-resident request descriptors.  Batch-1
 * engines only (micro-batch engines return PRE_ERR_UNSUPPORTED).  While the
 * loop runs it holds every CU: the engine's other calls return PRE_ERR_BUSY,
 * and the caller must not wait on other GPU work of the device until
 * pre_serve_stop. */
typedef struct pre_server pre_server;
typedef struct pre_serve_stats {
  int32_t steps;   /* decode steps the loop ran */
  int32_t served;  /* requests it finished (without a request error) */
  int32_t error;   /* the device error latched by the loop (PRE_DEV_*) */
} pre_serve_stats;

/* Allocate the ring (n_slots slots, prompts of up to max_prompt tokens, up
 * to max_out generated tokens each; coherent pinned host memory owned by
 * the server) and launch the resident loop on `stream`.  The loop ends by
 * itself after idle_ms milliseconds without a request (a bound for callers
 * that never stop it).  The engine's ready-flag epochs and device positions
 * continue across the loop. */
int pre_serve_start(pre_engine *e, int32_t n_slots, int32_t max_prompt, int32_t max_out, uint32_t idle_ms,
                    void *stream, pre_server **out);

/* Submit a request (host only, no GPU call): n_prompt >= 1 tokens (h_prompt,
 * host), decoded from position pos (the number of tokens already cached for
 * the sequence; -1 = the engine's current position), then up to budget
 * greedy tokens, stopping after a token equal to eos (-1: none).  The last
 * prompt token's greedy successor is the first output.  *slot receives the
 * slot to poll.  PRE_ERR_BUSY if every slot is taken, PRE_ERR_DEVICE if the
 * loop has ended; a request the kernel finds invalid (its steps would pass
 * max_ctx) is finished with that error in its slot and the loop goes on. */
int pre_serve_submit(pre_server *s, const int32_t *h_prompt, int32_t n_prompt, int32_t pos, int32_t budget,
                     int32_t eos, int32_t *slot);

/* Copy up to max_tokens of the slot's tokens produced so far into h_tokens;
 * *n_out = how many exist, *done = 1 once the request is finished (the slot
 * is then freed; *err = its PRE_DEV_* error or 0).  Returns PRE_ERR_DEVICE
 * if the loop ended before finishing the request. */
int pre_serve_poll(pre_server *s, int32_t slot, int32_t *h_tokens, int32_t max_tokens, int32_t *n_out,
                   int32_t *done, int32_t *err);

/* Ask the loop to end, wait for the kernel, report its counts and free the
 * ring and the server. */
int pre_serve_stop(pre_server *s, pre_serve_stats *stats);

/* Static description of an error code (PRE_ERR_* or PRE_DEV_* kinds are
 * told apart by sign: PRE_ERR_* are negative). */
const char *pre_strerror(int code);

/* ---- introspection (host only, no GPU needed) ------------------------- */
/* Summary of the task table built for cfg: stage instances per step, the
 * workgroups used, ready-flag slots, and the result of the table validator
 * (0 = every check passed, otherwise the number of the first failed check).
 * Also dumps up to max_tasks task records (8 int32 each: op, layer, r0, r1,
 * aux, wait_lo, wait_hi, signal) in table order when h_tasks is non-NULL.
 * Source: the compile-time task table with per-XCD placement ("Persistent
 * execution paradigm" section 5.1; "TileRT speed scaling law", future
 * directions). */
typedef struct pre_plan_info {
  int32_t n_stage_inst, n_wgs, n_slots, n_tasks, attn_splits, validator;
  int32_t xcd_local;  /* 1: per-KV-head XCD-local hand-offs; 2: every workgroup on one XCD; 0: none */
  int32_t fold_ffn;   /* 1: the decode kernel folds the down projection into the gate/up stage */
  int32_t fold_attn;  /* 1: the decode kernel folds the attention into the output projection */
  int64_t workspace_bytes;
} pre_plan_info;
int pre_plan_describe(const pre_config *cfg, pre_plan_info *out, int32_t *h_tasks,
                      int32_t max_tasks);

/* Run the table validator on a caller-supplied table (n_tasks records of 8
 * int32 in the layout pre_plan_describe dumps).  Returns 0 if it passes, the
 * number of the first failed check otherwise, or a negative PRE_ERR_* code.
 * Source: a task graph fixed ahead of time can be checked before it runs,
 * where a fault inside the resident kernel could not be recovered from
 * ("Persistent execution paradigm" sections 5.1 and 7.3). */
int pre_plan_validate(const pre_config *cfg, const int32_t *h_tasks, int32_t n_tasks);

/* Algorithmic bytes one decode step moves for sequences at the given
 * positions (h_pos[batch]): every weight read once (active experts only),
 * the attended K/V read once, the new K/V written.  For bandwidth figures.
 * Source: the bandwidth roofline, bytes per token over HBM bandwidth, as the
 * score of a decode engine (SemiAnalysis TileRT digest, its roofline
 * arithmetic; "TileRT speed scaling law", Fleet's Eq. (1)). */
int64_t pre_step_bytes(const pre_config *cfg, const int32_t *h_pos);

#ifdef __cplusplus
}
#endif
#endif /* PRE_H */
