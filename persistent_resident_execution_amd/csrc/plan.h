// Task table and workspace layout shared by the host builder (plan.cpp) and
// the device code (engine.hip).  Plain data only.
//
// The table is the ahead-of-time task graph of one decode step: a list of
// stage instances (per layer: QKV, ATTN, OPROJ, then GU/DOWN for a dense FFN
// or ROUTER/EGU/EDOWN for routed experts; finally LM), and for every stage
// instance one task per workgroup.  Each task names the contiguous range of
// ready-flag slots it waits on and the slot it sets when done.  This is the
// static task graph with per-XCD placement that the persistent-execution
// survey describes for chiplet GPUs (section 5.1) and the compile-time tile
// routing table the TileRT scaling-law critique proposes (future directions).
#pragma once
#include <stdint.h>

// The index helpers below are used by host code and by kernels.
#ifdef __HIP__
#define PRE_HD __host__ __device__
#else
#define PRE_HD
#endif

namespace pre {

// Most units (2 KB per wavefront) of a batch-1 GEMV stream loaded into LDS
// ahead of the register ring (fewer where the task's own LDS leaves less).
#ifndef PRE_UNITS
#define PRE_UNITS 4
#endif

// Folded FFN: most 16-byte units of Wd (8 columns each) one thread of a
// gate/up task holds for its row of the down projection's partial.
#define FOLD_U 4

enum Op : int32_t {
  OP_NONE = 0,
  OP_QKV = 1,    // RMSNorm-folded QKV rows (RoPE pairs), K/V append
  OP_ATTN = 2,   // one KV chunk of one (sequence, KV head); last arriver combines
  OP_OPROJ = 3,  // one KV head's slice of the output projection (split-K partial)
  OP_GU = 4,     // gate/up row pairs + SwiGLU
  OP_DOWN = 5,   // down projection rows + residual
  OP_ROUTER = 6, // router rows (MoE)
  OP_EGU = 7,    // expert gate/up row pairs (slot k of the chosen experts)
  OP_EDOWN = 8,  // expert down rows summed over chosen experts + residual
  OP_LM = 9,     // LM-head rows + per-task argmax
  OP_EMBED = 10, // micro-batch: embedding rows of every sequence, packed for the QKV stage
  OP_COMB = 11,  // micro-batch: attention chunk combine of one KV head, packed for the O projection
};

// One task: 8 x int32 = 32 bytes.
struct Task {
  int32_t op, layer;
  int32_t r0, r1;     // row / pair range [r0, r1); ATTN: r0 = chunk, r1 = chunks
  int32_t aux;        // ATTN, OPROJ: sequence * n_kv_heads + kv head (micro-batch ATTN, COMB: kv head)
  int32_t wait_lo, wait_hi;  // ready slots [lo, hi) that must reach this step's epoch
  int32_t signal;     // slot set to the epoch when done (ATTN: set by the combiner)
};

// Device-side copy of one layer's weight pointers.
struct DevLayer {
  const void *attn_norm, *wq, *wk, *wv, *wo, *ffn_norm;
  const void *wg, *wu, *wd;
  const void *router;
  const void *e_wg, *e_wu, *e_wd, *e_sg, *e_su, *e_sd;
  const void *s_wg, *s_wu, *s_wd, *s_sg, *s_su, *s_sd;
};

// Latched device status + control words (first bytes of the workspace).
struct DevStatus {
  int32_t error, step, stage, slot, wg;
  uint32_t observed, expected;
  int32_t xcc_mismatch;
  uint32_t abort;      // non-zero: every workgroup leaves at its next check
  uint32_t pad[7];
};

// Byte offsets of everything inside the caller's workspace.
struct Layout {
  int64_t status, flags, layers, tasks, rope, xcc;
  int64_t x_out, pbuf, q, u, rl, part, lmp, x_emb, a_norm, tok, xmid;
  int64_t pk, ssq;  // micro-batch: packed GEMM inputs, per-workgroup sums of squares
  int64_t ctx;      // the engine's own position array [B] (used when the caller passes none)
  int64_t cmd, req;  // serving loop: the scheduler's command words, the claimed prompt [max_ctx]
  int64_t kvnew;     // fp8 cache: the step's new K and V rows in fp32 [L][B][2][Hkv][d]
  int64_t dpart;     // folded FFN: each gate/up task's partial of the down projection [L][W][h]
  int64_t total;
};

// Shapes derived once from the config.
struct Dims {
  int32_t L, h, Hq, Hkv, d, ffn, V, B, max_ctx;
  int32_t E, top_k, n_shared, effn, moe;
  int32_t G;          // query heads per KV head
  int32_t qkv_pairs;  // RoPE pairs of all QKV rows: Hkv * (G + 2) * d / 2
  int32_t F;          // width of the FFN activation slot (ffn or (top_k+n_shared)*effn)
  int32_t mb;         // micro-batch path (batch > 1): MFMA GEMM stages, balanced attention
  int32_t W, X, NC;   // workgroups, XCDs, attention chunks per (sequence, KV head)
  int32_t local;      // QKV->attention->O-projection hand-offs stay inside one XCD's L2
  int32_t onexcd;     // every workgroup on XCD 0 (small grids): every hand-off stays in its L2
  int32_t Tg;         // workgroups per (sequence, KV head): W / (batch * n_kv_heads); micro-batch: per KV head
  int32_t n_si, stages_per_layer, threads;
  int32_t kmax;       // longest GEMV input, padded
  int32_t ymax;       // most GEMV results one task produces (x waves: LDS partials)
  int32_t segoff;     // LDS float offset of the GEMV segment table (0)
  int32_t mbst;       // micro-batch: longest GEMM input staged in LDS (0: none)
  int32_t npre;       // GEMV: most units of each wavefront's stream loaded straight into LDS first
  int32_t xsoff;      // LDS float offset of the staged GEMV input (segment table, reduction
                      // scratch and partials come first; a task's LDS units follow its input)
  int32_t cmax;       // longest attention chunk (positions; micro-batch: longest piece of one workgroup)
  int32_t lds_bytes;  // dynamic LDS per workgroup
  int32_t kv8;        // fp8 e4m3 K/V cache with an fp32 scale per cached row
  int32_t fold;       // resident kernel: the down projection folded into the gate/up stage
  int32_t inl;        // resident kernel: each O-projection task computes its head's attention itself
  int32_t aoff;       // inline attention: LDS float offset of its scratch (past the staged input)
  float eps, theta;
};

// Workgroup slot lambda (XCD-major logical position) of hardware block b.
// Blocks are dispatched round-robin over the X XCDs, so block b runs on XCD
// b % X; lambda = xcd * (W / X) + b / X keeps consecutive lambdas on one XCD.
PRE_HD inline int32_t lambda_of_block(int32_t b, int32_t W, int32_t X) {
  if (X <= 1 || W % X != 0) return b;
  return (b % X) * (W / X) + b / X;
}
PRE_HD inline int32_t block_of_lambda(int32_t lam, int32_t W, int32_t X) {
  if (X <= 1 || W % X != 0) return lam;
  int32_t per = W / X;
  return (lam % per) * X + lam / per;
}

}  // namespace pre
