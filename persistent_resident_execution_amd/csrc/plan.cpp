// Host-side construction and validation of the decode step's task table.
//
// Built once per engine: it fixes which workgroup computes which rows /
// chunks of every stage of every layer, which ready-flag slots each task
// waits on, and where every activation lives in the workspace.  The
// validator re-derives the producer/consumer relation from the shapes and
// checks the table against it, so a mistake in the builder is caught on the
// host before anything is launched.
#include <algorithm>
#include <cstring>
#include <vector>

#include "../../include/pre.h"
#include "plan.h"

namespace pre {

static int64_t align256(int64_t x) { return (x + 255) & ~int64_t(255); }
static int32_t pad_to(int32_t x, int32_t m) { return (x + m - 1) / m * m; }
static int32_t cdiv(int32_t a, int32_t b) { return (a + b - 1) / b; }
static inline void split(int64_t n, int W, int t, int32_t *lo, int32_t *hi);

int derive_dims(const pre_config *c, int n_cus, Dims *D) {
  if (!c || !D) return PRE_ERR_ARG;
  std::memset(D, 0, sizeof(*D));
  if (c->n_layers < 1 || c->hidden < 8 || c->n_q_heads < 1 || c->n_kv_heads < 1 ||
      c->vocab < 1 || c->max_ctx < 2 || c->batch < 1)
    return PRE_ERR_SHAPE;
  if (c->n_q_heads % c->n_kv_heads) return PRE_ERR_SHAPE;
  if (c->head_dim != 64 && c->head_dim != 128) return PRE_ERR_SHAPE;
  if (c->hidden % 8 || (c->n_q_heads * c->head_dim) % 8) return PRE_ERR_SHAPE;
  if (c->batch > 8) return PRE_ERR_SHAPE;
  // the K/V append addresses a layer's whole cache through one buffer
  // descriptor (32-bit size and offsets), the attention one head's
  if ((int64_t)c->batch * c->n_kv_heads * c->max_ctx * c->head_dim * 2 >= (1ll << 32)) return PRE_ERR_SHAPE;
  const bool moe = c->n_experts > 0;
  const bool mb = c->batch > 1;
  if (c->kv_dtype != 0 && c->kv_dtype != 1) return PRE_ERR_SHAPE;
  // the fp8 cache is built for the batch-1 attention tile
  if (c->kv_dtype == 1 && mb) return PRE_ERR_UNSUPPORTED;
  // micro-batch: dense models whose GEMM inputs come in whole 32-column
  // blocks of the packed MFMA layout
  if (mb && (moe || c->hidden % 32 || c->ffn_dim % 32 || (c->n_q_heads * c->head_dim) % 32))
    return PRE_ERR_UNSUPPORTED;
  if (moe) {
    if (c->expert_dtype != 1 || c->top_k < 1 || c->top_k > c->n_experts || c->top_k > 16 ||
        c->n_shared < 0 || c->n_shared > 4 || c->expert_ffn < 16 || c->expert_ffn % 16 ||
        c->hidden % 16 || c->n_experts > 1024)
      return PRE_ERR_SHAPE;
  } else {
    if (c->ffn_dim < 8 || c->ffn_dim % 8) return PRE_ERR_SHAPE;
  }
  D->kv8 = c->kv_dtype == 1;
  D->L = c->n_layers; D->h = c->hidden; D->Hq = c->n_q_heads; D->Hkv = c->n_kv_heads;
  D->d = c->head_dim; D->ffn = c->ffn_dim; D->V = c->vocab; D->B = c->batch;
  D->max_ctx = c->max_ctx;
  D->mb = mb;
  D->E = moe ? c->n_experts : 0; D->top_k = moe ? c->top_k : 0;
  D->n_shared = moe ? c->n_shared : 0; D->effn = moe ? c->expert_ffn : 0; D->moe = moe;
  D->G = c->n_q_heads / c->n_kv_heads;
  if (D->G > 8) return PRE_ERR_SHAPE;
  D->qkv_pairs = D->Hkv * (D->G + 2) * D->d / 2;
  D->F = moe ? (D->top_k + D->n_shared) * D->effn : D->ffn;
  // default grid: one workgroup per CU, unless a layer's weights are too
  // few to keep that many busy: then about one workgroup per 32 KB of a
  // layer's weights (a multiple of 8, so the XCDs get equal shares)
  if (c->grid_wgs > 0) {
    D->W = c->grid_wgs;
  } else {
    const int64_t h = c->hidden, qkv = (int64_t)(c->n_q_heads + 2 * c->n_kv_heads) * c->head_dim;
    int64_t lb = 2 * h * qkv + 2 * (int64_t)c->n_q_heads * c->head_dim * h;
    if (moe)
      lb += 2 * (int64_t)c->n_experts * h + (int64_t)(c->top_k + c->n_shared) * 3 * c->expert_ffn * h;
    else
      lb += 6 * (int64_t)c->ffn_dim * h;
    const int64_t by_size = std::max<int64_t>(8, lb / (32 * 1024) / 8 * 8);
    D->W = (int32_t)std::min<int64_t>(n_cus, by_size);
    // a small model (at most two XCDs' worth of workgroups) is latency-bound:
    // it runs on one XCD, where every hand-off stays in that XCD's L2
    if (!mb && D->W <= 2 * (n_cus / 8)) D->W = std::min(D->W, n_cus / 8);
  }
  if (D->W < 1 || D->W > 4096) return PRE_ERR_SHAPE;
  D->X = 8;
  const int bg = mb ? D->Hkv : D->B * D->Hkv;
  if (D->Hkv > 8 || D->W < bg) return PRE_ERR_SHAPE;
  // micro-batch: the attention work of KV head g lies on workgroups
  // [g * W / Hkv, (g + 1) * W / Hkv)
  if (mb && D->W % D->Hkv) return PRE_ERR_SHAPE;
  D->Tg = D->W / bg;
  // KV head g's QKV pairs, attention chunks and O-projection slice occupy
  // lambdas [g * W/8, (g + 1) * W/8): one XCD, when there are 8 KV heads and
  // the grid splits evenly over the 8 XCDs
  D->local = c->xcd_local >= 0 && D->Hkv == D->X && D->B == 1 && D->W % D->X == 0;
  // every workgroup on XCD 0 when the grid fits one XCD's CUs (and the
  // per-head placement does not apply)
  D->onexcd = c->xcd_local >= 0 && !D->local && D->B == 1 && D->W <= n_cus / 8;
  // about 128 positions per attention chunk at the longest context, at most
  // 16 chunks (longer chunks cost the matrix-core attention little, and the
  // O projection's combine reads one record per chunk) and at most one chunk
  // per workgroup of the (sequence, KV head)'s share
  D->NC = c->attn_splits > 0 ? c->attn_splits : std::min({D->Tg, 16, std::max(1, cdiv(c->max_ctx, 128))});
  if (mb) D->NC = 1;  // the micro-batch attention split follows the contexts of each step
  if (D->NC > D->Tg) return PRE_ERR_SHAPE;
  D->threads = c->wg_threads > 0 ? c->wg_threads : 512;
  if (D->threads % 64 || D->threads < 128 || D->threads > 512) return PRE_ERR_SHAPE;
  // micro-batch: wavefronts split a batch's row groups evenly (a power of
  // two), and the LM head keeps one wavefront per sequence
  if (mb && ((D->threads & (D->threads - 1)) || D->threads < 64 * D->B)) return PRE_ERR_SHAPE;
  // Folded FFN (small one-XCD dense engines with a bf16 cache, resident
  // kernel only): each
  // gate/up task also forms its slice's partial of the down projection, so
  // the down stage and its hand-off drop out.  Thread t of the task holds
  // row t of Wd's columns [r0, r1) in registers, in 16-byte units (so r0 is
  // a multiple of 8 and there are at most FOLD_U units); every workgroup
  // must produce QKV pairs, so that the output projection's waits cover
  // every workgroup's share of the residual it writes while staging.
  if (c->fold_ffn >= 0 && !moe && !mb && !D->kv8 && D->onexcd && D->h <= D->threads &&
      D->qkv_pairs >= D->W && D->W <= 32) {
    bool ok = true;
    for (int lam = 0; lam < D->W && ok; ++lam) {
      int32_t r0, r1;
      split(D->ffn, D->W, lam, &r0, &r1);
      ok = r0 % 8 == 0 && r1 - r0 <= 8 * FOLD_U;
    }
    D->fold = ok;
  }
  D->stages_per_layer = (moe || mb) ? 6 : 5;
  // micro-batch: an embedding stage first, then per layer QKV, ATTN, COMB,
  // OPROJ, GU, DOWN, then the LM head
  D->n_si = D->L * D->stages_per_layer + (mb ? 2 : 1);
  // longest staged GEMV input; the fp8 expert-down chunks of the last slot
  // read up to (slots - 1) * effn + effn rounded up to whole 1024-column chunks
  const int nk = D->top_k + D->n_shared;
  D->kmax = pad_to(std::max({D->h, D->Hq * D->d, D->F, moe ? D->E : 0,
                             moe ? (nk - 1) * D->effn + pad_to(D->effn, 1024) : 0}), 1024);
  // micro-batch: a workgroup's share of one KV head's positions of all sequences
  // (in sub-pieces of at most 16K / G positions: the scores stay within 64 KB of LDS)
  D->cmax = mb ? std::min(cdiv(D->B * D->max_ctx, D->Tg) + 1, std::max(64, 16384 / D->G))
               : cdiv(D->max_ctx, D->NC);
  const int waves = D->threads / 64;
  {
    // results (2 per row pair) of the largest task of any GEMV stage
    const int W = D->W;
    auto rows2 = [](int r) { return r + (r & 1); };  // consecutive-row pairs
    int y = std::max({2 * cdiv(D->qkv_pairs, W), rows2(cdiv(D->h, W)), rows2(cdiv(D->V, W)),
                      rows2(cdiv(D->h, D->Tg))});
    if (moe) y = std::max({y, rows2(cdiv(D->E, W)), 2 * cdiv(D->F, W), rows2(cdiv(D->h, W)) * nk});
    else y = std::max(y, 2 * cdiv(D->ffn, W));
    D->ymax = pad_to(y, 64);
  }
  // GEMV phase: segment table (80 entries of 12 words), reduction scratch,
  // per-row results, then the staged input; the output projection's chunk
  // combine writes its result into the staged input and needs no scratch.
  // Attention phase: q, scores, per-wave output partials, softmax stats.
  D->segoff = 0;
  D->xsoff = (int32_t)pad_to(80 * 12 + 256 + (int64_t)D->ymax * waves, 64);
  int64_t gemv = (int64_t)D->xsoff + D->kmax;
  int64_t attn = (int64_t)D->G * D->d + (int64_t)D->G * pad_to(D->cmax, 64) +
                 (int64_t)waves * D->G * D->d + 4 * D->G + 256;
  // the chunk's K and V row scales, the newest row's K and V codes
  if (D->kv8) attn += 2 * (int64_t)pad_to(D->cmax, 64) + D->d / 2;
  if (mb) {
    // MFMA stages: per-wavefront partials (8 sequences x 16 rows), the
    // sequences' norm scales and sums, per-thread partials, and the packed
    // input (32 bytes per column) when the hidden-size inputs fit beside
    // them; attention: the running state of a piece (output, max, sum)
    const int64_t base = (int64_t)waves * 8 * 16 + 16 + 512;
    // (staged in whole 128-column steps: the tail past K is zero-filled)
    const int64_t kst = pad_to(std::max(D->h, D->Hq * D->d), 128);
    D->mbst = (base + kst * 8) * 4 <= 150 * 1024 ? (int32_t)kst : 0;
    gemv = base + (int64_t)D->mbst * 8;
    attn += (int64_t)D->G * D->d + 4 * D->G;
  }
  // The head of every batch-1 GEMV stream (up to PRE_UNITS units of 2 KB per
  // wavefront) goes straight into LDS after the task's staged input, in
  // what the CU's 160 KB leave; the workgroup then takes all of them.  Not
  // on one XCD, where the streams are short and the hand-offs' latency is
  // the whole cost.
  int64_t base = std::max(gemv, attn);
  // Attention folded into the output projection (small one-XCD batch-1
  // engines, bf16 cache, resident kernel only): each O-projection task runs
  // its KV head's attention over every position before its own stream, with
  // the scores of the whole context in LDS past the staged input.
  if (c->fold_attn >= 0 && !mb && !D->kv8 && D->B == 1 && D->onexcd) {
    const int64_t aoff = pad_to(D->xsoff + (int64_t)D->kmax, 64);
    const int64_t need = (int64_t)D->G * D->d + (int64_t)D->G * pad_to(D->max_ctx, 64) +
                         (int64_t)waves * D->G * D->d + 4 * D->G + 256;
    if ((aoff + need) * 4 <= 150 * 1024) {
      D->inl = 1;
      D->aoff = (int32_t)aoff;
      base = std::max(base, aoff + need);
    }
  }
  D->npre = (mb || D->onexcd) ? 0 : PRE_UNITS;
  // (1 KB of the 160 KB stays for the kernels' static LDS)
  D->lds_bytes = (int32_t)((D->npre ? std::max<int64_t>(base, 40704) : base) * 4);
  if (D->lds_bytes > 160 * 1024) return PRE_ERR_SHAPE;
  D->eps = c->rms_eps;
  D->theta = c->rope_theta;
  return PRE_OK;
}

void build_layout(const Dims &D, Layout *Lo) {
  int64_t off = 0;
  auto take = [&](int64_t bytes) { int64_t o = off; off = align256(off + bytes); return o; };
  const int64_t f = 4;
  Lo->status = take(sizeof(DevStatus));
  Lo->flags = take((int64_t)D.n_si * D.W * 4);
  Lo->layers = take((int64_t)D.L * sizeof(DevLayer));
  Lo->tasks = take((int64_t)D.n_si * D.W * sizeof(Task));
  Lo->rope = take((int64_t)D.max_ctx * D.d * f);          // cos then sin, [pos][d/2] each
  Lo->xcc = take((int64_t)D.W * 4);
  Lo->x_out = take((int64_t)D.L * D.B * D.h * f);
  Lo->pbuf = take((int64_t)D.L * D.B * D.Hkv * D.h * f);  // O-projection partial per KV head
  Lo->q = take((int64_t)D.L * D.B * D.Hq * D.d * f);
  Lo->u = take((int64_t)D.L * D.B * D.F * f);
  Lo->rl = take((int64_t)D.L * D.B * std::max(D.E, 1) * f);
  Lo->part = take((int64_t)D.L * D.B * D.Hkv * D.NC * D.G * (D.d + 4) * f);  // records m, l, -, -, o[d]
  Lo->lmp = take((int64_t)D.W * D.B * 8);
  Lo->x_emb = take((int64_t)D.B * D.h * f);
  Lo->a_norm = take((int64_t)D.B * D.kmax * f);
  Lo->tok = take((int64_t)D.B * 4 * 4);
  Lo->xmid = take((int64_t)D.L * D.B * D.h * f);  // post-attention residual (MoE layers, micro-batch)
  Lo->ctx = take((int64_t)D.B * 4);
  Lo->cmd = take(64);
  Lo->req = take((int64_t)D.max_ctx * 4);
  Lo->kvnew = D.kv8 ? take((int64_t)D.L * D.B * 2 * D.Hkv * D.d * f) : 0;
  Lo->dpart = D.fold ? take((int64_t)D.L * D.W * D.h * f) : 0;
  if (D.mb) {
    // packed bf16 hi/lo GEMM inputs: 4 KB per 128 columns (whole steps, the
    // tail left zero); per layer the QKV input (plus the LM head's), the
    // gate/up input, the down input and the O-projection input
    const int64_t kh = (int64_t)cdiv(D.h, 128) * 4096, kf = (int64_t)cdiv(D.ffn, 128) * 4096,
                  ko = (int64_t)cdiv(D.Hq * D.d, 128) * 4096;
    Lo->pk = take((2 * (int64_t)D.L + 1) * kh + D.L * (kf + ko));
    Lo->ssq = take((2 * (int64_t)D.L + 1) * D.W * D.B * f);
    // attention records of every (workgroup, sequence) of a layer
    Lo->part = take((int64_t)D.L * D.W * D.B * D.G * (D.d + 4) * f);
  } else {
    Lo->pk = Lo->ssq = 0;
  }
  Lo->total = off;
}

// Balanced split of n items over W tasks.
static inline void split(int64_t n, int W, int t, int32_t *lo, int32_t *hi) {
  *lo = (int32_t)(n * t / W);
  *hi = (int32_t)(n * (t + 1) / W);
}

static inline int32_t slot(const Dims &D, int si, int i) { return si * D.W + i; }

// Balanced split of n items (a multiple of 8) in whole groups of 8.
static inline void split8(int64_t n, int W, int t, int32_t *lo, int32_t *hi) {
  const int64_t u = n / 8;
  *lo = (int32_t)(8 * (u * t / W));
  *hi = (int32_t)(8 * (u * (t + 1) / W));
}

// Micro-batch table.  Per step: EMBED; per layer QKV, ATTN, COMB, OPROJ,
// GU, DOWN; LM.  Every stage has one task per workgroup.  KV head g's QKV
// rows, attention share and combine lie on workgroups [g * Tw, (g + 1) * Tw)
// (Tw = W / Hkv, lambda XCD-major), the other stages split rows evenly.
static void build_tasks_mb(const Dims &D, std::vector<Task> &T) {
  const int W = D.W, Tw = D.Tg;
  T.assign((size_t)D.n_si * W, Task{});
  auto at = [&](int si, int lam) -> Task & { return T[(size_t)si * W + lam]; };
  auto all = [&](Task &t, int si_prod) { t.wait_lo = slot(D, si_prod, 0); t.wait_hi = slot(D, si_prod, W); };
  const int P = D.qkv_pairs, PG = P / D.Hkv;
  for (int lam = 0; lam < W; ++lam) {
    Task &t = at(0, lam);
    t.op = OP_EMBED; t.layer = 0;
    split8(D.h, W, lam, &t.r0, &t.r1);
    t.wait_lo = t.wait_hi = 0;  // the step's tokens are known to every workgroup
    t.signal = slot(D, 0, lam);
  }
  for (int l = 0; l < D.L; ++l) {
    const int s_q = 1 + 6 * l, s_a = s_q + 1, s_c = s_q + 2, s_o = s_q + 3, s_gu = s_q + 4, s_dn = s_q + 5;
    for (int lam = 0; lam < W; ++lam) {
      Task &q = at(s_q, lam);
      q.op = OP_QKV; q.layer = l;
      split(P, W, lam, &q.r0, &q.r1);
      all(q, s_q - 1);  // EMBED or the previous layer's DOWN
      q.signal = slot(D, s_q, lam);
      const int g = lam / Tw, i = lam % Tw;
      Task &a = at(s_a, lam);
      a.op = OP_ATTN; a.layer = l; a.aux = g; a.r0 = i; a.r1 = Tw;
      int lo = -1, hi = -1;  // QKV tasks whose pairs meet KV head g's
      for (int w = 0; w < W; ++w) {
        int32_t x0, x1;
        split(P, W, w, &x0, &x1);
        if (x0 < x1 && x0 < (g + 1) * PG && x1 > g * PG) {
          if (lo < 0) lo = w;
          hi = w + 1;
        }
      }
      a.wait_lo = slot(D, s_q, lo); a.wait_hi = slot(D, s_q, hi);
      a.signal = slot(D, s_a, lam);
      Task &c = at(s_c, lam);
      c.op = OP_COMB; c.layer = l; c.aux = g;
      split8((int64_t)D.B * D.G * D.d, Tw, i, &c.r0, &c.r1);
      c.wait_lo = slot(D, s_a, g * Tw); c.wait_hi = slot(D, s_a, (g + 1) * Tw);
      c.signal = slot(D, s_c, lam);
      Task &o = at(s_o, lam);
      o.op = OP_OPROJ; o.layer = l; o.aux = -1;
      split8(D.h, W, lam, &o.r0, &o.r1);
      all(o, s_c);
      o.signal = slot(D, s_o, lam);
      Task &gu = at(s_gu, lam);
      gu.op = OP_GU; gu.layer = l;
      split8(D.ffn, W, lam, &gu.r0, &gu.r1);
      all(gu, s_o);
      gu.signal = slot(D, s_gu, lam);
      Task &dn = at(s_dn, lam);
      dn.op = OP_DOWN; dn.layer = l;
      split8(D.h, W, lam, &dn.r0, &dn.r1);
      all(dn, s_gu);
      dn.signal = slot(D, s_dn, lam);
    }
  }
  const int s_lm = D.n_si - 1;
  for (int lam = 0; lam < W; ++lam) {
    Task &t = at(s_lm, lam);
    t.op = OP_LM; t.layer = D.L;
    split(D.V, W, lam, &t.r0, &t.r1);
    all(t, s_lm - 1);
    t.signal = slot(D, s_lm, lam);
  }
}

void build_tasks(const Dims &D, std::vector<Task> &T) {
  if (D.mb) { build_tasks_mb(D, T); return; }
  const int W = D.W, spl = D.stages_per_layer;
  T.assign((size_t)D.n_si * W, Task{});
  auto at = [&](int si, int lam) -> Task & { return T[(size_t)si * W + lam]; };
  const int P = D.qkv_pairs, PG = P / D.Hkv;  // pairs per KV group
  for (int l = 0; l < D.L; ++l) {
    const int s_qkv = l * spl, s_attn = s_qkv + 1, s_o = s_qkv + 2;
    const int s_prev = l > 0 ? l * spl - 1 : -1;  // previous layer's last FFN stage
    for (int lam = 0; lam < W; ++lam) {
      Task &t = at(s_qkv, lam);
      t.op = OP_QKV; t.layer = l;
      split(P, W, lam, &t.r0, &t.r1);
      t.wait_lo = s_prev >= 0 ? slot(D, s_prev, 0) : 0;
      t.wait_hi = s_prev >= 0 ? slot(D, s_prev, W) : 0;
      t.signal = slot(D, s_qkv, lam);
    }
    // attention chunk c of (sequence, KV head) bg on workgroup bg * Tg + c:
    // the XCD that computed that head's QKV rows (lambda is XCD-major)
    for (int lam = 0; lam < W; ++lam) {
      Task &t = at(s_attn, lam);
      const int bg = lam / D.Tg, c = lam % D.Tg;
      if (bg >= D.B * D.Hkv || c >= D.NC) { t.op = OP_NONE; t.signal = -1; continue; }
      const int g = bg % D.Hkv;
      t.op = OP_ATTN; t.layer = l; t.r0 = c; t.r1 = D.NC; t.aux = bg;
      // producers: QKV tasks whose pair range meets group g's pairs
      int lo = -1, hi = -1;
      for (int q = 0; q < W; ++q) {
        int32_t a, b;
        split(P, W, q, &a, &b);
        if (a < b && a < (g + 1) * PG && b > g * PG) {
          if (lo < 0) lo = q;
          hi = q + 1;
        }
      }
      t.wait_lo = slot(D, s_attn - 1, lo);
      t.wait_hi = slot(D, s_attn - 1, hi);
      t.signal = slot(D, s_attn, lam);
    }
    // output projection, split over KV heads: workgroup bg * Tg + i combines
    // head bg's chunks and multiplies rows i of Wo's column slice for bg
    for (int lam = 0; lam < W; ++lam) {
      Task &t = at(s_o, lam);
      const int bg = lam / D.Tg, i = lam % D.Tg;
      t.op = OP_OPROJ; t.layer = l;
      if (bg < D.B * D.Hkv) {
        t.aux = bg;
        split(D.h, D.Tg, i, &t.r0, &t.r1);
      } else {  // left-over workgroup: no rows, still takes part in the stage
        t.aux = 0; t.r0 = t.r1 = 0;
      }
      t.wait_lo = slot(D, s_attn, t.aux * D.Tg);
      t.wait_hi = slot(D, s_attn, t.aux * D.Tg + D.NC);
      t.signal = slot(D, s_o, lam);
    }
    if (!D.moe) {
      const int s_gu = s_qkv + 3, s_dn = s_qkv + 4;
      for (int lam = 0; lam < W; ++lam) {
        Task &g = at(s_gu, lam);
        g.op = OP_GU; g.layer = l;
        split(D.ffn, W, lam, &g.r0, &g.r1);
        g.wait_lo = slot(D, s_o, 0); g.wait_hi = slot(D, s_o, W);
        g.signal = slot(D, s_gu, lam);
        Task &dn = at(s_dn, lam);
        dn.op = OP_DOWN; dn.layer = l;
        split(D.h, W, lam, &dn.r0, &dn.r1);
        dn.wait_lo = slot(D, s_gu, 0); dn.wait_hi = slot(D, s_gu, W);
        dn.signal = slot(D, s_dn, lam);
      }
    } else {
      const int s_r = s_qkv + 3, s_egu = s_qkv + 4, s_ed = s_qkv + 5;
      for (int lam = 0; lam < W; ++lam) {
        Task &r = at(s_r, lam);
        r.op = OP_ROUTER; r.layer = l;
        split(D.E, W, lam, &r.r0, &r.r1);
        r.wait_lo = slot(D, s_o, 0); r.wait_hi = slot(D, s_o, W);
        r.signal = slot(D, s_r, lam);
        Task &g = at(s_egu, lam);
        g.op = OP_EGU; g.layer = l;
        split(D.F, W, lam, &g.r0, &g.r1);
        g.wait_lo = slot(D, s_r, 0); g.wait_hi = slot(D, s_r, W);
        g.signal = slot(D, s_egu, lam);
        Task &dn = at(s_ed, lam);
        dn.op = OP_EDOWN; dn.layer = l;
        split(D.h, W, lam, &dn.r0, &dn.r1);
        dn.wait_lo = slot(D, s_egu, 0); dn.wait_hi = slot(D, s_egu, W);
        dn.signal = slot(D, s_ed, lam);
      }
    }
  }
  const int s_lm = D.L * spl, s_last = s_lm - 1;
  for (int lam = 0; lam < W; ++lam) {
    Task &t = at(s_lm, lam);
    t.op = OP_LM; t.layer = D.L;
    split(D.V, W, lam, &t.r0, &t.r1);
    t.wait_lo = slot(D, s_last, 0); t.wait_hi = slot(D, s_last, W);
    t.signal = slot(D, s_lm, lam);
  }
}

// Expected op of a stage instance.
static int32_t op_of_stage(const Dims &D, int si) {
  if (D.mb) {
    static const int32_t mbs[6] = {OP_QKV, OP_ATTN, OP_COMB, OP_OPROJ, OP_GU, OP_DOWN};
    if (si == 0) return OP_EMBED;
    if (si == D.n_si - 1) return OP_LM;
    return mbs[(si - 1) % 6];
  }
  if (si == D.L * D.stages_per_layer) return OP_LM;
  const int k = si % D.stages_per_layer;
  static const int32_t dense[5] = {OP_QKV, OP_ATTN, OP_OPROJ, OP_GU, OP_DOWN};
  static const int32_t moe[6] = {OP_QKV, OP_ATTN, OP_OPROJ, OP_ROUTER, OP_EGU, OP_EDOWN};
  return D.moe ? moe[k] : dense[k];
}

// Rows (or pairs, or chunks) a GEMV stage must cover.
static int64_t coverage_target(const Dims &D, int32_t op) {
  switch (op) {
    case OP_QKV: return D.qkv_pairs;
    case OP_OPROJ: case OP_DOWN: case OP_EDOWN: return D.h;
    case OP_GU: return D.ffn;
    case OP_ROUTER: return D.E;
    case OP_EGU: return D.F;
    case OP_LM: return D.V;
    default: return -1;
  }
}

// Returns 0 if every check passes, else the number of the first failed one:
//  1 table size; 2 op of each task matches its stage; 3 wait ranges point
//  only at slots of earlier stage instances that some task sets; 4 no two
//  stage instances' tasks set the same slot and each GEMV task sets its own;
//  5 row/pair coverage exactly once per GEMV stage; 6 every attention
//  (sequence, KV head) has each chunk exactly once; 7 every consumer waits on
//  all producers of its input; 8 every workgroup takes part in every GEMV
//  stage (this orders slot reuse across steps); 9 layer numbers.
// The micro-batch table: checks 1-4 and 9 as below; 5 row coverage (in
// whole groups of 8 where the output is packed) and the combine's element
// coverage per KV head; 6 every KV head has Tw attention tasks numbered
// 0..Tw-1; 7 producer sets; 8 no empty task slot.
static int validate_mb(const Dims &D, const std::vector<Task> &T) {
  const int W = D.W, n_slots = D.n_si * W, Tw = D.Tg;
  if ((int64_t)T.size() != (int64_t)D.n_si * W) return 1;
  for (int si = 0; si < D.n_si; ++si)
    for (int lam = 0; lam < W; ++lam) {
      const Task &t = T[(size_t)si * W + lam];
      if (t.op == OP_NONE) return 8;
      if (t.op != op_of_stage(D, si)) return 2;
      if (t.signal != si * W + lam) return 4;
      if (t.wait_lo < 0 || t.wait_hi < t.wait_lo || t.wait_hi > si * W) return 3;
      const int want_layer = si == 0 ? 0 : (t.op == OP_LM ? D.L : (si - 1) / 6);
      if (t.layer != want_layer) return 9;
    }
  const int PG = D.qkv_pairs / D.Hkv;
  for (int si = 0; si < D.n_si; ++si) {
    const int32_t op = op_of_stage(D, si);
    const Task *row = &T[(size_t)si * W];
    if (op == OP_ATTN) {
      for (int lam = 0; lam < W; ++lam)
        if (row[lam].aux != lam / Tw || row[lam].r0 != lam % Tw || row[lam].r1 != Tw) return 6;
      continue;
    }
    if (op == OP_COMB) {
      const int64_t n = (int64_t)D.B * D.G * D.d;
      for (int g = 0; g < D.Hkv; ++g) {
        int64_t next = 0;
        for (int i = 0; i < Tw; ++i) {
          const Task &t = row[g * Tw + i];
          if (t.aux != g || t.r0 != next || t.r1 < t.r0 || t.r0 % 8 || t.r1 % 8) return 5;
          next = t.r1;
        }
        if (next != n) return 5;
      }
      continue;
    }
    const int64_t n = op == OP_EMBED || op == OP_OPROJ || op == OP_DOWN ? D.h
                      : op == OP_GU ? D.ffn : op == OP_QKV ? D.qkv_pairs : D.V;
    const bool by8 = op != OP_QKV && op != OP_LM;
    int64_t next = 0;
    for (int lam = 0; lam < W; ++lam) {  // contiguous, in workgroup order
      const Task &t = row[lam];
      if (t.r0 != next || t.r1 < t.r0 || (by8 && (t.r0 % 8 || t.r1 % 8))) return 5;
      next = t.r1;
    }
    if (next != n) return 5;
  }
  for (int si = 0; si < D.n_si; ++si) {
    const int32_t op = op_of_stage(D, si);
    for (int lam = 0; lam < W; ++lam) {
      const Task &t = T[(size_t)si * W + lam];
      bool ok = true;
      if (op == OP_EMBED) {
        ok = t.wait_lo == t.wait_hi;
      } else if (op == OP_ATTN) {
        const int g = t.aux;
        for (int q = 0; q < W && ok; ++q) {
          const Task &p = T[(size_t)(si - 1) * W + q];
          if (p.r0 < p.r1 && p.r0 < (g + 1) * PG && p.r1 > g * PG)
            ok = t.wait_lo <= (si - 1) * W + q && t.wait_hi > (si - 1) * W + q;
        }
      } else if (op == OP_COMB) {
        ok = t.wait_lo <= (si - 1) * W + t.aux * Tw && t.wait_hi >= (si - 1) * W + (t.aux + 1) * Tw;
      } else {
        ok = t.wait_lo <= (si - 1) * W && t.wait_hi >= si * W;
      }
      if (!ok) return 7;
    }
  }
  (void)n_slots;
  return 0;
}

int validate(const Dims &D, const std::vector<Task> &T) {
  if (D.mb) return validate_mb(D, T);
  const int W = D.W, n_slots = D.n_si * W;
  if ((int64_t)T.size() != (int64_t)D.n_si * W) return 1;
  std::vector<int> setter_si(n_slots, -1);
  for (int si = 0; si < D.n_si; ++si) {
    const int32_t want = op_of_stage(D, si);
    for (int lam = 0; lam < W; ++lam) {
      const Task &t = T[(size_t)si * W + lam];
      if (t.op != want && !(want == OP_ATTN && t.op == OP_NONE)) return 2;
      if (t.op == OP_NONE) continue;
      if (t.signal < 0 || t.signal >= n_slots || t.signal / W != si) return 4;
      if (setter_si[t.signal] >= 0 && setter_si[t.signal] != si) return 4;
      setter_si[t.signal] = si;
      if (t.signal != si * W + lam) return 4;
    }
  }
  for (int si = 0; si < D.n_si; ++si)
    for (int lam = 0; lam < W; ++lam) {
      const Task &t = T[(size_t)si * W + lam];
      if (t.op == OP_NONE) continue;
      if (t.wait_lo < 0 || t.wait_hi < t.wait_lo || t.wait_hi > n_slots) return 3;
      for (int s = t.wait_lo; s < t.wait_hi; ++s)
        if (setter_si[s] < 0 || setter_si[s] >= si) return 3;
      const int want_layer = (t.op == OP_LM) ? D.L : si / D.stages_per_layer;
      if (t.layer != want_layer) return 9;
    }
  // coverage
  for (int si = 0; si < D.n_si; ++si) {
    const int32_t op = op_of_stage(D, si);
    if (op == OP_ATTN) {
      std::vector<int> seen((size_t)D.B * D.Hkv * D.NC, 0);
      for (int lam = 0; lam < W; ++lam) {
        const Task &t = T[(size_t)si * W + lam];
        if (t.op != OP_ATTN) continue;
        if (t.aux < 0 || t.aux >= D.B * D.Hkv || t.r0 < 0 || t.r0 >= D.NC || t.r1 != D.NC) return 6;
        seen[(size_t)t.aux * D.NC + t.r0]++;
      }
      for (int v : seen) if (v != 1) return 6;
      continue;
    }
    const int64_t n = coverage_target(D, op);
    const int copies = op == OP_OPROJ ? D.B * D.Hkv : 1;  // O-projection: every row once per head
    std::vector<int> cnt((size_t)n * copies, 0);
    for (int lam = 0; lam < W; ++lam) {
      const Task &t = T[(size_t)si * W + lam];
      if (t.r0 < 0 || t.r1 < t.r0 || t.r1 > n) return 5;
      const int k = op == OP_OPROJ ? t.aux : 0;
      if (k < 0 || k >= copies) return 5;
      for (int r = t.r0; r < t.r1; ++r) cnt[(size_t)k * n + r]++;
    }
    for (int v : cnt) if (v != 1) return 5;
  }
  // dependencies: the exact producer set each consumer needs
  auto covers = [&](const Task &t, int si_prod, int lo, int hi) {
    // every slot si_prod*W + [lo, hi) inside the wait range
    return t.wait_lo <= si_prod * W + lo && t.wait_hi >= si_prod * W + hi;
  };
  const int spl = D.stages_per_layer;
  const int PG = D.qkv_pairs / D.Hkv;
  for (int si = 0; si < D.n_si; ++si) {
    const int32_t op = op_of_stage(D, si);
    for (int lam = 0; lam < W; ++lam) {
      const Task &t = T[(size_t)si * W + lam];
      if (t.op == OP_NONE) continue;
      bool ok = true;
      switch (op) {
        case OP_QKV: if (si > 0) ok = covers(t, si - 1, 0, W); break;
        case OP_ATTN: {
          const int g = t.aux % D.Hkv;
          for (int q = 0; q < W && ok; ++q) {
            const Task &p = T[(size_t)(si - 1) * W + q];
            if (p.r0 < p.r1 && p.r0 < (g + 1) * PG && p.r1 > g * PG) ok = covers(t, si - 1, q, q + 1);
          }
          break;
        }
        case OP_OPROJ:  // every chunk task of its (sequence, KV head)
          for (int q = 0; q < W && ok; ++q) {
            const Task &p = T[(size_t)(si - 1) * W + q];
            if (p.op == OP_ATTN && p.aux == t.aux) ok = covers(t, si - 1, q, q + 1);
          }
          break;
        case OP_LM: ok = covers(t, si - 1, 0, W); break;
        default: ok = covers(t, si - 1, 0, W); break;  // GU, DOWN, ROUTER, EGU, EDOWN
      }
      if (!ok) return 7;
    }
    if (op != OP_ATTN)
      for (int lam = 0; lam < W; ++lam)
        if (T[(size_t)si * W + lam].op == OP_NONE) return 8;
  }
  (void)spl;
  return 0;
}

int64_t step_bytes(const pre_config *c, const int32_t *pos) {
  if (c->n_layers < 1 || c->hidden < 1 || c->batch < 1 || c->batch > 8) return -1;
  const int64_t h = c->hidden, d = c->head_dim, L = c->n_layers;
  int64_t w = 0;
  w += (int64_t)(c->n_q_heads + 2 * c->n_kv_heads) * d * h * 2;  // qkv
  w += h * c->n_q_heads * d * 2;                                   // o
  w += 2 * h * 2;                                                  // norms
  if (c->n_experts > 0) {
    const int64_t f = c->expert_ffn;
    const int64_t blk_up = ((f + 127) / 128) * ((h + 127) / 128) * 2;
    const int64_t per = 3 * f * h + 3 * blk_up;
    w += (int64_t)c->n_experts * h * 2;                          // router
    w += (int64_t)(c->top_k + c->n_shared) * per;                // active experts
  } else {
    w += 3 * (int64_t)c->ffn_dim * h * 2;
  }
  int64_t total = w * L + (int64_t)c->vocab * h * 2 + h * 2;     // LM head + final norm
  for (int b = 0; b < c->batch; ++b) {
    total += h * 2;                                              // embedding row
    // one position, K or V: bf16 rows, or fp8 codes plus an fp32 scale per head
    const int64_t kv_row = c->kv_dtype == 1 ? (int64_t)c->n_kv_heads * (d + 4) : (int64_t)c->n_kv_heads * d * 2;
    total += L * 2 * kv_row * ((int64_t)pos[b] + 1);             // attend 0..pos
    total += L * 2 * kv_row;                                     // append at pos
  }
  return total;
}

}  // namespace pre

extern "C" int pre_plan_describe(const pre_config *cfg, pre_plan_info *out, int32_t *h_tasks,
                                 int32_t max_tasks) {
  if (!cfg || !out) return PRE_ERR_ARG;
  pre::Dims D;
  int rc = pre::derive_dims(cfg, 256, &D);
  if (rc != PRE_OK) return rc;
  std::vector<pre::Task> T;
  pre::build_tasks(D, T);
  pre::Layout Lo;
  pre::build_layout(D, &Lo);
  out->n_stage_inst = D.n_si;
  out->n_wgs = D.W;
  out->n_slots = D.n_si * D.W;
  out->n_tasks = (int32_t)T.size();
  out->attn_splits = D.NC;
  out->validator = pre::validate(D, T);
  out->xcd_local = D.local ? 1 : D.onexcd ? 2 : 0;
  out->fold_ffn = D.fold;
  out->fold_attn = D.inl;
  out->workspace_bytes = Lo.total;
  if (h_tasks)
    for (int32_t i = 0; i < max_tasks && i < (int32_t)T.size(); ++i)
      std::memcpy(h_tasks + 8 * (int64_t)i, &T[i], sizeof(pre::Task));
  return PRE_OK;
}

extern "C" int pre_plan_validate(const pre_config *cfg, const int32_t *h_tasks, int32_t n_tasks) {
  if (!cfg || !h_tasks) return PRE_ERR_ARG;
  pre::Dims D;
  int rc = pre::derive_dims(cfg, 256, &D);
  if (rc != PRE_OK) return rc;
  std::vector<pre::Task> T((size_t)std::max(n_tasks, 0));
  if (n_tasks > 0) std::memcpy(T.data(), h_tasks, sizeof(pre::Task) * (size_t)n_tasks);
  return pre::validate(D, T);
}

extern "C" int64_t pre_step_bytes(const pre_config *cfg, const int32_t *h_pos) {
  if (!cfg || !h_pos) return -1;
  return pre::step_bytes(cfg, h_pos);
}
