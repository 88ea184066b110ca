// Persistent resident decode engine: tile device functions, the resident
// kernel, the one-kernel-per-operator baseline and the C ABI of pre.h.
//
// One workgroup per CU walks the host-built task table (plan.h) once per
// decode step.  Before each task it spins on the ready flags of the task's
// producers, afterwards it publishes its own flag.  RMSNorm is folded into
// the projection that consumes it (each consumer normalises its staged copy
// of the residual stream), RoPE and the bf16 KV append run in the QKV
// epilogue, SwiGLU in the gate/up epilogue, residual adds in the O/down
// epilogues, and the greedy token is reduced on the device by every
// workgroup at the end of the step, so the next step starts without the host
// (persistent-execution survey sections 1, 4 and 6.2; TileRT notes,
// "persistent engine kernel" and "tile pipeline").
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../../include/pre.h"
#include "device.h"
#include "plan.h"

namespace pre {
int derive_dims(const pre_config *c, int n_cus, Dims *D);
void build_layout(const Dims &D, Layout *Lo);
void build_tasks(const Dims &D, std::vector<Task> &T);
int validate(const Dims &D, const std::vector<Task> &T);

// Everything a kernel needs, passed by value (kernel argument segment).
struct KP {
  // shapes
  int32_t L, h, Hq, Hkv, d, ffn, V, B, max_ctx, E, top_k, n_shared, effn, moe, G, F, W, X, NC, Tg;
  int32_t n_si, spl, kmax, ymax, cmax, lds_floats;
  int32_t nthr, nw;  // threads and wavefronts per workgroup (scalar: never re-read from the dispatch packet)
  float eps, attn_scale;
  // model
  const DevLayer *layers;
  const uint16_t *embed, *final_norm, *lm_head;
  uint16_t *kc, *vc;
  // workspace
  const Task *tasks;
  uint32_t *flags, *xcc;
  DevStatus *status;
  const float *rope;
  float *x_out, *pbuf, *q, *u, *rl, *part, *lmp, *x_emb, *a_norm;
  int32_t *tok_slot;
  // this call
  int32_t n_steps, pos0;
  uint32_t epoch_base, watchdog_ticks;
  const int32_t *in_tok, *forced;
  int32_t *out_tok;
  float *chk_logits, *chk_hidden;
  uint32_t *trace;
  uint32_t trace_cap;
  int32_t persistent;
};

// ---------------------------------------------------------------------------
// ---------------------------------------------------------------------------
// error latch / abort

__device__ __forceinline__ void latch_error(const KP &P, int kind, int step, int stage, int slot,
                                            uint32_t obs, uint32_t expd) {
  int32_t zero = 0;
  if (__hip_atomic_compare_exchange_strong(&P.status->error, &zero, kind, __ATOMIC_RELAXED,
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
    st_flag(reinterpret_cast<uint32_t *>(&P.status->step), (uint32_t)step);
    st_flag(reinterpret_cast<uint32_t *>(&P.status->stage), (uint32_t)stage);
    st_flag(reinterpret_cast<uint32_t *>(&P.status->slot), (uint32_t)slot);
    st_flag(reinterpret_cast<uint32_t *>(&P.status->wg), blockIdx.x);
    st_flag(&P.status->observed, obs);
    st_flag(&P.status->expected, expd);
  }
  drain();
  st_flag(&P.status->abort, 1u);
}

// Spin (wave 0) until flags[lo..hi) >= ep; all threads return the same
// verdict.  Bounded by the watchdog; leaves early if another workgroup
// aborted.
__device__ __forceinline__ bool wait_slots(const KP &P, int lo, int hi, uint32_t ep, int step,
                                           int stage, int *sh) {
  if (lo >= hi) return true;
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const uint64_t t0 = now_ticks();
    int verdict = 1, iter = 0;
    while (true) {
      bool ok = true;
      uint32_t seen = ep;
      int bad = -1;
      for (int i = lo + lane; i < hi; i += 64) {
        uint32_t v = ld_flag(P.flags + i);
        if ((int32_t)(v - ep) < 0) { ok = false; seen = v; bad = i; }
      }
      if (__all(ok)) break;
      if ((++iter & 15) == 0) {
        if (ld_flag(&P.status->abort)) { verdict = 0; break; }
        if (now_ticks() - t0 > P.watchdog_ticks) {
          uint64_t m = __ballot(!ok);
          int first = __ffsll((unsigned long long)m) - 1;
          if (lane == first) latch_error(P, PRE_DEV_TIMEOUT, step, stage, bad, seen, ep);
          verdict = 0;
          break;
        }
      }
      __builtin_amdgcn_s_sleep(1);
    }
    if (lane == 0) sh[0] = verdict;
  }
  __syncthreads();
  const bool r = sh[0] != 0;
  __syncthreads();
  return r;
}

// The dependency wait of one task (a no-op in the per-operator baseline).
struct Waiter {
  int active, lo, hi, step, stage;
  uint32_t ep;
  int *sh;
  __device__ __forceinline__ bool operator()(const KP &P) const {
    if (!active) return true;
    const bool ok = wait_slots(P, lo, hi, ep, step, stage, sh);
    if (threadIdx.x == 0) sh[3] = (int)(uint32_t)now_ticks();  // trace: end of the wait
    return ok;
  }
  // trace: time of phase k (0..3) of the task, taken by thread 0
  __device__ __forceinline__ void mark(int k) const {
    if (active && threadIdx.x == 0) sh[4 + k] = (int)(uint32_t)now_ticks();
  }
};

// Publish: every thread's stores are complete, then one sc1 flag store.
__device__ __forceinline__ void signal_slot(const KP &P, int slot, uint32_t ep) {
  drain();
  __syncthreads();
  if (threadIdx.x == 0 && slot >= 0) st_flag(P.flags + slot, ep);
}

// ---------------------------------------------------------------------------
// staging a GEMV input vector into LDS (fp32), optionally RMS-normalised

// x = base (+ the nparts partial vectors of the split output projection),
// then RMSNorm with `gain` when it is given.
struct Src {
  const float *f32;      // fp32 base vector (device-scope loads), or
  const uint16_t *bf16;  // bf16 base row (embedding)
  const float *parts;    // nparts fp32 vectors at stride pstride, added in order
  int nparts, pstride;
  const uint16_t *gain;  // non-NULL: fold RMSNorm with these gains
};
constexpr int MAXPARTS = 8;  // KV heads per sequence (partials of the split O projection)

// xs[0..K) = src (normalised if gain), xs[K..Kpad) = 0.  Ends with a barrier.
// The gains are fetched together with the data, so staging costs one device
// round trip (two when K exceeds GK * 4 * threads and gains are refetched).
constexpr int GK = 4;
__device__ __forceinline__ void stage_vec(const KP &P, float *xs, float *red, const Src &s, int K,
                                          int Kpad) {
  const int tid = threadIdx.x, T = P.nthr, n4 = K >> 2;
  float ss = 0.f;
  const Rsrc rg = mkbuf(s.gain, s.gain ? (uint32_t)K * 2 : 0u);
  v2i gr[GK];
#pragma unroll
  for (int k = 0; k < GK; ++k) gr[k] = s.gain ? ld64<CP_DEF>(rg, (uint32_t)(tid + k * T) * 8) : v2i{0, 0};
  if (s.f32 && s.nparts == 0) {
    const Rsrc r = mkbuf(s.f32, (uint32_t)K * 4);
    for (int i = tid; i < n4; i += 8 * T) {
      v4i a[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) a[j] = ld128<CP_SC1>(r, (uint32_t)(i + j * T) * 16);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (i + j * T < n4) {
          float4 f = __builtin_bit_cast(float4, a[j]);
          reinterpret_cast<float4 *>(xs)[i + j * T] = f;
          ss = fmaf(f.x, f.x, ss); ss = fmaf(f.y, f.y, ss);
          ss = fmaf(f.z, f.z, ss); ss = fmaf(f.w, f.w, ss);
        }
    }
  } else {
    // base (fp32 or bf16) plus partial vectors, two float4 per thread per round
    const Rsrc rb = mkbuf(s.f32 ? (const void *)s.f32 : (const void *)s.bf16, (uint32_t)K * (s.f32 ? 4 : 2));
    const Rsrc rp = mkbuf(s.parts, s.parts ? (uint32_t)((s.nparts - 1) * s.pstride + K) * 4 : 0u);
    for (int i0 = tid; i0 < n4; i0 += 2 * T) {
      v4i pv[2][MAXPARTS], bv[2];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int i = i0 + k * T;  // past n4 the buffers return 0
#pragma unroll
        for (int p = 0; p < MAXPARTS; ++p)
          if (p < s.nparts) pv[k][p] = ld128<CP_SC1>(rp, (uint32_t)(p * s.pstride + 4 * i) * 4);
        if (s.f32) {
          bv[k] = ld128<CP_SC1>(rb, (uint32_t)i * 16);
        } else {
          const v2i w = ld64<CP_DEF>(rb, (uint32_t)i * 8);
          bv[k] = __builtin_bit_cast(v4i, float4{bf_lo(w.x), bf_hi(w.x), bf_lo(w.y), bf_hi(w.y)});
        }
      }
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int i = i0 + k * T;
        if (i >= n4) break;
        float4 f = __builtin_bit_cast(float4, bv[k]);
#pragma unroll
        for (int p = 0; p < MAXPARTS; ++p)
          if (p < s.nparts) {
            const float4 q = __builtin_bit_cast(float4, pv[k][p]);
            f.x += q.x; f.y += q.y; f.z += q.z; f.w += q.w;
          }
        reinterpret_cast<float4 *>(xs)[i] = f;
        ss = fmaf(f.x, f.x, ss); ss = fmaf(f.y, f.y, ss);
        ss = fmaf(f.z, f.z, ss); ss = fmaf(f.w, f.w, ss);
      }
    }
  }
  for (int i = K + tid; i < Kpad; i += T) xs[i] = 0.f;
  if (s.gain) {
    const int wave = wave_id(), nw = P.nw;
    ss = wave_sum(ss);
    if ((tid & 63) == 0) red[wave] = ss;
    __syncthreads();
    float tot = 0.f;
    for (int w = 0; w < nw; ++w) tot += red[w];
    const float rinv = 1.0f / sqrtf(tot / (float)K + P.eps);
    for (int k = 0; k < GK; ++k) {
      const int i = tid + k * T;
      if (i < n4) {
        const float4 f = reinterpret_cast<float4 *>(xs)[i];
        reinterpret_cast<float4 *>(xs)[i] = float4{f.x * rinv * bf_lo(gr[k].x), f.y * rinv * bf_hi(gr[k].x),
                                                   f.z * rinv * bf_lo(gr[k].y), f.w * rinv * bf_hi(gr[k].y)};
      }
    }
    for (int i = tid + GK * T; i < n4; i += T) {  // beyond the gains held in registers
      const v2i g = ld64<CP_DEF>(rg, (uint32_t)i * 8);
      const float4 f = reinterpret_cast<float4 *>(xs)[i];
      reinterpret_cast<float4 *>(xs)[i] = float4{f.x * rinv * bf_lo(g.x), f.y * rinv * bf_hi(g.x),
                                                 f.z * rinv * bf_lo(g.y), f.w * rinv * bf_hi(g.y)};
    }
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Streamed GEMV core.
//
// A task computes groups [0, ng) of R weight rows that share the same K-long
// input (a RoPE pair, a gate/up pair, or single rows).  Each row is cut into
// chunks of one 16-byte load per lane (8 bf16 or 16 fp8 values; 512 or 1024
// columns per chunk), so every load instruction of a wavefront reads 1 KB of
// consecutive weight bytes.  The task's (group, chunk) units, group-major,
// are split into one contiguous span per wavefront (split-K across
// wavefronts where a span ends inside a group), so every wavefront streams
// the same amount.  A ring of D units (D * R loads) is kept in flight per
// wavefront: unit u is consumed while unit u + D is being fetched, across row
// boundaries, with no barrier.  The first D units are issued before the task
// waits for its producers (weights never wait on activations).  Loads past a
// row's end, or past the span's end, address a zero-length buffer and return
// 0 without touching memory, so every ring slot issues exactly R loads and
// the wait counts stay static.  A wavefront writes one partial sum per
// (group it touched, row) into LDS; the task's epilogue adds the wavefronts'
// partials in wavefront order (deterministic).

constexpr int CP_W = CP_NT;  // weight loads: streaming (read once per step)

template <int R, int D, bool FP8, int CP = CP_W>
struct Stream {
  v4i buf[D][R];
  float sc[D][R];
  const void *rp[R];      // rows of the group being issued
  uint32_t rb[R];
  const uint16_t *sp[R];  // fp8: block-scale row of each row
  uint32_t sb[R];
  int ig, ic, cg, cc, nch, left;  // issue / compute cursors, units left to issue
  int wave, nw;                   // this wavefront, wavefronts per workgroup
  float acc[R];
};

// Issue the next unit of the span into ring slot j (the caller knows one is
// left).
template <int R, int D, bool FP8, int CP, class RowFn>
__device__ __forceinline__ void st_issue(Stream<R, D, FP8, CP> &S, int j, RowFn &rowfn) {
  const int lane = threadIdx.x & 63;
  const int col = FP8 ? S.ic * 1024 + lane * 16 : S.ic * 512 + lane * 8;
  const uint32_t off = FP8 ? (uint32_t)col : (uint32_t)col * 2;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    S.buf[j][r] = ld128<CP>(mkbuf(S.rp[r], S.rb[r]), off);
    if (FP8) {
      // two bf16 scales per dword; this lane's 16 columns share one 128-wide block
      const int blk = col >> 7;
      const uint32_t w = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(mkbuf(S.sp[r], S.sb[r]),
                                                                         (uint32_t)(blk >> 1) * 4, 0, CP_DEF);
      S.sc[j][r] = bf16f((uint16_t)((blk & 1) ? (w >> 16) : (w & 0xffffu)));
    }
  }
  --S.left;
  if (++S.ic == S.nch) {
    S.ic = 0;
    ++S.ig;
    if (S.left > 0) rowfn(S.ig, S);
  }
}

// This wavefront's span of the task's ng * nch units; issues its first D
// units (all of them when the span is shorter).  Returns the span length.
// When the span covers a whole ring the D issues are unconditional, so the
// ring's wait counts stay static through the main loop.
template <int R, int D, bool FP8, int CP, class RowFn>
__device__ __forceinline__ int st_begin(Stream<R, D, FP8, CP> &S, RowFn &rowfn, int ng, int K, int nw) {
  const int wave = wave_id();
  S.wave = wave;
  S.nw = nw;
  S.nch = FP8 ? (K + 1023) >> 10 : (K + 511) >> 9;
  const int N = ng * S.nch, u0 = (int)((int64_t)N * wave / nw), u1 = (int)((int64_t)N * (wave + 1) / nw);
  const int n = u1 - u0;
  S.ig = S.cg = u0 / S.nch;
  S.ic = S.cc = u0 % S.nch;
  S.left = n;
#pragma unroll
  for (int r = 0; r < R; ++r) { S.acc[r] = 0.f; S.rp[r] = nullptr; S.rb[r] = 0; S.sp[r] = nullptr; S.sb[r] = 0; }
  if (n > 0) rowfn(S.ig, S);
  if (n >= D) {
#pragma unroll
    for (int j = 0; j < D; ++j) st_issue(S, j, rowfn);
  } else {
#pragma unroll
    for (int j = 0; j < D; ++j)
      if (j < n) st_issue(S, j, rowfn);
  }
  return n;
}

// Unit in ring slot j: accumulate; at the end of a group (or of the span)
// write the wavefront's partial of that group to ys[(g * nw + wave) * R + r].
template <int R, int D, bool FP8, int CP, class XFn>
__device__ __forceinline__ void st_compute(Stream<R, D, FP8, CP> &S, int j, bool span_end, XFn &xfn,
                                           float *ys) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float *xb = xfn(S.cg, r) + (FP8 ? S.cc * 1024 + lane * 16 : S.cc * 512 + lane * 8);
    if (FP8) {
      S.acc[r] = fmaf(S.sc[j][r], dot16_fp8(S.buf[j][r], xb), S.acc[r]);
    } else {
      const float4 *x4 = reinterpret_cast<const float4 *>(xb);
      S.acc[r] = dot8_bf16(S.buf[j][r], x4[0], x4[1], S.acc[r]);
    }
  }
  const bool row_end = ++S.cc == S.nch;
  if (row_end || span_end) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float y = wave_sum(S.acc[r]);
      S.acc[r] = 0.f;
      if (lane == 0) ys[(S.cg * S.nw + S.wave) * R + r] = y;
    }
    if (row_end) { S.cc = 0; ++S.cg; }
  }
}

// Consume the span of n units: xfn(g, r) is the LDS input of row r of group g.
// Full rounds of the ring first (one unconditional issue per consumed unit),
// then the last one or two rounds without further issues past the span.
template <int R, int D, bool FP8, int CP, class RowFn, class XFn>
__device__ __forceinline__ void st_run(Stream<R, D, FP8, CP> &S, int n, RowFn &rowfn, XFn xfn, float *ys) {
  if (n >= D) {
    const int m = (n - D) / D;  // rounds whose every issue lies inside the span
    for (int q = 0; q < m; ++q) {
#pragma unroll
      for (int j = 0; j < D; ++j) {
        st_compute(S, j, false, xfn, ys);
        st_issue(S, j, rowfn);
      }
    }
    const int rem = n - m * D;  // D <= rem < 2D
#pragma unroll
    for (int j = 0; j < D; ++j) {
      st_compute(S, j, j == rem - 1, xfn, ys);
      if (j + D < rem) st_issue(S, j, rowfn);
    }
#pragma unroll
    for (int j = 0; j < D; ++j)
      if (j + D < rem) st_compute(S, j, j + D == rem - 1, xfn, ys);
  } else {
#pragma unroll
    for (int j = 0; j < D; ++j)
      if (j < n) st_compute(S, j, j == n - 1, xfn, ys);
  }
}

// Zero the partial-sum buffer of ng groups (before the task's staging barrier).
__device__ __forceinline__ void ys_clear(float *ys, int ng, int R, int nw, int nthr) {
  const int n = ng * nw * R;
  for (int i = threadIdx.x; i < n; i += nthr) ys[i] = 0.f;
}
// Result r of group g: the wavefronts' partials added in wavefront order.
__device__ __forceinline__ float ys_get(const float *ys, int g, int r, int R, int nw) {
  float y = 0.f;
  for (int w = 0; w < nw; ++w) y += ys[(g * nw + w) * R + r];
  return y;
}

// ---------------------------------------------------------------------------
// per-layer addressing helpers

__device__ __forceinline__ int64_t vec_off(const KP &P, int l, int b, int width) {
  return ((int64_t)l * P.B + b) * width;
}
// The residual stream entering layer l: the embedding row of the token (the
// baseline keeps it in x_emb) or the previous layer's output.
__device__ __forceinline__ Src layer_input(const KP &P, int l, int tok, const uint16_t *gain) {
  Src s{nullptr, nullptr, nullptr, 0, 0, gain};
  if (l > 0) s.f32 = P.x_out + vec_off(P, l - 1, 0, P.h);
  else if (P.persistent) s.bf16 = P.embed + (int64_t)tok * P.h;
  else s.f32 = P.x_emb;
  return s;
}
// The residual stream after attention of layer l: layer input plus the KV
// heads' output-projection partials.
__device__ __forceinline__ Src mid_input(const KP &P, int l, int tok, const uint16_t *gain) {
  Src s = layer_input(P, l, tok, gain);
  s.parts = P.pbuf + vec_off(P, l, 0, P.Hkv * P.h);
  s.nparts = P.Hkv;
  s.pstride = P.h;
  return s;
}
// Element i of the layer-l post-attention residual (same addition order as
// stage_vec).
__device__ __forceinline__ float mid_elem(const KP &P, int l, int tok, int i) {
  float x;
  if (l > 0) x = ld_sc1(P.x_out + vec_off(P, l - 1, 0, P.h) + i);
  else if (P.persistent) x = bf16f(P.embed[(int64_t)tok * P.h + i]);
  else x = ld_sc1(P.x_emb + i);
  const float *pb = P.pbuf + vec_off(P, l, 0, P.Hkv * P.h) + i;
  float pv[MAXPARTS];
#pragma unroll
  for (int p = 0; p < MAXPARTS; ++p) pv[p] = p < P.Hkv ? ld_sc1(pb + (int64_t)p * P.h) : 0.f;
#pragma unroll
  for (int p = 0; p < MAXPARTS; ++p)
    if (p < P.Hkv) x += pv[p];
  return x;
}

// Field f of a layer's pointer table (the order of DevLayer): selecting a
// matrix by index keeps the choice in scalar registers.
enum LField { F_WQ = 1, F_WK = 2, F_WV = 3, F_EWG = 10, F_EWU = 11, F_EWD = 12, F_ESG = 13,
              F_ESU = 14, F_ESD = 15, F_SWG = 16, F_SWU = 17, F_SWD = 18, F_SSG = 19,
              F_SSU = 20, F_SSD = 21 };
__device__ __forceinline__ const void *lptr(const DevLayer *L, int f) {
  return reinterpret_cast<const void *const *>(L)[f];
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// LDS layout of the GEMV tasks: xs[kmax] | ys[ymax * waves] | red[256]
struct GemvLds {
  float *xs, *ys, *red;
};
__device__ __forceinline__ GemvLds gemv_lds(const KP &P, float *lds) {
  float *ys = lds + P.kmax;
  return GemvLds{lds, ys, ys + P.ymax * P.nw};
}

// Row-wise GEMV over one bf16 matrix W [rows][K] starting at row r0.
struct RowsBf16 {
  const uint16_t *W;
  int K, r0;
  __device__ __forceinline__ void operator()(int g, Stream<1, 8, false> &S) const {
    S.rp[0] = W + (int64_t)(r0 + g) * K;
    S.rb[0] = (uint32_t)K * 2;
  }
};

// ---------------------------------------------------------------------------
// tasks.  Each: prefetch the first weight units, wait for producers, stage
// the input, stream the rows, run the epilogue with all threads.  Returns
// false if the wait was aborted.

// QKV: pairs [r0, r1) in group-major order (per KV head g: its G query
// heads, then k head g, then v head g; d/2 RoPE pairs (j, j + d/2) each).
__device__ __forceinline__ bool task_qkv(const KP &P, const Task &t, int pos, int tok, float *lds,
                                         const Waiter &wait) {
  const int l = t.layer, ng = t.r1 - t.r0;
  const GemvLds M = gemv_lds(P, lds);
  const int half = P.d >> 1, per_group = (P.G + 2) * half, h = P.h;
  const DevLayer *Lp = P.layers + l;
  const int G = P.G, dd = P.d, r0 = t.r0;
  auto rowfn = [=](int gi, Stream<2, 8, false> &S) {
    const int p = r0 + gi, g = p / per_group, rem = p % per_group, hh = rem / half, j = rem % half;
    const uint16_t *W = (const uint16_t *)lptr(Lp, hh < G ? F_WQ : (hh == G ? F_WK : F_WV));
    const int head = hh < G ? g * G + hh : g;
    S.rp[0] = W + ((int64_t)head * dd + j) * h;
    S.rp[1] = W + ((int64_t)head * dd + j + half) * h;
    S.rb[0] = S.rb[1] = (uint32_t)h * 2;
  };
  Stream<2, 8, false> S;
  const int n = st_begin(S, rowfn, ng, h, P.nw);
  ys_clear(M.ys, ng, 2, P.nw, P.nthr);
  if (!wait(P)) return false;
  if (P.persistent) stage_vec(P, M.xs, M.red, layer_input(P, l, tok, (const uint16_t *)Lp->attn_norm), h, P.kmax);
  else stage_vec(P, M.xs, M.red, Src{P.a_norm, nullptr, nullptr, 0, 0, nullptr}, h, P.kmax);
  wait.mark(0);
  st_run(S, n, rowfn, [=](int, int) { return (const float *)M.xs; }, M.ys);
  __syncthreads();
  wait.mark(1);
  const float *cosT = P.rope + (int64_t)pos * half;
  const float *sinT = P.rope + (int64_t)P.max_ctx * half + (int64_t)pos * half;
  for (int i = threadIdx.x; i < ng; i += P.nthr) {
    const int p = t.r0 + i, g = p / per_group, rem = p % per_group, hh = rem / half, j = rem % half;
    float a = ys_get(M.ys, i, 0, 2, P.nw), b = ys_get(M.ys, i, 1, 2, P.nw);
    if (hh <= P.G) {  // RoPE on q and k
      const float c = cosT[j], s = sinT[j];
      const float a2 = a * c - b * s, b2 = b * c + a * s;
      a = a2; b = b2;
    }
    if (hh < P.G) {
      float *qd = P.q + vec_off(P, l, 0, P.Hq * P.d) + (int64_t)(g * P.G + hh) * P.d;
      st_sc1(qd + j, a);
      st_sc1(qd + j + half, b);
    } else {
      uint16_t *cache = (hh == P.G) ? P.kc : P.vc;
      const int64_t base = (((int64_t)l * P.B + 0) * P.Hkv + g) * P.max_ctx * P.d;
      const Rsrc r = mkbuf(cache + base, (uint32_t)P.max_ctx * P.d * 2);
      st16<CP_SC1>(r, (uint32_t)((int64_t)pos * P.d + j) * 2, f2bf(a));
      st16<CP_SC1>(r, (uint32_t)((int64_t)pos * P.d + j + half) * 2, f2bf(b));
    }
  }
  return true;
}

// Combine the NC chunk partials of (sequence b, KV head g) into
// xs[0 .. G*d): o_h = sum_c e^{m_c - M} o_c / sum_c e^{m_c - M} l_c with
// M = max_c m_c.  The partial block [NC][G][d + 2] is contiguous; it is read
// with wide loads into the LDS behind xs (in slices of chunks when it does
// not fit), so the combine costs one device round trip (two with slices).
__device__ __forceinline__ void attn_combine_lds(const KP &P, int l, int bg, float *lds, int lds_n, float *xs) {
  const int b = bg / P.Hkv, g = bg % P.Hkv, G = P.G, d = P.d, NC = P.NC, rec = d + 2;
  const int tid = threadIdx.x, T = P.nthr;
  const float *src = P.part + (((int64_t)l * P.B + b) * P.Hkv + g) * NC * G * rec;
  const int go = (G * d + 3) & ~3;
  float *wt = lds + go;          // [NC][G] e^{m - M}
  float *den = wt + NC * G;      // [G] sum, [G] max
  float *blk = lds + ((go + NC * G + 2 * G + 3) & ~3);
  const int room = (lds_n - (int)(blk - lds)) / (G * rec);
  const int per = max(1, min(NC, room));
  const Rsrc r = mkbuf(src, (uint32_t)NC * G * rec * 4);
  float num[4] = {0.f, 0.f, 0.f, 0.f}, dsum = 0.f;
  for (int c0 = 0; c0 < NC; c0 += per) {
    const int c1 = min(NC, c0 + per), nf = (c1 - c0) * G * rec;  // nf is even
    const uint32_t base = (uint32_t)c0 * G * rec * 4;
    for (int i = tid * 2; i < nf; i += 16 * T) {
      v2i a[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int e = i + k * 2 * T;
        a[k] = e < nf ? ld64<CP_SC1>(r, base + (uint32_t)e * 4) : v2i{0, 0};
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int e = i + k * 2 * T;
        if (e < nf) *reinterpret_cast<float2 *>(blk + e) = __builtin_bit_cast(float2, a[k]);
      }
    }
    __syncthreads();
    if (c0 == 0) {  // the maxima; every slice after the first must reload them
      if (tid < G) {
        float Mx = -INFINITY;
        if (per == NC)
          for (int cc = 0; cc < NC; ++cc) Mx = fmaxf(Mx, blk[(cc * G + tid) * rec]);
        else
          for (int cc = 0; cc < NC; ++cc) Mx = fmaxf(Mx, ldf<CP_SC1>(r, (uint32_t)(cc * G + tid) * rec * 4));
        den[G + tid] = Mx;
      }
      __syncthreads();
    }
    for (int i = tid; i < (c1 - c0) * G; i += T) wt[c0 * G + i] = expf(blk[i * rec] - den[G + i % G]);
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = tid + q * T;
      if (i < G * d) {
        const int hh = i / d, j = i % d;
        for (int cc = c0; cc < c1; ++cc)
          num[q] = fmaf(wt[cc * G + hh], blk[((cc - c0) * G + hh) * rec + 2 + j], num[q]);
      }
    }
    if (tid < G)
      for (int cc = c0; cc < c1; ++cc) dsum = fmaf(wt[cc * G + tid], blk[((cc - c0) * G + tid) * rec + 1], dsum);
    __syncthreads();
  }
  if (tid < G) den[tid] = dsum;
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int i = tid + q * T;
    if (i < G * d) xs[i] = num[q] / den[i / d];
  }
}

// Output projection of one KV head: rows [r0, r1) of Wo restricted to the
// head group's G*d columns, times that group's attention output (combined
// here from its chunk partials).  Writes the split-K partial
// pbuf[l][b][g][rows]; the residual add happens where the partials are read.
__device__ __forceinline__ bool task_oproj(const KP &P, const Task &t, float *lds, const Waiter &wait) {
  const int l = t.layer, bg = t.aux, b = bg / P.Hkv, g = bg % P.Hkv, ng = t.r1 - t.r0;
  const int K = P.G * P.d, ld = P.Hq * P.d;
  const GemvLds M = gemv_lds(P, lds);
  RowsBf16 rowfn{(const uint16_t *)P.layers[l].wo + (int64_t)g * K, ld, t.r0};
  // row g of the slice: W + row * ld; K columns
  auto rows = [=](int gi, Stream<1, 16, false> &S) {
    S.rp[0] = rowfn.W + (int64_t)(rowfn.r0 + gi) * ld;
    S.rb[0] = (uint32_t)K * 2;
  };
  Stream<1, 16, false> S;
  const int n = st_begin(S, rows, ng, K, P.nw);
  ys_clear(M.ys, ng, 1, P.nw, P.nthr);
  if (!wait(P)) return false;
  // combine into xs[0..K); its scratch lies behind the padded input and
  // overlaps ys, which is cleared again once the combine is done
  const int Kp = (K + 511) & ~511;
  attn_combine_lds(P, l, bg, lds + Kp, P.lds_floats - Kp, M.xs);
  __syncthreads();
  wait.mark(0);
  for (int i = K + threadIdx.x; i < Kp; i += P.nthr) M.xs[i] = 0.f;
  ys_clear(M.ys, ng, 1, P.nw, P.nthr);
  __syncthreads();
  st_run(S, n, rows, [=](int, int) { return (const float *)M.xs; }, M.ys);
  __syncthreads();
  wait.mark(1);
  float *dst = P.pbuf + ((int64_t)(l * P.B + b) * P.Hkv + g) * P.h + t.r0;
  for (int i = threadIdx.x; i < ng; i += P.nthr) st_sc1(dst + i, ys_get(M.ys, i, 0, 1, P.nw));
  return true;
}

// Dense gate/up row pairs [r0, r1): u_j = silu(Wg_j b) * (Wu_j b).
__device__ __forceinline__ bool task_gu(const KP &P, const Task &t, int tok, float *lds, const Waiter &wait) {
  const int l = t.layer, h = P.h, ng = t.r1 - t.r0;
  const DevLayer &Lw = P.layers[l];
  const GemvLds M = gemv_lds(P, lds);
  const uint16_t *wg = (const uint16_t *)Lw.wg, *wu = (const uint16_t *)Lw.wu;
  const int r0 = t.r0;
  auto rowfn = [=](int gi, Stream<2, 4, false> &S) {
    S.rp[0] = wg + (int64_t)(r0 + gi) * h;
    S.rp[1] = wu + (int64_t)(r0 + gi) * h;
    S.rb[0] = S.rb[1] = (uint32_t)h * 2;
  };
  Stream<2, 4, false> S;
  const int n = st_begin(S, rowfn, ng, h, P.nw);
  ys_clear(M.ys, ng, 2, P.nw, P.nthr);
  if (!wait(P)) return false;
  if (P.persistent) stage_vec(P, M.xs, M.red, mid_input(P, l, tok, (const uint16_t *)Lw.ffn_norm), h, P.kmax);
  else stage_vec(P, M.xs, M.red, Src{P.a_norm, nullptr, nullptr, 0, 0, nullptr}, h, P.kmax);
  wait.mark(0);
  st_run(S, n, rowfn, [=](int, int) { return (const float *)M.xs; }, M.ys);
  __syncthreads();
  wait.mark(1);
  float *u = P.u + vec_off(P, l, 0, P.F);
  for (int i = threadIdx.x; i < ng; i += P.nthr)
    st_sc1(u + t.r0 + i, silu(ys_get(M.ys, i, 0, 2, P.nw)) * ys_get(M.ys, i, 1, 2, P.nw));
  return true;
}

// Dense down rows [r0, r1) + residual: x_out = x_mid + Wd u.
__device__ __forceinline__ bool task_down(const KP &P, const Task &t, int step, int tok, float *lds,
                                          const Waiter &wait) {
  const int l = t.layer, ng = t.r1 - t.r0;
  const GemvLds M = gemv_lds(P, lds);
  RowsBf16 rowfn{(const uint16_t *)P.layers[l].wd, P.ffn, t.r0};
  Stream<1, 8, false> S;
  const int n = st_begin(S, rowfn, ng, P.ffn, P.nw);
  ys_clear(M.ys, ng, 1, P.nw, P.nthr);
  // the post-attention residual was final before the gate/up stage this
  // workgroup passed: fetch it now
  const int tid = threadIdx.x;
  const float res0 = tid < ng ? mid_elem(P, l, tok, t.r0 + tid) : 0.f;
  if (!wait(P)) return false;
  stage_vec(P, M.xs, M.red, Src{P.u + vec_off(P, l, 0, P.F), nullptr, nullptr, 0, 0, nullptr}, P.ffn, P.kmax);
  wait.mark(0);
  st_run(S, n, rowfn, [=](int, int) { return (const float *)M.xs; }, M.ys);
  __syncthreads();
  wait.mark(1);
  float *xo = P.x_out + vec_off(P, l, 0, P.h);
  float *hid = (P.chk_hidden && l == P.L - 1) ? P.chk_hidden + (int64_t)step * P.B * P.h : nullptr;
  for (int i = tid; i < ng; i += P.nthr) {
    const int row = t.r0 + i;
    const float v = (i == tid ? res0 : mid_elem(P, l, tok, row)) + ys_get(M.ys, i, 0, 1, P.nw);
    st_sc1(xo + row, v);
    if (hid) hid[row] = v;
  }
  return true;
}

// Router rows [r0, r1): rl = Wr b (MoE).
__device__ __forceinline__ bool task_router(const KP &P, const Task &t, int tok, float *lds,
                                            const Waiter &wait) {
  const int l = t.layer, h = P.h, ng = t.r1 - t.r0;
  const DevLayer &Lw = P.layers[l];
  const GemvLds M = gemv_lds(P, lds);
  RowsBf16 rowfn{(const uint16_t *)Lw.router, h, t.r0};
  Stream<1, 8, false> S;
  const int n = st_begin(S, rowfn, ng, h, P.nw);
  ys_clear(M.ys, ng, 1, P.nw, P.nthr);
  if (!wait(P)) return false;
  if (P.persistent) stage_vec(P, M.xs, M.red, mid_input(P, l, tok, (const uint16_t *)Lw.ffn_norm), h, P.kmax);
  else stage_vec(P, M.xs, M.red, Src{P.a_norm, nullptr, nullptr, 0, 0, nullptr}, h, P.kmax);
  st_run(S, n, rowfn, [=](int, int) { return (const float *)M.xs; }, M.ys);
  __syncthreads();
  float *rl = P.rl + vec_off(P, l, 0, P.E);
  for (int i = threadIdx.x; i < ng; i += P.nthr) st_sc1(rl + t.r0 + i, ys_get(M.ys, i, 0, 1, P.nw));
  return true;
}

// Softmax over the router logits and top-k selection (ties -> lower expert
// id), then the n_shared shared experts with weight 1.  Every workgroup
// that needs the choice computes it; the inputs and the order of operations
// are the same everywhere, so all of them agree.  sel/selw in LDS.
__device__ __forceinline__ void route(const KP &P, int l, int *sel, float *selw, float *scratch) {
  const int tid = threadIdx.x, T = P.nthr;
  const float *rl = P.rl + vec_off(P, l, 0, P.E);
  for (int i = tid; i < P.E; i += T) scratch[i] = ld_sc1(rl + i);
  __syncthreads();
  if (tid < 64) {
    const int lane = tid;
    float m = -INFINITY;
    for (int i = lane; i < P.E; i += 64) m = fmaxf(m, scratch[i]);
    m = wave_max(m);
    float s = 0.f;
    for (int i = lane; i < P.E; i += 64) s += expf(scratch[i] - m);
    s = wave_sum(s);
    uint32_t taken = 0;  // bit li: local index lane + 64 * li already chosen (E <= 1024)
    for (int k = 0; k < P.top_k; ++k) {
      float bv = -INFINITY;
      int bi = 0x7fffffff, li = 0;
      for (int i = lane; i < P.E; i += 64, ++li)
        if (!((taken >> li) & 1u) && (scratch[i] > bv || (scratch[i] == bv && i < bi))) { bv = scratch[i]; bi = i; }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        const float ov = __shfl_xor(bv, o);
        const int oi = __shfl_xor(bi, o);
        if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
      }
      if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
      if (lane == 0) { sel[k] = bi; selw[k] = expf(bv - m) / s; }
    }
    if (lane == 0)
      for (int k = 0; k < P.n_shared; ++k) { sel[P.top_k + k] = k; selw[P.top_k + k] = 1.0f; }
  }
  __syncthreads();
}

// Expert gate/up pairs [r0, r1) over (slot k, row j): u[k][j].  The rows
// depend on the routing, so the stream starts after it.
__device__ __forceinline__ bool task_egu(const KP &P, const Task &t, int tok, float *lds, const Waiter &wait) {
  const int l = t.layer, h = P.h, ng = t.r1 - t.r0;
  const DevLayer &Lw = P.layers[l];
  const GemvLds M = gemv_lds(P, lds);
  int *sel = reinterpret_cast<int *>(M.red + 64);
  float *selw = M.red + 96;
  if (!wait(P)) return false;
  route(P, l, sel, selw, M.xs);
  const int f = P.effn, hb = (h + 127) / 128, fb = (f + 127) / 128;
  const int top_k = P.top_k, r0 = t.r0;
  const DevLayer *Lp = P.layers + l;
  auto rowfn = [=](int gi, Stream<2, 4, true> &S) {
    const int p = r0 + gi, k = p / f, j = p % f, e = sel[k];
    const int sh = k >= top_k ? F_SWG - F_EWG : 0;
    const uint8_t *wg = (const uint8_t *)lptr(Lp, F_EWG + sh);
    const uint8_t *wu = (const uint8_t *)lptr(Lp, F_EWU + sh);
    const uint16_t *sg = (const uint16_t *)lptr(Lp, F_ESG + sh);
    const uint16_t *su = (const uint16_t *)lptr(Lp, F_ESU + sh);
    const int64_t wofs = ((int64_t)e * f + j) * h, sofs = ((int64_t)e * fb + j / 128) * hb;
    S.rp[0] = wg + wofs; S.rp[1] = wu + wofs;
    S.rb[0] = S.rb[1] = (uint32_t)h;
    S.sp[0] = sg + sofs; S.sp[1] = su + sofs;
    S.sb[0] = S.sb[1] = (uint32_t)hb * 2;
  };
  Stream<2, 4, true> S;
  const int n = st_begin(S, rowfn, ng, h, P.nw);
  ys_clear(M.ys, ng, 2, P.nw, P.nthr);
  if (P.persistent) stage_vec(P, M.xs, M.red, mid_input(P, l, tok, (const uint16_t *)Lw.ffn_norm), h, P.kmax);
  else stage_vec(P, M.xs, M.red, Src{P.a_norm, nullptr, nullptr, 0, 0, nullptr}, h, P.kmax);
  st_run(S, n, rowfn, [=](int, int) { return (const float *)M.xs; }, M.ys);
  __syncthreads();
  float *u = P.u + vec_off(P, l, 0, P.F);
  for (int i = threadIdx.x; i < ng; i += P.nthr)
    st_sc1(u + t.r0 + i, silu(ys_get(M.ys, i, 0, 2, P.nw)) * ys_get(M.ys, i, 1, 2, P.nw));
  return true;
}

// Expert down rows [r0, r1): x_out = x_mid + sum_k w_k Wd_{e_k} u_k.  The
// stream runs over (row, slot) pairs; the epilogue sums the slots of a row
// in slot order.
__device__ __forceinline__ bool task_edown(const KP &P, const Task &t, int step, int tok, float *lds,
                                           const Waiter &wait) {
  const int l = t.layer, rows = t.r1 - t.r0;
  const GemvLds M = gemv_lds(P, lds);
  int *sel = reinterpret_cast<int *>(M.red + 64);
  float *selw = M.red + 96;
  const int tid = threadIdx.x;
  const float res0 = tid < rows ? mid_elem(P, l, tok, t.r0 + tid) : 0.f;
  if (!wait(P)) return false;
  route(P, l, sel, selw, M.xs);
  const int f = P.effn, hb = (P.h + 127) / 128, fb = (f + 127) / 128;
  const int nk = P.top_k + P.n_shared;
  const int top_k = P.top_k, hh = P.h, r0 = t.r0;
  const DevLayer *Lp = P.layers + l;
  auto rowfn = [=](int q, Stream<1, 8, true> &S) {
    const int i = r0 + q / nk, k = q % nk, e = sel[k];
    const int sh = k >= top_k ? F_SWG - F_EWG : 0;
    S.rp[0] = (const uint8_t *)lptr(Lp, F_EWD + sh) + ((int64_t)e * hh + i) * f;
    S.rb[0] = (uint32_t)f;
    S.sp[0] = (const uint16_t *)lptr(Lp, F_ESD + sh) + ((int64_t)e * hb + i / 128) * fb;
    S.sb[0] = (uint32_t)fb * 2;
  };
  Stream<1, 8, true> S;
  const int n = st_begin(S, rowfn, rows * nk, f, P.nw);
  ys_clear(M.ys, rows * nk, 1, P.nw, P.nthr);
  stage_vec(P, M.xs, M.red, Src{P.u + vec_off(P, l, 0, P.F), nullptr, nullptr, 0, 0, nullptr}, P.F, P.kmax);
  st_run(S, n, rowfn, [=](int q, int) { return (const float *)(M.xs + (q % nk) * f); }, M.ys);
  __syncthreads();
  float *xo = P.x_out + vec_off(P, l, 0, P.h);
  float *hid = (P.chk_hidden && l == P.L - 1) ? P.chk_hidden + (int64_t)step * P.B * P.h : nullptr;
  for (int i = tid; i < rows; i += P.nthr) {
    float acc = 0.f;
    for (int k = 0; k < nk; ++k) acc = fmaf(selw[k], ys_get(M.ys, i * nk + k, 0, 1, P.nw), acc);
    const float v = (i == tid ? res0 : mid_elem(P, l, tok, t.r0 + i)) + acc;
    st_sc1(xo + t.r0 + i, v);
    if (hid) hid[t.r0 + i] = v;
  }
  return true;
}

// Best (value, lowest index) of two candidates.
__device__ __forceinline__ void argmax_merge(float &bv, int &bi, float ov, int oi) {
  if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
}

// LM head rows [r0, r1): logits (check mode) and this task's (max, lowest
// index) partial.  A NaN logit makes the partial NaN.
__device__ __forceinline__ bool task_lm(const KP &P, const Task &t, int lam, int step, float *lds,
                                        const Waiter &wait) {
  const GemvLds M = gemv_lds(P, lds);
  const int wave = wave_id(), nw = P.nw, lane = threadIdx.x & 63, ng = t.r1 - t.r0;
  RowsBf16 rowfn{P.lm_head, P.h, t.r0};
  Stream<1, 8, false> S;
  const int n = st_begin(S, rowfn, ng, P.h, P.nw);
  ys_clear(M.ys, ng, 1, P.nw, P.nthr);
  if (!wait(P)) return false;
  if (P.persistent)
    stage_vec(P, M.xs, M.red, Src{P.x_out + vec_off(P, P.L - 1, 0, P.h), nullptr, nullptr, 0, 0, P.final_norm},
              P.h, P.kmax);
  else stage_vec(P, M.xs, M.red, Src{P.a_norm, nullptr, nullptr, 0, 0, nullptr}, P.h, P.kmax);
  wait.mark(0);
  st_run(S, n, rowfn, [=](int, int) { return (const float *)M.xs; }, M.ys);
  __syncthreads();
  wait.mark(1);
  float *lg = P.chk_logits ? P.chk_logits + (int64_t)step * P.B * P.V : nullptr;
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  bool nan = false;
  for (int i = threadIdx.x; i < ng; i += P.nthr) {
    const float y = ys_get(M.ys, i, 0, 1, P.nw);
    if (y != y) nan = true;
    else argmax_merge(bv, bi, y, t.r0 + i);
    if (lg) lg[t.r0 + i] = y;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) argmax_merge(bv, bi, __shfl_xor(bv, o), __shfl_xor(bi, o));
  const bool wnan = __any(nan);
  float *wv = M.red + 128;
  int *wi = reinterpret_cast<int *>(M.red + 160);
  int *wn = reinterpret_cast<int *>(M.red + 192);
  if (lane == 0) { wv[wave] = bv; wi[wave] = bi; wn[wave] = wnan; }
  __syncthreads();
  if (threadIdx.x == 0) {
    float v = -INFINITY;
    int ix = 0x7fffffff, anynan = 0;
    for (int w = 0; w < nw; ++w) { anynan |= wn[w]; argmax_merge(v, ix, wv[w], wi[w]); }
    if (anynan) v = __builtin_nanf("");
    st_sc1(P.lmp + 2 * lam, v);
    st_flag(reinterpret_cast<uint32_t *>(P.lmp) + 2 * lam + 1, (uint32_t)ix);
  }
  return true;
}

// Global greedy token from the W partials (all threads get it); -1 on NaN.
__device__ __forceinline__ int reduce_lm(const KP &P, int *sh) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    bool nan = false;
    for (int i = lane; i < P.W; i += 64) {
      const float v = ld_sc1(P.lmp + 2 * i);
      const int ix = (int)ld_flag(reinterpret_cast<const uint32_t *>(P.lmp) + 2 * i + 1);
      if (v != v) nan = true;
      else argmax_merge(bv, bi, v, ix);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) argmax_merge(bv, bi, __shfl_xor(bv, o), __shfl_xor(bi, o));
    const bool anynan = __any(nan);
    if (lane == 0) sh[1] = anynan ? -1 : bi;
  }
  __syncthreads();
  const int r = sh[1];
  __syncthreads();
  return r;
}

// ---------------------------------------------------------------------------
// Split-KV attention: chunk c of (sequence b, KV head g), all G query heads
// of the group at once so K/V are read once (query-head folding).  The chunk's
// cached rows were written in earlier steps, so their loads are issued before
// the dependency wait; only the newest position (written by this step's QKV
// tasks) and q are read after it.  Writes the chunk's (max, sum,
// unnormalised output) per head; the output projection combines the chunks.

constexpr int APB = 4;  // attention passes whose K/V rows are held in registers

__device__ __forceinline__ bool attn_chunk(const KP &P, const Task &t, int pos, float *lds,
                                           const Waiter &wait) {
  const int l = t.layer, bg = t.aux, b = bg / P.Hkv, g = bg % P.Hkv, c = t.r0, NC = t.r1;
  const int G = P.G, d = P.d, tid = threadIdx.x, T = P.nthr;
  const int wave = wave_id(), nw = P.nw, lane = tid & 63;
  const int n = pos + 1, C = (n + NC - 1) / NC, t0 = c * C;
  const int cnt = max(0, min(n, t0 + C) - t0);
  const int cpad = ((P.cmax + 63) / 64) * 64;
  float *qs = lds, *sc = qs + G * d, *ored = sc + G * cpad, *st = ored + nw * G * d;
  const int64_t cbase = (((int64_t)l * P.B + b) * P.Hkv + g) * P.max_ctx * d;
  const Rsrc kr = mkbuf(P.kc + cbase, (uint32_t)P.max_ctx * d * 2);
  const Rsrc vr = mkbuf(P.vc + cbase, (uint32_t)P.max_ctx * d * 2);
  const int LPP = d / 8, PPW = 64 / LPP, sub = lane % LPP, grp = lane / LPP;
  const int PASS = nw * PPW;
  auto koff = [=](int tt) { return (uint32_t)((int64_t)(t0 + tt) * d + sub * 8) * 2; };
  // cached rows of the first batch, before the wait
  v4i kb[APB], vb[APB];
#pragma unroll
  for (int p = 0; p < APB; ++p) {
    const int tt = p * PASS + wave * PPW + grp;
    const bool old = tt < cnt && t0 + tt != pos;
    kb[p] = old ? ld128<CP_SC1>(kr, koff(tt)) : v4i{0, 0, 0, 0};
    vb[p] = old ? ld128<CP_SC1>(vr, koff(tt)) : v4i{0, 0, 0, 0};
  }
  if (!wait(P)) return false;
  // q of the group and the newest row
  const float *qsrc = P.q + vec_off(P, l, b, P.Hq * d) + (int64_t)g * G * d;
  for (int i = tid; i < G * d; i += T) qs[i] = ld_sc1(qsrc + i) * P.attn_scale;
#pragma unroll
  for (int p = 0; p < APB; ++p) {
    const int tt = p * PASS + wave * PPW + grp;
    if (tt < cnt && t0 + tt == pos) {
      kb[p] = ld128<CP_SC1>(kr, koff(tt));
      vb[p] = ld128<CP_SC1>(vr, koff(tt));
    }
  }
  __syncthreads();
  wait.mark(0);
  // scores
  for (int base = 0; base < cnt; base += APB * PASS) {
    if (base > 0) {
#pragma unroll
      for (int p = 0; p < APB; ++p) {
        const int tt = base + p * PASS + wave * PPW + grp;
        kb[p] = tt < cnt ? ld128<CP_SC1>(kr, koff(tt)) : v4i{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int p = 0; p < APB; ++p) {
      const int tt = base + p * PASS + wave * PPW + grp;
      if (base + p * PASS < cnt) {
        for (int hh = 0; hh < G; ++hh) {
          const float4 *q4 = reinterpret_cast<const float4 *>(qs + hh * d + sub * 8);
          float s = dot8_bf16(kb[p], q4[0], q4[1], 0.f);
          s = (LPP == 16) ? sum16(s) : sum8(s);
          if (tt < cnt && sub == 0) sc[hh * cpad + tt] = s;
        }
      }
    }
  }
  __syncthreads();
  // per-head max and exponentials
  for (int hh = wave; hh < G; hh += nw) {
    float m = -INFINITY;
    for (int i = lane; i < cnt; i += 64) m = fmaxf(m, sc[hh * cpad + i]);
    m = wave_max(m);
    float s = 0.f;
    for (int i = lane; i < cnt; i += 64) {
      const float e = expf(sc[hh * cpad + i] - m);
      sc[hh * cpad + i] = e;
      s += e;
    }
    s = wave_sum(s);
    if (lane == 0) { st[2 * hh] = cnt > 0 ? m : -1e30f; st[2 * hh + 1] = s; }
  }
  __syncthreads();
  wait.mark(1);
  // o = sum_t p_t V_t: a lane owns 8 dims of one position per pass
  float acc[8][8];
#pragma unroll
  for (int hh = 0; hh < 8; ++hh)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[hh][e] = 0.f;
  for (int base = 0; base < cnt; base += APB * PASS) {
    if (base > 0) {
#pragma unroll
      for (int p = 0; p < APB; ++p) {
        const int tt = base + p * PASS + wave * PPW + grp;
        vb[p] = tt < cnt ? ld128<CP_SC1>(vr, koff(tt)) : v4i{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int p = 0; p < APB; ++p) {
      const int tt = base + p * PASS + wave * PPW + grp;
      if (tt < cnt) {
        const v4i vw = vb[p];
        const float v[8] = {bf_lo(vw.x), bf_hi(vw.x), bf_lo(vw.y), bf_hi(vw.y),
                            bf_lo(vw.z), bf_hi(vw.z), bf_lo(vw.w), bf_hi(vw.w)};
#pragma unroll
        for (int hh = 0; hh < 8; ++hh)
          if (hh < G) {
            const float pr = sc[hh * cpad + tt];
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[hh][e] = fmaf(pr, v[e], acc[hh][e]);
          }
      }
    }
  }
  // reduce the PPW position groups of the wave (lanes sub, sub + LPP, ...):
  // the two 8-lane halves of a row first when LPP = 8, then across rows
#pragma unroll
  for (int hh = 0; hh < 8; ++hh)
    if (hh < G) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float v = acc[hh][e];
        if (LPP == 8) v += dpp<0x128>(v);  // row_ror:8
        acc[hh][e] = xrow_sum(v);
      }
    }
  if (grp == 0) {
#pragma unroll
    for (int hh = 0; hh < 8; ++hh)
      if (hh < G)
#pragma unroll
        for (int e = 0; e < 8; ++e) ored[(wave * G + hh) * d + sub * 8 + e] = acc[hh][e];
  }
  __syncthreads();
  wait.mark(2);
  float *pdst = P.part + ((((int64_t)l * P.B + b) * P.Hkv + g) * NC + c) * G * (d + 2);
  for (int i = tid; i < G * d; i += T) {
    const int hh = i / d, j = i % d;
    float s = 0.f;
    for (int w = 0; w < nw; ++w) s += ored[(w * G + hh) * d + j];
    st_sc1(pdst + hh * (d + 2) + 2 + j, s);
  }
  for (int hh = tid; hh < G; hh += T) {
    st_sc1(pdst + hh * (d + 2), st[2 * hh]);
    st_sc1(pdst + hh * (d + 2) + 1, st[2 * hh + 1]);
  }
  return true;
}

__device__ __forceinline__ void trace_rec(const KP &P, int step, int si, int lam, uint32_t a, uint32_t b,
                                          uint32_t c, const int *sh) {
  if (!P.trace || threadIdx.x != 0) return;
  const uint64_t idx = ((uint64_t)step * P.n_si + si) * P.W + lam;
  if (idx >= P.trace_cap) return;
  uint32_t *r = P.trace + 8 * idx;
  r[0] = (uint32_t)si | ((uint32_t)lam << 16);
  r[1] = a; r[2] = b; r[3] = c;
  for (int k = 0; k < 4; ++k) r[4 + k] = (uint32_t)sh[4 + k];
}

__device__ __forceinline__ bool token_ok(const KP &P, int tok, int step) {
  if (tok >= 0 && tok < P.V) return true;
  if (threadIdx.x == 0) latch_error(P, PRE_DEV_BAD_TOKEN, step, -1, -1, (uint32_t)tok, 0);
  return false;
}

// Run one task of the table (both paths).
__device__ __forceinline__ bool run_task(const KP &P, const Task &t, int lam, int step, int pos, int tok,
                                         float *lds, const Waiter &wait) {
  switch (t.op) {
    case OP_QKV: return task_qkv(P, t, pos, tok, lds, wait);
    case OP_ATTN: return attn_chunk(P, t, pos, lds, wait);
    case OP_OPROJ: return task_oproj(P, t, lds, wait);
    case OP_GU: return task_gu(P, t, tok, lds, wait);
    case OP_DOWN: return task_down(P, t, step, tok, lds, wait);
    case OP_ROUTER: return task_router(P, t, tok, lds, wait);
    case OP_EGU: return task_egu(P, t, tok, lds, wait);
    case OP_EDOWN: return task_edown(P, t, step, tok, lds, wait);
    case OP_LM: return task_lm(P, t, lam, step, lds, wait);
    default: return true;
  }
}

// ---------------------------------------------------------------------------
// the resident kernel

extern "C" __global__ void __launch_bounds__(512) pre_persistent(KP P) {
  extern __shared__ __attribute__((aligned(16))) float lds[];
  __shared__ int sh[8];
  const int lam = lambda_of_block(blockIdx.x, P.W, P.X);
  if (threadIdx.x == 0) {
    const uint32_t x = xcc_id();
    P.xcc[lam] = x;
    if (P.W % P.X == 0 && (int)x != (int)(blockIdx.x % P.X))
      __hip_atomic_fetch_add(&P.status->xcc_mismatch, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  int tok = P.forced ? P.forced[0] : P.in_tok[0];
  for (int s = 0; s < P.n_steps; ++s) {
    const uint32_t ep = P.epoch_base + (uint32_t)s + 1u;
    const int pos = P.pos0 + s;
    if (P.forced) tok = P.forced[(int64_t)s * P.B];
    if (!token_ok(P, tok, s)) return;
    for (int si = 0; si < P.n_si; ++si) {
      const Task t = P.tasks[(int64_t)si * P.W + lam];
      if (t.op == OP_NONE) continue;
      const uint32_t tw = (uint32_t)now_ticks();
      const Waiter wait{1, t.wait_lo, t.wait_hi, s, si, ep, sh};
      if (!run_task(P, t, lam, s, pos, tok, lds, wait)) return;
      signal_slot(P, t.signal, ep);
      trace_rec(P, s, si, lam, tw, (uint32_t)sh[3], (uint32_t)now_ticks(), sh);
    }
    // greedy token of step s: every workgroup when it feeds the next step,
    // workgroup 0 always (it writes the output)
    const bool need = (!P.forced && s + 1 < P.n_steps) || lam == 0;
    if (need) {
      const int s_lm = P.n_si - 1;
      if (!wait_slots(P, s_lm * P.W, (s_lm + 1) * P.W, ep, s, s_lm, sh)) return;
      const int nt = reduce_lm(P, sh);
      if (nt < 0) {
        if (threadIdx.x == 0) latch_error(P, PRE_DEV_NAN, s, s_lm, -1, 0, 0);
        return;
      }
      if (lam == 0 && threadIdx.x == 0) P.out_tok[(int64_t)s * P.B] = nt;
      if (!P.forced) tok = nt;
    }
  }
}

// ---------------------------------------------------------------------------
// baseline: one kernel per operator, stream order as the only sync

extern "C" __global__ void __launch_bounds__(512) pre_k_embed(KP P, int step) {
  int tok = P.forced ? P.forced[(int64_t)step * P.B] : (step == 0 ? P.in_tok[0] : P.tok_slot[0]);
  if (tok < 0 || tok >= P.V) {
    if (threadIdx.x == 0) latch_error(P, PRE_DEV_BAD_TOKEN, step, -1, -1, (uint32_t)tok, 0);
    tok = 0;
  }
  if (threadIdx.x == 0 && blockIdx.x == 0) P.tok_slot[1] = tok;  // token of this step
  for (int i = threadIdx.x; i < P.h; i += P.nthr) P.x_emb[i] = bf16f(P.embed[(int64_t)tok * P.h + i]);
}

// a_norm = RMSNorm(x, gain) with x the layer input (mid = 0), the
// post-attention residual (mid = 1) or the last layer's output (mid = 2).
extern "C" __global__ void __launch_bounds__(512) pre_k_norm(KP P, int l, int mid, const uint16_t *gain) {
  extern __shared__ __attribute__((aligned(16))) float lds[];
  float *xs = lds, *red = lds + P.kmax;
  Src s = mid == 2 ? Src{P.x_out + vec_off(P, P.L - 1, 0, P.h), nullptr, nullptr, 0, 0, gain}
                   : (mid ? mid_input(P, l, 0, gain) : layer_input(P, l, 0, gain));
  stage_vec(P, xs, red, s, P.h, P.kmax);
  for (int i = threadIdx.x; i < P.kmax; i += P.nthr) P.a_norm[i] = xs[i];
}

extern "C" __global__ void __launch_bounds__(512) pre_k_task(KP P, int si, int step) {
  extern __shared__ __attribute__((aligned(16))) float lds[];
  __shared__ int sh[8];
  const int lam = blockIdx.x;
  const Task t = P.tasks[(int64_t)si * P.W + lam];
  const Waiter none{0, 0, 0, 0, 0, 0u, sh};
  run_task(P, t, lam, step, P.pos0 + step, P.tok_slot[1], lds, none);
}

extern "C" __global__ void __launch_bounds__(512) pre_k_argmax(KP P, int step) {
  __shared__ int sh[8];
  const int nt = reduce_lm(P, sh);
  if (threadIdx.x == 0) {
    if (nt < 0) latch_error(P, PRE_DEV_NAN, step, P.n_si - 1, -1, 0, 0);
    P.tok_slot[0] = nt < 0 ? 0 : nt;
    P.out_tok[(int64_t)step * P.B] = nt;
  }
}

// Debug: the wavefront primitives on one wave of input (64 floats):
// out[0..64) sum8, [64..128) sum16, [128] wave_sum, [129] wave_max,
// [192..256) row_ror:8 pair sums, [256..320) xrow_sum.
extern "C" __global__ void pre_k_lane_ops(const float *in, float *out) {
  const int lane = threadIdx.x & 63;
  const float v = in[lane];
  out[lane] = sum8(v);
  out[64 + lane] = sum16(v);
  const float ws = wave_sum(v), wm = wave_max(v);
  if (lane == 0) { out[128] = ws; out[129] = wm; }
  out[192 + lane] = v + dpp<0x128>(v);
  out[256 + lane] = xrow_sum(v);
}

// Debug: decode n fp8 codes with the GEMV's unpacking (checks the format).
extern "C" __global__ void pre_k_fp8_decode(const uint8_t *in, float *out, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (4 * i + 3 < n) {
    float f[4];
    fp8x4(*reinterpret_cast<const uint32_t *>(in + 4 * i), f);
    for (int k = 0; k < 4; ++k) out[4 * i + k] = f[k];
  }
}

// Debug / tuning: the streamed GEMV alone, y = W x over rows split evenly
// across the grid, for a given ring depth and weight cache policy.
template <int D, int CP>
__global__ void __launch_bounds__(1024) pre_k_gemv_bench(const uint16_t *W, int rows, int K, const float *x,
                                                         float *y) {
  extern __shared__ __attribute__((aligned(16))) float lds[];
  const int nthr = __builtin_amdgcn_readfirstlane(blockDim.x), nw = nthr >> 6;
  const int Kp = (K + 511) / 512 * 512;
  for (int i = threadIdx.x; i < Kp; i += nthr) lds[i] = i < K ? x[i] : 0.f;
  float *ys = lds + Kp;
  const int r0 = (int)((int64_t)rows * blockIdx.x / gridDim.x);
  const int r1 = (int)((int64_t)rows * (blockIdx.x + 1) / gridDim.x);
  struct Rows {
    const uint16_t *W;
    int K, r0;
    __device__ void operator()(int g, Stream<1, D, false, CP> &S) const {
      S.rp[0] = W + (int64_t)(r0 + g) * K;
      S.rb[0] = (uint32_t)K * 2;
    }
  } rowfn{W, K, r0};
  Stream<1, D, false, CP> S;
  const int n = st_begin(S, rowfn, r1 - r0, K, nw);
  ys_clear(ys, r1 - r0, 1, nw, nthr);
  __syncthreads();
  st_run(S, n, rowfn, [=](int, int) { return (const float *)lds; }, ys);
  __syncthreads();
  for (int i = threadIdx.x; i < r1 - r0; i += nthr) y[r0 + i] = ys_get(ys, i, 0, 1, nw);
}

}  // namespace pre

// ===========================================================================
// host side: the C ABI

using namespace pre;

struct pre_engine {
  pre_config cfg;
  Dims D;
  Layout Lo;
  char *ws;
  size_t ws_bytes;
  pre_kv kv;
  const void *embed, *final_norm, *lm_head;
  int32_t pos[8];
  uint32_t epoch_base;
  uint32_t watchdog_ms;
  int lds_dyn;
  int broken;
  hipStream_t stream;
  std::vector<pre_layer_w> lw;  // host copy of the layer pointers (norm gains for the baseline)
  uint32_t *trace;
  size_t trace_bytes;
  int device;
};

static inline bool al16(const void *p) { return ((uintptr_t)p & 15) == 0; }

static int device_cus(int *cus, int *lds_max, int *dev) {
  if (hipGetDevice(dev) != hipSuccess) return PRE_ERR_HIP;
  hipDeviceProp_t pr;
  if (hipGetDeviceProperties(&pr, *dev) != hipSuccess) return PRE_ERR_HIP;
  *cus = pr.multiProcessorCount;
  *lds_max = (int)pr.sharedMemPerBlock;
  return PRE_OK;
}

extern "C" int pre_workspace_size(const pre_config *cfg, size_t *bytes) {
  if (!cfg || !bytes) return PRE_ERR_ARG;
  int cus = 256, ldsm = 0, dev = 0;
  if (cfg->grid_wgs <= 0 && device_cus(&cus, &ldsm, &dev) != PRE_OK) cus = 256;
  Dims D;
  int rc = derive_dims(cfg, cus, &D);
  if (rc != PRE_OK) return rc;
  Layout Lo;
  build_layout(D, &Lo);
  *bytes = (size_t)Lo.total;
  return PRE_OK;
}

static int check_layer(const Dims &D, const pre_layer_w &L) {
  const void *need_dense[] = {L.attn_norm, L.wq, L.wk, L.wv, L.wo, L.ffn_norm, L.wg, L.wu, L.wd};
  const void *need_moe[] = {L.attn_norm, L.wq, L.wk, L.wv, L.wo, L.ffn_norm, L.router,
                            L.e_wg, L.e_wu, L.e_wd, L.e_sg, L.e_su, L.e_sd};
  if (!D.moe) {
    for (const void *p : need_dense) { if (!p) return PRE_ERR_ARG; if (!al16(p)) return PRE_ERR_ALIGN; }
  } else {
    for (const void *p : need_moe) { if (!p) return PRE_ERR_ARG; if (!al16(p)) return PRE_ERR_ALIGN; }
    if (D.n_shared > 0) {
      const void *sh[] = {L.s_wg, L.s_wu, L.s_wd, L.s_sg, L.s_su, L.s_sd};
      for (const void *p : sh) { if (!p) return PRE_ERR_ARG; if (!al16(p)) return PRE_ERR_ALIGN; }
    }
  }
  return PRE_OK;
}

extern "C" int pre_engine_create(const pre_config *cfg, const pre_weights *w, const pre_kv *kv,
                                 void *d_workspace, size_t ws_bytes, void *stream, pre_engine **out) {
  if (!out) return PRE_ERR_ARG;
  *out = nullptr;
  if (!cfg || !w || !kv || !d_workspace || !w->layers) return PRE_ERR_ARG;
  int cus, ldsm, dev;
  if (device_cus(&cus, &ldsm, &dev) != PRE_OK) return PRE_ERR_HIP;
  Dims D;
  int rc = derive_dims(cfg, cus, &D);
  if (rc != PRE_OK) return rc;
  if (!w->embed || !w->final_norm || !w->lm_head || !kv->k || !kv->v) return PRE_ERR_ARG;
  if (!al16(w->embed) || !al16(w->final_norm) || !al16(w->lm_head) || !al16(kv->k) || !al16(kv->v) ||
      !al16(d_workspace))
    return PRE_ERR_ALIGN;
  for (int l = 0; l < D.L; ++l)
    if ((rc = check_layer(D, w->layers[l])) != PRE_OK) return rc;
  if ((int64_t)D.max_ctx * D.d * 2 >= (1ll << 32)) return PRE_ERR_SHAPE;
  Layout Lo;
  build_layout(D, &Lo);
  if ((int64_t)ws_bytes < Lo.total) return PRE_ERR_WORKSPACE;
  std::vector<Task> T;
  build_tasks(D, T);
  if (validate(D, T) != 0) return PRE_ERR_SHAPE;

  // LDS: what the tiles need, raised past half a CU's LDS so that exactly one
  // workgroup fits per CU (one resident workgroup per CU).
  int dyn = D.lds_bytes;
  const int want = std::min(ldsm, 96 * 1024);
  if (want > dyn && want > ldsm / 2) dyn = want;
  if (dyn > ldsm) return PRE_ERR_SHAPE;
  if (hipFuncSetAttribute((const void *)pre_persistent, hipFuncAttributeMaxDynamicSharedMemorySize, dyn) !=
          hipSuccess ||
      hipFuncSetAttribute((const void *)pre_k_task, hipFuncAttributeMaxDynamicSharedMemorySize, dyn) !=
          hipSuccess ||
      hipFuncSetAttribute((const void *)pre_k_norm, hipFuncAttributeMaxDynamicSharedMemorySize, dyn) !=
          hipSuccess)
    return PRE_ERR_HIP;
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void *)pre_persistent, D.threads, dyn) !=
      hipSuccess)
    return PRE_ERR_HIP;
  if (per_cu < 1 || (int64_t)per_cu * cus < D.W) return PRE_ERR_SHAPE;

  std::vector<DevLayer> dl(D.L);
  for (int l = 0; l < D.L; ++l) std::memcpy(&dl[l], &w->layers[l], sizeof(DevLayer));
  const int half = D.d / 2;
  std::vector<float> rope((size_t)D.max_ctx * D.d);
  for (int p = 0; p < D.max_ctx; ++p)
    for (int i = 0; i < half; ++i) {
      const double inv = std::pow((double)cfg->rope_theta, -2.0 * i / (double)D.d);
      const double a = (double)p * inv;
      rope[(size_t)p * half + i] = (float)std::cos(a);
      rope[(size_t)D.max_ctx * half + (size_t)p * half + i] = (float)std::sin(a);
    }
  hipStream_t st = (hipStream_t)stream;
  char *ws = (char *)d_workspace;
  if (hipMemsetAsync(ws, 0, (size_t)Lo.total, st) != hipSuccess ||
      hipMemcpyAsync(ws + Lo.layers, dl.data(), dl.size() * sizeof(DevLayer), hipMemcpyHostToDevice, st) !=
          hipSuccess ||
      hipMemcpyAsync(ws + Lo.tasks, T.data(), T.size() * sizeof(Task), hipMemcpyHostToDevice, st) != hipSuccess ||
      hipMemcpyAsync(ws + Lo.rope, rope.data(), rope.size() * sizeof(float), hipMemcpyHostToDevice, st) !=
          hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    return PRE_ERR_HIP;

  pre_engine *e = new pre_engine();
  e->cfg = *cfg;
  e->D = D;
  e->Lo = Lo;
  e->ws = ws;
  e->ws_bytes = ws_bytes;
  e->kv = *kv;
  e->embed = w->embed;
  e->final_norm = w->final_norm;
  e->lm_head = w->lm_head;
  std::memset(e->pos, 0, sizeof(e->pos));
  e->epoch_base = 0;
  const char *wd = std::getenv("PRE_WATCHDOG_MS");
  e->watchdog_ms = wd ? (uint32_t)std::max(1, std::atoi(wd)) : 2000u;
  e->lds_dyn = dyn;
  e->broken = 0;
  e->stream = st;
  e->trace = nullptr;
  e->trace_bytes = 0;
  e->device = dev;
  e->lw.assign(w->layers, w->layers + D.L);
  *out = e;
  return PRE_OK;
}

extern "C" int pre_engine_set_positions(pre_engine *e, const int32_t *h_pos) {
  if (!e || !h_pos) return PRE_ERR_ARG;
  for (int b = 0; b < e->D.B; ++b)
    if (h_pos[b] < 0 || h_pos[b] >= e->D.max_ctx) return PRE_ERR_CONTEXT;
  for (int b = 0; b < e->D.B; ++b) e->pos[b] = h_pos[b];
  return PRE_OK;
}

extern "C" int pre_engine_get_positions(const pre_engine *e, int32_t *h_pos) {
  if (!e || !h_pos) return PRE_ERR_ARG;
  for (int b = 0; b < e->D.B; ++b) h_pos[b] = e->pos[b];
  return PRE_OK;
}

static void fill_kp(const pre_engine *e, KP &P, int persistent) {
  const Dims &D = e->D;
  std::memset(&P, 0, sizeof(P));
  P.L = D.L; P.h = D.h; P.Hq = D.Hq; P.Hkv = D.Hkv; P.d = D.d; P.ffn = D.ffn; P.V = D.V; P.B = D.B;
  P.max_ctx = D.max_ctx; P.E = D.E; P.top_k = D.top_k; P.n_shared = D.n_shared; P.effn = D.effn;
  P.moe = D.moe; P.G = D.G; P.F = D.F; P.W = D.W; P.X = D.X; P.NC = D.NC; P.Tg = D.Tg; P.n_si = D.n_si;
  P.spl = D.stages_per_layer; P.kmax = D.kmax; P.ymax = D.ymax; P.cmax = D.cmax;
  P.lds_floats = e->lds_dyn / 4;
  P.nthr = D.threads;
  P.nw = D.threads / 64;
  P.eps = D.eps;
  P.attn_scale = (float)(1.0 / std::sqrt((double)D.d));
  char *ws = e->ws;
  const Layout &Lo = e->Lo;
  P.layers = (const DevLayer *)(ws + Lo.layers);
  P.embed = (const uint16_t *)e->embed;
  P.final_norm = (const uint16_t *)e->final_norm;
  P.lm_head = (const uint16_t *)e->lm_head;
  P.kc = (uint16_t *)e->kv.k;
  P.vc = (uint16_t *)e->kv.v;
  P.tasks = (const Task *)(ws + Lo.tasks);
  P.flags = (uint32_t *)(ws + Lo.flags);
  P.xcc = (uint32_t *)(ws + Lo.xcc);
  P.status = (DevStatus *)(ws + Lo.status);
  P.rope = (const float *)(ws + Lo.rope);
  P.x_out = (float *)(ws + Lo.x_out);
  P.pbuf = (float *)(ws + Lo.pbuf);
  P.q = (float *)(ws + Lo.q);
  P.u = (float *)(ws + Lo.u);
  P.rl = (float *)(ws + Lo.rl);
  P.part = (float *)(ws + Lo.part);
  P.lmp = (float *)(ws + Lo.lmp);
  P.x_emb = (float *)(ws + Lo.x_emb);
  P.a_norm = (float *)(ws + Lo.a_norm);
  P.tok_slot = (int32_t *)(ws + Lo.tok);
  P.watchdog_ticks = (uint32_t)std::min<uint64_t>((uint64_t)e->watchdog_ms * 100000ull, 0xffffffffull);
  P.persistent = persistent;
}

static int check_call(const pre_engine *e, int32_t n_steps, const int32_t *d_in, const int32_t *d_forced,
                      const int32_t *d_out) {
  if (!e || n_steps < 0 || !d_out || (!d_in && !d_forced)) return PRE_ERR_ARG;
  if (e->broken) return PRE_ERR_BROKEN;
  for (int b = 0; b < e->D.B; ++b)
    if ((int64_t)e->pos[b] + n_steps > e->D.max_ctx) return PRE_ERR_CONTEXT;
  return PRE_OK;
}

extern "C" int pre_engine_decode(pre_engine *e, int32_t n_steps, const int32_t *d_in_tokens,
                                 const int32_t *d_forced, int32_t *d_out_tokens, const pre_check *chk,
                                 void *stream) {
  int rc = check_call(e, n_steps, d_in_tokens, d_forced, d_out_tokens);
  if (rc != PRE_OK || n_steps == 0) return rc;
  KP P;
  fill_kp(e, P, 1);
  P.n_steps = n_steps;
  P.pos0 = e->pos[0];
  P.epoch_base = e->epoch_base;
  P.in_tok = d_in_tokens;
  P.forced = d_forced;
  P.out_tok = d_out_tokens;
  P.chk_logits = chk ? chk->logits : nullptr;
  P.chk_hidden = chk ? chk->hidden : nullptr;
  P.trace = e->trace;
  P.trace_cap = (uint32_t)std::min<size_t>(e->trace_bytes / 32, 0xffffffffu);
  void *args[] = {&P};
  hipError_t err = hipLaunchCooperativeKernel((const void *)pre_persistent, dim3(e->D.W),
                                              dim3(e->D.threads), args, (unsigned)e->lds_dyn,
                                              (hipStream_t)stream);
  if (err != hipSuccess) return PRE_ERR_HIP;
  e->epoch_base += (uint32_t)n_steps;
  for (int b = 0; b < e->D.B; ++b) e->pos[b] += n_steps;
  return PRE_OK;
}

extern "C" int pre_baseline_decode(pre_engine *e, int32_t n_steps, const int32_t *d_in_tokens,
                                   const int32_t *d_forced, int32_t *d_out_tokens, const pre_check *chk,
                                   void *stream) {
  int rc = check_call(e, n_steps, d_in_tokens, d_forced, d_out_tokens);
  if (rc != PRE_OK || n_steps == 0) return rc;
  KP P;
  fill_kp(e, P, 0);
  P.in_tok = d_in_tokens;
  P.forced = d_forced;
  P.out_tok = d_out_tokens;
  P.chk_logits = chk ? chk->logits : nullptr;
  P.chk_hidden = chk ? chk->hidden : nullptr;
  P.pos0 = e->pos[0];
  hipStream_t st = (hipStream_t)stream;
  const Dims &D = e->D;
  const dim3 blk(D.threads);
  const unsigned lds = (unsigned)e->lds_dyn;
  const std::vector<pre_layer_w> &lw = e->lw;
  for (int s = 0; s < n_steps; ++s) {
    hipLaunchKernelGGL(pre_k_embed, dim3(1), blk, 0, st, P, s);
    for (int l = 0; l < D.L; ++l) {
      const int si0 = l * D.stages_per_layer;
      hipLaunchKernelGGL(pre_k_norm, dim3(D.B), blk, lds, st, P, l, 0, (const uint16_t *)lw[l].attn_norm);
      for (int k = 0; k < 3; ++k)  // QKV, attention chunks, O projection
        hipLaunchKernelGGL(pre_k_task, dim3(D.W), blk, lds, st, P, si0 + k, s);
      hipLaunchKernelGGL(pre_k_norm, dim3(D.B), blk, lds, st, P, l, 1, (const uint16_t *)lw[l].ffn_norm);
      for (int k = 3; k < D.stages_per_layer; ++k)
        hipLaunchKernelGGL(pre_k_task, dim3(D.W), blk, lds, st, P, si0 + k, s);
    }
    hipLaunchKernelGGL(pre_k_norm, dim3(D.B), blk, lds, st, P, D.L - 1, 2, (const uint16_t *)e->final_norm);
    hipLaunchKernelGGL(pre_k_task, dim3(D.W), blk, lds, st, P, D.n_si - 1, s);
    hipLaunchKernelGGL(pre_k_argmax, dim3(1), dim3(64), 0, st, P, s);
  }
  if (hipGetLastError() != hipSuccess) return PRE_ERR_HIP;
  for (int b = 0; b < D.B; ++b) e->pos[b] += n_steps;
  return PRE_OK;
}

extern "C" int pre_engine_status(pre_engine *e, pre_status *out) {
  if (!e || !out) return PRE_ERR_ARG;
  DevStatus ds;
  if (hipStreamSynchronize(e->stream) != hipSuccess ||
      hipMemcpy(&ds, e->ws + e->Lo.status, sizeof(ds), hipMemcpyDeviceToHost) != hipSuccess)
    return PRE_ERR_HIP;
  out->error = ds.error;
  out->step = ds.step;
  out->stage = ds.stage;
  out->slot = ds.slot;
  out->wg = ds.wg;
  out->observed = ds.observed;
  out->expected = ds.expected;
  out->xcc_mismatch = ds.xcc_mismatch;
  if (ds.error != PRE_DEV_OK) {
    e->broken = 1;
    return PRE_ERR_DEVICE;
  }
  return PRE_OK;
}

extern "C" int pre_engine_reset(pre_engine *e, void *stream) {
  if (!e) return PRE_ERR_ARG;
  hipStream_t st = (hipStream_t)stream;
  const Layout &Lo = e->Lo;
  if (hipMemsetAsync(e->ws + Lo.status, 0, sizeof(DevStatus), st) != hipSuccess ||
      hipMemsetAsync(e->ws + Lo.flags, 0, (size_t)(Lo.layers - Lo.flags), st) != hipSuccess)
    return PRE_ERR_HIP;
  e->epoch_base = 0;
  e->broken = 0;
  return PRE_OK;
}

extern "C" int pre_engine_set_watchdog(pre_engine *e, uint32_t ms) {
  if (!e || ms == 0) return PRE_ERR_ARG;
  e->watchdog_ms = ms;
  return PRE_OK;
}

extern "C" int pre_engine_set_trace(pre_engine *e, void *d_buf, size_t bytes) {
  if (!e) return PRE_ERR_ARG;
  if (d_buf && !al16(d_buf)) return PRE_ERR_ALIGN;
  e->trace = (uint32_t *)d_buf;
  e->trace_bytes = d_buf ? bytes : 0;
  return PRE_OK;
}

extern "C" int pre_engine_destroy(pre_engine *e) {
  if (!e) return PRE_ERR_ARG;
  delete e;
  return PRE_OK;
}

extern "C" const char *pre_strerror(int code) {
  switch (code) {
    case PRE_OK: return "ok";
    case PRE_ERR_ARG: return "invalid argument";
    case PRE_ERR_SHAPE: return "configuration not supported by the tile shapes";
    case PRE_ERR_ALIGN: return "pointer not 16-byte aligned";
    case PRE_ERR_WORKSPACE: return "workspace too small";
    case PRE_ERR_HIP: return "HIP runtime call failed";
    case PRE_ERR_UNSUPPORTED: return "configuration valid but not built";
    case PRE_ERR_DEVICE: return "device latched an error (see pre_engine_status)";
    case PRE_ERR_BROKEN: return "engine broken by an earlier device error; reset it";
    case PRE_ERR_CONTEXT: return "position would reach max_ctx";
    default: return "unknown error";
  }
}

// Debug entry: decode n (multiple of 4) fp8 codes with the kernels' unpacking.
extern "C" int pre_debug_fp8_decode(const void *d_codes, float *d_out, int n, void *stream) {
  if (!d_codes || !d_out || n <= 0 || (n & 3)) return PRE_ERR_ARG;
  const int th = 64, nb = (n / 4 + th - 1) / th;
  hipLaunchKernelGGL(pre_k_fp8_decode, dim3(nb), dim3(th), 0, (hipStream_t)stream, (const uint8_t *)d_codes,
                     d_out, n);
  return hipGetLastError() == hipSuccess ? PRE_OK : PRE_ERR_HIP;
}

// Debug / tuning entry: time the streamed GEMV variants.  variant = 2 * i + c
// with ring depth {8, 16, 24, 32}[i] and weight cache policy {default,
// streaming}[c]; rows are split over `grid` workgroups of `threads` threads,
// each given at least lds_min bytes of LDS (96 KB keeps one per CU).
extern "C" int pre_debug_gemv(int variant, const void *d_w, int rows, int K, const float *d_x, float *d_y,
                              int grid, int threads, int lds_min, void *stream) {
  if (!d_w || !d_x || !d_y || rows < 1 || K < 8 || K % 8 || grid < 1 || threads < 64 || threads > 1024)
    return PRE_ERR_ARG;
  const int Kp = (K + 511) / 512 * 512;
  const size_t lds = std::max<size_t>((size_t)(Kp + (rows + grid - 1) / grid + 64) * 4, (size_t)lds_min);
  if (lds > 160 * 1024) return PRE_ERR_SHAPE;
  const void *fns[8] = {(const void *)pre_k_gemv_bench<8, CP_DEF>, (const void *)pre_k_gemv_bench<8, CP_NT>,
                        (const void *)pre_k_gemv_bench<16, CP_DEF>, (const void *)pre_k_gemv_bench<16, CP_NT>,
                        (const void *)pre_k_gemv_bench<24, CP_DEF>, (const void *)pre_k_gemv_bench<24, CP_NT>,
                        (const void *)pre_k_gemv_bench<32, CP_DEF>, (const void *)pre_k_gemv_bench<32, CP_NT>};
  if (variant < 0 || variant >= 8) return PRE_ERR_ARG;
  if (hipFuncSetAttribute(fns[variant], hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
    return PRE_ERR_HIP;
  const uint16_t *w = (const uint16_t *)d_w;
  void *args[] = {&w, &rows, &K, &d_x, &d_y};
  if (hipLaunchKernel(fns[variant], dim3(grid), dim3(threads), args, lds, (hipStream_t)stream) != hipSuccess)
    return PRE_ERR_HIP;
  return PRE_OK;
}

// Debug: byte offsets of the workspace regions (status, flags, layers, tasks,
// rope, xcc, x_out, pbuf, q, u, rl, part, lmp, x_emb, a_norm, tok, total) --
// 17 int64 values.
extern "C" int pre_debug_layout(const pre_engine *e, int64_t *out) {
  if (!e || !out) return PRE_ERR_ARG;
  const Layout &L = e->Lo;
  const int64_t v[17] = {L.status, L.flags, L.layers, L.tasks, L.rope, L.xcc, L.x_out, L.pbuf, L.q, L.u,
                         L.rl, L.part, L.lmp, L.x_emb, L.a_norm, L.tok, L.total};
  for (int i = 0; i < 17; ++i) out[i] = v[i];
  return PRE_OK;
}

// Debug entry: run pre_k_lane_ops on 64 inputs (see the kernel for the layout
// of the 320 outputs).
extern "C" int pre_debug_lane_ops(const float *d_in, float *d_out, void *stream) {
  if (!d_in || !d_out) return PRE_ERR_ARG;
  hipLaunchKernelGGL(pre_k_lane_ops, dim3(1), dim3(64), 0, (hipStream_t)stream, d_in, d_out);
  return hipGetLastError() == hipSuccess ? PRE_OK : PRE_ERR_HIP;
}
