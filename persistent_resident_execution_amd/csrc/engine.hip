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
  int32_t L, h, Hq, Hkv, d, ffn, V, B, max_ctx, E, top_k, n_shared, effn, moe, G, F, W, X, NC;
  int32_t n_si, spl, kmax, cmax;
  float eps, attn_scale;
  // model
  const DevLayer *layers;
  const uint16_t *embed, *final_norm, *lm_head;
  uint16_t *kc, *vc;
  // workspace
  const Task *tasks;
  uint32_t *flags, *counters, *xcc;
  DevStatus *status;
  const float *rope;
  float *x_out, *xm, *q, *o, *u, *rl, *part, *lmp, *x_emb, *a_norm;
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
// error latch / abort

__device__ __forceinline__ void latch_error(const KP &P, int kind, int step, int stage, int slot, uint32_t obs,
                            uint32_t expd) {
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
__device__ __forceinline__ bool wait_slots(const KP &P, int lo, int hi, uint32_t ep, int step, int stage,
                           int *sh) {
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
          // the lowest lane still waiting reports its slot
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

// Publish: every thread's stores are complete, then one sc1 flag store.
__device__ __forceinline__ void signal_slot(const KP &P, int slot, uint32_t ep) {
  drain();
  __syncthreads();
  if (threadIdx.x == 0 && slot >= 0) st_flag(P.flags + slot, ep);
}

// ---------------------------------------------------------------------------
// staging a GEMV input vector into LDS (fp32), optionally RMS-normalised

struct Src {
  const float *f32;      // fp32 slot (device-scope loads), or
  const uint16_t *bf16;  // bf16 row (embedding)
  const uint16_t *gain;  // non-NULL: fold RMSNorm with these gains
};

// xs[0..K) = src (normalised if gain), xs[K..Kpad) = 0.  Ends with a barrier.
__device__ __forceinline__ void stage_vec(const KP &P, float *xs, float *red, const Src &s, int K, int Kpad) {
  const int tid = threadIdx.x, T = blockDim.x;
  float ss = 0.f;
  if (s.f32) {
    const Rsrc r = mkbuf(s.f32, (uint32_t)K * 4);
    const int n4 = K >> 2;
    for (int i = tid; i < n4; i += 4 * T) {
      v4i a[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) a[j] = ld128<CP_SC1>(r, (uint32_t)(i + j * T) * 16);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (i + j * T < n4) {
          float4 f = __builtin_bit_cast(float4, a[j]);
          reinterpret_cast<float4 *>(xs)[i + j * T] = f;
          ss = fmaf(f.x, f.x, ss); ss = fmaf(f.y, f.y, ss);
          ss = fmaf(f.z, f.z, ss); ss = fmaf(f.w, f.w, ss);
        }
    }
  } else {
    const Rsrc r = mkbuf(s.bf16, (uint32_t)K * 2);
    const int n8 = K >> 3;
    for (int i = tid; i < n8; i += T) {
      v4i w = ld128<CP_DEF>(r, (uint32_t)i * 16);
      float f[8] = {bf_lo(w.x), bf_hi(w.x), bf_lo(w.y), bf_hi(w.y),
                    bf_lo(w.z), bf_hi(w.z), bf_lo(w.w), bf_hi(w.w)};
#pragma unroll
      for (int j = 0; j < 8; ++j) { xs[i * 8 + j] = f[j]; ss = fmaf(f[j], f[j], ss); }
    }
  }
  for (int i = K + tid; i < Kpad; i += T) xs[i] = 0.f;
  if (s.gain) {
    const int wave = wave_id(), nw = T >> 6;
    ss = wave_sum(ss);
    if ((tid & 63) == 0) red[wave] = ss;
    __syncthreads();
    float tot = 0.f;
    for (int w = 0; w < nw; ++w) tot += red[w];
    const float rinv = 1.0f / sqrtf(tot / (float)K + P.eps);
    const Rsrc g = mkbuf(s.gain, (uint32_t)K * 2);
    for (int i = tid; i < (K >> 3); i += T) {
      v4i w = ld128<CP_DEF>(g, (uint32_t)i * 16);
      float gf[8] = {bf_lo(w.x), bf_hi(w.x), bf_lo(w.y), bf_hi(w.y),
                     bf_lo(w.z), bf_hi(w.z), bf_lo(w.w), bf_hi(w.w)};
#pragma unroll
      for (int j = 0; j < 8; ++j) xs[i * 8 + j] = xs[i * 8 + j] * rinv * gf[j];
    }
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// GEMV cores: RF rows at a time per wavefront, K split across the 64 lanes
// (8 bf16 or 16 fp8 per lane per 16-byte load), U loads per row in flight.

constexpr int U = 8;

// out[r] = sum_k W_r[k] * xs_r[k] over K (bf16 rows; NULL row -> 0).
template <int RF>
__device__ __forceinline__ void dot_bf16(const uint16_t *const (&row)[RF], const float *const (&xs)[RF],
                                         int K, float (&out)[RF]) {
  const int lane = threadIdx.x & 63;
  float acc[RF];
  Rsrc rs[RF];
#pragma unroll
  for (int r = 0; r < RF; ++r) {
    acc[r] = 0.f;
    rs[r] = mkbuf(row[r], row[r] ? (uint32_t)K * 2 : 0u);
  }
  const int nch = (K + 511) >> 9;
  for (int c0 = 0; c0 < nch; c0 += U) {
    v4i w[RF][U];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int r = 0; r < RF; ++r)
        w[r][u] = (c0 + u < nch) ? ld128<CP_DEF>(rs[r], (uint32_t)((c0 + u) * 512 + lane * 8) * 2)
                                 : v4i{0, 0, 0, 0};
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (c0 + u < nch) {
#pragma unroll
        for (int r = 0; r < RF; ++r) {
          const float4 *x4 = reinterpret_cast<const float4 *>(xs[r] + (c0 + u) * 512 + lane * 8);
          acc[r] = dot8_bf16(w[r][u], x4[0], x4[1], acc[r]);
        }
      }
  }
#pragma unroll
  for (int r = 0; r < RF; ++r) out[r] = wave_sum(acc[r]);
}

// fp8 rows with one bf16 scale per 128-column block (scale row pointer srow).
template <int RF>
__device__ __forceinline__ void dot_fp8(const uint8_t *const (&row)[RF], const uint16_t *const (&srow)[RF],
                                        const float *const (&xs)[RF], int K, float (&out)[RF]) {
  const int lane = threadIdx.x & 63;
  float acc[RF];
  Rsrc rs[RF];
#pragma unroll
  for (int r = 0; r < RF; ++r) {
    acc[r] = 0.f;
    rs[r] = mkbuf(row[r], row[r] ? (uint32_t)K : 0u);
  }
  const int nch = (K + 1023) >> 10;
  for (int c0 = 0; c0 < nch; c0 += U) {
    v4i w[RF][U];
    float sc[RF][U];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int r = 0; r < RF; ++r) {
        const int k = (c0 + u) * 1024 + lane * 16;
        const bool in = (c0 + u < nch) && row[r] && k < K;
        w[r][u] = in ? ld128<CP_DEF>(rs[r], (uint32_t)k) : v4i{0, 0, 0, 0};
        sc[r][u] = in ? bf16f(srow[r][k >> 7]) : 0.f;
      }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (c0 + u < nch) {
#pragma unroll
        for (int r = 0; r < RF; ++r)
          acc[r] = fmaf(sc[r][u], dot16_fp8(w[r][u], xs[r] + (c0 + u) * 1024 + lane * 16), acc[r]);
      }
  }
#pragma unroll
  for (int r = 0; r < RF; ++r) out[r] = wave_sum(acc[r]);
}

// ---------------------------------------------------------------------------
// per-layer addressing helpers

__device__ __forceinline__ int64_t vec_off(const KP &P, int l, int b, int width) {
  return ((int64_t)l * P.B + b) * width;
}
// x entering layer l: the embedding row (l == 0) or the previous layer's output.
__device__ __forceinline__ Src layer_input(const KP &P, int l, int tok, const uint16_t *gain) {
  Src s{nullptr, nullptr, gain};
  if (l == 0) s.bf16 = P.embed + (int64_t)tok * P.h;
  else s.f32 = P.x_out + vec_off(P, l - 1, 0, P.h);
  return s;
}
__device__ __forceinline__ float residual_in(const KP &P, int l, int tok, int i) {
  if (l == 0) return P.persistent ? bf16f(P.embed[(int64_t)tok * P.h + i]) : ld_sc1(P.x_emb + i);
  return ld_sc1(P.x_out + vec_off(P, l - 1, 0, P.h) + i);
}

// ---------------------------------------------------------------------------
// tasks

// QKV: pairs [r0, r1) in group-major order (per KV head g: its G query
// heads, then k head g, then v head g; d/2 RoPE pairs (j, j + d/2) each).
__device__ __forceinline__ void task_qkv(const KP &P, const Task &t, int pos, int tok, float *lds) {
  const int l = t.layer;
  const DevLayer &Lw = P.layers[l];
  float *xs = lds, *red = lds + P.kmax;
  if (P.persistent) stage_vec(P, xs, red, layer_input(P, l, tok, (const uint16_t *)Lw.attn_norm), P.h, P.kmax);
  else stage_vec(P, xs, red, Src{P.a_norm, nullptr, nullptr}, P.h, P.kmax);
  const int wave = wave_id(), nw = blockDim.x >> 6, lane = threadIdx.x & 63;
  const int half = P.d >> 1, per_group = (P.G + 2) * half;
  const float *cosT = P.rope + (int64_t)pos * half;
  const float *sinT = P.rope + (int64_t)P.max_ctx * half + (int64_t)pos * half;
  for (int p = t.r0 + wave; p < t.r1; p += nw) {
    const int g = p / per_group, rem = p % per_group, hh = rem / half, j = rem % half;
    const uint16_t *W;
    int head;
    if (hh < P.G) { W = (const uint16_t *)Lw.wq; head = g * P.G + hh; }
    else if (hh == P.G) { W = (const uint16_t *)Lw.wk; head = g; }
    else { W = (const uint16_t *)Lw.wv; head = g; }
    const uint16_t *rows[2] = {W + ((int64_t)head * P.d + j) * P.h,
                               W + ((int64_t)head * P.d + j + half) * P.h};
    const float *xsr[2] = {xs, xs};
    float y[2];
    dot_bf16<2>(rows, xsr, P.h, y);
    if (lane == 0) {
      float a = y[0], b = y[1];
      if (hh <= P.G) {  // RoPE on q and k
        const float c = cosT[j], s = sinT[j];
        const float a2 = a * c - b * s, b2 = b * c + a * s;
        a = a2; b = b2;
      }
      if (hh < P.G) {
        float *qd = P.q + vec_off(P, l, 0, P.Hq * P.d) + (int64_t)head * P.d;
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
  }
}

// O projection rows [r0, r1) + residual: xm = x_in + Wo o.
__device__ __forceinline__ void task_oproj(const KP &P, const Task &t, int tok, float *lds) {
  const int l = t.layer;
  const DevLayer &Lw = P.layers[l];
  const int K = P.Hq * P.d;
  float *xs = lds, *red = lds + P.kmax;
  stage_vec(P, xs, red, Src{P.o + vec_off(P, l, 0, K), nullptr, nullptr}, K, P.kmax);
  const int wave = wave_id(), nw = blockDim.x >> 6, lane = threadIdx.x & 63;
  const uint16_t *W = (const uint16_t *)Lw.wo;
  float *xm = P.xm + vec_off(P, l, 0, P.h);
  for (int i = t.r0 + 2 * wave; i < t.r1; i += 2 * nw) {
    const bool two = i + 1 < t.r1;
    const uint16_t *rows[2] = {W + (int64_t)i * K, two ? W + (int64_t)(i + 1) * K : nullptr};
    const float *xsr[2] = {xs, xs};
    float y[2];
    dot_bf16<2>(rows, xsr, K, y);
    if (lane == 0) st_sc1(xm + i, residual_in(P, l, tok, i) + y[0]);
    if (lane == 1 && two) st_sc1(xm + i + 1, residual_in(P, l, tok, i + 1) + y[1]);
  }
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// Dense gate/up row pairs [r0, r1): u_j = silu(Wg_j b) * (Wu_j b).
__device__ __forceinline__ void task_gu(const KP &P, const Task &t, float *lds) {
  const int l = t.layer;
  const DevLayer &Lw = P.layers[l];
  float *xs = lds, *red = lds + P.kmax;
  if (P.persistent)
    stage_vec(P, xs, red, Src{P.xm + vec_off(P, l, 0, P.h), nullptr, (const uint16_t *)Lw.ffn_norm}, P.h, P.kmax);
  else stage_vec(P, xs, red, Src{P.a_norm, nullptr, nullptr}, P.h, P.kmax);
  const int wave = wave_id(), nw = blockDim.x >> 6, lane = threadIdx.x & 63;
  float *u = P.u + vec_off(P, l, 0, P.F);
  for (int j = t.r0 + wave; j < t.r1; j += nw) {
    const uint16_t *rows[2] = {(const uint16_t *)Lw.wg + (int64_t)j * P.h,
                               (const uint16_t *)Lw.wu + (int64_t)j * P.h};
    const float *xsr[2] = {xs, xs};
    float y[2];
    dot_bf16<2>(rows, xsr, P.h, y);
    if (lane == 0) st_sc1(u + j, silu(y[0]) * y[1]);
  }
}

// Dense down rows [r0, r1) + residual: x_out = xm + Wd u.
__device__ __forceinline__ void task_down(const KP &P, const Task &t, int step, float *lds) {
  const int l = t.layer;
  const DevLayer &Lw = P.layers[l];
  float *xs = lds, *red = lds + P.kmax;
  stage_vec(P, xs, red, Src{P.u + vec_off(P, l, 0, P.F), nullptr, nullptr}, P.ffn, P.kmax);
  const int wave = wave_id(), nw = blockDim.x >> 6, lane = threadIdx.x & 63;
  const uint16_t *W = (const uint16_t *)Lw.wd;
  const float *xm = P.xm + vec_off(P, l, 0, P.h);
  float *xo = P.x_out + vec_off(P, l, 0, P.h);
  float *hid = (P.chk_hidden && l == P.L - 1) ? P.chk_hidden + (int64_t)step * P.B * P.h : nullptr;
  for (int i = t.r0 + 2 * wave; i < t.r1; i += 2 * nw) {
    const bool two = i + 1 < t.r1;
    const uint16_t *rows[2] = {W + (int64_t)i * P.ffn, two ? W + (int64_t)(i + 1) * P.ffn : nullptr};
    const float *xsr[2] = {xs, xs};
    float y[2];
    dot_bf16<2>(rows, xsr, P.ffn, y);
    if (lane < 2 && (lane == 0 || two)) {
      const int ii = i + lane;
      const float v = ld_sc1(xm + ii) + (lane == 0 ? y[0] : y[1]);
      st_sc1(xo + ii, v);
      if (hid) hid[ii] = v;
    }
  }
}

// Router rows [r0, r1): rl = Wr b (MoE).
__device__ __forceinline__ void task_router(const KP &P, const Task &t, float *lds) {
  const int l = t.layer;
  const DevLayer &Lw = P.layers[l];
  float *xs = lds, *red = lds + P.kmax;
  if (P.persistent)
    stage_vec(P, xs, red, Src{P.xm + vec_off(P, l, 0, P.h), nullptr, (const uint16_t *)Lw.ffn_norm}, P.h, P.kmax);
  else stage_vec(P, xs, red, Src{P.a_norm, nullptr, nullptr}, P.h, P.kmax);
  const int wave = wave_id(), nw = blockDim.x >> 6, lane = threadIdx.x & 63;
  const uint16_t *W = (const uint16_t *)Lw.router;
  float *rl = P.rl + vec_off(P, l, 0, P.E);
  for (int i = t.r0 + 2 * wave; i < t.r1; i += 2 * nw) {
    const bool two = i + 1 < t.r1;
    const uint16_t *rows[2] = {W + (int64_t)i * P.h, two ? W + (int64_t)(i + 1) * P.h : nullptr};
    const float *xsr[2] = {xs, xs};
    float y[2];
    dot_bf16<2>(rows, xsr, P.h, y);
    if (lane == 0) st_sc1(rl + i, y[0]);
    if (lane == 1 && two) st_sc1(rl + i + 1, y[1]);
  }
}

// Softmax over the router logits and top-k selection (ties -> lower expert
// id), then the n_shared shared experts with weight 1.  Every workgroup
// that needs the choice computes it; the inputs and the order of operations
// are the same everywhere, so all of them agree.  sel/selw in LDS.
__device__ __forceinline__ void route(const KP &P, int l, int *sel, float *selw, float *scratch) {
  const int tid = threadIdx.x, T = blockDim.x;
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
    uint64_t taken_lo = 0;  // per-lane bitmask of taken local indices (E <= 1024 -> 16 per lane)
    for (int k = 0; k < P.top_k; ++k) {
      float bv = -INFINITY;
      int bi = 0x7fffffff;
      int li = 0;
      for (int i = lane; i < P.E; i += 64, ++li)
        if (!((taken_lo >> li) & 1) && (scratch[i] > bv || (scratch[i] == bv && i < bi))) { bv = scratch[i]; bi = i; }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        const float ov = __shfl_xor(bv, o);
        const int oi = __shfl_xor(bi, o);
        if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
      }
      if ((bi & 63) == lane) taken_lo |= 1ull << (bi >> 6);
      if (lane == 0) { sel[k] = bi; selw[k] = expf(bv - m) / s; }
    }
    if (lane == 0)
      for (int k = 0; k < P.n_shared; ++k) { sel[P.top_k + k] = k; selw[P.top_k + k] = 1.0f; }
  }
  __syncthreads();
}

// Expert gate/up pairs [r0, r1) over (slot k, row j): u[k][j].
__device__ __forceinline__ void task_egu(const KP &P, const Task &t, float *lds) {
  const int l = t.layer;
  const DevLayer &Lw = P.layers[l];
  float *xs = lds, *red = lds + P.kmax;
  int *sel = reinterpret_cast<int *>(red + 64);
  float *selw = red + 96;
  route(P, l, sel, selw, xs);  // uses xs as scratch before the input is staged
  if (P.persistent)
    stage_vec(P, xs, red, Src{P.xm + vec_off(P, l, 0, P.h), nullptr, (const uint16_t *)Lw.ffn_norm}, P.h, P.kmax);
  else stage_vec(P, xs, red, Src{P.a_norm, nullptr, nullptr}, P.h, P.kmax);
  const int wave = wave_id(), nw = blockDim.x >> 6, lane = threadIdx.x & 63;
  const int f = P.effn, hb = (P.h + 127) / 128, fb = (f + 127) / 128;
  float *u = P.u + vec_off(P, l, 0, P.F);
  for (int p = t.r0 + wave; p < t.r1; p += nw) {
    const int k = p / f, j = p % f;
    const int e = sel[k];
    const bool shared = k >= P.top_k;
    const uint8_t *wg = (const uint8_t *)(shared ? Lw.s_wg : Lw.e_wg);
    const uint8_t *wu = (const uint8_t *)(shared ? Lw.s_wu : Lw.e_wu);
    const uint16_t *sg = (const uint16_t *)(shared ? Lw.s_sg : Lw.e_sg);
    const uint16_t *su = (const uint16_t *)(shared ? Lw.s_su : Lw.e_su);
    const int64_t wofs = ((int64_t)e * f + j) * P.h;
    const int64_t sofs = ((int64_t)e * fb + j / 128) * hb;
    const uint8_t *rows[2] = {wg + wofs, wu + wofs};
    const uint16_t *srows[2] = {sg + sofs, su + sofs};
    const float *xsr[2] = {xs, xs};
    float y[2];
    dot_fp8<2>(rows, srows, xsr, P.h, y);
    if (lane == 0) st_sc1(u + p, silu(y[0]) * y[1]);
  }
}

// Expert down rows [r0, r1): x_out = xm + sum_k w_k Wd_{e_k} u_k.
__device__ __forceinline__ void task_edown(const KP &P, const Task &t, int step, float *lds) {
  const int l = t.layer;
  const DevLayer &Lw = P.layers[l];
  float *xs = lds, *red = lds + P.kmax;
  int *sel = reinterpret_cast<int *>(red + 64);
  float *selw = red + 96;
  route(P, l, sel, selw, xs);
  stage_vec(P, xs, red, Src{P.u + vec_off(P, l, 0, P.F), nullptr, nullptr}, P.F, P.kmax);
  const int wave = wave_id(), nw = blockDim.x >> 6, lane = threadIdx.x & 63;
  const int f = P.effn, hb = (P.h + 127) / 128, fb = (f + 127) / 128;
  const int nk = P.top_k + P.n_shared;
  const float *xm = P.xm + vec_off(P, l, 0, P.h);
  float *xo = P.x_out + vec_off(P, l, 0, P.h);
  float *hid = (P.chk_hidden && l == P.L - 1) ? P.chk_hidden + (int64_t)step * P.B * P.h : nullptr;
  for (int i = t.r0 + wave; i < t.r1; i += nw) {
    float acc = 0.f;
    for (int k0 = 0; k0 < nk; k0 += 2) {
      const uint8_t *rows[2];
      const uint16_t *srows[2];
      const float *xsr[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int k = k0 + q;
        if (k < nk) {
          const bool shared = k >= P.top_k;
          const int e = sel[k];
          rows[q] = (const uint8_t *)(shared ? Lw.s_wd : Lw.e_wd) + ((int64_t)e * P.h + i) * f;
          srows[q] = (const uint16_t *)(shared ? Lw.s_sd : Lw.e_sd) + ((int64_t)e * hb + i / 128) * fb;
          xsr[q] = xs + (int64_t)k * f;
        } else {
          rows[q] = nullptr; srows[q] = nullptr; xsr[q] = xs;
        }
      }
      float y[2];
      dot_fp8<2>(rows, srows, xsr, f, y);
      acc += selw[k0] * y[0];
      if (k0 + 1 < nk) acc += selw[k0 + 1] * y[1];
    }
    if (lane == 0) {
      const float v = ld_sc1(xm + i) + acc;
      st_sc1(xo + i, v);
      if (hid) hid[i] = v;
    }
  }
}

// LM head rows [r0, r1): logits (check mode) and this task's (max, lowest
// index) partial.  A NaN logit makes the partial NaN.
__device__ __forceinline__ void task_lm(const KP &P, const Task &t, int lam, int step, float *lds) {
  float *xs = lds, *red = lds + P.kmax;
  if (P.persistent)
    stage_vec(P, xs, red, Src{P.x_out + vec_off(P, P.L - 1, 0, P.h), nullptr, P.final_norm}, P.h, P.kmax);
  else stage_vec(P, xs, red, Src{P.a_norm, nullptr, nullptr}, P.h, P.kmax);
  const int wave = wave_id(), nw = blockDim.x >> 6, lane = threadIdx.x & 63;
  float best = -INFINITY;
  int bidx = 0x7fffffff;
  bool nan = false;
  float *lg = P.chk_logits ? P.chk_logits + (int64_t)step * P.B * P.V : nullptr;
  for (int i = t.r0 + 2 * wave; i < t.r1; i += 2 * nw) {
    const bool two = i + 1 < t.r1;
    const uint16_t *rows[2] = {P.lm_head + (int64_t)i * P.h, two ? P.lm_head + (int64_t)(i + 1) * P.h : nullptr};
    const float *xsr[2] = {xs, xs};
    float y[2];
    dot_bf16<2>(rows, xsr, P.h, y);
    if (y[0] != y[0] || (two && y[1] != y[1])) nan = true;
    if (y[0] > best) { best = y[0]; bidx = i; }
    if (two && y[1] > best) { best = y[1]; bidx = i + 1; }
    if (lg) {
      if (lane == 0) lg[i] = y[0];
      if (lane == 1 && two) lg[i + 1] = y[1];
    }
  }
  float *wv = red + 128;
  int *wi = reinterpret_cast<int *>(red + 160);
  int *wn = reinterpret_cast<int *>(red + 192);
  if (lane == 0) { wv[wave] = best; wi[wave] = bidx; wn[wave] = nan; }
  __syncthreads();
  if (threadIdx.x == 0) {
    float bv = -INFINITY;
    int bi = 0x7fffffff, anynan = 0;
    for (int w = 0; w < nw; ++w) {
      anynan |= wn[w];
      if (wv[w] > bv || (wv[w] == bv && wi[w] < bi)) { bv = wv[w]; bi = wi[w]; }
    }
    if (anynan) bv = __builtin_nanf("");
    st_sc1(P.lmp + 2 * lam, bv);
    st_flag(reinterpret_cast<uint32_t *>(P.lmp) + 2 * lam + 1, (uint32_t)bi);
  }
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
      else if (v > bv || (v == bv && ix < bi)) { bv = v; bi = ix; }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float ov = __shfl_xor(bv, o);
      const int oi = __shfl_xor(bi, o);
      if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
    }
    const bool anynan = __any(nan);
    if (lane == 0) sh[1] = anynan ? -1 : bi;
  }
  __syncthreads();
  const int r = sh[1];
  __syncthreads();
  return r;
}

// Split-KV attention: chunk c of (sequence b, KV head g), all G query heads
// of the group at once so K/V are read once (query-head folding).  Writes the
// chunk's (max, sum, unnormalised output) per head.
__device__ __forceinline__ void attn_chunk(const KP &P, const Task &t, int pos, float *lds) {
  const int l = t.layer, bg = t.aux, b = bg / P.Hkv, g = bg % P.Hkv, c = t.r0, NC = t.r1;
  const int G = P.G, d = P.d, tid = threadIdx.x, T = blockDim.x;
  const int wave = wave_id(), nw = T >> 6, lane = tid & 63;
  const int n = pos + 1, C = (n + NC - 1) / NC, t0 = c * C;
  const int cnt = max(0, min(n, t0 + C) - t0);
  const int cpad = ((P.cmax + 63) / 64) * 64;
  float *qs = lds, *sc = qs + G * d, *ored = sc + G * cpad, *st = ored + nw * G * d;
  const float *qsrc = P.q + vec_off(P, l, b, P.Hq * d) + (int64_t)g * G * d;
  for (int i = tid; i < G * d; i += T) qs[i] = ld_sc1(qsrc + i) * P.attn_scale;
  __syncthreads();
  const int64_t cbase = (((int64_t)l * P.B + b) * P.Hkv + g) * P.max_ctx * d;
  const Rsrc kr = mkbuf(P.kc + cbase, (uint32_t)P.max_ctx * d * 2);
  const Rsrc vr = mkbuf(P.vc + cbase, (uint32_t)P.max_ctx * d * 2);
  const int LPP = d / 8, PPW = 64 / LPP, sub = lane % LPP, grp = lane / LPP;
  // scores
  for (int base = wave * PPW; base < cnt; base += nw * PPW) {
    const int tt = base + grp;
    const bool live = tt < cnt;
    v4i kw = live ? ld128<CP_SC1>(kr, (uint32_t)((int64_t)(t0 + tt) * d + sub * 8) * 2) : v4i{0, 0, 0, 0};
    for (int hh = 0; hh < G; ++hh) {
      const float4 *q4 = reinterpret_cast<const float4 *>(qs + hh * d + sub * 8);
      float s = dot8_bf16(kw, q4[0], q4[1], 0.f);
      s = (LPP == 16) ? sum16(s) : sum8(s);
      if (live && sub == 0) sc[hh * cpad + tt] = s;
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
  // o = sum_t p_t V_t: lane owns 8 dims of one position per pass
  float acc[8][8];
#pragma unroll
  for (int hh = 0; hh < 8; ++hh)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[hh][e] = 0.f;
  for (int base = wave * PPW; base < cnt; base += nw * PPW) {
    const int tt = base + grp;
    if (tt >= cnt) continue;
    const v4i vw = ld128<CP_SC1>(vr, (uint32_t)((int64_t)(t0 + tt) * d + sub * 8) * 2);
    const float v[8] = {bf_lo(vw.x), bf_hi(vw.x), bf_lo(vw.y), bf_hi(vw.y),
                        bf_lo(vw.z), bf_hi(vw.z), bf_lo(vw.w), bf_hi(vw.w)};
#pragma unroll
    for (int hh = 0; hh < 8; ++hh)
      if (hh < G) {
        const float p = sc[hh * cpad + tt];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[hh][e] = fmaf(p, v[e], acc[hh][e]);
      }
  }
  // reduce the PPW position groups of the wave (lanes sub, sub+LPP, ...)
#pragma unroll
  for (int hh = 0; hh < 8; ++hh)
    if (hh < G) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float v = acc[hh][e];
        for (int o = LPP; o < 64; o <<= 1) v += __shfl_xor(v, o);
        acc[hh][e] = v;
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
}

// Combine the NC chunk partials of (sequence b, KV head g) into o.
__device__ __forceinline__ void attn_combine(const KP &P, int l, int bg, float *lds) {
  const int b = bg / P.Hkv, g = bg % P.Hkv, G = P.G, d = P.d, NC = P.NC;
  const int tid = threadIdx.x, T = blockDim.x;
  const float *src = P.part + (((int64_t)l * P.B + b) * P.Hkv + g) * NC * G * (d + 2);
  float *ml = lds;  // [NC][G][2]
  for (int i = tid; i < NC * G; i += T) {
    const int cc = i / G, hh = i % G;
    ml[2 * i] = ld_sc1(src + ((int64_t)cc * G + hh) * (d + 2));
    ml[2 * i + 1] = ld_sc1(src + ((int64_t)cc * G + hh) * (d + 2) + 1);
  }
  __syncthreads();
  float *dst = P.o + vec_off(P, l, b, P.Hq * d) + (int64_t)g * G * d;
  for (int i = tid; i < G * d; i += T) {
    const int hh = i / d, j = i % d;
    float M = -INFINITY;
    for (int cc = 0; cc < NC; ++cc) M = fmaxf(M, ml[2 * (cc * G + hh)]);
    float num = 0.f, den = 0.f;
    for (int cc = 0; cc < NC; ++cc) {
      const float wgt = expf(ml[2 * (cc * G + hh)] - M);
      den = fmaf(wgt, ml[2 * (cc * G + hh) + 1], den);
      num = fmaf(wgt, ld_sc1(src + ((int64_t)cc * G + hh) * (d + 2) + 2 + j), num);
    }
    st_sc1(dst + i, num / den);
  }
}

// Persistent attention task: chunk, then the last of the NC chunk tasks of
// this (sequence, KV head) to arrive combines and publishes the group.
__device__ __forceinline__ void task_attn(const KP &P, const Task &t, int pos, uint32_t ep, float *lds, int *sh) {
  attn_chunk(P, t, pos, lds);
  drain();
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t *cnt = P.counters + (int64_t)t.layer * P.B * P.Hkv + t.aux;
    const uint32_t old = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sh[2] = (old == (uint32_t)t.r1 * ep - 1u);
  }
  __syncthreads();
  const bool last = sh[2] != 0;
  __syncthreads();
  if (last) {
    attn_combine(P, t.layer, t.aux, lds);
    signal_slot(P, t.signal, ep);
  }
}

__device__ __forceinline__ void trace_rec(const KP &P, int step, int si, int lam, uint32_t a, uint32_t b,
                                          uint32_t c) {
  if (!P.trace || threadIdx.x != 0) return;
  const uint64_t idx = ((uint64_t)step * P.n_si + si) * P.W + lam;
  if (idx >= P.trace_cap) return;
  uint32_t *r = P.trace + 4 * idx;
  r[0] = (uint32_t)si | ((uint32_t)lam << 16);
  r[1] = a; r[2] = b; r[3] = c;
}

__device__ __forceinline__ bool token_ok(const KP &P, int tok, int step) {
  if (tok >= 0 && tok < P.V) return true;
  if (threadIdx.x == 0) latch_error(P, PRE_DEV_BAD_TOKEN, step, -1, -1, (uint32_t)tok, 0);
  return false;
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
      if (!wait_slots(P, t.wait_lo, t.wait_hi, ep, s, si, sh)) return;
      const uint32_t ts = (uint32_t)now_ticks();
      switch (t.op) {
        case OP_QKV: task_qkv(P, t, pos, tok, lds); break;
        case OP_ATTN: task_attn(P, t, pos, ep, lds, sh); break;
        case OP_OPROJ: task_oproj(P, t, tok, lds); break;
        case OP_GU: task_gu(P, t, lds); break;
        case OP_DOWN: task_down(P, t, s, lds); break;
        case OP_ROUTER: task_router(P, t, lds); break;
        case OP_EGU: task_egu(P, t, lds); break;
        case OP_EDOWN: task_edown(P, t, s, lds); break;
        case OP_LM: task_lm(P, t, lam, s, lds); break;
        default: break;
      }
      if (t.op != OP_ATTN) signal_slot(P, t.signal, ep);
      trace_rec(P, s, si, lam, tw, ts, (uint32_t)now_ticks());
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
  for (int i = threadIdx.x; i < P.h; i += blockDim.x) P.x_emb[i] = bf16f(P.embed[(int64_t)tok * P.h + i]);
}

// a_norm = RMSNorm(src, gain)
extern "C" __global__ void __launch_bounds__(512) pre_k_norm(KP P, const float *src, const uint16_t *gain) {
  extern __shared__ __attribute__((aligned(16))) float lds[];
  float *xs = lds, *red = lds + P.kmax;
  stage_vec(P, xs, red, Src{src, nullptr, gain}, P.h, P.kmax);
  for (int i = threadIdx.x; i < P.kmax; i += blockDim.x) P.a_norm[i] = xs[i];
}

extern "C" __global__ void __launch_bounds__(512) pre_k_task(KP P, int si, int step) {
  extern __shared__ __attribute__((aligned(16))) float lds[];
  const int lam = blockIdx.x;
  const Task t = P.tasks[(int64_t)si * P.W + lam];
  const int pos = P.pos0 + step;
  const int tok = P.tok_slot[1];
  switch (t.op) {
    case OP_QKV: task_qkv(P, t, pos, tok, lds); break;
    case OP_ATTN: attn_chunk(P, t, pos, lds); break;
    case OP_OPROJ: task_oproj(P, t, tok, lds); break;
    case OP_GU: task_gu(P, t, lds); break;
    case OP_DOWN: task_down(P, t, step, lds); break;
    case OP_ROUTER: task_router(P, t, lds); break;
    case OP_EGU: task_egu(P, t, lds); break;
    case OP_EDOWN: task_edown(P, t, step, lds); break;
    case OP_LM: task_lm(P, t, lam, step, lds); break;
    default: break;
  }
}

extern "C" __global__ void __launch_bounds__(512) pre_k_combine(KP P, int l) {
  extern __shared__ __attribute__((aligned(16))) float lds[];
  attn_combine(P, l, blockIdx.x, lds);
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

// Debug: decode n fp8 codes with the GEMV's unpacking (checks the format).
extern "C" __global__ void pre_k_fp8_decode(const uint8_t *in, float *out, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (4 * i + 3 < n) {
    float f[4];
    fp8x4(*reinterpret_cast<const uint32_t *>(in + 4 * i), f);
    for (int k = 0; k < 4; ++k) out[4 * i + k] = f[k];
  }
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
          hipSuccess ||
      hipFuncSetAttribute((const void *)pre_k_combine, hipFuncAttributeMaxDynamicSharedMemorySize, dyn) !=
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
  P.moe = D.moe; P.G = D.G; P.F = D.F; P.W = D.W; P.X = D.X; P.NC = D.NC; P.n_si = D.n_si;
  P.spl = D.stages_per_layer; P.kmax = D.kmax; P.cmax = D.cmax;
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
  P.counters = (uint32_t *)(ws + Lo.counters);
  P.xcc = (uint32_t *)(ws + Lo.xcc);
  P.status = (DevStatus *)(ws + Lo.status);
  P.rope = (const float *)(ws + Lo.rope);
  P.x_out = (float *)(ws + Lo.x_out);
  P.xm = (float *)(ws + Lo.xm);
  P.q = (float *)(ws + Lo.q);
  P.o = (float *)(ws + Lo.o);
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
  P.trace_cap = (uint32_t)std::min<size_t>(e->trace_bytes / 16, 0xffffffffu);
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
  const char *ws = e->ws;
  const float *x_out = (const float *)(ws + e->Lo.x_out), *xm = (const float *)(ws + e->Lo.xm);
  const float *x_emb = (const float *)(ws + e->Lo.x_emb);
  const std::vector<pre_layer_w> &lw = e->lw;
  static_assert(sizeof(pre_layer_w) == sizeof(DevLayer), "layer table layout");
  for (int s = 0; s < n_steps; ++s) {
    hipLaunchKernelGGL(pre_k_embed, dim3(1), blk, 0, st, P, s);
    for (int l = 0; l < D.L; ++l) {
      const int si0 = l * D.stages_per_layer;
      const float *xin = l == 0 ? x_emb : x_out + (int64_t)(l - 1) * D.B * D.h;
      hipLaunchKernelGGL(pre_k_norm, dim3(D.B), blk, lds, st, P, xin, (const uint16_t *)lw[l].attn_norm);
      hipLaunchKernelGGL(pre_k_task, dim3(D.W), blk, lds, st, P, si0 + 0, s);
      hipLaunchKernelGGL(pre_k_task, dim3(D.B * D.Hkv * D.NC), blk, lds, st, P, si0 + 1, s);
      hipLaunchKernelGGL(pre_k_combine, dim3(D.B * D.Hkv), blk, lds, st, P, l);
      hipLaunchKernelGGL(pre_k_task, dim3(D.W), blk, lds, st, P, si0 + 2, s);
      hipLaunchKernelGGL(pre_k_norm, dim3(D.B), blk, lds, st, P, xm + (int64_t)l * D.B * D.h,
                         (const uint16_t *)lw[l].ffn_norm);
      for (int k = 3; k < D.stages_per_layer; ++k)
        hipLaunchKernelGGL(pre_k_task, dim3(D.W), blk, lds, st, P, si0 + k, s);
    }
    hipLaunchKernelGGL(pre_k_norm, dim3(D.B), blk, lds, st, P, x_out + (int64_t)(D.L - 1) * D.B * D.h,
                       (const uint16_t *)e->final_norm);
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
      hipMemsetAsync(e->ws + Lo.flags, 0, (size_t)(Lo.counters - Lo.flags) + (size_t)(Lo.layers - Lo.counters),
                     st) != hipSuccess)
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
