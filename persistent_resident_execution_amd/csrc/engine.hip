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
#include <mutex>
#include <type_traits>
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
  int32_t n_si, spl, kmax, ymax, segoff, cmax, lds_floats;
  int32_t npre, xsoff;  // GEMV: most units per wavefront loaded into LDS first; staged input offset
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
  float *x_out, *pbuf, *q, *u, *rl, *part, *lmp, *x_emb, *a_norm, *xmid;
  int32_t *tok_slot;
  // this call
  int32_t n_steps;
  int32_t *ctx_len;      // [B] each sequence's position (= cached tokens) at the call's start;
                         // read by every workgroup at the start, advanced at the end
  uint32_t epoch_base, watchdog_ticks;
  const int32_t *in_tok, *forced;
  int32_t *out_tok;
  float *chk_logits, *chk_hidden;
  uint32_t *trace;
  uint32_t trace_cap;
  int32_t persistent;
  int32_t b_si, b_step;  // baseline launches: the stage and step to run
  int32_t b_nsteps;      // baseline: steps of the whole call (the position check)
  int32_t local;         // XCD-local hand-offs (QKV -> attention -> O projection)
  int32_t onexcd;        // every workgroup on XCD 0: every hand-off in that XCD's L2
  int32_t drop_slot;     // debug: the task setting this ready flag skips the store (-1: none)
  // micro-batch
  int32_t mbst;          // longest GEMM input staged in LDS (columns; longer ones stream from memory)
  int32_t Bc;            // sequences of the K/V cache (a chunk of one sequence: 1)
  int32_t chunk;         // the B columns are consecutive tokens of sequence 0 (prefill, verify)
  int32_t chunk_n;       // chunk mode: tokens of the call (the last step may be ragged)
  int32_t verify;        // chunk mode, one step: accept the drafts, commit the accepted tokens
  int32_t *v_accept;     // verify: the number of accepted drafts
  int32_t kv8;           // fp8 e4m3 cache: kc / vc hold codes, ksc / vsc one fp32 scale per row
  float *ksc, *vsc;      // [L][B][Hkv][max_ctx]
  float *kvnew;          // the step's new K and V rows in fp32 [L][B][2][Hkv][d]
  uint8_t *pk;           // packed GEMM inputs
  float *ssq;            // per-workgroup sums of squares of the normalised inputs
  // serving loop: the request ring (coherent host memory) and the
  // scheduler's broadcast area in the workspace
  uint32_t *ring;        // header (16 words) then ring_slots slots of ring_words words
  int32_t *cmd;          // workspace: command sequence number and the claimed request
  int32_t *req_tok;      // workspace: the claimed request's prompt [max_ctx]
  int32_t ring_slots, ring_prompt, ring_out, ring_words;
  uint32_t idle_ticks;   // the loop ends after this long without a request
  // folded FFN (small-model kernel): the gate/up tasks leave the down
  // projection's partials, the down stage is skipped
  int32_t fold;
  float *dpart;          // [L][W][h]
  // attention folded into the output projection (small-model kernel): the
  // attention stage is skipped, every O-projection task attends itself
  int32_t inl, aoff;     // on; LDS float offset of the attention's scratch
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
template <bool PIPE = false>
__device__ __forceinline__ bool wait_slots(const KP &P, int lo, int hi, uint32_t ep, int step,
                                           int stage, int *sh) {
  if (lo >= hi) return true;
  if (PIPE && threadIdx.x < 64 && hi - lo <= 256) {
    // Up to 256 producers: two polls in flight.  Each check uses the older
    // poll while the newer one is already on its way, so a flag that lands
    // is seen about half a memory round trip sooner than with one poll at a
    // time.
    const int lane = threadIdx.x;
    const uint64_t t0 = now_ticks();
    int verdict = 1, iter = 0;
    auto poll = [&](uint32_t (&v)[4]) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int i = lo + lane + 64 * k;
        v[k] = i < hi ? ld_flag(P.flags + i) : ep;
      }
    };
    auto done = [&](const uint32_t (&v)[4]) {
      bool ok = true;
#pragma unroll
      for (int k = 0; k < 4; ++k) ok &= (int32_t)(v[k] - ep) >= 0;
      return __all(ok);
    };
    uint32_t a[4], b[4];
    poll(a);
    while (true) {
      poll(b);
      if (done(a)) break;
      poll(a);
      if (done(b)) break;
      if ((++iter & 7) == 0) {
        if (ld_flag(&P.status->abort)) { verdict = 0; break; }
        if (now_ticks() - t0 > P.watchdog_ticks) {
          uint32_t seen = ep;
          int bad = -1;
#pragma unroll
          for (int k = 0; k < 4; ++k)
            if ((int32_t)(b[k] - ep) < 0 && lo + lane + 64 * k < hi) { seen = b[k]; bad = lo + lane + 64 * k; }
          const uint64_t m = __ballot(bad >= 0);
          const int first = __ffsll((unsigned long long)m) - 1;
          if (lane == first) latch_error(P, PRE_DEV_TIMEOUT, step, stage, bad, seen, ep);
          verdict = 0;
          break;
        }
      }
    }
    if (lane == 0) sh[0] = verdict;
  } else if (threadIdx.x < 64) {
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
// Timestamps are taken only when a trace buffer is set: reading the clock is
// a scalar-memory round trip that the barrier after it would make every
// wavefront wait for.
// PIPE: two polls in flight (the batch-1 kernel; the micro-batch kernel's
// register budget keeps the single poll).
template <bool PIPE>
struct WaiterT {
  int active, lo, hi, step, stage;
  uint32_t ep;
  int *sh;
  int tr;  // tracing on
  __device__ __forceinline__ bool operator()(const KP &P) const {
    if (!active) return true;
    const bool ok = wait_slots<PIPE>(P, lo, hi, ep, step, stage, sh);
    if (tr && threadIdx.x == 0) sh[3] = (int)(uint32_t)now_ticks();  // trace: end of the wait
    return ok;
  }
  // trace: time of phase k (0..3) of the task, taken by thread 0
  __device__ __forceinline__ void mark(int k) const {
    if (tr && threadIdx.x == 0) sh[4 + k] = (int)(uint32_t)now_ticks();
  }
};
using Waiter = WaiterT<true>;
using MbWaiter = WaiterT<false>;

// Publish: every thread's stores are complete, then one flag store.  When
// all of the flag's readers are on this XCD (the QKV and attention stages
// with XCD-local placement) the flag goes into the XCD's L2 (sc0), where the
// readers' device-scope polls find it without a round trip to memory; the
// data itself is always written through at device scope: under the weight
// stream, L2-scope stores of partly written lines drain several times
// slower.
__device__ __forceinline__ void signal_slot(const KP &P, int slot, uint32_t ep, bool local) {
  drain();
  __syncthreads();
  if (threadIdx.x == 0 && slot >= 0 && slot != P.drop_slot) {
    if (local) __builtin_amdgcn_raw_buffer_store_b32(ep, mkbuf(P.flags + slot, 4), 0, 0, CP_SC0);
    else st_flag(P.flags + slot, ep);
  }
}

// A result other workgroups read: written through at device scope, or, with
// one-XCD placement (every reader shares this XCD's L2), left in the L2,
// where the readers' device-scope loads find it without a memory round trip.
__device__ __forceinline__ void st_out(const KP &P, float *p, float v) {
  if (P.onexcd)
    __hip_atomic_store(reinterpret_cast<uint32_t *>(p), __builtin_bit_cast(uint32_t, v), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_WORKGROUP);
  else
    st_sc1(p, v);
}
// A result whose every reader runs on this XCD (the QKV -> attention ->
// O-projection hand-offs of one KV head with XCD-local placement): left in
// the XCD's L2 like those stages' flags, so the readers' device-scope loads
// find it there instead of in memory.
__device__ __forceinline__ void st_xcd(const KP &P, float *p, float v) {
  if (P.local || P.onexcd)
    __hip_atomic_store(reinterpret_cast<uint32_t *>(p), __builtin_bit_cast(uint32_t, v), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_WORKGROUP);
  else
    st_sc1(p, v);
}
__device__ __forceinline__ void st_xcd16(const KP &P, Rsrc r, uint32_t off, uint16_t v) {
  if (P.local || P.onexcd) st16<CP_SC0>(r, off, v);
  else st16<CP_SC1>(r, off, v);
}
__device__ __forceinline__ void st_out16(const KP &P, Rsrc r, uint32_t off, uint16_t v) {
  if (P.onexcd) st16<CP_SC0>(r, off, v);
  else st16<CP_SC1>(r, off, v);
}
__device__ __forceinline__ void st_out128(const KP &P, Rsrc r, uint32_t off, v4i v) {
  if (P.onexcd) st128<CP_SC0>(r, off, v);
  else st128<CP_SC1>(r, off, v);
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
  float *dump;           // non-NULL: write float4s [d0, d1) of the summed vector here
  int d0, d1;
};
constexpr int MAXPARTS = 8;  // KV heads per sequence (partials of the split O projection)
constexpr int MAXW = 8;      // wavefronts per workgroup (at most 512 threads)
constexpr int PREC_O = 4;    // attention chunk record: m, l, two unused words, then o[d]

// xs[0..K) = src (times the gains if given), xs[K..Kpad) = 0.  Ends with a
// barrier.  RMSNorm is folded: with gains, each wavefront's sum of squares
// of the unscaled input goes to red[wave], and the consumer multiplies its
// results by norm_scale() -- W (x * g) / rms(x) equals W (x * g / rms(x)) --
// so staging needs neither a second pass nor a barrier before it.  The gains
// are fetched together with the data: staging costs one device round trip.
__device__ __forceinline__ void stage_vec(const KP &P, float *xs, float *red, const Src &s, int K,
                                          int Kpad) {
  const int tid = threadIdx.x, T = P.nthr, n4 = K >> 2;
  float ss = 0.f;
  const Rsrc rg = mkbuf(uni_ptr(s.gain), s.gain ? (uint32_t)K * 2 : 0u);
  auto scaled = [](float4 f, v2i g) {
    return float4{f.x * bf_lo(g.x), f.y * bf_hi(g.x), f.z * bf_lo(g.y), f.w * bf_hi(g.y)};
  };
  if (s.f32 && s.nparts == 0) {
    const Rsrc r = mkbuf(uni_ptr(s.f32), (uint32_t)K * 4);
    for (int i = tid; i < n4; i += 8 * T) {
      v4i a[8];
      v2i g[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {  // loads past the input are not issued
        a[j] = v4i{0, 0, 0, 0};
        g[j] = v2i{0, 0};
        if (i + j * T < n4) {
          a[j] = ld128<CP_SC1>(r, (uint32_t)(i + j * T) * 16);
          if (s.gain) g[j] = ld64<CP_DEF>(rg, (uint32_t)(i + j * T) * 8);
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (i + j * T < n4) {
          const float4 f = __builtin_bit_cast(float4, a[j]);
          reinterpret_cast<float4 *>(xs)[i + j * T] = s.gain ? scaled(f, g[j]) : f;
          ss = fmaf(f.x, f.x, ss); ss = fmaf(f.y, f.y, ss);
          ss = fmaf(f.z, f.z, ss); ss = fmaf(f.w, f.w, ss);
        }
    }
  } else {
    // base (fp32 or bf16) plus partial vectors, two float4 per thread per round
    const Rsrc rb = mkbuf(uni_ptr(s.f32 ? (const void *)s.f32 : (const void *)s.bf16), (uint32_t)K * (s.f32 ? 4 : 2));
    const Rsrc rp = mkbuf(uni_ptr(s.parts), s.parts ? (uint32_t)((s.nparts - 1) * s.pstride + K) * 4 : 0u);
    const Rsrc rd = mkbuf(uni_ptr(s.dump), s.dump ? (uint32_t)K * 4 : 0u);
    for (int i0 = tid; i0 < n4; i0 += 2 * T) {
      v4i pv[2][MAXPARTS], bv[2];
      v2i g[2];
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
        g[k] = s.gain ? ld64<CP_DEF>(rg, (uint32_t)i * 8) : v2i{0, 0};
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
        reinterpret_cast<float4 *>(xs)[i] = s.gain ? scaled(f, g[k]) : f;
        if (s.dump && i >= s.d0 && i < s.d1)
          st_out128(P, rd, (uint32_t)i * 16, __builtin_bit_cast(v4i, f));
        ss = fmaf(f.x, f.x, ss); ss = fmaf(f.y, f.y, ss);
        ss = fmaf(f.z, f.z, ss); ss = fmaf(f.w, f.w, ss);
      }
    }
  }
  for (int i = K + tid; i < Kpad; i += T) xs[i] = 0.f;
  if (s.gain) {
    const float w = wave_sum2_l63(ss, 0.f).x;
    if ((tid & 63) == 63) red[wave_id()] = w;
  }
  __syncthreads();
}

// 1 / rms of the input staged with gains: from the per-wavefront sums of
// squares that stage_vec left in red (read after a later barrier).
__device__ __forceinline__ float norm_scale(const KP &P, const float *red, int K) {
  float rw[MAXW];
#pragma unroll
  for (int w = 0; w < MAXW; ++w) rw[w] = w < P.nw ? red[w] : 0.f;
  float tot = 0.f;
#pragma unroll
  for (int w = 0; w < MAXW; ++w) tot += rw[w];
  return 1.0f / sqrtf(tot / (float)K + P.eps);
}

// Staging of the folded FFN's consumers (the next layer's QKV stage, the LM
// head): x = base + the np partials of the down projection (vectors of K
// floats, np <= 32), times the gains, RMSNorm folded as in stage_vec.  The 8
// lanes of a group share one float4 slot: lane j adds partials j, j + 8, ...
// (lane 0 starts from the base), the group's sums meet by a butterfly over
// the 8 lanes (the same order on every run), and lane 0 writes the slot.
// Float4s [d0, d1) of x (before the gains) also go to dump and, if given,
// dump2.  All loads of a round are in flight together: one device round
// trip for up to 32 partials.  Ends with a barrier.
__device__ __forceinline__ void stage_fold(const KP &P, float *xs, float *red, const float *base,
                                           const float *parts, int np, const uint16_t *gain, float *dump,
                                           float *dump2, int d0, int d1, int K, int Kpad) {
  const int tid = threadIdx.x, T = P.nthr, n4 = K >> 2, j = tid & 7, per = T >> 3;
  constexpr uint32_t OOB = 0x80000000u;
  const Rsrc rb = mkbuf(uni_ptr(base), (uint32_t)K * 4);
  const Rsrc rp = mkbuf(uni_ptr(parts), (uint32_t)np * K * 4);
  const Rsrc rg = mkbuf(uni_ptr(gain), (uint32_t)K * 2);
  const Rsrc rd = mkbuf(uni_ptr(dump), dump ? (uint32_t)K * 4 : 0u);
  const Rsrc rd2 = mkbuf(uni_ptr(dump2), dump2 ? (uint32_t)K * 4 : 0u);
  float ss = 0.f;
  for (int i0 = 0; i0 < n4; i0 += per) {
    const int i = i0 + (tid >> 3);
    const bool in = i < n4;
    v4i a[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int p = j + 8 * k;
      a[k] = ld128<CP_SC1>(rp, in && p < np ? (uint32_t)(p * K + 4 * i) * 4 : OOB);
    }
    const v4i b = ld128<CP_SC1>(rb, in && j == 0 ? (uint32_t)i * 16 : OOB);
    const v2i g = ld64<CP_DEF>(rg, in && j == 0 ? (uint32_t)i * 8 : OOB);
    float4 f = __builtin_bit_cast(float4, b);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float4 q = __builtin_bit_cast(float4, a[k]);
      f.x += q.x; f.y += q.y; f.z += q.z; f.w += q.w;
    }
#pragma unroll
    for (int m = 1; m < 8; m <<= 1) {
      f.x += __shfl_xor(f.x, m); f.y += __shfl_xor(f.y, m);
      f.z += __shfl_xor(f.z, m); f.w += __shfl_xor(f.w, m);
    }
    if (in && j == 0) {
      reinterpret_cast<float4 *>(xs)[i] = float4{f.x * bf_lo(g.x), f.y * bf_hi(g.x), f.z * bf_lo(g.y), f.w * bf_hi(g.y)};
      ss = fmaf(f.x, f.x, ss); ss = fmaf(f.y, f.y, ss);
      ss = fmaf(f.z, f.z, ss); ss = fmaf(f.w, f.w, ss);
      if (i >= d0 && i < d1) {
        if (dump) st_out128(P, rd, (uint32_t)i * 16, __builtin_bit_cast(v4i, f));
        if (dump2) st_out128(P, rd2, (uint32_t)i * 16, __builtin_bit_cast(v4i, f));
      }
    }
  }
  for (int i = K + tid; i < Kpad; i += T) xs[i] = 0.f;
  const float w = wave_sum2_l63(ss, 0.f).x;
  if ((tid & 63) == 63) red[wave_id()] = w;
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Streamed GEMV core.
//
// Every projection of the step runs as a stream of row *pairs* that share
// one input vector: a RoPE pair (j, j + d/2) of one q/k/v head, a gate/up
// pair, or two consecutive rows (the second one absent at a ragged end).  A
// task's pairs form a few segments -- runs of pairs inside one matrix (a
// head, an expert slot, a row range) -- listed in LDS.  Each row is cut into
// chunks of one 16-byte load per lane (512 bf16 or 1024 fp8 columns), so
// every load instruction of a wavefront reads 1 KB of consecutive weight
// bytes.  The task's (pair, chunk) units are split into one contiguous span
// per wavefront (split-K across wavefronts where a span ends inside a pair),
// so every wavefront streams the same amount.  A ring of D units (2D loads)
// is kept in flight per wavefront: unit u is consumed while unit u + D is
// being fetched, across row and segment boundaries, with no barrier.  The
// first D units are issued before the task waits for its producers (weights
// never wait on activations).  Loads past a row's end, or past the span's
// end, address a zero-length buffer and return 0 without touching memory.
// A wavefront writes one partial sum per (pair it touched, row) into LDS;
// the epilogue adds the wavefronts' partials in wavefront order
// (deterministic).
//
// Every projection shares this one loop -- one copy for bf16 weights, one
// for fp8 experts -- so the code the resident kernel runs stays small enough
// to stay in the instruction cache across task switches.

constexpr int CP_W = CP_NT;  // weight loads: streaming (read once per step)
constexpr int RING = 4;      // units (pairs of 16-byte loads per lane) in flight

// A run of n pairs inside one matrix.  Pair i of the run has its A row at
// a + i * pstride and its B row at b + i * pstride (pairs i >= nB have no B
// row); its row index, for the fp8 block scales, is j0 + i * gstep.
struct Seg {
  uint64_t a, b;    // byte addresses of the first pair's A and B rows (b = 0: none)
  uint64_t sa, sb;  // fp8: block-scale matrices of A and B (row block 0)
  int32_t j0, n, nB, xo;  // first row index, pairs, pairs with a B row, input offset (floats)
};
[[maybe_unused]] constexpr int SEGMAX = 80;  // most segments of one task (every q/k/v head of a layer)

// Geometry shared by all pairs of a task (wave-uniform).
struct Geo {
  int K;             // columns of every row
  uint32_t rowbytes; // bytes of one row's K columns
  uint32_t pstride;  // bytes from one pair's A row to the next pair's
  int gstep, jb;     // rows from one pair's A row to the next's; B row index - A row index
  uint32_t srow;     // fp8: bytes per row block of a block-scale matrix
  int nseg, NG;      // segments, pairs in all
};

// The geometry as scalar values.  Builders compute it next to a branch taken
// by one thread (the one writing the table); the compiler may then merge the
// two copies into a value it must treat as per-lane, which would turn every
// weight load into a loop over lanes.  Reading each field through
// readfirstlane keeps it scalar.
__device__ __forceinline__ int rfl(int v);
__device__ __forceinline__ Geo geo_uniform(const Geo &g) {
  return Geo{rfl(g.K), (uint32_t)rfl((int)g.rowbytes), (uint32_t)rfl((int)g.pstride), rfl(g.gstep), rfl(g.jb),
             (uint32_t)rfl((int)g.srow), rfl(g.nseg), rfl(g.NG)};
}

template <bool FP8, int D = RING, int CP = CP_W>
struct PStream {
  v4i buf[D][2];
  uint16_t sc[D][2];  // fp8: the bf16 block scale of each lane's 16 weights, as loaded (widened where
                      // used, so that issuing a unit never waits for its scale)
  int xo[D];       // fp8: input offset of the unit in each slot
  // issue cursor (wave-uniform)
  uint64_t pa, pb, sa, sb;
  int j, ig, is, ic, segn, segnB, segxo;
  uint32_t rbA;
  // compute cursor
  int cg, cc;
  int nch, left, wave, nw;
  int np;        // units of the span held in LDS (the span's first ones)
  uint32_t pre;  // LDS byte address of this wavefront's units there
  float acc[2];
};

__device__ __forceinline__ int rfl(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ uint64_t rfl64(uint64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ Rsrc mkbuf64(uint64_t p, uint32_t bytes) {
  return mkbuf(reinterpret_cast<const void *>(p), bytes);
}

// Point the issue cursor at the first pair of segment s (past the last
// segment every row has length 0).
template <bool FP8, int D, int CP>
__device__ __forceinline__ void seg_enter(PStream<FP8, D, CP> &S, const Seg *tab, const Geo &G, int s) {
  S.ig = 0;
  if (s < G.nseg) {
    const Seg &e = tab[s];
    S.pa = rfl64(e.a);
    S.pb = rfl64(e.b);
    if (FP8) { S.sa = rfl64(e.sa); S.sb = rfl64(e.sb); }
    S.j = rfl(e.j0);
    S.segn = rfl(e.n);
    S.segnB = rfl(e.nB);
    S.segxo = rfl(e.xo);
    S.rbA = G.rowbytes;
  } else {
    S.pa = S.pb = S.sa = S.sb = 0;
    S.j = 0;
    S.segn = 0x7fffffff;
    S.segnB = 0;
    S.segxo = 0;
    S.rbA = 0;
  }
}

// Move the issue cursor to the next unit of the span.  Once the span is used
// up every further issue reads nothing.
template <bool FP8, int D, int CP>
__device__ __forceinline__ void st_advance(PStream<FP8, D, CP> &S, const Seg *tab, const Geo &G) {
  if (--S.left <= 0) {
    S.rbA = 0;
  } else if (++S.ic == S.nch) {
    S.ic = 0;
    if (++S.ig == S.segn) {
      seg_enter(S, tab, G, ++S.is);
    } else {
      S.pa += G.pstride;
      S.pb += G.pstride;
      S.j += G.gstep;
    }
  }
}

// Issue the unit under the cursor into ring slot jj and advance the cursor.
template <bool FP8, int D, int CP>
__device__ __forceinline__ void st_issue(PStream<FP8, D, CP> &S, int jj, const Seg *tab, const Geo &G) {
  const int lane = threadIdx.x & 63;
  const uint32_t col = FP8 ? (uint32_t)S.ic * 1024 + lane * 16 : (uint32_t)S.ic * 512 + lane * 8;
  const uint32_t off = FP8 ? col : col * 2;
  const uint32_t rbB = S.ig < S.segnB ? S.rbA : 0u;
  S.buf[jj][0] = ld128<CP>(mkbuf64(S.pa, S.rbA), off);
  S.buf[jj][1] = ld128<CP>(mkbuf64(S.pb, rbB), off);
  if (FP8) {
    // this lane's 16 columns share one 128-wide block: one bf16 scale each
    const uint32_t so = (col >> 7) * 2;
    S.sc[jj][0] = __builtin_amdgcn_raw_buffer_load_b16(
        mkbuf64(S.sa + (uint64_t)(S.j >> 7) * G.srow, S.rbA ? G.srow : 0u), so, 0, CP_DEF);
    S.sc[jj][1] = __builtin_amdgcn_raw_buffer_load_b16(
        mkbuf64(S.sb + (uint64_t)((S.j + G.jb) >> 7) * G.srow, rbB ? G.srow : 0u), so, 0, CP_DEF);
    S.xo[jj] = S.segxo;
  }
  st_advance(S, tab, G);
}

// Issue the unit under the cursor (bf16) straight into LDS at byte address
// dst: row A's 1 KB, then row B's (zeros past a task's last B row), lane i's
// 16 bytes at 16 i; no register holds it.
template <bool FP8, int D, int CP>
__device__ __forceinline__ void st_issue_lds(PStream<FP8, D, CP> &S, uint32_t dst, const Seg *tab, const Geo &G) {
  static_assert(!FP8, "the LDS head is for bf16 streams");
  const int lane = threadIdx.x & 63;
  const uint32_t off = ((uint32_t)S.ic * 512 + lane * 8) * 2;
  const uint32_t rbB = S.ig < S.segnB ? S.rbA : 0u;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(mkbuf64(S.pa, S.rbA), lds_ptr(dst), 16, off, 0, 0, CP);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(mkbuf64(S.pb, rbB), lds_ptr(dst + 1024), 16, off, 0, 0, CP);
  st_advance(S, tab, G);
}

// This wavefront's span of the task's NG * nch units; issues its first D
// units (reading nothing past the span).  Returns the span length.
// With npre > 0 (bf16), the span's first min(npre, n) units go straight into
// LDS at pre (2 KB each; the wavefront's own area) before the ring's D:
// twice the bytes on their way while the task waits for its producers and
// stages its input, without the registers a deeper ring would take.
template <bool FP8, int D, int CP>
__device__ __forceinline__ int st_begin(PStream<FP8, D, CP> &S, const Seg *tab, const Geo &G, int nw,
                                        int npre = 0, const float *pre = nullptr) {
  const int wave = wave_id();
  S.wave = wave;
  S.nw = nw;
  S.nch = FP8 ? (G.K + 1023) >> 10 : (G.K + 511) >> 9;
  const uint32_t N = (uint32_t)(G.NG * S.nch);  // < 2^26 for every supported shape
  const int u0 = (int)(N * (uint32_t)wave / (uint32_t)nw), u1 = (int)(N * (uint32_t)(wave + 1) / (uint32_t)nw);
  const int n = u1 - u0;
  int g = u0 / S.nch;
  S.cg = g;
  S.cc = S.ic = u0 - g * S.nch;
  S.left = n;
  S.acc[0] = S.acc[1] = 0.f;
  int s = 0;
  while (s < G.nseg) {  // the segment holding the span's first pair
    const int ns = rfl(tab[s].n);
    if (g < ns) break;
    g -= ns;
    ++s;
  }
  S.is = s;
  seg_enter(S, tab, G, s);
  S.ig = g;
  S.pa += (uint64_t)g * G.pstride;
  S.pb += (uint64_t)g * G.pstride;
  S.j += g * G.gstep;
  if (n <= 0) S.rbA = 0;
  S.np = 0;
  if constexpr (!FP8) {
    S.np = rfl(min(npre, n));
    S.pre = lds_u32(pre);
    for (int e = 0; e < S.np; ++e) st_issue_lds(S, S.pre + e * 2048, tab, G);
  }
#pragma unroll
  for (int jj = 0; jj < D; ++jj) st_issue(S, jj, tab, G);
  return n;
}

// Unit in ring slot jj: accumulate; at the end of a pair (or of the span)
// lane 63 writes the wavefront's partials of that pair to
// ys[(pair * nw + wave) * 2 + {0, 1}].
template <bool FP8, int D, int CP>
__device__ __forceinline__ void st_compute_w(PStream<FP8, D, CP> &S, int jj, v4i w0, v4i w1, bool span_end,
                                             const float *xs, float *ys) {
  const int lane = threadIdx.x & 63;
  const float *xb = xs + (FP8 ? S.xo[jj] + S.cc * 1024 + lane * 16 : S.cc * 512 + lane * 8);
  if (FP8) {
    S.acc[0] = fmaf(bf16f(S.sc[jj][0]), dot16_fp8(w0, xb), S.acc[0]);
    S.acc[1] = fmaf(bf16f(S.sc[jj][1]), dot16_fp8(w1, xb), S.acc[1]);
  } else {
    const float4 *x4 = reinterpret_cast<const float4 *>(xb);
    const float4 x0 = x4[0], x1 = x4[1];
    S.acc[0] = dot8_bf16(w0, x0, x1, S.acc[0]);
    S.acc[1] = dot8_bf16(w1, x0, x1, S.acc[1]);
  }
  const bool row_end = ++S.cc == S.nch;
  if (row_end || span_end) {
    const float2 y = wave_sum2_l63(S.acc[0], S.acc[1]);
    S.acc[0] = S.acc[1] = 0.f;
    if (lane == 63) *reinterpret_cast<float2 *>(ys + (S.cg * S.nw + S.wave) * 2) = y;
    if (row_end) { S.cc = 0; ++S.cg; }
  }
}
template <bool FP8, int D, int CP>
__device__ __forceinline__ void st_compute(PStream<FP8, D, CP> &S, int jj, bool span_end, const float *xs,
                                           float *ys) {
  st_compute_w(S, jj, S.buf[jj][0], S.buf[jj][1], span_end, xs, ys);
}

// Consume the span of n units.  Full rounds of the ring first (one issue per
// consumed unit, all inside the span), then the last one or two rounds.
template <bool FP8, int D, int CP>
__device__ __forceinline__ void st_run(PStream<FP8, D, CP> &S, int n, const Seg *tab, const Geo &G,
                                       const float *xs, float *ys) {
  if constexpr (!FP8) {
    // the units in LDS first.  Their loads were issued before the ring's,
    // so once every load of this wavefront is complete (by now they have
    // landed: the staging after them waited for its own) the LDS holds
    // them; the wait and the reads share one asm block, which no memory
    // access crosses.
    for (int e = 0; e < S.np; ++e) {
      v4i w0, w1;
      asm volatile(
          "s_waitcnt vmcnt(0)\n\t"
          "ds_read_b128 %0, %2\n\t"
          "ds_read_b128 %1, %2 offset:1024\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(w0), "=&v"(w1)
          : "v"(S.pre + e * 2048 + (threadIdx.x & 63) * 16)
          : "memory");
      st_compute_w(S, 0, w0, w1, e == n - 1, xs, ys);
    }
    n -= S.np;
  }
  const int m = n >= D ? (n - D) / D : 0;  // rounds whose every issue lies inside the span
  for (int q = 0; q < m; ++q) {
#pragma unroll
    for (int jj = 0; jj < D; ++jj) {
      st_compute(S, jj, false, xs, ys);
      st_issue(S, jj, tab, G);
    }
  }
  const int rem = n - m * D;  // 0 <= rem < 2D
#pragma unroll
  for (int jj = 0; jj < D; ++jj) {
    if (jj < rem) st_compute(S, jj, jj == rem - 1, xs, ys);
    if (jj + D < rem) st_issue(S, jj, tab, G);
  }
#pragma unroll
  for (int jj = 0; jj < D; ++jj)
    if (jj + D < rem) st_compute(S, jj, jj + D == rem - 1, xs, ys);
}

// Zero the partials of ng pairs (before the task's staging barrier).
__device__ __forceinline__ void ys_clear(float *ys, int ng, int nw, int nthr) {
  const int n = ng * nw * 2;
  for (int i = threadIdx.x; i < n; i += nthr) ys[i] = 0.f;
}
// Row r (0: A, 1: B) of pair g: the wavefronts' partials in wavefront order.
// All loads are issued before the first add (one LDS round trip).
__device__ __forceinline__ float ys_get(const float *ys, int g, int r, int nw) {
  const float *p = ys + g * nw * 2 + r;
  float v[MAXW];
#pragma unroll
  for (int w = 0; w < MAXW; ++w) v[w] = w < nw ? p[2 * w] : 0.f;
  float y = 0.f;
#pragma unroll
  for (int w = 0; w < MAXW; ++w) y += v[w];
  return y;
}
// Row e of a task made of consecutive-row pairs.
__device__ __forceinline__ float ys_row(const float *ys, int e, int nw) { return ys_get(ys, e >> 1, e & 1, nw); }

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
// stage_vec).  MoE layers in the resident kernel have it materialised by the
// router stage.
__device__ __forceinline__ float mid_elem(const KP &P, int l, int tok, int i) {
  if (P.persistent && P.moe) return ld_sc1(P.xmid + vec_off(P, l, 0, P.h) + i);
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

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// LDS layout of the GEMV tasks: xs[kmax] | ys[ymax * waves] | red[256] | ... |
// seg table at segoff (the gap, if any, is for the attention chunk combine)
struct GemvLds {
  float *xs, *ys, *red;
  Seg *seg;
};
__device__ __forceinline__ GemvLds gemv_lds(const KP &P, float *lds) {
  float *red = lds + SEGMAX * 12, *ys = red + 256;
  return GemvLds{lds + P.xsoff, ys, red, reinterpret_cast<Seg *>(lds + P.segoff)};
}

// Best (value, lowest index) of two candidates.
__device__ __forceinline__ void argmax_merge(float &bv, int &bi, float ov, int oi) {
  if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
}
template <int CTRL, int RM = 0xf>
__device__ __forceinline__ void argmax_dpp(float &bv, int &bi) {
  const float ov = dpp_keep<CTRL, RM>(bv);
  const int oi = __builtin_amdgcn_update_dpp(bi, bi, CTRL, RM, 0xf, false);
  argmax_merge(bv, bi, ov, oi);
}
// (max, lowest index) over the 64 lanes with DPP moves (the merge is
// commutative and associative); the result is valid in lane 63.
__device__ __forceinline__ void wave_argmax_l63(float &bv, int &bi) {
  argmax_dpp<0xb1>(bv, bi);
  argmax_dpp<0x4e>(bv, bi);
  argmax_dpp<0x141>(bv, bi);
  argmax_dpp<0x140>(bv, bi);
  argmax_dpp<0x142, 0xa>(bv, bi);
  argmax_dpp<0x143, 0xc>(bv, bi);
}

// Softmax over the router logits and top-k selection (ties -> lower expert
// id), then the n_shared shared experts with weight 1.  Every workgroup
// that needs the choice computes it; the inputs and the order of operations
// are the same everywhere, so all of them agree.  sel/selw in LDS.
//
// The selection is one parallel pass, not k rounds of an argmax: expert e's
// rank is the number of experts ahead of it in the order (logit descending,
// lower id first on ties, a NaN logit last), counted by tpe threads of
// consecutive lanes over E / tpe experts each; ranks below top_k are the
// choice, in that order.  (A NaN logit makes the softmax sum NaN, so every
// weight is NaN and the LM head's NaN check reports it.)
__device__ __forceinline__ void route(const KP &P, int l, int *sel, float *selw, float *scratch) {
  const int tid = threadIdx.x, T = P.nthr, E = P.E, lane = tid & 63;
  const float *rl = P.rl + vec_off(P, l, 0, E);
  for (int i = tid; i < E; i += T) scratch[i] = ld_sc1(rl + i);
  __syncthreads();
  // softmax statistics: every wavefront, in the same order
  float m = -INFINITY;
  for (int i = lane; i < E; i += 64) m = fmaxf(m, scratch[i]);
  m = wave_max(m);
  float s = 0.f;
  for (int i = lane; i < E; i += 64) s += expf(scratch[i] - m);
  s = wave_sum(s);
  int tpe = 1;  // threads per expert: T / E rounded down to a power of two, at most 64
  while (tpe < 64 && tpe * 2 * E <= T) tpe *= 2;
  const int part = tid & (tpe - 1), per = T / tpe;
  for (int base = 0; base < E; base += per) {  // (the same trip count in every lane)
    const int e = base + tid / tpe;
    const float ve = e < E ? scratch[e] : 0.f;
    const float ke = ve != ve ? -INFINITY : ve;
    int c = 0;
    for (int j = part; j < E; j += tpe) {
      const float vj = scratch[j];
      const float kj = vj != vj ? -INFINITY : vj;
      c += (kj > ke || (kj == ke && j < e)) ? 1 : 0;
    }
    for (int o = 1; o < tpe; o <<= 1) c += __shfl_xor(c, o);
    if (e < E && part == 0 && c < P.top_k) {
      sel[c] = e;
      selw[c] = expf(ve - m) / s;
    }
  }
  if (tid == 0)
    for (int k = 0; k < P.n_shared; ++k) { sel[P.top_k + k] = k; selw[P.top_k + k] = 1.0f; }
  __syncthreads();
}

// Field f of a layer's pointer table (the order of DevLayer).
enum LField { F_WQ = 1, F_WK = 2, F_WV = 3, F_EWG = 10, F_EWU = 11, F_EWD = 12, F_ESG = 13,
              F_ESU = 14, F_ESD = 15, F_SWG = 16 };
__device__ __forceinline__ uint64_t lptr(const DevLayer *L, int f) {
  return (uint64_t)reinterpret_cast<const void *const *>(L)[f];
}

// One run of consecutive-row pairs: rows [r0, r0 + rows) of a matrix whose
// rows are `stride` bytes apart.
__device__ __forceinline__ void seg_rows(Seg *tab, uint64_t a, int r0, int rows, uint32_t stride, int xo) {
  tab->a = a + (uint64_t)r0 * stride;
  tab->b = tab->a + stride;
  tab->sa = tab->sb = 0;
  tab->j0 = r0;
  tab->n = (rows + 1) >> 1;
  tab->nB = rows >> 1;
  tab->xo = xo;
}
__device__ __forceinline__ Geo geo_rows(int K, uint32_t elt, uint32_t stride, int rows) {
  return Geo{K, (uint32_t)K * elt, 2 * stride, 2, 1, 0u, rows > 0 ? 1 : 0, (rows + 1) >> 1};
}

// Segments of the bf16 tasks (QKV, OPROJ, GU, DOWN, ROUTER, LM); thread 0
// writes single-segment tables, the QKV heads are written in parallel.
__device__ __forceinline__ Geo segs_bf16(const KP &P, const Task &t, Seg *tab) {
  const int l = t.layer, r0 = t.r0, rows = t.r1 - t.r0, tid = threadIdx.x, h = P.h;
  const DevLayer *Lp = P.layers + l;
  Geo G;
  switch (t.op) {
    case OP_QKV: {
      // pairs [r0, r1) in group-major order: per KV head g its G query heads,
      // then k head g, then v head g; d/2 RoPE pairs (j, j + d/2) per head
      const int half = P.d >> 1;
      const int H0 = r0 / half, nseg = rows > 0 ? (t.r1 - 1) / half - H0 + 1 : 0;
      G = Geo{h, (uint32_t)h * 2, (uint32_t)h * 2, 1, 0, 0u, nseg, rows};
      for (int s = tid; s < nseg; s += P.nthr) {
        const int hr = H0 + s, g = hr / (P.G + 2), hh = hr - g * (P.G + 2);
        const int jlo = max(r0, hr * half) - hr * half, jhi = min(t.r1, (hr + 1) * half) - hr * half;
        const uint64_t W = lptr(Lp, hh < P.G ? F_WQ : (hh == P.G ? F_WK : F_WV));
        const int head = hh < P.G ? g * P.G + hh : g;
        Seg &e = tab[s];
        e.a = W + ((uint64_t)head * P.d + jlo) * h * 2;
        e.b = e.a + (uint64_t)half * h * 2;
        e.sa = e.sb = 0;
        e.j0 = jlo;
        e.n = e.nB = jhi - jlo;
        e.xo = 0;
      }
      return G;
    }
    case OP_OPROJ: {
      // rows [r0, r1) of Wo restricted to KV head g's G*d columns
      const int K = P.G * P.d, ld = P.Hq * P.d, g = t.aux % P.Hkv;
      if (tid == 0) seg_rows(tab, (uint64_t)Lp->wo + (uint64_t)g * K * 2, r0, rows, (uint32_t)ld * 2, 0);
      return geo_rows(K, 2, (uint32_t)ld * 2, rows);
    }
    case OP_GU:
      if (tid == 0) {
        tab->a = (uint64_t)Lp->wg + (uint64_t)r0 * h * 2;
        tab->b = (uint64_t)Lp->wu + (uint64_t)r0 * h * 2;
        tab->sa = tab->sb = 0;
        tab->j0 = r0;
        tab->n = tab->nB = rows;
        tab->xo = 0;
      }
      return Geo{h, (uint32_t)h * 2, (uint32_t)h * 2, 1, 0, 0u, rows > 0 ? 1 : 0, rows};
    case OP_DOWN:
      if (tid == 0) seg_rows(tab, (uint64_t)Lp->wd, r0, rows, (uint32_t)P.ffn * 2, 0);
      return geo_rows(P.ffn, 2, (uint32_t)P.ffn * 2, rows);
    case OP_ROUTER:
      if (tid == 0) seg_rows(tab, (uint64_t)Lp->router, r0, rows, (uint32_t)h * 2, 0);
      return geo_rows(h, 2, (uint32_t)h * 2, rows);
    default:  // OP_LM
      if (tid == 0) seg_rows(tab, (uint64_t)P.lm_head, r0, rows, (uint32_t)h * 2, 0);
      return geo_rows(h, 2, (uint32_t)h * 2, rows);
  }
}

// Segments of the routed-expert tasks (after routing: sel in LDS).
__device__ __forceinline__ Geo segs_fp8(const KP &P, const Task &t, const int *sel, Seg *tab) {
  const int l = t.layer, r0 = t.r0, rows = t.r1 - t.r0, tid = threadIdx.x;
  const int f = P.effn, h = P.h, hb = (h + 127) / 128, fb = (f + 127) / 128, nk = P.top_k + P.n_shared;
  const DevLayer *Lp = P.layers + l;
  if (t.op == OP_EGU) {
    // flat rows [r0, r1) over (slot k, row j of expert sel[k]): gate/up pairs
    const int K0 = r0 / f, nseg = rows > 0 ? (t.r1 - 1) / f - K0 + 1 : 0;
    for (int s = tid; s < nseg; s += P.nthr) {
      const int k = K0 + s, e = sel[k], sh = k >= P.top_k ? F_SWG - F_EWG : 0;
      const int jlo = max(r0, k * f) - k * f, jhi = min(t.r1, (k + 1) * f) - k * f;
      Seg &g = tab[s];
      g.a = lptr(Lp, F_EWG + sh) + ((uint64_t)e * f + jlo) * h;
      g.b = lptr(Lp, F_EWU + sh) + ((uint64_t)e * f + jlo) * h;
      g.sa = lptr(Lp, F_ESG + sh) + (uint64_t)e * fb * hb * 2;
      g.sb = lptr(Lp, F_ESU + sh) + (uint64_t)e * fb * hb * 2;
      g.j0 = jlo;
      g.n = g.nB = jhi - jlo;
      g.xo = 0;
    }
    return Geo{h, (uint32_t)h, (uint32_t)h, 1, 0, (uint32_t)hb * 2, nseg, rows};
  }
  // OP_EDOWN: rows [r0, r1) of every chosen expert's down matrix, slot-major;
  // slot k reads its own part u[k] of the activation
  for (int k = tid; k < nk; k += P.nthr) {
    const int e = sel[k], sh = k >= P.top_k ? F_SWG - F_EWG : 0;
    seg_rows(tab + k, lptr(Lp, F_EWD + sh) + (uint64_t)e * h * f, r0, rows, (uint32_t)f, k * f);
    tab[k].sa = tab[k].sb = lptr(Lp, F_ESD + sh) + (uint64_t)e * hb * fb * 2;
  }
  return Geo{f, (uint32_t)f, 2u * f, 2, 1, (uint32_t)fb * 2, rows > 0 ? nk : 0, rows > 0 ? nk * ((rows + 1) >> 1) : 0};
}

// Combine the NC chunk partials of (sequence b, KV head g) into
// xs[0 .. G*d): o_h = sum_c e^{m_c - M} o_c / sum_c e^{m_c - M} l_c with
// M = max_c m_c.  A record is m, l, two unused words, o[d] (16-byte
// aligned).  Each thread forms its output elements straight from the
// records: up to 16 chunks per round with all their loads in flight (the
// m, l pair of a head is one address for the whole wavefront), the running
// max carried across rounds -- one memory round trip for up to 16 chunks,
// no LDS staging and no barrier.
__device__ __forceinline__ void attn_combine(const KP &P, int l, int bg, float *xs) {
  const int b = bg / P.Hkv, g = bg % P.Hkv, G = P.G, d = P.d, NC = P.NC, rec = d + PREC_O;
  const int tid = threadIdx.x, T = P.nthr;
  const Rsrc r = mkbuf(uni_ptr(P.part + (((int64_t)l * P.B + b) * P.Hkv + g) * NC * G * rec),
                       (uint32_t)NC * G * rec * 4);
  for (int i = tid; i < G * d; i += T) {
    const int hh = i / d, j = i - hh * d;
    float M = -INFINITY, num = 0.f, den = 0.f;
    for (int c0 = 0; c0 < NC; c0 += 16) {
      v2i ml[16];
      float ov[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const uint32_t base = c0 + k < NC ? (uint32_t)(((c0 + k) * G + hh) * rec) * 4 : 0x80000000u;
        ml[k] = ld64<CP_SC1>(r, base);
        ov[k] = ldf<CP_SC1>(r, base + (uint32_t)(PREC_O + j) * 4);
      }
      float mv[16], Mn = M;
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int mb = ml[k].x;  // copied out as a value before the bit cast
        mv[k] = c0 + k < NC ? __int_as_float(mb) : -INFINITY;
        Mn = fmaxf(Mn, mv[k]);
      }
      if (Mn != M) {  // rescale what earlier rounds summed (nothing in the first)
        const float sc = expf(M - Mn);
        num *= sc;
        den *= sc;
        M = Mn;
      }
#pragma unroll
      for (int k = 0; k < 16; ++k)
        if (c0 + k < NC) {
          const int lb = ml[k].y;
          const float w = expf(mv[k] - M);
          num = fmaf(w, ov[k], num);
          den = fmaf(w, __int_as_float(lb), den);
        }
    }
    xs[i] = num / den;
  }
}

// ---------------------------------------------------------------------------
// The GEMV tasks.  Each: list its segments, prefetch the first weight units,
// wait for producers, stage the input (RMSNorm folded in where the input is
// a residual stream; the attention combine for the O projection), stream,
// then the task's epilogue with all threads.  Returns false if the wait was
// aborted.  FP8 selects the routed-expert tasks (EGU, EDOWN), whose rows
// depend on the routing and so are listed after the wait.
//
//   QKV    RoPE pairs of q/k/v rows; epilogue: RoPE, q to the workspace,
//          k/v appended to the bf16 cache
//   OPROJ  one KV head's slice of Wo times that head group's attention
//          output; epilogue: the split-K partial pbuf[l][b][g]
//   GU     gate/up pairs; epilogue: SwiGLU u = silu(g) * up
//   DOWN   Wd rows; epilogue: residual x_out = x_mid + Wd u
//   ROUTER router rows; epilogue: router logits
//   EGU    expert gate/up pairs over (slot, row); epilogue: SwiGLU
//   EDOWN  expert down rows, slot-major; epilogue: x_mid + sum_k w_k Wd_k u_k
//   LM     LM-head rows; epilogue: logits (check mode) and the task's
//          (max, lowest index) partial, NaN if any logit is NaN

// SM: the small-model kernel, which can fold stages (the large models'
// kernels are compiled without that code).
template <bool FP8, bool SM>
__device__ __forceinline__ bool task_gemv(const KP &P, const Task &t, int lam, int step, int pos, int tok,
                                          float *lds, const Waiter &wait) {
  const int l = t.layer, rows = t.r1 - t.r0, tid = threadIdx.x, nw = P.nw, op = t.op;
  const GemvLds M = gemv_lds(P, lds);
  int *sel = reinterpret_cast<int *>(M.red + 64);
  float *selw = M.red + 96;
  Geo G;
  // The rows are known before the wait except for the routed experts' gate/up
  // task (and every expert task on the per-operator path): in the resident
  // kernel the down task of a layer runs on the workgroup that just routed
  // the same layer for its gate/up task, and the choice is still in LDS.
  const bool known = !FP8 || (P.persistent && op == OP_EDOWN);
  // The resident kernel's expert gate/up task: its input (the post-attention
  // residual, summed once by the router stage) is final once the router is,
  // so it is copied into LDS before the routing reads the router's logits,
  // and the weight loads follow the choice (late).
  const bool late = FP8 && !known && P.persistent;
  if (FP8) {
    if (!known) {
      if (!wait(P)) return false;
      if (!late) route(P, l, sel, selw, M.xs);
    }
    if (!late) G = segs_fp8(P, t, sel, M.seg);
  } else {
    G = segs_bf16(P, t, M.seg);
  }
  if (!late) G = geo_uniform(G);
  __syncthreads();
  PStream<FP8> S;
  // this task's LDS units: past its staged input, as many as the LDS holds
  int npre = 0;
  const float *pre = nullptr;
  if (!FP8 && P.npre) {
    const int hoff = (P.xsoff + min(P.kmax, (G.K + 1023) & ~1023) + 63) & ~63;
    npre = rfl(min(P.npre, (P.lds_floats - hoff) / (nw * 512)));
    pre = lds + hoff + wave_id() * npre * 512;
  }
  int n = 0;
  if (!late) {
    n = st_begin(S, M.seg, G, nw, npre, pre);
    ys_clear(M.ys, G.NG, nw, P.nthr);
  }
  // the post-attention residual was final before the gate/up stage this
  // workgroup passed: fetch it now
  const bool down = op == OP_DOWN || op == OP_EDOWN;
  const float res0 = down && tid < rows ? mid_elem(P, l, tok, t.r0 + tid) : 0.f;
  // QKV: this thread's first pair's RoPE factors (a table lookup; fetched
  // now so the epilogue does not wait for memory)
  float cos0 = 1.f, sin0 = 0.f;
  if (!FP8 && op == OP_QKV && tid < rows) {
    const int half = P.d >> 1, j = (t.r0 + tid) % ((P.G + 2) * half) % half;
    cos0 = P.rope[(int64_t)pos * half + j];
    sin0 = P.rope[(int64_t)P.max_ctx * half + (int64_t)pos * half + j];
  }
  // folded FFN: this thread's Wd weights for the gate/up task's partial of
  // the down projection (row tid, the task's columns in 16-byte units; a
  // unit's columns past the task's are not used), fetched before the wait
  const bool fold = SM && !FP8 && P.fold && op == OP_GU;
  v4i wdv[FOLD_U];
  if (fold) {
    const Rsrc rw = mkbuf(uni_ptr(P.layers[l].wd), (uint32_t)P.h * P.ffn * 2);
#pragma unroll
    for (int u = 0; u < FOLD_U; ++u)
      wdv[u] = ld128<CP_DEF>(rw, tid < P.h && 8 * u < rows ? (uint32_t)((int64_t)tid * P.ffn + t.r0 + 8 * u) * 2
                                                          : 0x80000000u);
  }
  if (known && !wait(P)) {
    __builtin_amdgcn_s_waitcnt(0);  // no load into LDS outlives the task
    return false;
  }
  bool normed = false;  // RMSNorm folded into the staging: results scale by norm_scale
  int Kst = 0;
  if (op == OP_OPROJ) {
    // combine into xs[0..K) and zero the padding of the last chunk (with the
    // attention folded in, xs already holds the head group's output)
    const int Kp = (G.K + 511) & ~511;
    if (!(SM && P.inl)) attn_combine(P, l, t.aux, M.xs);
    for (int i = G.K + tid; i < Kp; i += P.nthr) M.xs[i] = 0.f;
    __syncthreads();
  } else if (late) {
    // x = the post-attention residual into xs through LDS-destination loads
    // (1 KB per instruction, no registers held while the routing runs; past
    // K they write zeros) and this thread's gains into registers; then the
    // routing (the partials' area as its scratch), the segments and the
    // weight loads; then xs = x * g and the sums of squares for the folded
    // RMSNorm.
    const int K = P.h, n4 = K >> 2, T = P.nthr, lane = tid & 63, wave = wave_id(), nc = (K + 255) >> 8;
    const Rsrc rx = mkbuf(uni_ptr(P.xmid + vec_off(P, l, 0, P.h)), (uint32_t)K * 4);
    const Rsrc rg = mkbuf(uni_ptr(P.layers[l].ffn_norm), (uint32_t)K * 2);
    const uint32_t xb = lds_u32(M.xs);
    for (int c = wave; c < nc; c += nw)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, lds_ptr(xb + c * 1024), 16, (uint32_t)(c * 256 + lane * 4) * 4,
                                               0, 0, CP_SC1);
    constexpr int GJ = 4;  // gains held for K <= 16 T (the rest read after)
    v2i gv[GJ];
#pragma unroll
    for (int j = 0; j < GJ; ++j)
      gv[j] = tid + j * T < n4 ? ld64<CP_DEF>(rg, (uint32_t)(tid + j * T) * 8) : v2i{0, 0};
    route(P, l, sel, selw, M.ys);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wavefront's copies and gains
    G = geo_uniform(segs_fp8(P, t, sel, M.seg));
    __syncthreads();  // the segment table and every wavefront's copy of x
    // xs = x * g and the sums of squares, then the weight loads: nothing in
    // the staging waits behind them
    float ss = 0.f;
    float4 *x4 = reinterpret_cast<float4 *>(M.xs);
    auto scale4 = [&](int i, v2i g) {
      const float4 f = x4[i];
      ss = fmaf(f.x, f.x, ss); ss = fmaf(f.y, f.y, ss);
      ss = fmaf(f.z, f.z, ss); ss = fmaf(f.w, f.w, ss);
      x4[i] = float4{f.x * bf_lo(g.x), f.y * bf_hi(g.x), f.z * bf_lo(g.y), f.w * bf_hi(g.y)};
    };
#pragma unroll
    for (int j = 0; j < GJ; ++j)
      if (tid + j * T < n4) scale4(tid + j * T, gv[j]);
    for (int i = tid + GJ * T; i < n4; i += T) scale4(i, ld64<CP_DEF>(rg, (uint32_t)i * 8));
    for (int i = nc * 256 + tid; i < P.kmax; i += T) M.xs[i] = 0.f;
    const float w = wave_sum2_l63(ss, 0.f).x;
    if (lane == 63) M.red[wave] = w;
    ys_clear(M.ys, G.NG, nw, P.nthr);
    __syncthreads();
    n = st_begin(S, M.seg, G, nw, npre, pre);
    normed = true;
    Kst = K;
  } else {
    Src src{P.a_norm, nullptr, nullptr, 0, 0, nullptr};  // the baseline's normalised input
    int K = P.h;
    Kst = K;
    if (down) {
      src.f32 = P.u + vec_off(P, l, 0, P.F);
      K = P.F;
    } else if (P.persistent) {
      const DevLayer &Lw = P.layers[l];
      if (SM && P.fold && (op == OP_LM || (op == OP_QKV && l > 0))) {
        // folded FFN: the previous layer's output is its post-attention
        // residual plus the gate/up tasks' partials of the down projection,
        // summed here; this task's share of it is kept (the next gate/up
        // stage's residual, the checked hidden state)
        const int lp = op == OP_LM ? P.L - 1 : l - 1, n4 = P.h >> 2;
        float *hid = (op == OP_LM && P.chk_hidden) ? P.chk_hidden + (int64_t)step * P.B * P.h : nullptr;
        stage_fold(P, M.xs, M.red, P.xmid + vec_off(P, lp, 0, P.h), P.dpart + (int64_t)lp * P.W * P.h, P.W,
                   op == OP_LM ? P.final_norm : (const uint16_t *)Lw.attn_norm, P.x_out + vec_off(P, lp, 0, P.h),
                   hid, (int)((int64_t)n4 * lam / P.W), (int)((int64_t)n4 * (lam + 1) / P.W), K,
                   min(P.kmax, (K + 1023) & ~1023));
        src.f32 = nullptr;
      } else if (op == OP_QKV) {
        src = layer_input(P, l, tok, (const uint16_t *)Lw.attn_norm);
      } else if (op == OP_LM) {
        src = Src{P.x_out + vec_off(P, P.L - 1, 0, P.h), nullptr, nullptr, 0, 0, P.final_norm};
      } else if (op == OP_EGU) {
        // the post-attention residual, summed once by the router stage
        src = Src{P.xmid + vec_off(P, l, 0, P.h), nullptr, nullptr, 0, 0, (const uint16_t *)Lw.ffn_norm};
      } else {
        src = mid_input(P, l, tok, (const uint16_t *)Lw.ffn_norm);
        if (op == OP_ROUTER || fold) {  // sum the residual once for the expert stages (folded FFN: for
                                        // the next layer's input): this task's share
          const int n4 = P.h >> 2;
          src.dump = P.xmid + vec_off(P, l, 0, P.h);
          src.d0 = (int)((int64_t)n4 * lam / P.W);
          src.d1 = (int)((int64_t)n4 * (lam + 1) / P.W);
        }
      }
    }
    // zero padding up to what the stream reads: whole 512-column chunks
    // (fp8 expert slots start at their own offsets: up to kmax)
    if (!SM || src.f32 || src.bf16) {
      stage_vec(P, M.xs, M.red, src, K, FP8 ? P.kmax : min(P.kmax, (K + 1023) & ~1023));
      normed = src.gain != nullptr;
    } else {
      normed = true;  // staged by stage_fold
    }
    Kst = K;
  }
  wait.mark(0);
  st_run(S, n, M.seg, G, M.xs, M.ys);
  __syncthreads();
  wait.mark(1);
  const float *ys = M.ys;
  const float rs = normed ? norm_scale(P, M.red, Kst) : 1.f;
  if (FP8) {
    if (op == OP_EGU) {
      float *u = P.u + vec_off(P, l, 0, P.F) + t.r0;
      for (int i = tid; i < rows; i += P.nthr)
        st_out(P, u + i, silu(rs * ys_get(ys, i, 0, nw)) * (rs * ys_get(ys, i, 1, nw)));
    } else {
      const int nk = P.top_k + P.n_shared, np = (rows + 1) >> 1;
      float *xo = P.x_out + vec_off(P, l, 0, P.h) + t.r0;
      float *hid = (P.chk_hidden && l == P.L - 1) ? P.chk_hidden + (int64_t)step * P.B * P.h + t.r0 : nullptr;
      for (int i = tid; i < rows; i += P.nthr) {
        float acc = 0.f;
        for (int k = 0; k < nk; ++k) acc = fmaf(selw[k], ys_get(ys, k * np + (i >> 1), i & 1, nw), acc);
        const float v = (i == tid ? res0 : mid_elem(P, l, tok, t.r0 + i)) + acc;
        st_out(P, xo + i, v);
        if (hid) hid[i] = v;
      }
    }
    return true;
  }
  switch (op) {
    case OP_QKV: {
      const int half = P.d >> 1, per_group = (P.G + 2) * half;
      const float *cosT = P.rope + (int64_t)pos * half;
      const float *sinT = P.rope + (int64_t)P.max_ctx * half + (int64_t)pos * half;
      for (int i = tid; i < rows; i += P.nthr) {
        const int p = t.r0 + i, g = p / per_group, rem = p % per_group, hh = rem / half, j = rem % half;
        float a = rs * ys_get(ys, i, 0, nw), b = rs * ys_get(ys, i, 1, nw);
        if (hh <= P.G) {  // RoPE on q and k
          const float c = i == tid ? cos0 : cosT[j], s = i == tid ? sin0 : sinT[j];
          const float a2 = a * c - b * s, b2 = b * c + a * s;
          a = a2; b = b2;
        }
        if (hh < P.G) {
          float *qd = P.q + vec_off(P, l, 0, P.Hq * P.d) + (int64_t)(g * P.G + hh) * P.d;
          st_xcd(P, qd + j, a);
          st_xcd(P, qd + j + half, b);
        } else if (P.kv8) {  // fp8 cache: the new row in fp32, quantized by the attention task owning it
          float *kn = P.kvnew + ((((int64_t)l * P.B) * 2 + (hh == P.G ? 0 : 1)) * P.Hkv + g) * P.d;
          st_xcd(P, kn + j, a);
          st_xcd(P, kn + j + half, b);
        } else {  // the layer's K or V cache of every KV head under one descriptor each
          const int64_t lbase = (int64_t)l * P.B * P.Hkv * P.max_ctx * P.d;
          const uint32_t bytes = (uint32_t)((int64_t)P.B * P.Hkv * P.max_ctx * P.d * 2);
          const uint32_t o0 = (uint32_t)(((int64_t)g * P.max_ctx + pos) * P.d + j) * 2, o1 = o0 + (uint32_t)half * 2;
          if (hh == P.G) {
            const Rsrc r = mkbuf(P.kc + lbase, bytes);
            st_xcd16(P, r, o0, f2bf(a));
            st_xcd16(P, r, o1, f2bf(b));
          } else {
            const Rsrc r = mkbuf(P.vc + lbase, bytes);
            st_xcd16(P, r, o0, f2bf(a));
            st_xcd16(P, r, o1, f2bf(b));
          }
        }
      }
      return true;
    }
    case OP_OPROJ: {
      const int b = t.aux / P.Hkv, g = t.aux % P.Hkv;
      float *dst = P.pbuf + ((int64_t)(l * P.B + b) * P.Hkv + g) * P.h + t.r0;
      for (int i = tid; i < rows; i += P.nthr) st_out(P, dst + i, ys_row(ys, i, nw));
      return true;
    }
    case OP_GU: {
      float *u = P.u + vec_off(P, l, 0, P.F) + t.r0;
      for (int i = tid; i < rows; i += P.nthr) {
        const float v = silu(rs * ys_get(ys, i, 0, nw)) * (rs * ys_get(ys, i, 1, nw));
        if (fold) M.xs[i] = v;  // (every wavefront is past the stream: xs is free; u has no reader)
        else st_out(P, u + i, v);
      }
      if (fold) {
        // the down projection's partial over this task's columns: row tid of
        // Wd times u[r0 .. r1), in column order
        __syncthreads();
        if (tid < P.h) {
          float y = 0.f;
#pragma unroll
          for (int u = 0; u < FOLD_U; ++u) {
            const int w4[4] = {wdv[u].x, wdv[u].y, wdv[u].z, wdv[u].w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int c = 8 * u + e;
              if (c < rows) y = fmaf((e & 1) ? bf_hi(w4[e >> 1]) : bf_lo(w4[e >> 1]), M.xs[c], y);
            }
          }
          st_out(P, P.dpart + ((int64_t)l * P.W + lam) * P.h + tid, y);
        }
      }
      return true;
    }
    case OP_DOWN: {
      float *xo = P.x_out + vec_off(P, l, 0, P.h) + t.r0;
      float *hid = (P.chk_hidden && l == P.L - 1) ? P.chk_hidden + (int64_t)step * P.B * P.h + t.r0 : nullptr;
      for (int i = tid; i < rows; i += P.nthr) {
        const float v = (i == tid ? res0 : mid_elem(P, l, tok, t.r0 + i)) + ys_row(ys, i, nw);
        st_out(P, xo + i, v);
        if (hid) hid[i] = v;
      }
      return true;
    }
    case OP_ROUTER: {
      float *rl = P.rl + vec_off(P, l, 0, P.E) + t.r0;
      for (int i = tid; i < rows; i += P.nthr) st_out(P, rl + i, rs * ys_row(ys, i, nw));
      return true;
    }
    default: {  // OP_LM
      float *lg = P.chk_logits ? P.chk_logits + (int64_t)step * P.B * P.V + t.r0 : nullptr;
      const int wave = wave_id(), lane = tid & 63;
      float bv = -INFINITY;
      int bi = 0x7fffffff;
      bool nan = false;
      for (int i = tid; i < rows; i += P.nthr) {
        const float y = rs * ys_row(ys, i, nw);
        if (y != y) nan = true;
        else argmax_merge(bv, bi, y, t.r0 + i);
        if (lg) lg[i] = y;
      }
      wave_argmax_l63(bv, bi);
      const bool wnan = __any(nan);
      float *wv = M.red + 128;
      int *wi = reinterpret_cast<int *>(M.red + 160);
      int *wn = reinterpret_cast<int *>(M.red + 192);
      if (lane == 63) { wv[wave] = bv; wi[wave] = bi; wn[wave] = wnan; }
      __syncthreads();
      if (tid == 0) {
        float v = -INFINITY;
        int ix = 0x7fffffff, anynan = 0;
        for (int w = 0; w < nw; ++w) { anynan |= wn[w]; argmax_merge(v, ix, wv[w], wi[w]); }
        if (anynan) v = __builtin_nanf("");
        st_out(P, P.lmp + 2 * lam, v);
        st_out(P, P.lmp + 2 * lam + 1, __builtin_bit_cast(float, (uint32_t)ix));
      }
      return true;
    }
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
      else argmax_merge(bv, bi, v, ix);
    }
    wave_argmax_l63(bv, bi);
    const bool anynan = __any(nan);
    if (lane == 63) sh[1] = anynan ? -1 : bi;
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

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// D(16x16) += A(16 rows x 32) * B(32 x 16 columns).  Lane l supplies row
// (l % 16) of A and column (l % 16) of B, each as the 8 consecutive k of
// group l / 16; it receives D rows 4 * (l / 16) .. + 3 of column l % 16.
__device__ __forceinline__ f32x4_t mfma_16x16x32(v4i a, v4i b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                 c, 0, 0, 0);
}

// Attention of one piece on the matrix cores: positions [t0, t0 + cnt) of
// sequence b, KV head g, layer l, all G query heads (cnt <= the score
// buffer's cpad columns).  NQ = d / 32 column quarters of a head; NS = sets
// of 16 / NQ query heads in the score columns.
//  * Scores, with the diagonal operand mapping of the micro-batch GEMM
//    stream: A row i = (position i / NQ, quarter i % NQ) of 16 / NQ
//    consecutive cached K rows -- one 16-byte load per lane reads them
//    whole, 1 KB contiguous -- and B column j = (query head j / NQ, quarter
//    j % NQ), the scaled q as hi + lo bf16 parts.  The diagonal entries,
//    added over the quarters, are the scores; they go to sc[head][position].
//    The first RA loads are issued before the wait with the step's newest
//    row left out, and that row is reloaded after it.
//  * Softmax per head (max, exponentials, sum into st[2h], st[2h + 1]; max
//    -1e30 for an empty piece), with zeros to whole 32-position chunks.
//  * o = sum_t p_t V_t in chunks of 32 positions: A rows (head, hi/lo part of
//    p), B column j = one of the head's dimensions, the 8 positions of a
//    k-group packed from 8 V loads (each lane loads its own 8-dimension slice
//    of 8 consecutive rows, so the packing stays in the lane).  Wavefront w
//    leaves its share in ored[(w * G + h) * d + j].
// VPRE: each wavefront's first V chunk is also loaded before the wait (the
// newest row again left out and reloaded), for short pieces whose V rows
// would otherwise arrive only after the scores.  Ends after a barrier; false
// if the wait was aborted.  Phase marks 0-2 after the scores, the softmax
// and the weighted sums.
template <int NQ, int NS, bool VPRE, bool F8, class WaitT>
__device__ __forceinline__ bool attn_core(const KP &P, int l, int b, int g, int t0, int cnt, int pos, float *sc,
                                          int cpad, float *ored, float *st, float *ksl, float *vsl,
                                          uint8_t *nrow, const WaitT *wait) {
  constexpr int D = 32 * NQ;  // head dimension
  constexpr int PL = 16 / NQ;  // positions per K load
  constexpr int RA = 8;  // K loads in flight per wavefront
  constexpr int EB = F8 ? 1 : 2;  // bytes per cached element
  constexpr uint32_t OOB = 0x80000000u;
  // a load of one lane: 8 elements (16 bytes of bf16, 8 bytes of fp8 codes)
  using KV8 = typename std::conditional<F8, v2i, v4i>::type;
  auto ld8e = [](Rsrc r, uint32_t off) -> KV8 {
    if constexpr (F8) return ld64<CP_SC1>(r, off);
    else return ld128<CP_SC1>(r, off);
  };
  auto as_bf16 = [](const KV8 &w) -> v4i {
    if constexpr (F8) return fp8x8_bf16(w);
    else return w;
  };
  const int G = P.G;
  const int wave = wave_id(), nw = P.nw, lane = threadIdx.x & 63, ii = lane & 15, qg = lane >> 4;
  const int64_t cbase = (((int64_t)l * P.B + b) * P.Hkv + g) * P.max_ctx * D;
  const Rsrc kr = mkbuf(reinterpret_cast<const uint8_t *>(P.kc) + cbase * EB, (uint32_t)P.max_ctx * D * EB);
  const Rsrc vr = mkbuf(reinterpret_cast<const uint8_t *>(P.vc) + cbase * EB, (uint32_t)P.max_ctx * D * EB);
  // K load u: positions u * PL ..; this lane's row and 8 elements.  Before
  // the wait the row this step's QKV stage writes is left out (reloaded after).
  // (With the fp8 cache the newest row is never read back from memory: the
  // task owning it quantizes it into LDS, nrow, and patches its operands.)
  auto koff = [&](int u, bool pre) -> uint32_t {
    const int tt = u * PL + ii / NQ;
    const bool in = tt < cnt && !((pre || F8) && t0 + tt == pos);
    return in ? ((uint32_t)(t0 + tt) * (uint32_t)D + (uint32_t)((ii % NQ) * 32 + qg * 8)) * EB : OOB;
  };
  const int nL = (cnt + PL - 1) / PL;
  const int nk = nL > wave ? (nL - wave + nw - 1) / nw : 0;  // this wavefront's loads u = wave + nw * k
  // V chunk c (positions c * 32 ..): load r of this lane = position
  // c * 32 + 8 qg + r, dimensions 8 (ii % (D / 8)) ..
  const uint32_t vcol = (uint32_t)(ii % (D / 8)) * 8u * EB;
  auto vload = [&](KV8 (&x)[8], int c, bool pre) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int tt = c * 32 + 8 * qg + r;
      const bool in = tt < cnt && !((pre || F8) && t0 + tt == pos);
      x[r] = ld8e(vr, in ? (uint32_t)(t0 + tt) * (uint32_t)(D * EB) + vcol : OOB);
    }
  };
  const int nC = (cnt + 31) >> 5;
  const int nkc = nC > wave ? (nC - wave + nw - 1) / nw : 0;  // this wavefront's chunks c = wave + nw * k
  KV8 ka[RA], va[8], vn[8];
#pragma unroll
  for (int s = 0; s < RA; ++s) ka[s] = ld8e(kr, koff(wave + nw * s, true));
  if (VPRE) vload(va, wave, true);
  const int64_t srow = (((int64_t)l * P.B + b) * P.Hkv + g) * P.max_ctx;  // scale of row t: [srow + t]
  if (F8) {
    // the earlier rows' scales into LDS (0 past the piece, where p is 0 too)
    for (int i = threadIdx.x; i < nC * 32; i += P.nthr) {
      const bool in = i < cnt && t0 + i != pos;
      ksl[i] = in ? ld_sc1(P.ksc + srow + t0 + i) : 0.f;
      vsl[i] = in ? ld_sc1(P.vsc + srow + t0 + i) : 0.f;
    }
  }
  if (wait && !(*wait)(P)) return false;
  const bool own = t0 <= pos && pos < t0 + cnt;  // this piece holds the step's newest row
  // fp8 cache: the newest row's fp32 K and V values, loaded together with q
  // (one round trip for both)
  float kx = 0.f, vx = 0.f;
  if (F8 && own && threadIdx.x < D) {
    const float *kn = P.kvnew + (((int64_t)l * P.B + b) * 2 * P.Hkv + g) * D;
    kx = ld_sc1(kn + threadIdx.x);
    vx = ld_sc1(kn + (int64_t)P.Hkv * D + threadIdx.x);
  }
  // q as the score columns: set s, column j = (head s * 16 / NQ + j / NQ, quarter j % NQ)
  v4i qh[NS], ql[NS];
  {
    // (written by other workgroups this step: read at device scope; absent heads read 0)
    const Rsrc rq = mkbuf(uni_ptr(P.q + vec_off(P, l, b, P.Hq * D) + (int64_t)g * G * D), (uint32_t)(G * D * 4));
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int hh = s * (16 / NQ) + ii / NQ;
      const uint32_t qo = hh < G ? (uint32_t)(hh * D + (ii % NQ) * 32 + qg * 8) * 4u : OOB;
      const float4 x0 = __builtin_bit_cast(float4, ld128<CP_SC1>(rq, qo));
      const float4 x1 = __builtin_bit_cast(float4, ld128<CP_SC1>(rq, qo + 16u));
      const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float a0 = x[2 * i] * P.attn_scale, a1 = x[2 * i + 1] * P.attn_scale;
        const uint16_t h0 = f2bf(a0), h1 = f2bf(a1);
        const uint16_t l0 = f2bf(a0 - bf16f(h0)), l1 = f2bf(a1 - bf16f(h1));
        qh[s][i] = (int)((uint32_t)h0 | ((uint32_t)h1 << 16));
        ql[s][i] = (int)((uint32_t)l0 | ((uint32_t)l1 << 16));
      }
    }
  }
  if (F8 && own) {
    // Quantize the step's row from the fp32 values the QKV stage left
    // (scale = amax / 448, e4m3 codes of x / scale) into LDS for this task's
    // own products, and append it to the cache for the later steps (the
    // stores complete before this task's flag).
    const int tid = threadIdx.x;
    if (tid < D) {
      const float km = wave_max(__builtin_fabsf(kx)), vm = wave_max(__builtin_fabsf(vx));
      if ((tid & 63) == 0) { st[2 * wave] = km; st[2 * wave + 1] = vm; }
    }
    __syncthreads();
    float km = st[0], vm = st[1];
    if (D > 64) { km = fmaxf(km, st[2]); vm = fmaxf(vm, st[3]); }
    const float ks = km > 0.f ? km / 448.0f : 1.0f, vs = vm > 0.f ? vm / 448.0f : 1.0f;
    if (tid < D) {
      const uint32_t ck = f2e4m3(kx / ks), cv = f2e4m3(vx / vs), o = (uint32_t)(pos * D + tid);
      nrow[tid] = (uint8_t)ck;
      nrow[D + tid] = (uint8_t)cv;
      __builtin_amdgcn_raw_buffer_store_b8((uint8_t)ck, kr, o, 0, CP_SC1);
      __builtin_amdgcn_raw_buffer_store_b8((uint8_t)cv, vr, o, 0, CP_SC1);
    }
    if (tid == 0) {
      st_sc1(P.ksc + srow + pos, ks);
      st_sc1(P.vsc + srow + pos, vs);
      ksl[pos - t0] = ks;
      vsl[pos - t0] = vs;
    }
    __syncthreads();
  } else if (F8) {
    __syncthreads();  // the scales staged above
  }
  if (!F8 && own) {  // the newest row, now written
    const int up = (pos - t0) / PL;
    if (up % nw == wave && up / nw < RA) {
#pragma unroll
      for (int s = 0; s < RA; ++s)
        if (s == up / nw) ka[s] = ld8e(kr, koff(up, false));
    }
    const int tp = pos - t0 - 32 * wave;  // in this wavefront's first V chunk: load (tp % 8) of every lane
    if (VPRE && tp >= 0 && tp < 32) {
#pragma unroll
      for (int r = 0; r < 8; ++r)
        if (r == (tp & 7)) {
          const int tt = 32 * wave + 8 * qg + r;
          va[r] = ld8e(vr, tt < cnt ? (uint32_t)(t0 + tt) * (uint32_t)(D * EB) + vcol : OOB);
        }
    }
  }
  // fp8: the newest row's lanes take their 8 codes from nrow
  const int tnew = F8 && own ? pos - t0 : -1;
  auto knew = [&](KV8 &a, int u) {
    if constexpr (F8) {
      if (u * PL + ii / NQ == tnew) a = *reinterpret_cast<const v2i *>(nrow + (ii % NQ) * 32 + qg * 8);
    }
  };
  // scores of K load u (positions u * PL ..) into sc (fp8: of the codes; the
  // rows' scales are applied in the softmax pass)
  auto scores = [&](KV8 araw, int u) {
    knew(araw, u);
    const v4i a = as_bf16(araw);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      f32x4_t c = mfma_16x16x32(a, qh[s], f32x4_t{0.f, 0.f, 0.f, 0.f});
      c = mfma_16x16x32(a, ql[s], c);
      if (NQ == 4) {  // lane (qg, 4c + h): position qg, head c, quarter h in element h
        const int h = ii & 3;
        float v = h == 0 ? c[0] : h == 1 ? c[1] : h == 2 ? c[2] : c[3];
        v += dpp<0xB1>(v);  // quad_perm [1, 0, 3, 2]
        v += dpp<0x4E>(v);  // quad_perm [2, 3, 0, 1]
        const int tt = u * PL + qg, hh = s * 4 + (ii >> 2);
        if (h == 0 && tt < cnt && hh < G) sc[hh * cpad + tt] = v;
      } else {  // lane (qg, 2c + h): positions 2 qg (element h) and 2 qg + 1 (element 2 + h), head c
        const int h = ii & 1;
        float v0 = h ? c[1] : c[0], v1 = h ? c[3] : c[2];
        v0 += dpp<0xB1>(v0);
        v1 += dpp<0xB1>(v1);
        const int tt = u * PL + 2 * qg, hh = s * 8 + (ii >> 1);
        if (h == 0 && hh < G) {
          if (tt < cnt) sc[hh * cpad + tt] = v0;
          if (tt + 1 < cnt) sc[hh * cpad + tt + 1] = v1;
        }
      }
    }
  };
  for (int k0 = 0; k0 < nk; k0 += RA) {
#pragma unroll
    for (int s = 0; s < RA; ++s) {
      if (k0 + s < nk) scores(ka[s], wave + nw * (k0 + s));
      ka[s] = ld8e(kr, koff(wave + nw * (k0 + s + RA), false));
    }
  }
  if (!VPRE) vload(va, wave, false);  // the first V chunk, during the softmax
  __syncthreads();
  if (wait) wait->mark(0);
  // softmax per head; with the fp8 cache each score takes its K row's scale
  // here, and the stored p its V row's (the sum stays unscaled), so the
  // products below run on the codes as they are
  for (int hh = wave; hh < G; hh += nw) {
    float m = -INFINITY;
    for (int i = lane; i < cnt; i += 64) {
      float v = sc[hh * cpad + i];
      if (F8) {
        v *= ksl[i];
        sc[hh * cpad + i] = v;
      }
      m = fmaxf(m, v);
    }
    m = wave_max(m);
    float sm = 0.f;
    for (int i = lane; i < cnt; i += 64) {
      const float e = expf(sc[hh * cpad + i] - m);
      sc[hh * cpad + i] = F8 ? e * vsl[i] : e;
      sm += e;
    }
    for (int i = cnt + lane; i < nC * 32; i += 64) sc[hh * cpad + i] = 0.f;  // whole chunks
    sm = wave_sum(sm);
    if (lane == 0) { st[2 * hh] = cnt > 0 ? m : -1e30f; st[2 * hh + 1] = sm; }
  }
  __syncthreads();
  if (wait) wait->mark(1);
  f32x4_t acc[D / 16];
#pragma unroll
  for (int m = 0; m < D / 16; ++m) acc[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  auto pv = [&](const KV8 (&xr)[8], int c) {
    // A: row ii = (head ii / 2, part ii % 2) of p, positions c * 32 + 8 qg ..
    // (with the fp8 cache, p already carries each row's V scale)
    const int hh = ii >> 1;
    float p[8];
    if (hh < G) {
      const float4 *p4 = reinterpret_cast<const float4 *>(sc + hh * cpad + c * 32 + 8 * qg);
      const float4 p0 = p4[0], p1 = p4[1];
      p[0] = p0.x; p[1] = p0.y; p[2] = p0.z; p[3] = p0.w; p[4] = p1.x; p[5] = p1.y; p[6] = p1.z; p[7] = p1.w;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) p[e] = 0.f;
    }
    v4i x[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      KV8 w = xr[r];
      if constexpr (F8) {
        if (c * 32 + 8 * qg + r == tnew) w = *reinterpret_cast<const v2i *>(nrow + D + vcol);
      }
      x[r] = as_bf16(w);
    }
    v4i pa;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint16_t w0 = f2bf(p[2 * i]), w1 = f2bf(p[2 * i + 1]);
      if (ii & 1) { w0 = f2bf(p[2 * i] - bf16f(w0)); w1 = f2bf(p[2 * i + 1] - bf16f(w1)); }
      pa[i] = (int)((uint32_t)w0 | ((uint32_t)w1 << 16));
    }
    // B for output dimension 8 (ii % (D / 8)) + e: element e of the 8 rows
#pragma unroll
    for (int m = 0; m < D / 16; ++m) {
      v4i bw;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const v4i &X = x[2 * u], &Y = x[2 * u + 1];
        uint32_t xa, ya;
        if (NQ == 4) {
          xa = (uint32_t)X[m >> 1];
          ya = (uint32_t)Y[m >> 1];
        } else {  // D = 64: lanes ii >= 8 take dimensions 4..7 of their slice
          xa = (uint32_t)(ii >= 8 ? X[(m >> 1) + 2] : X[m >> 1]);
          ya = (uint32_t)(ii >= 8 ? Y[(m >> 1) + 2] : Y[m >> 1]);
        }
        bw[u] = (int)((m & 1) ? (xa >> 16) | (ya & 0xffff0000u) : (xa & 0xffffu) | (ya << 16));
      }
      acc[m] = mfma_16x16x32(pa, bw, acc[m]);
    }
  };
  for (int k = 0; k < nkc; k += 2) {
    vload(vn, wave + nw * (k + 1), false);
    pv(va, wave + nw * k);
    if (k + 1 >= nkc) break;
    vload(va, wave + nw * (k + 2), false);
    pv(vn, wave + nw * (k + 1));
  }
  // this wavefront's partial outputs: rows 4 qg + e = (head 2 qg + e / 2, part e % 2)
#pragma unroll
  for (int m = 0; m < D / 16; ++m) {
    const int dim = NQ == 4 ? ii * 8 + m : (ii & 7) * 8 + m + 4 * (ii >> 3);
    const int h0 = 2 * qg, h1 = 2 * qg + 1;
    if (h0 < G) ored[(wave * G + h0) * D + dim] = acc[m][0] + acc[m][1];
    if (h1 < G) ored[(wave * G + h1) * D + dim] = acc[m][2] + acc[m][3];
  }
  __syncthreads();
  if (wait) wait->mark(2);
  return true;
}

// One attention chunk task: chunk c of NC of (sequence b, KV head g)'s
// positions, all G query heads, on the matrix cores; the record (m, l, -, -,
// o[d]) per head goes to the O-projection task's combine.
// xo != NULL (the attention folded into the output projection): one piece
// over every position, its normalised output o / l per head written to xo
// (LDS) instead of a record.
template <bool KV8>
__device__ __forceinline__ bool attn_chunk(const KP &P, const Task &t, int pos, float *lds,
                                           const Waiter &wait, float *xo = nullptr) {
  const int l = t.layer, bg = t.aux, b = bg / P.Hkv, g = bg % P.Hkv, c = t.r0, NC = t.r1;
  const int G = P.G, d = P.d, tid = threadIdx.x, T = P.nthr, nw = P.nw;
  const int n = pos + 1, C = (n + NC - 1) / NC, t0 = c * C;
  const int cnt = max(0, min(n, t0 + C) - t0);
  const int cpad = (((xo ? P.max_ctx : P.cmax) + 63) / 64) * 64;
  float *qs = lds, *sc = qs + G * d, *ored = sc + G * cpad, *st = ored + nw * G * d;
  // fp8 cache: the piece's row scales, and the newest row's codes (K then V)
  float *ksl = st + 4 * G, *vsl = ksl + cpad;
  uint8_t *nrow = reinterpret_cast<uint8_t *>(vsl + cpad);
  bool ok;
  if (KV8)
    ok = d == 64 ? attn_core<2, 1, true, true>(P, l, b, g, t0, cnt, pos, sc, cpad, ored, st, ksl, vsl, nrow, &wait)
         : G <= 4
             ? attn_core<4, 1, true, true>(P, l, b, g, t0, cnt, pos, sc, cpad, ored, st, ksl, vsl, nrow, &wait)
             : attn_core<4, 2, true, true>(P, l, b, g, t0, cnt, pos, sc, cpad, ored, st, ksl, vsl, nrow, &wait);
  else
    ok = d == 64
             ? attn_core<2, 1, true, false>(P, l, b, g, t0, cnt, pos, sc, cpad, ored, st, ksl, vsl, nrow, &wait)
         : G <= 4
             ? attn_core<4, 1, true, false>(P, l, b, g, t0, cnt, pos, sc, cpad, ored, st, ksl, vsl, nrow, &wait)
             : attn_core<4, 2, true, false>(P, l, b, g, t0, cnt, pos, sc, cpad, ored, st, ksl, vsl, nrow, &wait);
  if (!ok) return false;
  if (xo) {
    for (int i = tid; i < G * d; i += T) {
      const int hh = i / d, j = i % d;
      float s = 0.f;
      float ov[MAXW];
#pragma unroll
      for (int w = 0; w < MAXW; ++w) ov[w] = w < nw ? ored[(w * G + hh) * d + j] : 0.f;
#pragma unroll
      for (int w = 0; w < MAXW; ++w) s += ov[w];
      xo[i] = s / st[2 * hh + 1];
    }
    __syncthreads();
    return true;
  }
  const int rec = d + PREC_O;
  float *pdst = P.part + ((((int64_t)l * P.B + b) * P.Hkv + g) * NC + c) * G * rec;
  for (int i = tid; i < G * d; i += T) {
    const int hh = i / d, j = i % d;
    float s = 0.f;
    float ov[MAXW];
#pragma unroll
    for (int w = 0; w < MAXW; ++w) ov[w] = w < nw ? ored[(w * G + hh) * d + j] : 0.f;
#pragma unroll
    for (int w = 0; w < MAXW; ++w) s += ov[w];
    st_xcd(P, pdst + hh * rec + PREC_O + j, s);
  }
  for (int hh = tid; hh < G; hh += T) {
    st_xcd(P, pdst + hh * rec, st[2 * hh]);
    st_xcd(P, pdst + hh * rec + 1, st[2 * hh + 1]);
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

// Sequence b's position at the start of the call, checked against the
// cache: every step of the call must stay below max_ctx.  Every workgroup
// reads the same value and takes the same branch, so on an error they all
// leave (one latches PRE_DEV_CONTEXT) and no wait is left pending.  Returns
// -1 on an error.
__device__ __forceinline__ int call_position(const KP &P, int b) {
  const int p = __builtin_amdgcn_readfirstlane((int)ld_flag(reinterpret_cast<const uint32_t *>(P.ctx_len) + b));
  const int n = P.chunk ? P.chunk_n : P.persistent ? P.n_steps : P.b_nsteps;
  if (p >= 0 && (int64_t)p + n <= P.max_ctx) return p;
  if (threadIdx.x == 0 && blockIdx.x == 0) latch_error(P, PRE_DEV_CONTEXT, 0, -1, b, (uint32_t)p, (uint32_t)P.max_ctx);
  return -1;
}

__device__ __forceinline__ bool token_ok(const KP &P, int tok, int step) {
  if (tok >= 0 && tok < P.V) return true;
  if (threadIdx.x == 0) latch_error(P, PRE_DEV_BAD_TOKEN, step, -1, -1, (uint32_t)tok, 0);
  return false;
}

// The kernel arguments, re-read from the argument segment by the caller.
// The compiler treats argument loads as invariant and would hoist every
// field a task ever reads to the start of the kernel, where they do not fit
// in scalar registers and get spilled; reading them through a pointer it
// cannot look through confines each field to the task that uses it.
__device__ __forceinline__ const KP &kp_fresh() {
  const __attribute__((address_space(4))) KP *p =
      (const __attribute__((address_space(4))) KP *)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(p));
  return *(const KP *)p;
}

// Run one task of the table (both paths).
// KV8: the attention tile of the fp8 cache; it is compiled into kernels of
// its own (pre_persistent_kv8, pre_serve_kv8) so that the bf16 kernels keep
// their register allocation (one kernel takes the budget of its heaviest
// task).
template <bool KV8, bool SM>
__device__ __forceinline__ bool run_task(const Task &t, int lam, int step, int pos, int tok, float *lds,
                                         const Waiter &wait) {
  const KP &P = kp_fresh();
  if constexpr (!SM) {
    switch (t.op) {
      case OP_NONE: return true;
      case OP_ATTN: return attn_chunk<KV8>(P, t, pos, lds, wait);
      case OP_EGU:
      case OP_EDOWN: return task_gemv<true, false>(P, t, lam, step, pos, tok, lds, wait);
      default: return task_gemv<false, false>(P, t, lam, step, pos, tok, lds, wait);
    }
  } else {
    if (t.op == OP_NONE) return true;
    // attention folded into the output projection: the task's KV head over
    // every position (its wait is the head's QKV producers), the output
    // straight into the projection's staged input, then the projection with
    // nothing left to wait for
    const bool inl = !KV8 && P.inl && t.op == OP_OPROJ;
    if (t.op == OP_ATTN || inl) {
      Task a = t;
      if (inl) { a.r0 = 0; a.r1 = 1; }
      if (!attn_chunk<KV8>(P, a, pos, inl ? lds + P.aoff : lds, wait, inl ? lds + P.xsoff : nullptr)) return false;
      if (!inl) return true;
    }
    if (t.op == OP_EGU || t.op == OP_EDOWN) return task_gemv<true, true>(P, t, lam, step, pos, tok, lds, wait);
    Waiter w = wait;
    if (inl) w.lo = w.hi;
    return task_gemv<false, true>(P, t, lam, step, pos, tok, lds, w);
  }
}

// The folded stages of the small-model kernel, applied to the task table as
// it is read (false: skip the task).  Folded FFN: the down stage's tasks are
// skipped, and the stages that waited for them (the next layer's QKV, the LM
// head) wait for the gate/up stage of the same layer instead -- the stage
// right before, whose tasks now leave the down projection's partials.
// Attention folded into the output projection: the attention stage's tasks
// are skipped, and each O-projection task waits for what the first attention
// task of its (sequence, KV head) would have: that head's QKV producers.
__device__ __forceinline__ bool fold_task(const KP &P, Task &t, int si) {
  if (P.inl) {
    if (t.op == OP_ATTN) return false;
    if (t.op == OP_OPROJ) {
      const Task a = P.tasks[(int64_t)(si - 1) * P.W + t.aux * P.Tg];
      t.wait_lo = a.wait_lo;
      t.wait_hi = a.wait_hi;
    }
  }
  if (!P.fold) return true;
  if (t.op == OP_DOWN) return false;
  if ((t.op == OP_QKV && t.layer > 0) || t.op == OP_LM) {
    t.wait_lo -= P.W;
    t.wait_hi -= P.W;
  }
  return true;
}

// ---------------------------------------------------------------------------
// the resident kernel

// The resident kernel.  With P.persistent = 0 it is the per-operator
// baseline's task kernel instead: every workgroup runs its task of stage
// P.b_si for step P.b_step once, without waits or flags (stream order is the
// only synchronisation).  Both modes go through the one call of run_task, so
// the task code exists once in the binary.
template <bool KV8, bool SM>
__device__ __forceinline__ void resident_body(KP &P) {
  extern __shared__ __attribute__((aligned(16))) float lds[];
  __shared__ int sh[8];
  const bool res = P.persistent != 0;
  // one-XCD placement: the grid has 8 blocks per workgroup and only the
  // blocks dispatched to XCD 0 (b % 8 == 0) take part; the others leave
  if (res && P.onexcd && blockIdx.x % P.X != 0) return;
  const int lam = !res ? blockIdx.x : P.onexcd ? blockIdx.x / P.X : lambda_of_block(blockIdx.x, P.W, P.X);
  if (res) {
    // the XCD this workgroup runs on; the task placement assumes block b on
    // XCD b % 8, and the XCD-local hand-offs need it
    if (threadIdx.x == 0) {
      const uint32_t x = xcc_id();
      P.xcc[lam] = x;
      const int bad = (P.W % P.X == 0 || P.onexcd) && (int)x != (int)(blockIdx.x % P.X);
      if (bad) __hip_atomic_fetch_add(&P.status->xcc_mismatch, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (bad && (P.local || P.onexcd)) latch_error(P, PRE_DEV_PLACEMENT, 0, -1, lam, x, blockIdx.x % P.X);
      sh[2] = bad;
    }
    __syncthreads();
    if ((P.local || P.onexcd) && sh[2]) return;
  }
  const int s_end = res ? P.n_steps : P.b_step + 1;
  const int si0 = res ? 0 : P.b_si, si1 = res ? P.n_si : P.b_si + 1;
  // the position of the call's first step, from the device array (every
  // workgroup reads it here; workgroup 0 advances it after the last step)
  const int pos0 = call_position(P, 0);
  if (pos0 < 0) return;
  int tok = res ? (P.forced ? P.forced[0] : P.in_tok[0]) : P.tok_slot[1];
  for (int s = res ? 0 : P.b_step; s < s_end; ++s) {
    const uint32_t ep = P.epoch_base + (uint32_t)s + 1u;
    const int pos = pos0 + s;
    if (res) {
      if (P.forced) tok = P.forced[(int64_t)s * P.B];
      if (!token_ok(P, tok, s)) return;
    }
    for (int si = si0; si < si1; ++si) {
      Task t = P.tasks[(int64_t)si * P.W + lam];
      if (t.op == OP_NONE) continue;
      if constexpr (SM) {
        if (!fold_task(P, t, si)) continue;
      }
      const int tr = res && P.trace != nullptr;
      const uint32_t tw = tr ? (uint32_t)now_ticks() : 0u;
      const Waiter wait{res ? 1 : 0, t.wait_lo, t.wait_hi, s, si, ep, sh, tr};
      if (!run_task<KV8, SM>(t, lam, s, pos, tok, lds, wait)) return;
      if (res) {
        signal_slot(P, t.signal, ep, P.onexcd || (P.local && (t.op == OP_QKV || t.op == OP_ATTN)));
        if (tr) trace_rec(P, s, si, lam, tw, (uint32_t)sh[3], (uint32_t)now_ticks(), sh);
      }
    }
    if (!res) return;
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
  // Workgroup 0 has seen every workgroup's LM flag of the last step, so every
  // workgroup has read the start position: advance it.
  if (lam == 0 && threadIdx.x == 0) st_flag(reinterpret_cast<uint32_t *>(P.ctx_len), (uint32_t)(pos0 + P.n_steps));
}

extern "C" __global__ void __launch_bounds__(512) pre_persistent(KP P) { resident_body<false, false>(P); }
extern "C" __global__ void __launch_bounds__(512) pre_persistent_kv8(KP P) { resident_body<true, false>(P); }
// Small one-XCD engines whose stages are folded (bf16 cache): a kernel of its
// own, so that the large models' kernel keeps its code and register budget.
extern "C" __global__ void __launch_bounds__(512) pre_persistent_small(KP P) { resident_body<false, true>(P); }

// the micro-batch task set and kernel
#include "mb.h"

// the serving loop (request ring)
#include "serve.h"

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
  const float r = norm_scale(P, red, P.h);
  for (int i = threadIdx.x; i < P.kmax; i += P.nthr) P.a_norm[i] = xs[i] * r;
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

// Baseline: every sequence's position advances by the call's steps (the
// last launch of the call, after every stage has read the start positions).
extern "C" __global__ void pre_k_advance(KP P, int n) {
  const int b = threadIdx.x;
  if (b < P.B) {
    const int p = P.ctx_len[b];
    if (p >= 0 && (int64_t)p + n <= P.max_ctx) P.ctx_len[b] = p + n;
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

// Debug: encode n fp32 values with the fp8 cache's encoder (checks the format).
extern "C" __global__ void pre_k_fp8_encode(const float *in, uint8_t *out, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = (uint8_t)f2e4m3(in[i]);
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

// Plain copy of n16 16-byte words (reference kernel for the memory-traffic
// counters: it reads and writes exactly 16 * n16 bytes).
extern "C" __global__ void __launch_bounds__(256) pre_k_copy(const v4i *src, v4i *dst, int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

// Debug / tuning: the streamed GEMV alone, y = W x over rows split evenly
// across the grid (consecutive-row pairs), for a given ring depth and weight
// cache policy.
template <int D, int CP>
__global__ void __launch_bounds__(1024) pre_k_gemv_bench(const uint16_t *W, int rows, int K, const float *x,
                                                         float *y) {
  extern __shared__ __attribute__((aligned(16))) float lds[];
  const int nthr = __builtin_amdgcn_readfirstlane(blockDim.x), nw = nthr >> 6;
  const int Kp = (K + 511) / 512 * 512;
  for (int i = threadIdx.x; i < Kp; i += nthr) lds[i] = i < K ? x[i] : 0.f;
  const int r0 = (int)((int64_t)rows * blockIdx.x / gridDim.x);
  const int r1 = (int)((int64_t)rows * (blockIdx.x + 1) / gridDim.x);
  Seg *tab = reinterpret_cast<Seg *>(lds + Kp);
  float *ys = lds + Kp + 64;
  if (threadIdx.x == 0) seg_rows(tab, (uint64_t)W, r0, r1 - r0, (uint32_t)K * 2, 0);
  const Geo G = geo_uniform(geo_rows(K, 2, (uint32_t)K * 2, r1 - r0));
  __syncthreads();
  PStream<false, D, CP> S;
  const int n = st_begin(S, tab, G, nw);
  ys_clear(ys, G.NG, nw, nthr);
  __syncthreads();
  st_run(S, n, tab, G, lds, ys);
  __syncthreads();
  for (int i = threadIdx.x; i < r1 - r0; i += nthr) y[r0 + i] = ys_row(ys, i, nw);
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
  int32_t *ctx;  // device position array [B]: the caller's, or the workspace's own
  uint32_t epoch_base;
  uint32_t watchdog_ms;
  int lds_dyn;
  int broken;
  hipStream_t stream;
  std::vector<pre_layer_w> lw;  // host copy of the layer pointers (norm gains for the baseline)
  uint32_t *trace;
  size_t trace_bytes;
  int device;
  int32_t drop_slot;  // debug: ready flag never published (-1: none)
  uint32_t static_gen;  // non-zero: created over the static workspace, with this generation
  int serving;          // a serving loop holds the GPU: other calls return PRE_ERR_BUSY
  // chunk task set (prefill / verify): its dims, layout, offset in the
  // workspace and its own ready-flag epochs
  int has_chunk;
  Dims Dc;
  Layout Lc;
  int64_t coff;
  uint32_t chunk_epoch;
};

static bool static_taken_over(const pre_engine *e);

static inline bool al16(const void *p) { return ((uintptr_t)p & 15) == 0; }

static int device_cus(int *cus, int *lds_max, int *dev) {
  if (hipGetDevice(dev) != hipSuccess) return PRE_ERR_HIP;
  hipDeviceProp_t pr;
  if (hipGetDeviceProperties(&pr, *dev) != hipSuccess) return PRE_ERR_HIP;
  *cus = pr.multiProcessorCount;
  *lds_max = (int)pr.sharedMemPerBlock;
  return PRE_OK;
}

// The chunk task set of a batch-1 engine (pre_config.chunk > 0): the
// micro-batch task table with `chunk` columns that are consecutive tokens of
// the engine's one sequence (prefill, speculative verify).  Dense models
// whose GEMM inputs come in whole 32-column blocks only.
static int chunk_dims(const pre_config *cfg, int cus, Dims *Dc) {
  if (cfg->chunk == 0) return PRE_OK;
  if (cfg->chunk < 2 || cfg->chunk > 8) return PRE_ERR_SHAPE;
  if (cfg->batch != 1 || cfg->n_experts > 0) return PRE_ERR_UNSUPPORTED;
  pre_config c = *cfg;
  c.batch = cfg->chunk;
  c.attn_splits = 0;
  return derive_dims(&c, cus, Dc);
}

static int64_t align256h(int64_t x) { return (x + 255) & ~int64_t(255); }

extern "C" int pre_workspace_size(const pre_config *cfg, size_t *bytes) {
  if (!cfg || !bytes) return PRE_ERR_ARG;
  int cus = 256, ldsm = 0, dev = 0;
  if (cfg->grid_wgs <= 0 && device_cus(&cus, &ldsm, &dev) != PRE_OK) cus = 256;
  Dims D, Dc;
  int rc = derive_dims(cfg, cus, &D);
  if (rc != PRE_OK) return rc;
  if ((rc = chunk_dims(cfg, cus, &Dc)) != PRE_OK) return rc;
  Layout Lo, Lc;
  build_layout(D, &Lo);
  int64_t total = Lo.total;
  if (cfg->chunk) {
    build_layout(Dc, &Lc);
    total = align256h(total) + Lc.total;
  }
  *bytes = (size_t)total;
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

static int create_engine(const pre_config *cfg, const pre_weights *w, const pre_kv *kv, void *d_workspace,
                         size_t ws_bytes, void *stream, pre_engine **out, uint32_t static_gen);

extern "C" int pre_engine_create(const pre_config *cfg, const pre_weights *w, const pre_kv *kv,
                                 void *d_workspace, size_t ws_bytes, void *stream, pre_engine **out) {
  return create_engine(cfg, w, kv, d_workspace, ws_bytes, stream, out, 0);
}

// ---- the engine over the library's static workspace ----------------------
// For callers that cannot allocate device memory.  The workspace is this
// file-scope device array; each GPU the library runs on holds its own copy
// until the process ends.  In host code `scratch` names a host-side stand-in,
// not the device array: its device address is looked up once per device
// (hipGetSymbolAddress with that device current) and only that address is
// ever used.  Engines created over it share it: each create takes it over
// (a generation count per device), and calls on an engine created before
// the latest one on that device return PRE_ERR_BROKEN.
static __device__ __align__(256) char scratch[PRE_STATIC_WORKSPACE_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];
uint32_t g_scratch_gen[kMaxDevices];
}  // namespace

extern "C" int pre_engine_create_static(const pre_config *cfg, const pre_weights *w, const pre_kv *kv,
                                        void *stream, pre_engine **out) {
  if (!out) return PRE_ERR_ARG;
  *out = nullptr;
  if (!cfg) return PRE_ERR_ARG;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PRE_ERR_HIP;
  size_t need = 0;
  int rc = pre_workspace_size(cfg, &need);
  if (rc != PRE_OK) return rc;
  if (need > (size_t)PRE_STATIC_WORKSPACE_BYTES) return PRE_ERR_WORKSPACE;
  void *ptr;
  uint32_t gen;
  {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
      void *p = nullptr;
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return PRE_ERR_HIP;
      g_scratch_ptr[dev] = p;
    }
    ptr = g_scratch_ptr[dev];
    gen = ++g_scratch_gen[dev];
    if (gen == 0) gen = ++g_scratch_gen[dev];
  }
  return create_engine(cfg, w, kv, ptr, (size_t)PRE_STATIC_WORKSPACE_BYTES, stream, out, gen);
}

static int create_engine(const pre_config *cfg, const pre_weights *w, const pre_kv *kv, void *d_workspace,
                         size_t ws_bytes, void *stream, pre_engine **out, uint32_t static_gen) {
  if (!out) return PRE_ERR_ARG;
  *out = nullptr;
  if (!cfg || !w || !kv || !d_workspace || !w->layers) return PRE_ERR_ARG;
  int cus, ldsm, dev;
  if (device_cus(&cus, &ldsm, &dev) != PRE_OK) return PRE_ERR_HIP;
  Dims D;
  int rc = derive_dims(cfg, cus, &D);
  if (rc != PRE_OK) return rc;
  if (!w->embed || !w->final_norm || !w->lm_head || !kv->k || !kv->v) return PRE_ERR_ARG;
  if (D.kv8 && (!kv->k_scale || !kv->v_scale)) return PRE_ERR_ARG;
  if (((uintptr_t)kv->k_scale & 3) || ((uintptr_t)kv->v_scale & 3)) return PRE_ERR_ALIGN;
  if (!al16(w->embed) || !al16(w->final_norm) || !al16(w->lm_head) || !al16(kv->k) || !al16(kv->v) ||
      !al16(d_workspace) || ((uintptr_t)kv->d_ctx_len & 3))
    return PRE_ERR_ALIGN;
  for (int l = 0; l < D.L; ++l)
    if ((rc = check_layer(D, w->layers[l])) != PRE_OK) return rc;
  Layout Lo, Lc;
  build_layout(D, &Lo);
  Dims Dc;
  std::memset(&Dc, 0, sizeof(Dc));
  std::memset(&Lc, 0, sizeof(Lc));
  if ((rc = chunk_dims(cfg, cus, &Dc)) != PRE_OK) return rc;
  const int64_t coff = align256h(Lo.total);
  if (cfg->chunk) build_layout(Dc, &Lc);
  if ((int64_t)ws_bytes < (cfg->chunk ? coff + Lc.total : Lo.total)) return PRE_ERR_WORKSPACE;
  std::vector<Task> T, Tc;
  build_tasks(D, T);
  if (validate(D, T) != 0) return PRE_ERR_SHAPE;
  if (cfg->chunk) {
    build_tasks(Dc, Tc);
    if (validate(Dc, Tc) != 0) return PRE_ERR_SHAPE;
  }

  // LDS: what the tiles need, raised past half a CU's LDS so that exactly one
  // workgroup fits per CU (one resident workgroup per CU).
  int dyn = std::max(D.lds_bytes, cfg->chunk ? Dc.lds_bytes : 0);
  const int want = std::min(ldsm, 96 * 1024);
  if (want > dyn && want > ldsm / 2) dyn = want;
  if (dyn > ldsm) return PRE_ERR_SHAPE;
  const void *kern = D.mb                 ? (const void *)pre_persistent_mb
                     : D.kv8              ? (const void *)pre_persistent_kv8
                     : (D.fold || D.inl) ? (const void *)pre_persistent_small
                                          : (const void *)pre_persistent;
  const void *serve_kern = D.kv8 ? (const void *)pre_serve_kv8 : (const void *)pre_serve;
  if ((!D.mb && hipFuncSetAttribute(serve_kern, hipFuncAttributeMaxDynamicSharedMemorySize, dyn) != hipSuccess) ||
      hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, dyn) != hipSuccess ||
      hipFuncSetAttribute((const void *)pre_persistent, hipFuncAttributeMaxDynamicSharedMemorySize, dyn) !=
          hipSuccess ||
      hipFuncSetAttribute((const void *)pre_k_norm, hipFuncAttributeMaxDynamicSharedMemorySize, dyn) !=
          hipSuccess)
    return PRE_ERR_HIP;
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, D.threads, dyn) != hipSuccess)
    return PRE_ERR_HIP;
  if (per_cu < 1 || (int64_t)per_cu * cus < (int64_t)D.W * (D.onexcd ? D.X : 1)) return PRE_ERR_SHAPE;
  if (cfg->chunk) {
    int per_cu_c = 0;
    if (hipFuncSetAttribute((const void *)pre_persistent_mb, hipFuncAttributeMaxDynamicSharedMemorySize, dyn) !=
            hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu_c, (const void *)pre_persistent_mb, Dc.threads, dyn) !=
            hipSuccess)
      return PRE_ERR_HIP;
    if (per_cu_c < 1 || (int64_t)per_cu_c * cus < (int64_t)Dc.W) return PRE_ERR_SHAPE;
  }

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
          hipSuccess)
    return PRE_ERR_HIP;
  if (cfg->chunk) {
    char *wc = ws + coff;
    if (hipMemsetAsync(wc, 0, (size_t)Lc.total, st) != hipSuccess ||
        hipMemcpyAsync(wc + Lc.layers, dl.data(), dl.size() * sizeof(DevLayer), hipMemcpyHostToDevice, st) !=
            hipSuccess ||
        hipMemcpyAsync(wc + Lc.tasks, Tc.data(), Tc.size() * sizeof(Task), hipMemcpyHostToDevice, st) !=
            hipSuccess ||
        hipMemcpyAsync(wc + Lc.rope, rope.data(), rope.size() * sizeof(float), hipMemcpyHostToDevice, st) !=
            hipSuccess)
      return PRE_ERR_HIP;
  }
  if (hipStreamSynchronize(st) != hipSuccess) return PRE_ERR_HIP;

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
  e->ctx = kv->d_ctx_len ? kv->d_ctx_len : (int32_t *)(ws + Lo.ctx);
  e->epoch_base = 0;
  const char *wd = std::getenv("PRE_WATCHDOG_MS");
  e->watchdog_ms = wd ? (uint32_t)std::max(1, std::atoi(wd)) : 2000u;
  e->lds_dyn = dyn;
  e->broken = 0;
  e->stream = st;
  e->trace = nullptr;
  e->trace_bytes = 0;
  e->device = dev;
  e->drop_slot = -1;
  e->static_gen = static_gen;
  e->serving = 0;
  e->has_chunk = cfg->chunk > 0;
  e->Dc = Dc;
  e->Lc = Lc;
  e->coff = coff;
  e->chunk_epoch = 0;
  e->lw.assign(w->layers, w->layers + D.L);
  *out = e;
  return PRE_OK;
}

// Host helpers over the device position array: both wait for the device
// (every queued call has advanced the positions) before they copy.
extern "C" int pre_engine_set_positions(pre_engine *e, const int32_t *h_pos) {
  if (!e || !h_pos) return PRE_ERR_ARG;
  if (e->serving) return PRE_ERR_BUSY;
  if (static_taken_over(e)) return PRE_ERR_BROKEN;
  for (int b = 0; b < e->D.B; ++b)
    if (h_pos[b] < 0 || h_pos[b] >= e->D.max_ctx) return PRE_ERR_CONTEXT;
  if (hipDeviceSynchronize() != hipSuccess ||
      hipMemcpy(e->ctx, h_pos, sizeof(int32_t) * e->D.B, hipMemcpyHostToDevice) != hipSuccess)
    return PRE_ERR_HIP;
  return PRE_OK;
}

extern "C" int pre_engine_get_positions(const pre_engine *e, int32_t *h_pos) {
  if (!e || !h_pos) return PRE_ERR_ARG;
  if (e->serving) return PRE_ERR_BUSY;
  if (static_taken_over(e)) return PRE_ERR_BROKEN;
  if (hipDeviceSynchronize() != hipSuccess ||
      hipMemcpy(h_pos, e->ctx, sizeof(int32_t) * e->D.B, hipMemcpyDeviceToHost) != hipSuccess)
    return PRE_ERR_HIP;
  return PRE_OK;
}

static void fill_kp_dims(const pre_engine *e, const Dims &D, const Layout &Lo, char *ws, KP &P, int persistent);

static void fill_kp(const pre_engine *e, KP &P, int persistent) {
  fill_kp_dims(e, e->D, e->Lo, e->ws, P, persistent);
}

// The chunk task set's arguments: its own table, flags and activations; the
// engine's status word, cache (one sequence) and position array.
static void fill_kp_chunk(const pre_engine *e, KP &P) {
  fill_kp_dims(e, e->Dc, e->Lc, e->ws + e->coff, P, 1);
  P.status = (DevStatus *)(e->ws + e->Lo.status);
  P.Bc = 1;
  P.chunk = 1;
}

static void fill_kp_dims(const pre_engine *e, const Dims &D, const Layout &Lo, char *ws, KP &P, int persistent) {
  std::memset(&P, 0, sizeof(P));
  P.L = D.L; P.h = D.h; P.Hq = D.Hq; P.Hkv = D.Hkv; P.d = D.d; P.ffn = D.ffn; P.V = D.V; P.B = D.B;
  P.max_ctx = D.max_ctx; P.E = D.E; P.top_k = D.top_k; P.n_shared = D.n_shared; P.effn = D.effn;
  P.moe = D.moe; P.G = D.G; P.F = D.F; P.W = D.W; P.X = D.X; P.NC = D.NC; P.Tg = D.Tg; P.n_si = D.n_si;
  P.spl = D.stages_per_layer; P.kmax = D.kmax; P.ymax = D.ymax; P.segoff = D.segoff; P.cmax = D.cmax;
  P.npre = D.npre; P.xsoff = D.xsoff;
  P.lds_floats = e->lds_dyn / 4;
  P.nthr = D.threads;
  P.nw = D.threads / 64;
  P.eps = D.eps;
  P.attn_scale = (float)(1.0 / std::sqrt((double)D.d));
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
  P.xmid = (float *)(ws + Lo.xmid);
  P.pk = D.mb ? (uint8_t *)(ws + Lo.pk) : nullptr;
  P.ssq = D.mb ? (float *)(ws + Lo.ssq) : nullptr;
  P.ctx_len = e->ctx;
  P.drop_slot = e->drop_slot;
  P.mbst = D.mbst;
  P.Bc = D.B;
  P.kv8 = D.kv8;
  P.ksc = e->kv.k_scale;
  P.vsc = e->kv.v_scale;
  P.kvnew = D.kv8 ? (float *)(ws + Lo.kvnew) : nullptr;
  P.tok_slot = (int32_t *)(ws + Lo.tok);
  P.watchdog_ticks = (uint32_t)std::min<uint64_t>((uint64_t)e->watchdog_ms * 100000ull, 0xffffffffull);
  P.persistent = persistent;
  P.local = D.local;
  P.onexcd = persistent ? D.onexcd : 0;  // the per-operator launches spread over every XCD
  P.fold = persistent ? D.fold : 0;      // the per-operator path runs the down stage
  P.dpart = D.fold ? (float *)(ws + Lo.dpart) : nullptr;
  P.inl = persistent ? D.inl : 0;        // the per-operator path runs the attention stage
  P.aoff = D.aoff;
}

static int check_call(const pre_engine *e, int32_t n_steps, const int32_t *d_in, const int32_t *d_forced,
                      const int32_t *d_out) {
  if (!e || n_steps < 0) return PRE_ERR_ARG;
  if (n_steps == 0) return PRE_OK;  // nothing to do; the buffers are not read
  if (!d_out || (!d_in && !d_forced)) return PRE_ERR_ARG;
  if (e->serving) return PRE_ERR_BUSY;
  if (e->broken || static_taken_over(e)) return PRE_ERR_BROKEN;
  if (n_steps > e->D.max_ctx) return PRE_ERR_CONTEXT;  // (positions live on the device: checked there)
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
  P.epoch_base = e->epoch_base;
  P.in_tok = d_in_tokens;
  P.forced = d_forced;
  P.out_tok = d_out_tokens;
  P.chk_logits = chk ? chk->logits : nullptr;
  P.chk_hidden = chk ? chk->hidden : nullptr;
  P.trace = e->trace;
  P.trace_cap = (uint32_t)std::min<size_t>(e->trace_bytes / 32, 0xffffffffu);
  void *args[] = {&P};
  const void *kern = e->D.mb                    ? (const void *)pre_persistent_mb
                     : e->D.kv8                 ? (const void *)pre_persistent_kv8
                     : (e->D.fold || e->D.inl) ? (const void *)pre_persistent_small
                                                : (const void *)pre_persistent;
  const unsigned nblk = (unsigned)(e->D.W * (e->D.onexcd ? e->D.X : 1));  // one-XCD: 8 blocks per workgroup
  hipError_t err = hipLaunchCooperativeKernel(kern, dim3(nblk), dim3(e->D.threads), args, (unsigned)e->lds_dyn,
                                              (hipStream_t)stream);
  if (err != hipSuccess) return PRE_ERR_HIP;
  e->epoch_base += (uint32_t)n_steps;
  return PRE_OK;
}

// One launch of the chunk task set over n tokens of the engine's sequence.
static int chunk_launch(pre_engine *e, int32_t n, const int32_t *d_tokens, int32_t *d_out, const pre_check *chk,
                        int32_t *d_accept, void *stream) {
  KP P;
  fill_kp_chunk(e, P);
  const int C = e->Dc.B;
  P.n_steps = (n + C - 1) / C;
  P.chunk_n = n;
  P.verify = d_accept != nullptr;
  P.v_accept = d_accept;
  P.epoch_base = e->chunk_epoch;
  P.forced = d_tokens;
  P.out_tok = d_out;
  P.chk_logits = chk ? chk->logits : nullptr;
  P.chk_hidden = chk ? chk->hidden : nullptr;
  void *args[] = {&P};
  if (hipLaunchCooperativeKernel((const void *)pre_persistent_mb, dim3(e->Dc.W), dim3(e->Dc.threads), args,
                                 (unsigned)e->lds_dyn, (hipStream_t)stream) != hipSuccess)
    return PRE_ERR_HIP;
  e->chunk_epoch += (uint32_t)P.n_steps;
  return PRE_OK;
}

extern "C" int pre_engine_prefill(pre_engine *e, int32_t n_tokens, const int32_t *d_tokens, int32_t *d_out_tokens,
                                  const pre_check *chk, void *stream) {
  if (!e || n_tokens < 0) return PRE_ERR_ARG;
  if (n_tokens == 0) return PRE_OK;
  if (!d_tokens || !d_out_tokens) return PRE_ERR_ARG;
  if (!e->has_chunk) return PRE_ERR_UNSUPPORTED;
  if (e->serving) return PRE_ERR_BUSY;
  if (e->broken || static_taken_over(e)) return PRE_ERR_BROKEN;
  if (n_tokens > e->D.max_ctx) return PRE_ERR_CONTEXT;
  return chunk_launch(e, n_tokens, d_tokens, d_out_tokens, chk, nullptr, stream);
}

extern "C" int pre_engine_verify(pre_engine *e, int32_t n_draft, const int32_t *d_tokens, int32_t *d_out_tokens,
                                 int32_t *d_accepted, const pre_check *chk, void *stream) {
  if (!e || !d_tokens || !d_out_tokens || !d_accepted || n_draft < 1) return PRE_ERR_ARG;
  if (!e->has_chunk) return PRE_ERR_UNSUPPORTED;
  if (n_draft + 1 > e->Dc.B) return PRE_ERR_SHAPE;
  if (e->serving) return PRE_ERR_BUSY;
  if (e->broken || static_taken_over(e)) return PRE_ERR_BROKEN;
  return chunk_launch(e, n_draft + 1, d_tokens, d_out_tokens, chk, d_accepted, stream);
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
  P.b_nsteps = n_steps;
  hipStream_t st = (hipStream_t)stream;
  const Dims &D = e->D;
  const dim3 blk(D.threads);
  const unsigned lds = (unsigned)e->lds_dyn;
  const std::vector<pre_layer_w> &lw = e->lw;
  // one stage of one step per launch of the task kernel
  auto stage = [&](int si, int s) {
    P.b_si = si;
    P.b_step = s;
    if (D.mb) hipLaunchKernelGGL(pre_persistent_mb, dim3(D.W), blk, lds, st, P);
    else if (D.kv8) hipLaunchKernelGGL(pre_persistent_kv8, dim3(D.W), blk, lds, st, P);
    else hipLaunchKernelGGL(pre_persistent, dim3(D.W), blk, lds, st, P);
  };
  for (int s = 0; s < n_steps && D.mb; ++s) {  // micro-batch: every stage is a task kernel
    for (int si = 0; si < D.n_si; ++si) stage(si, s);
    hipLaunchKernelGGL(pre_k_argmax_mb, dim3(1), blk, 0, st, P, s);
  }
  for (int s = 0; s < n_steps && !D.mb; ++s) {
    hipLaunchKernelGGL(pre_k_embed, dim3(1), blk, 0, st, P, s);
    for (int l = 0; l < D.L; ++l) {
      const int si0 = l * D.stages_per_layer;
      hipLaunchKernelGGL(pre_k_norm, dim3(D.B), blk, lds, st, P, l, 0, (const uint16_t *)lw[l].attn_norm);
      for (int k = 0; k < 3; ++k) stage(si0 + k, s);  // QKV, attention chunks, O projection
      hipLaunchKernelGGL(pre_k_norm, dim3(D.B), blk, lds, st, P, l, 1, (const uint16_t *)lw[l].ffn_norm);
      for (int k = 3; k < D.stages_per_layer; ++k) stage(si0 + k, s);
    }
    hipLaunchKernelGGL(pre_k_norm, dim3(D.B), blk, lds, st, P, D.L - 1, 2, (const uint16_t *)e->final_norm);
    stage(D.n_si - 1, s);
    hipLaunchKernelGGL(pre_k_argmax, dim3(1), dim3(64), 0, st, P, s);
  }
  hipLaunchKernelGGL(pre_k_advance, dim3(1), dim3(64), 0, st, P, n_steps);
  if (hipGetLastError() != hipSuccess) return PRE_ERR_HIP;
  return PRE_OK;
}

static bool static_taken_over(const pre_engine *e) {
  if (!e->static_gen) return false;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  return g_scratch_gen[e->device] != e->static_gen;
}

extern "C" int pre_engine_status(pre_engine *e, pre_status *out) {
  if (!e || !out) return PRE_ERR_ARG;
  if (e->serving) return PRE_ERR_BUSY;
  if (static_taken_over(e)) return PRE_ERR_BROKEN;
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
  if (e->serving) return PRE_ERR_BUSY;
  if (static_taken_over(e)) return PRE_ERR_BROKEN;
  hipStream_t st = (hipStream_t)stream;
  const Layout &Lo = e->Lo;
  if (hipMemsetAsync(e->ws + Lo.status, 0, sizeof(DevStatus), st) != hipSuccess ||
      hipMemsetAsync(e->ws + Lo.flags, 0, (size_t)(Lo.layers - Lo.flags), st) != hipSuccess)
    return PRE_ERR_HIP;
  if (e->has_chunk &&
      hipMemsetAsync(e->ws + e->coff + e->Lc.flags, 0, (size_t)(e->Lc.layers - e->Lc.flags), st) != hipSuccess)
    return PRE_ERR_HIP;
  e->epoch_base = 0;
  e->chunk_epoch = 0;
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

// ---- the serving loop (request ring) -------------------------------------

struct pre_server {
  pre_engine *e;
  uint32_t *ring_h;  // coherent host memory (the host's view)
  uint32_t *ring_d;  // the same memory as the kernel addresses it
  int32_t slots, max_prompt, max_out, words;
  int32_t next_seq;
  hipStream_t stream;
};

static inline uint32_t ring_ld(const uint32_t *p) { return __atomic_load_n(p, __ATOMIC_ACQUIRE); }
static inline void ring_st(uint32_t *p, uint32_t v) { __atomic_store_n(p, v, __ATOMIC_RELEASE); }

extern "C" int pre_serve_start(pre_engine *e, int32_t n_slots, int32_t max_prompt, int32_t max_out,
                               uint32_t idle_ms, void *stream, pre_server **out) {
  if (!out) return PRE_ERR_ARG;
  *out = nullptr;
  if (!e || n_slots < 1 || n_slots > 64 || max_prompt < 1 || max_out < 1 || idle_ms == 0) return PRE_ERR_ARG;
  if (e->D.mb) return PRE_ERR_UNSUPPORTED;
  if (e->serving) return PRE_ERR_BUSY;
  if (e->broken || static_taken_over(e)) return PRE_ERR_BROKEN;
  if (max_prompt > e->D.max_ctx || max_out > e->D.max_ctx) return PRE_ERR_CONTEXT;
  const int32_t words = (16 + max_prompt + max_out + 15) / 16 * 16;
  const size_t bytes = 4 * ((size_t)RING_HDR + (size_t)n_slots * words);
  void *h = nullptr, *d = nullptr;
  if (hipHostMalloc(&h, bytes, hipHostMallocCoherent | hipHostMallocMapped) != hipSuccess || !h) return PRE_ERR_HIP;
  std::memset(h, 0, bytes);
  if (hipHostGetDevicePointer(&d, h, 0) != hipSuccess || !d) {
    (void)hipHostFree(h);
    return PRE_ERR_HIP;
  }
  KP P;
  fill_kp(e, P, 1);
  P.fold = P.inl = 0;  // the serving loop runs every stage (its kernels carry no folded stages)
  P.epoch_base = e->epoch_base;
  P.ring = (uint32_t *)d;
  P.cmd = (int32_t *)(e->ws + e->Lo.cmd);
  P.req_tok = (int32_t *)(e->ws + e->Lo.req);
  P.ring_slots = n_slots;
  P.ring_prompt = max_prompt;
  P.ring_out = max_out;
  P.ring_words = words;
  P.idle_ticks = (uint32_t)std::min<uint64_t>((uint64_t)idle_ms * 100000ull, 0xffffffffull);
  hipStream_t st = (hipStream_t)stream;
  void *args[] = {&P};
  const unsigned nblk = (unsigned)(e->D.W * (e->D.onexcd ? e->D.X : 1));
  if (hipMemsetAsync(P.cmd, 0, 64, st) != hipSuccess ||
      hipLaunchCooperativeKernel(e->D.kv8 ? (const void *)pre_serve_kv8 : (const void *)pre_serve, dim3(nblk),
                                 dim3(e->D.threads), args,
                                 (unsigned)e->lds_dyn, st) != hipSuccess) {
    (void)hipHostFree(h);
    return PRE_ERR_HIP;
  }
  pre_server *s = new pre_server();
  s->e = e;
  s->ring_h = (uint32_t *)h;
  s->ring_d = (uint32_t *)d;
  s->slots = n_slots;
  s->max_prompt = max_prompt;
  s->max_out = max_out;
  s->words = words;
  s->next_seq = 1;
  s->stream = st;
  e->serving = 1;
  *out = s;
  return PRE_OK;
}

extern "C" int pre_serve_submit(pre_server *s, const int32_t *h_prompt, int32_t n_prompt, int32_t pos,
                                int32_t budget, int32_t eos, int32_t *slot) {
  if (!s || !h_prompt || !slot || n_prompt < 1 || n_prompt > s->max_prompt || budget < 1 ||
      budget > s->max_out || pos < -1)
    return PRE_ERR_ARG;
  const Dims &D = s->e->D;
  for (int i = 0; i < n_prompt; ++i)
    if (h_prompt[i] < 0 || h_prompt[i] >= D.V) return PRE_ERR_ARG;
  if (pos >= 0 && (int64_t)pos + n_prompt + budget - 1 > D.max_ctx) return PRE_ERR_CONTEXT;
  if (ring_ld(s->ring_h + 1) == 2u) return PRE_ERR_DEVICE;  // the loop has ended
  for (int i = 0; i < s->slots; ++i) {
    uint32_t *sl = s->ring_h + RING_HDR + (size_t)i * s->words;
    if (ring_ld(sl) != (uint32_t)SLOT_FREE) continue;
    for (int k = 0; k < n_prompt; ++k) sl[16 + k] = (uint32_t)h_prompt[k];
    sl[1] = (uint32_t)n_prompt;
    sl[2] = (uint32_t)pos;
    sl[3] = (uint32_t)budget;
    sl[4] = (uint32_t)eos;
    sl[5] = 0u;
    sl[6] = 0u;
    sl[7] = (uint32_t)s->next_seq++;
    ring_st(sl, SLOT_READY);  // published after every field above
    *slot = i;
    return PRE_OK;
  }
  return PRE_ERR_BUSY;
}

extern "C" int pre_serve_poll(pre_server *s, int32_t slot, int32_t *h_tokens, int32_t max_tokens, int32_t *n_out,
                              int32_t *done, int32_t *err) {
  if (!s || slot < 0 || slot >= s->slots || !n_out || !done || max_tokens < 0 || (max_tokens && !h_tokens))
    return PRE_ERR_ARG;
  uint32_t *sl = s->ring_h + RING_HDR + (size_t)slot * s->words;
  const uint32_t state = ring_ld(sl);
  if (state == (uint32_t)SLOT_FREE) return PRE_ERR_ARG;
  const int32_t n = (int32_t)ring_ld(sl + 5);  // tokens written before the count
  for (int i = 0; i < n && i < max_tokens; ++i) h_tokens[i] = (int32_t)sl[16 + s->max_prompt + i];
  *n_out = n;
  *done = state == (uint32_t)SLOT_DONE;
  if (err) *err = *done ? (int32_t)sl[6] : 0;
  if (*done) ring_st(sl, SLOT_FREE);
  else if (ring_ld(s->ring_h + 1) == 2u) return PRE_ERR_DEVICE;  // the loop ended before this request
  return PRE_OK;
}

extern "C" int pre_serve_stop(pre_server *s, pre_serve_stats *stats) {
  if (!s) return PRE_ERR_ARG;
  ring_st(s->ring_h, 1u);
  const hipError_t err = hipStreamSynchronize(s->stream);
  pre_engine *e = s->e;
  const uint32_t steps = ring_ld(s->ring_h + 2);
  if (stats) {
    stats->steps = (int32_t)steps;
    stats->served = (int32_t)ring_ld(s->ring_h + 3);
    stats->error = (int32_t)ring_ld(s->ring_h + 4);
  }
  e->epoch_base += steps;
  e->serving = 0;
  (void)hipHostFree(s->ring_h);
  delete s;
  return err == hipSuccess ? PRE_OK : PRE_ERR_HIP;
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
    case PRE_ERR_BROKEN:
      return "engine broken by an earlier device error (reset it), or its static workspace was taken over";
    case PRE_ERR_CONTEXT: return "position would reach max_ctx";
    case PRE_ERR_BUSY: return "busy: a serving loop holds the engine, or the request ring is full";
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

// Debug entry: encode n fp32 values with the fp8 cache's encoder.
extern "C" int pre_debug_fp8_encode(const float *d_in, void *d_out, int n, void *stream) {
  if (!d_in || !d_out || n <= 0) return PRE_ERR_ARG;
  const int th = 256, nb = (n + th - 1) / th;
  hipLaunchKernelGGL(pre_k_fp8_encode, dim3(nb), dim3(th), 0, (hipStream_t)stream, d_in, (uint8_t *)d_out, n);
  return hipGetLastError() == hipSuccess ? PRE_OK : PRE_ERR_HIP;
}

// Debug / tuning entry: time the streamed GEMV variants.  variant = 2 * i + c
// with ring depth {2, 4, 8, 12}[i] row pairs and weight cache policy {default,
// streaming}[c]; rows are split over `grid` workgroups of `threads` threads,
// each given at least lds_min bytes of LDS (96 KB keeps one per CU).
extern "C" int pre_debug_gemv(int variant, const void *d_w, int rows, int K, const float *d_x, float *d_y,
                              int grid, int threads, int lds_min, void *stream) {
  if (!d_w || !d_x || !d_y || rows < 1 || K < 8 || K % 8 || grid < 1 || threads < 64 || threads > 1024)
    return PRE_ERR_ARG;
  const int Kp = (K + 511) / 512 * 512;
  const size_t lds = std::max<size_t>((size_t)(Kp + 64 + ((rows + grid - 1) / grid + 1) * (threads / 64)) * 4,
                                      (size_t)lds_min);
  if (lds > 160 * 1024) return PRE_ERR_SHAPE;
  const void *fns[8] = {(const void *)pre_k_gemv_bench<2, CP_DEF>, (const void *)pre_k_gemv_bench<2, CP_NT>,
                        (const void *)pre_k_gemv_bench<4, CP_DEF>, (const void *)pre_k_gemv_bench<4, CP_NT>,
                        (const void *)pre_k_gemv_bench<8, CP_DEF>, (const void *)pre_k_gemv_bench<8, CP_NT>,
                        (const void *)pre_k_gemv_bench<12, CP_DEF>, (const void *)pre_k_gemv_bench<12, CP_NT>};
  if (variant < 0 || variant >= 8) return PRE_ERR_ARG;
  if (hipFuncSetAttribute(fns[variant], hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
    return PRE_ERR_HIP;
  const uint16_t *w = (const uint16_t *)d_w;
  void *args[] = {&w, &rows, &K, &d_x, &d_y};
  if (hipLaunchKernel(fns[variant], dim3(grid), dim3(threads), args, lds, (hipStream_t)stream) != hipSuccess)
    return PRE_ERR_HIP;
  return PRE_OK;
}

// Debug entry: copy `bytes` (a multiple of 16, 16-byte aligned buffers) with
// pre_k_copy -- the calibration kernel for memory-traffic counters.
extern "C" int pre_debug_copy(const void *d_src, void *d_dst, size_t bytes, void *stream) {
  if (!d_src || !d_dst || bytes == 0 || (bytes & 15) || !al16(d_src) || !al16(d_dst)) return PRE_ERR_ARG;
  const int64_t n16 = (int64_t)(bytes / 16);
  hipLaunchKernelGGL(pre_k_copy, dim3(2048), dim3(256), 0, (hipStream_t)stream, (const v4i *)d_src, (v4i *)d_dst,
                     n16);
  return hipGetLastError() == hipSuccess ? PRE_OK : PRE_ERR_HIP;
}

// Debug: the MFMA lane-layout probe (A 16x32, B 32x16 bf16 row-major; D
// 16x16 fp32).
extern "C" int pre_debug_mfma(const void *d_a, const void *d_b, float *d_d, void *stream) {
  if (!d_a || !d_b || !d_d) return PRE_ERR_ARG;
  hipLaunchKernelGGL(pre_k_mfma_probe, dim3(1), dim3(64), 0, (hipStream_t)stream, (const uint16_t *)d_a,
                     (const uint16_t *)d_b, d_d);
  return hipGetLastError() == hipSuccess ? PRE_OK : PRE_ERR_HIP;
}

// Debug: byte offsets of the workspace regions (status, flags, layers, tasks,
// rope, xcc, x_out, pbuf, q, u, rl, part, lmp, x_emb, a_norm, tok, xmid, pk,
// ssq, ctx, kvnew, total) -- 22 int64 values.
extern "C" int pre_debug_layout(const pre_engine *e, int64_t *out) {
  if (!e || !out) return PRE_ERR_ARG;
  const Layout &L = e->Lo;
  const int64_t v[22] = {L.status, L.flags, L.layers, L.tasks, L.rope, L.xcc, L.x_out, L.pbuf, L.q, L.u, L.rl,
                         L.part, L.lmp, L.x_emb, L.a_norm, L.tok, L.xmid, L.pk, L.ssq, L.ctx, L.kvnew, L.total};
  for (int i = 0; i < 22; ++i) out[i] = v[i];
  return PRE_OK;
}

// Debug: from the next decode call on, the task that sets ready flag `slot`
// (an index into the step's slots, 0 .. n_slots-1) skips the store; -1 turns
// this off.  Every consumer of that flag then waits until the watchdog fires,
// latches PRE_DEV_TIMEOUT and raises the abort word, and every other
// workgroup leaves at its next wait: the way to exercise the watchdog path
// with every kernel still ending normally.
extern "C" int pre_debug_drop_signal(pre_engine *e, int32_t slot) {
  if (!e || slot < -1 || slot >= e->D.n_si * e->D.W) return PRE_ERR_ARG;
  e->drop_slot = slot;
  return PRE_OK;
}

// Debug entry: run pre_k_lane_ops on 64 inputs (see the kernel for the layout
// of the 320 outputs).
extern "C" int pre_debug_lane_ops(const float *d_in, float *d_out, void *stream) {
  if (!d_in || !d_out) return PRE_ERR_ARG;
  hipLaunchKernelGGL(pre_k_lane_ops, dim3(1), dim3(64), 0, (hipStream_t)stream, d_in, d_out);
  return hipGetLastError() == hipSuccess ? PRE_OK : PRE_ERR_HIP;
}
