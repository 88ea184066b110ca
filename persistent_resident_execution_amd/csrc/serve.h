// The serving loop: the resident kernel that never returns between requests.
// Included by engine.hip after the batch-1 tiles, whose task code it runs.
//
// Instead of one launch per pre_engine_decode call, the host launches this
// kernel once and then hands it requests through a ring of descriptors in
// coherent host memory (persistent-execution survey, sections 4 and 5.6: the
// GPU polls host-written descriptors, a per-slot state machine moves each
// request from submitted to running to done; XL-Persistent-Kernel's
// lifecycle of a request: prompt, then decode until EOS or budget).
//
//  * Ring (host memory, system-coherent): a 16-word header -- word 0 the
//    host's stop request, 1 the loop's state (1 running, 2 ended), 2 decode
//    steps run, 3 requests served, 4 the latched device error -- then
//    ring_slots slots of ring_words words: 16 header words (0 state: FREE,
//    READY, RUNNING, DONE; 1 prompt length; 2 start position, -1 = where the
//    sequence stands; 3 budget of generated tokens; 4 EOS token, -1 = none;
//    5 tokens produced so far; 6 the request's error), ring_prompt prompt
//    tokens, ring_out output tokens.  The host moves a slot FREE -> READY and
//    DONE -> FREE, the kernel READY -> RUNNING -> DONE; there is one claimant
//    (workgroup 0), so the claim is a plain store and no atomic crosses PCIe.
//  * Workgroup 0 schedules: lanes of its first wavefront scan the slots'
//    states in one round trip, claim the oldest READY slot (lowest sequence
//    number), copy its prompt into device memory, check it (tokens in range,
//    the steps within max_ctx; a bad request is finished with its error and
//    the loop goes on), and broadcast it to every workgroup through the
//    command words (fields first, then the command's sequence number, all at
//    device scope).  Every other workgroup waits on that number.
//  * Every workgroup then runs the request's steps through the same task
//    table as a decode call: the prompt teacher-forced, then greedy tokens
//    fed back; each workgroup reduces the greedy token itself, so all of
//    them stop at the same step (EOS or budget).  Workgroup 0 writes each
//    token to the slot as it is produced, then the count.  The ready flags'
//    epochs continue across requests (every workgroup counts the steps).
//  * The loop ends when the host asks for it, or by itself after idle_ticks
//    without a request (so an abandoned loop cannot hold the GPU), or when a
//    device error is latched (every workgroup leaves through the abort word).

enum : int32_t { SLOT_FREE = 0, SLOT_READY = 1, SLOT_RUNNING = 2, SLOT_DONE = 3 };
constexpr int RING_HDR = 16;
enum : int32_t { CMD_SEQ = 0, CMD_KIND = 1, CMD_SLOT = 2, CMD_NPROMPT = 3, CMD_POS = 4, CMD_BUDGET = 5,
                 CMD_EOS = 6 };
enum : int32_t { KIND_REQUEST = 1, KIND_EXIT = 2 };

__device__ __forceinline__ uint32_t ld_sys(const uint32_t *p) {
  return __hip_atomic_load(const_cast<uint32_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ void st_sys(uint32_t *p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ uint32_t *ring_slot(const KP &P, int i) {
  return P.ring + RING_HDR + (int64_t)i * P.ring_words;
}

// Workgroup 0: wait for a READY slot (or the stop request, or the idle
// limit), claim it, copy and check its prompt, and publish the command.
// Returns the command's kind.  sh[0..7] is scratch.
__device__ __forceinline__ int serve_schedule(const KP &P, uint32_t seq, int *sh) {
  const int tid = threadIdx.x;
  while (true) {
    if (tid < 64) {
      const int lane = tid;
      const uint64_t t0 = now_ticks();
      int kind = 0, pick = -1;
      while (true) {
        // one round trip: every lane reads one slot's state and sequence
        int best = 0x7fffffff, who = -1;
        for (int i = lane; i < P.ring_slots; i += 64) {
          const uint32_t *sl = ring_slot(P, i);
          if ((int)ld_sys(sl) == SLOT_READY) {
            const int q = (int)ld_sys(sl + 7);
            if (q < best) { best = q; who = i; }
          }
        }
        // the oldest READY slot over the lanes (lowest sequence, then index)
        for (int o = 32; o >= 1; o >>= 1) {
          const int ob = __shfl_xor(best, o), ow = __shfl_xor(who, o);
          if (ob < best || (ob == best && ow >= 0 && (who < 0 || ow < who))) { best = ob; who = ow; }
        }
        if (who >= 0) { pick = who; kind = KIND_REQUEST; break; }
        if (ld_sys(P.ring) != 0u) { kind = KIND_EXIT; break; }            // the host's stop request
        if (ld_flag(&P.status->abort)) { kind = KIND_EXIT; break; }
        if (now_ticks() - t0 > P.idle_ticks) { kind = KIND_EXIT; break; }  // nobody is submitting
        __builtin_amdgcn_s_sleep(8);
      }
      if (lane == 0) { sh[0] = kind; sh[1] = pick; }
    }
    __syncthreads();
    const int kind = sh[0], pick = sh[1];
    __syncthreads();
    if (kind == KIND_EXIT) {
      if (tid == 0) {
        st_flag(reinterpret_cast<uint32_t *>(P.cmd + CMD_KIND), KIND_EXIT);
        drain();
        st_flag(reinterpret_cast<uint32_t *>(P.cmd + CMD_SEQ), seq);
      }
      return KIND_EXIT;
    }
    uint32_t *sl = ring_slot(P, pick);
    if (tid == 0) {
      st_sys(sl, SLOT_RUNNING);  // the claim: this workgroup is the only claimant
      const int p = (int)ld_sys(sl + 2);
      sh[2] = (int)ld_sys(sl + 1);
      sh[3] = p < 0 ? (int)ld_flag(reinterpret_cast<const uint32_t *>(P.ctx_len)) : p;
      sh[4] = (int)ld_sys(sl + 3);
      sh[5] = (int)ld_sys(sl + 4);
    }
    __syncthreads();
    const int np = sh[2], pos = sh[3], budget = sh[4], eos = sh[5];
    __syncthreads();
    // the prompt into device memory, checked
    int bad = 0;
    for (int i = tid; i < np && i < P.ring_prompt; i += P.nthr) {
      const int t = (int)ld_sys(sl + 16 + i);
      if (t < 0 || t >= P.V) bad = 1;
      st_flag(reinterpret_cast<uint32_t *>(P.req_tok + i), (uint32_t)t);
    }
    bad = __syncthreads_or(bad);
    int err = 0;
    if (np < 1 || np > P.ring_prompt || budget < 1 || budget > P.ring_out) err = PRE_DEV_BAD_TOKEN;
    else if (bad) err = PRE_DEV_BAD_TOKEN;
    else if (pos < 0 || (int64_t)pos + np + budget - 1 > P.max_ctx) err = PRE_DEV_CONTEXT;
    if (err) {  // finish the slot with its error and keep serving
      if (tid == 0) {
        st_sys(sl + 5, 0u);
        st_sys(sl + 6, (uint32_t)err);
        drain();
        st_sys(sl, SLOT_DONE);
      }
      __syncthreads();
      continue;
    }
    if (tid == 0) {
      st_flag(reinterpret_cast<uint32_t *>(P.cmd + CMD_KIND), KIND_REQUEST);
      st_flag(reinterpret_cast<uint32_t *>(P.cmd + CMD_SLOT), (uint32_t)pick);
      st_flag(reinterpret_cast<uint32_t *>(P.cmd + CMD_NPROMPT), (uint32_t)np);
      st_flag(reinterpret_cast<uint32_t *>(P.cmd + CMD_POS), (uint32_t)pos);
      st_flag(reinterpret_cast<uint32_t *>(P.cmd + CMD_BUDGET), (uint32_t)budget);
      st_flag(reinterpret_cast<uint32_t *>(P.cmd + CMD_EOS), (uint32_t)eos);
    }
    drain();
    __syncthreads();  // every thread's prompt stores and the fields are complete
    if (tid == 0) st_flag(reinterpret_cast<uint32_t *>(P.cmd + CMD_SEQ), seq);
    return KIND_REQUEST;
  }
}

// Every other workgroup: wait (no watchdog: idling is legitimate) for
// command `seq`; false if a device error aborted the loop.
__device__ __forceinline__ bool serve_wait_cmd(const KP &P, uint32_t seq, int *sh) {
  if (threadIdx.x == 0) {
    int ok = 1;
    while (ld_flag(reinterpret_cast<const uint32_t *>(P.cmd + CMD_SEQ)) != seq) {
      if (ld_flag(&P.status->abort)) { ok = 0; break; }
      __builtin_amdgcn_s_sleep(8);
    }
    sh[0] = ok;
  }
  __syncthreads();
  const bool r = sh[0] != 0;
  __syncthreads();
  return r;
}

template <bool KV8>
__device__ __forceinline__ void serve_body(KP &P) {
  extern __shared__ __attribute__((aligned(16))) float lds[];
  __shared__ int sh[8];
  if (P.onexcd && blockIdx.x % P.X != 0) return;
  const int lam = P.onexcd ? blockIdx.x / P.X : lambda_of_block(blockIdx.x, P.W, P.X);
  if (threadIdx.x == 0) {
    const uint32_t x = xcc_id();
    const int bad = (P.W % P.X == 0 || P.onexcd) && (int)x != (int)(blockIdx.x % P.X);
    if (bad && (P.local || P.onexcd)) latch_error(P, PRE_DEV_PLACEMENT, 0, -1, lam, x, blockIdx.x % P.X);
    sh[2] = bad;
  }
  __syncthreads();
  if ((P.local || P.onexcd) && sh[2]) return;
  if (lam == 0 && threadIdx.x == 0) st_sys(P.ring + 1, 1u);
  uint32_t ep_base = P.epoch_base, steps_done = 0, served = 0;
  const int s_lm = P.n_si - 1;
  for (uint32_t seq = 1;; ++seq) {
    int kind;
    if (lam == 0) {
      kind = serve_schedule(P, seq, sh);
    } else {
      if (!serve_wait_cmd(P, seq, sh)) break;
      kind = (int)ld_flag(reinterpret_cast<const uint32_t *>(P.cmd + CMD_KIND));
    }
    if (kind != KIND_REQUEST) break;
    const KP &Q = kp_fresh();
    const int slot = (int)ld_flag(reinterpret_cast<const uint32_t *>(Q.cmd + CMD_SLOT));
    const int np = __builtin_amdgcn_readfirstlane((int)ld_flag(reinterpret_cast<const uint32_t *>(Q.cmd + CMD_NPROMPT)));
    const int pos0 = __builtin_amdgcn_readfirstlane((int)ld_flag(reinterpret_cast<const uint32_t *>(Q.cmd + CMD_POS)));
    const int budget = (int)ld_flag(reinterpret_cast<const uint32_t *>(Q.cmd + CMD_BUDGET));
    const int eos = (int)ld_flag(reinterpret_cast<const uint32_t *>(Q.cmd + CMD_EOS));
    uint32_t *sl = ring_slot(Q, slot);
    int tok = (int)ld_flag(reinterpret_cast<const uint32_t *>(Q.req_tok));
    int ngen = 0, s = 0;
    bool alive = true;
    for (;; ++s) {
      const uint32_t ep = ep_base + (uint32_t)s + 1u;
      const int pos = pos0 + s;
      for (int si = 0; si < Q.n_si && alive; ++si) {
        const Task t = Q.tasks[(int64_t)si * Q.W + lam];
        if (t.op == OP_NONE) continue;
        const Waiter wait{1, t.wait_lo, t.wait_hi, s, si, ep, sh, 0};
        if (!run_task<KV8, false>(t, lam, s, pos, tok, lds, wait)) { alive = false; break; }
        const KP &R = kp_fresh();
        signal_slot(R, t.signal, ep, R.onexcd || (R.local && (t.op == OP_QKV || t.op == OP_ATTN)));
      }
      if (!alive) break;
      const KP &R = kp_fresh();
      const bool gen = s >= np - 1;  // this step's greedy token is an output
      if (gen || lam == 0) {
        if (!wait_slots(R, s_lm * R.W, (s_lm + 1) * R.W, ep, s, s_lm, sh)) { alive = false; break; }
        const int nt = reduce_lm(R, sh);
        if (nt < 0) {
          if (threadIdx.x == 0) latch_error(R, PRE_DEV_NAN, s, s_lm, -1, 0, 0);
          alive = false;
          break;
        }
        if (gen) {
          if (lam == 0 && threadIdx.x == 0) {
            st_sys(sl + 16 + R.ring_prompt + ngen, (uint32_t)nt);
            drain();
            st_sys(sl + 5, (uint32_t)(ngen + 1));
          }
          ++ngen;
          if (ngen >= budget || nt == eos) break;
          tok = nt;
          continue;
        }
      }
      tok = (int)ld_flag(reinterpret_cast<const uint32_t *>(R.req_tok) + s + 1);
    }
    if (!alive) break;
    ep_base += (uint32_t)s + 1u;
    steps_done += (uint32_t)s + 1u;
    ++served;
    if (lam == 0 && threadIdx.x == 0) {
      const KP &R = kp_fresh();
      st_flag(reinterpret_cast<uint32_t *>(R.ctx_len), (uint32_t)(pos0 + s + 1));
      st_sys(sl + 6, 0u);
      drain();
      st_sys(sl, SLOT_DONE);
      st_sys(R.ring + 2, steps_done);
      st_sys(R.ring + 3, served);
    }
  }
  if (lam == 0 && threadIdx.x == 0) {
    const KP &R = kp_fresh();
    st_sys(R.ring + 2, steps_done);
    st_sys(R.ring + 3, served);
    st_sys(R.ring + 4, (uint32_t)ld_flag(reinterpret_cast<const uint32_t *>(&R.status->error)));
    drain();
    st_sys(R.ring + 1, 2u);
  }
}

extern "C" __global__ void __launch_bounds__(512) pre_serve(KP P) { serve_body<false>(P); }
extern "C" __global__ void __launch_bounds__(512) pre_serve_kv8(KP P) { serve_body<true>(P); }
