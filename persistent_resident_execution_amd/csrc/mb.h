// Micro-batch decode (2..8 sequences in lockstep, each at its own context
// length): the resident kernel's second task set.  Included by engine.hip
// after the batch-1 tiles, whose helpers it shares (waits, flags, scalar
// reductions, the attention tile's inner loops).
//
// What changes with a batch (TileRT notes, "tile pipeline" and the skinny
// GEMM discussion; persistent-execution survey, section 6.2):
//
//  * Projections become skinny GEMMs.  Each weight is still read once per
//    step, but now multiplies up to 8 activation columns, so the work runs on
//    the matrix cores: v_mfma_f32_16x16x32_bf16 on 16 weight rows x 32
//    columns per instruction.  The activations enter as two bf16 columns per
//    sequence, hi = bf16(x) and lo = bf16(x - hi): their products with the
//    bf16 weights are exact in the fp32 accumulator, so the result carries
//    about 16 bits of the activation (better than one fp32 rounding of a
//    long dot product needs).  16 columns = 8 sequences x (hi, lo).
//  * The producers write their outputs straight into that packed layout,
//    ordered for the stream's operand mapping (below): 128 GEMM columns per
//    4 KB step, [fragment f][k-group q of 4][column c of 4][quarter h of
//    4][8 bf16], so the 16 bytes lane l of an MFMA takes for fragment f of
//    step s sit at s * 4096 + f * 1024 + l * 16.  The
//    RMSNorm that precedes a projection is folded as in the batch-1 tiles:
//    the producer packs x * g and leaves its share of sum(x^2) per sequence;
//    the consumer scales its outputs by 1 / rms.
//  * Attention is balanced over the workgroups of each KV head: the head's
//    (sequence, position) pairs of this step are cut into equal contiguous
//    shares, so long and short contexts cost the same per workgroup.  A
//    share that crosses a sequence boundary leaves one record per sequence;
//    a combine stage merges each sequence's records and packs the heads'
//    outputs for the O projection, which then runs like every other GEMM.

// ---------------------------------------------------------------------------
// MFMA operands and the packed layout

// Byte offset of the 16 bytes that hold columns k8 * 8 .. + 7 of GEMM input
// column `col` (sequence b: col b = hi, col 8 + b = lo).  Within step
// k8 / 16: quarter h = (k8 % 16) / 4, k-group q = k8 % 4; column col is
// c = col % 4 of fragment f (bit 0: col / 8, bit 1: (col / 4) % 2).
__device__ __forceinline__ uint32_t pk_off(int k8, int col) {
  const uint32_t k = (uint32_t)k8, c = (uint32_t)col;
  const uint32_t f = ((c >> 3) & 1u) | (((c >> 2) & 1u) << 1);
  return (k >> 4) * 4096u + f * 1024u + (k & 3u) * 256u + (c & 3u) * 64u + ((k >> 2) & 3u) * 16u;
}
// (whole steps; the columns past K stay zero)
__device__ __forceinline__ int64_t pk_bytes(int K) { return (int64_t)((K + 127) >> 7) * 4096; }
// The packed inputs of layer l: QKV (l = L: the LM head), gate/up, down, O.
__device__ __forceinline__ uint8_t *pk_x(const KP &P, int l) { return P.pk + (int64_t)l * pk_bytes(P.h); }
__device__ __forceinline__ uint8_t *pk_m(const KP &P, int l) {
  return P.pk + (int64_t)(P.L + 1 + l) * pk_bytes(P.h);
}
__device__ __forceinline__ uint8_t *pk_u(const KP &P, int l) {
  return P.pk + (int64_t)(2 * P.L + 1) * pk_bytes(P.h) + (int64_t)l * pk_bytes(P.ffn);
}
__device__ __forceinline__ uint8_t *pk_o(const KP &P, int l) {
  return P.pk + (int64_t)(2 * P.L + 1) * pk_bytes(P.h) + (int64_t)P.L * pk_bytes(P.ffn) +
         (int64_t)l * pk_bytes(P.Hq * P.d);
}

// Write 8 consecutive GEMM input values of sequence b as hi and lo bf16.
__device__ __forceinline__ void pk_store8(uint8_t *pk, int K, int k8, int b, const float (&v)[8]) {
  v4i hw, lw;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint16_t h0 = f2bf(v[2 * i]), h1 = f2bf(v[2 * i + 1]);
    const uint16_t l0 = f2bf(v[2 * i] - bf16f(h0)), l1 = f2bf(v[2 * i + 1] - bf16f(h1));
    hw[i] = (int)((uint32_t)h0 | ((uint32_t)h1 << 16));
    lw[i] = (int)((uint32_t)l0 | ((uint32_t)l1 << 16));
  }
  const Rsrc r = mkbuf(uni_ptr(pk), (uint32_t)pk_bytes(K));
  st128<CP_SC1>(r, pk_off(k8, b), hw);
  st128<CP_SC1>(r, pk_off(k8, 8 + b), lw);
}

// Per-workgroup sums of squares: index 2l = the QKV input of layer l (2L:
// the LM head's), 2l + 1 = the gate/up input of layer l.
__device__ __forceinline__ float *ssq_at(const KP &P, int idx, int lam) {
  return P.ssq + ((int64_t)idx * P.W + lam) * P.B;
}

// ---------------------------------------------------------------------------
// row groups: up to 16 rows of one weight matrix at a fixed stride

struct MbRg {
  uint64_t base;  // address of the group's first row
  int32_t nr;     // rows (0: none)
  int32_t rs;     // bytes from one row to the next
  int32_t o0;     // output index of the first row (QKV: RoPE pair index)
};

// The k-th run of at most 16 RoPE pairs of a QKV task that stays inside one
// q/k/v head; returns its length (0 past the last) and its first pair.
__device__ __forceinline__ int qkv_group(const KP &P, const Task &t, int k, int *p0) {
  const int half = P.d >> 1;
  int p = t.r0;
  for (int i = 0; p < t.r1; ++i) {
    const int n = min(16, min(t.r1, (p / half + 1) * half) - p);
    if (i == k) { *p0 = p; return n; }
    p += n;
  }
  *p0 = t.r1;
  return 0;
}

// Row groups of a task: QKV and gate/up list (A, B) partners next to each
// other (A = RoPE rows j / gate rows, B = rows j + d/2 / up rows).
__device__ __forceinline__ int mb_nrg(const KP &P, const Task &t) {
  const int rows = t.r1 - t.r0;
  if (t.op == OP_QKV) {
    int n = 0, p;
    while (qkv_group(P, t, n, &p) > 0) ++n;
    return 2 * n;
  }
  if (t.op == OP_GU) return 2 * ((rows + 15) >> 4);
  return (rows + 15) >> 4;
}

__device__ __forceinline__ MbRg mb_rg(const KP &P, const Task &t, int j) {
  const DevLayer &Lw = P.layers[min(t.layer, P.L - 1)];
  const int h2 = P.h * 2;
  if (t.op == OP_QKV) {
    int p;
    const int n = qkv_group(P, t, j >> 1, &p);
    const int half = P.d >> 1, gh = p / half, g = gh / (P.G + 2), hh = gh % (P.G + 2);
    const int jj = p % half + (j & 1) * half;
    const uint16_t *m;
    int64_t row;
    if (hh < P.G) { m = (const uint16_t *)Lw.wq; row = (int64_t)(g * P.G + hh) * P.d + jj; }
    else { m = (const uint16_t *)(hh == P.G ? Lw.wk : Lw.wv); row = (int64_t)g * P.d + jj; }
    return MbRg{(uint64_t)(m + row * P.h), n, h2, p};
  }
  if (t.op == OP_GU) {
    const int r = t.r0 + 16 * (j >> 1), n = max(0, min(16, t.r1 - r));
    const uint16_t *m = (const uint16_t *)((j & 1) ? Lw.wu : Lw.wg);
    return MbRg{(uint64_t)(m + (int64_t)r * P.h), n, h2, r};
  }
  const int r = t.r0 + 16 * j, n = max(0, min(16, t.r1 - r));
  if (t.op == OP_OPROJ) {
    const int K = P.Hq * P.d;
    return MbRg{(uint64_t)((const uint16_t *)Lw.wo + (int64_t)r * K), n, K * 2, r};
  }
  if (t.op == OP_DOWN)
    return MbRg{(uint64_t)((const uint16_t *)Lw.wd + (int64_t)r * P.ffn), n, P.ffn * 2, r};
  return MbRg{(uint64_t)(P.lm_head + (int64_t)r * P.h), n, h2, r};  // OP_LM
}

// ---------------------------------------------------------------------------
// The GEMM stream of one batch of nb row groups (nb = 1, 2, 4 or 8).
//
// Wavefront w takes row group jr = w % nb of the batch and k-part
// kp = w / nb of the nw / nb equal parts of the 128-column steps (with 8
// row groups every wavefront owns one group over all of K; with one group
// the eight wavefronts split K).
//
// Operand mapping ("diagonal"): the 16 rows of the MFMA's A operand are
// (weight row rho = i / 4, column quarter h = i % 4) of a set of 4 weight
// rows, so one 16-byte load per lane covers 4 rows x 256 contiguous bytes
// (the 16-rows x 64-bytes footprint of the plain mapping streams markedly
// slower).  The 16 B columns are (input column c = j / 4, quarter h = j % 4)
// of 4 packed input columns.  Entry (i, j) of the product is a true partial
// dot product only where h(i) = h(j); the other entries are discarded, so a
// 128-column step of 16 rows takes 4 loads (row sets s) and 16 MFMAs
// (4 row sets x {hi, lo} x {sequences 0-3, 4-7}), against 4 MFMAs for the
// plain mapping -- the matrix cores have that headroom.  hi and lo share an
// accumulator.  A ring of DS steps of A fragments is kept in flight; the
// first DS are issued before the dependency wait (weights never wait for
// activations), then the wait, the staging of the input (STAGED) and the
// loop.  At the end each lane keeps its diagonal entry, a quad of lanes adds
// the four quarters, and the 16 x B partials go to
// ys[((kp * nb + jr) * 8 + b) * 16 + row].
template <bool STAGED, int DS, class AfterWait, class AfterStage>
__device__ __forceinline__ bool mb_stream(const KP &P, const Task &t, int j0, int nb, int nrg, const uint8_t *act,
                                          float *lact, int K, const MbWaiter *wait, float *ys,
                                          const AfterWait &after_wait, const AfterStage &after_stage) {
  const int lane = tid_task() & 63, wave = wave_task(), nw = P.nw;
  const int ii = lane & 15, q = lane >> 4, h = ii & 3;
  const int jr = wave % nb, kp = wave / nb, nkp = nw / nb;
  MbRg g{0, 0, 0, 0};
  if (j0 + jr < nrg) g = mb_rg(P, t, j0 + jr);
  const int nr = rfl(g.nr), rs = rfl(g.rs);
  // rows past nr fall outside the buffer and read 0
  const Rsrc ra = mkbuf64(rfl64(g.base), (uint32_t)(nr * rs));
  const int nkb = K >> 5, nks = (nkb + 3) >> 2;
  const int ks0 = nks * kp / nkp, n = nks * (kp + 1) / nkp - ks0;
  const Rsrc rb = mkbuf(uni_ptr(act), (uint32_t)nks * 4096u);
  // Every out-of-range marker sits in the per-lane offset (the one the
  // buffer range check covers), set by masks rather than branches so the
  // ring's waits stay exact: steps past the span, and weight quarters of the
  // last step past the K / 32 blocks (the input there is zero).
  constexpr uint32_t OOB = 0x80000000u;
  const uint32_t va = (uint32_t)((ii >> 2) * rs + h * 64 + q * 16);  // row set 0, step 0
  auto span_mask = [&](int st) -> uint32_t { return (uint32_t)(st >= n) * OOB; };
  auto a_off = [&](int st, int s, uint32_t sm) -> uint32_t {  // step st of the span, row set s
    const int ks = ks0 + st;
    return (va + (uint32_t)(4 * s * rs) + (uint32_t)ks * 256u) | sm | ((uint32_t)(ks * 4 + h >= nkb) * OOB);
  };
  // B fragment f (bit 0 = lo, bit 1 = sequences 4..7): 1 KB, lane-linear
  auto b_off = [&](int st, int f) -> uint32_t {
    return (uint32_t)(ks0 + st) * 4096u + (uint32_t)f * 1024u + (uint32_t)lane * 16u;
  };
  v4i a[DS][4], bq[STAGED ? 1 : DS][4];
  f32x4_t acc[4][2];
#pragma unroll
  for (int s = 0; s < 4; ++s) acc[s][0] = acc[s][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int st = 0; st < DS; ++st)
#pragma unroll
    for (int s = 0; s < 4; ++s) a[st][s] = ld128<CP_W>(ra, a_off(st, s, span_mask(st)));
  if (wait) {
    if (!(*wait)(P)) return false;
    after_wait();  // loads of the producers' other results, in flight with the staging
    if (STAGED) {  // the packed input, once, into LDS (one round trip for the workgroup)
      const int n16 = nks * 256;
      for (int i0 = tid_task(); i0 < n16; i0 += 16 * P.nthr) {  // 4096 columns: one round
        v4i x[16];
#pragma unroll
        for (int k = 0; k < 16; ++k)
          x[k] = i0 + k * P.nthr < n16 ? ld128<CP_SC1>(rb, (uint32_t)(i0 + k * P.nthr) * 16u) : v4i{0, 0, 0, 0};
#pragma unroll
        for (int k = 0; k < 16; ++k)
          if (i0 + k * P.nthr < n16) reinterpret_cast<v4i *>(lact)[i0 + k * P.nthr] = x[k];
      }
      __syncthreads();
    }
    after_stage();  // (their values: landed with the staging)
  }
  if (!STAGED) {
#pragma unroll
    for (int st = 0; st < DS; ++st)
#pragma unroll
      for (int f = 0; f < 4; ++f) bq[STAGED ? 0 : st][f] = ld128<CP_SC1>(rb, b_off(st, f) | span_mask(st));
  }
  auto consume = [&](int slot, int st) {
    v4i b[4];
    if (STAGED) {
#pragma unroll
      for (int f = 0; f < 4; ++f) b[f] = reinterpret_cast<const v4i *>(lact)[b_off(st, f) >> 4];
    } else {
#pragma unroll
      for (int f = 0; f < 4; ++f) b[f] = bq[STAGED ? 0 : slot][f];
    }
    // the accumulator changes with every MFMA: no back-to-back dependence
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int s = 0; s < 4; ++s) acc[s][f >> 1] = mfma_16x16x32(a[slot][s], b[f], acc[s][f >> 1]);
  };
  // (inside the span: issues of the steady loop and the tail)
  auto issue = [&](int slot, int st) {
#pragma unroll
    for (int s = 0; s < 4; ++s) a[slot][s] = ld128<CP_W>(ra, a_off(st, s, 0u));
    if (!STAGED) {
#pragma unroll
      for (int f = 0; f < 4; ++f) bq[STAGED ? 0 : slot][f] = ld128<CP_SC1>(rb, b_off(st, f));
    }
  };
  const int m = n >= DS ? (n - DS) / DS : 0;  // rounds whose every issue lies inside the span
  // The first round is peeled: it still has the prologue's order of loads in
  // flight; the loop after it sees the steady order only, so its waits are
  // exact (one slot at a time).
  if (m > 0) {
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      consume(s, s);
      issue(s, DS + s);
    }
    for (int r = 1; r < m; ++r) {
#pragma unroll
      for (int s = 0; s < DS; ++s) {
        consume(s, r * DS + s);
        issue(s, (r + 1) * DS + s);
      }
    }
  }
  const int rem = n - m * DS;  // 0 <= rem < 2 DS
#pragma unroll
  for (int s = 0; s < DS; ++s) {
    if (s < rem) consume(s, m * DS + s);
    if (s + DS < rem) issue(s, (m + 1) * DS + s);
  }
#pragma unroll
  for (int s = 0; s < DS; ++s)
    if (s + DS < rem) consume(s, (m + 1) * DS + s);
  // diagonal entries: lane (q, 4c + h) holds row 4s + q, column c of
  // sequence set m, quarter h, in element h
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int ms = 0; ms < 2; ++ms) {
      const f32x4_t x = acc[s][ms];
      float v = h == 0 ? x[0] : h == 1 ? x[1] : h == 2 ? x[2] : x[3];
      v += dpp<0xB1>(v);  // quad_perm [1, 0, 3, 2]
      v += dpp<0x4E>(v);  // quad_perm [2, 3, 0, 1]
      const int b = 4 * ms + (ii >> 2);
      if (h == 0 && b < P.B) ys[((kp * nb + jr) * 8 + b) * 16 + 4 * s + q] = v;
    }
  return true;
}

// Output (row i of row group j, sequence b) of a batch of nb row groups:
// the nkp k-parts' partials added in order.
__device__ __forceinline__ float mb_y(const float *ys, int nb, int nkp, int j, int b, int i) {
  float v[MAXW];
#pragma unroll
  for (int w = 0; w < MAXW; ++w) v[w] = w < nkp ? ys[((w * nb + j) * 8 + b) * 16 + i] : 0.f;
  float y = 0.f;
#pragma unroll
  for (int w = 0; w < MAXW; ++w) y += v[w];
  return y;
}

// 1 / rms of each sequence's input from the producers' sums of squares
// (wavefront b sums sequence b's W partials in workgroup order).
__device__ __forceinline__ void mb_norm_scales(const KP &P, int idx, int K, float *rs) {
  const int wave = wave_task(), lane = tid_task() & 63;
  if (wave < P.B) {
    float s = 0.f;
    for (int w = lane; w < P.W; w += 64) s += ld_sc1(ssq_at(P, idx, w) + wave);
    s = wave_sum(s);
    if (lane == 0) rs[wave] = 1.0f / sqrtf(s / (float)K + P.eps);
  }
}

__device__ __forceinline__ int mb_tok(const int *toks, int b) { return toks[b]; }

// Buffer descriptors are scalar: every access below takes a per-workgroup
// base and a per-lane byte offset (a per-lane base would make the compiler
// loop over the lanes' distinct descriptors).

__device__ __forceinline__ void bf8(v4i w, float (&o)[8]) {
  o[0] = bf_lo(w.x); o[1] = bf_hi(w.x); o[2] = bf_lo(w.y); o[3] = bf_hi(w.y);
  o[4] = bf_lo(w.z); o[5] = bf_hi(w.z); o[6] = bf_lo(w.w); o[7] = bf_hi(w.w);
}
__device__ __forceinline__ void f8(v4i a, v4i c, float (&x)[8]) {
  const float4 p = __builtin_bit_cast(float4, a), q = __builtin_bit_cast(float4, c);
  x[0] = p.x; x[1] = p.y; x[2] = p.z; x[3] = p.w; x[4] = q.x; x[5] = q.y; x[6] = q.z; x[7] = q.w;
}
// Rows r..r+7 of sequence b of a layer's [B][h] fp32 vector (device scope).
__device__ __forceinline__ void ld8_vec(const KP &P, const float *vec, int b, int r, float (&x)[8]) {
  const Rsrc rr = mkbuf(uni_ptr(vec), (uint32_t)P.B * P.h * 4);
  const uint32_t o = ((uint32_t)b * P.h + r) * 4;
  f8(ld128<CP_SC1>(rr, o), ld128<CP_SC1>(rr, o + 16), x);
}
__device__ __forceinline__ void st8_vec(const KP &P, float *vec, int b, int r, const float (&v)[8]) {
  const Rsrc rr = mkbuf(uni_ptr(vec), (uint32_t)P.B * P.h * 4);
  const uint32_t o = ((uint32_t)b * P.h + r) * 4;
  st128<CP_SC1>(rr, o, __builtin_bit_cast(v4i, float4{v[0], v[1], v[2], v[3]}));
  st128<CP_SC1>(rr, o + 16, __builtin_bit_cast(v4i, float4{v[4], v[5], v[6], v[7]}));
}

// The residual entering layer l at rows r..r+7 of sequence b.
__device__ __forceinline__ void mb_x_in(const KP &P, int l, int b, int r, const int *toks, float (&x)[8]) {
  if (l == 0) {
    const Rsrc re = mkbuf(P.embed, (uint32_t)P.V * P.h * 2);
    bf8(ld128<CP_DEF>(re, ((uint32_t)mb_tok(toks, b) * P.h + r) * 2), x);
  } else {
    ld8_vec(P, P.x_out + vec_off(P, l - 1, 0, P.h), b, r, x);
  }
}

__device__ __forceinline__ void mb_gain8(const KP &P, const uint16_t *g, int r, float (&o)[8]) {
  bf8(ld128<CP_DEF>(mkbuf(uni_ptr(g), (uint32_t)P.h * 2), (uint32_t)r * 2), o);
}

// LDS of the micro-batch GEMM tasks: ys[nw * 8 * 16] | rs[8] | ssq[8] |
// per-thread partials[512] | staged packed input (K * 8 floats).
struct MbLds {
  float *ys, *rs, *ssq, *ep, *act;
};
__device__ __forceinline__ MbLds mb_lds(const KP &P, float *lds) {
  float *ys = lds, *rs = ys + P.nw * 8 * 16;
  return MbLds{ys, rs, rs + 8, rs + 16, rs + 16 + 512};
}

// One GEMM task: batches of up to 8 row groups, each streamed, reduced and
// finished by its operator's epilogue.
__device__ __forceinline__ bool mb_gemm(const KP &P, const Task &t, int lam, int step, const int *toks, float *lds,
                                        const MbWaiter &wait) {
  const int l = t.layer, op = t.op, tid = tid_task(), T = P.nthr, nw = P.nw, B = P.B;
  const MbLds M = mb_lds(P, lds);
  const int nrg = rfl(mb_nrg(P, t));
  const int nb = min(nw, nrg <= 1 ? 1 : nrg <= 2 ? 2 : nrg <= 4 ? 4 : 8);  // row groups per batch
  const int nkp = nw / nb;  // k-parts per row group
  const uint8_t *act;
  int K, nidx = -1;  // sums of squares this task's input is normalised with
  if (op == OP_QKV) { act = pk_x(P, l); K = P.h; nidx = 2 * l; }
  else if (op == OP_GU) { act = pk_m(P, l); K = P.h; nidx = 2 * l + 1; }
  else if (op == OP_DOWN) { act = pk_u(P, l); K = P.ffn; }
  else if (op == OP_OPROJ) { act = pk_o(P, l); K = P.Hq * P.d; }
  else { act = pk_x(P, P.L); K = P.h; nidx = 2 * P.L; }
  if (tid < 8) M.ssq[tid] = 0.f;
  // The producers' sums of squares of this input (wavefront b, sequence b),
  // loaded once the input is staged, in flight with the weight stream, and
  // folded into the norm scales after it.
  float sq4[4] = {0.f, 0.f, 0.f, 0.f};
  const bool early_ss = nidx >= 0 && P.W <= 256 && K <= P.mbst;  // staged inputs only
  auto load_ss = [&]() {
    const int wave = wave_task(), lane = tid & 63;
    if (early_ss && wave < B) {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (lane + 64 * k < P.W) sq4[k] = ld_sc1(ssq_at(P, nidx, lane + 64 * k) + wave);
    }
  };
  auto fold_ss = [&]() {
    const int wave = wave_task(), lane = tid & 63;
    if (early_ss && wave < B) {
      const float s = wave_sum(sq4[0] + sq4[1] + sq4[2] + sq4[3]);
      if (lane == 0) M.rs[wave] = 1.0f / sqrtf(s / (float)K + P.eps);
    }
  };
  // LM: each sequence's running best, kept by wavefront b
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  bool nan = false;
  bool waited = false;
  for (int j0 = 0; j0 < max(nrg, 1); j0 += nb) {
    const MbWaiter *wp = waited ? nullptr : &wait;
    const bool ok =
        K <= P.mbst ? mb_stream<true, 3>(P, t, j0, nb, nrg, act, M.act, K, wp, M.ys, [] {}, load_ss)
                    : mb_stream<false, 3>(P, t, j0, nb, nrg, act, M.act, K, wp, M.ys, [] {}, [] {});
    if (!ok) return false;
    if (!waited) {
      if (early_ss) {
        fold_ss();
      } else if (nidx >= 0) {
        mb_norm_scales(P, nidx, K, M.rs);
      } else if (tid < 8) {
        M.rs[tid] = 1.f;
      }
      waited = true;
    }
    __syncthreads();
    wait.mark(1);
    const float *ys = M.ys;
    switch (op) {
      case OP_QKV: {
        const int half = P.d >> 1;
        for (int e = tid; e < (nb >> 1) * 16 * B; e += T) {
          const int b = e % B, i = (e / B) % 16, k = e / (16 * B), jA = 2 * k;
          if (j0 + jA >= nrg) continue;
          int p;
          const int n = qkv_group(P, t, (j0 + jA) >> 1, &p);
          if (i >= n) continue;
          p += i;
          const int gh = p / half, g = gh / (P.G + 2), hh = gh % (P.G + 2), jj = p % half;
          const float r = M.rs[b];
          float a = r * mb_y(ys, nb, nkp, jA, b, i), c = r * mb_y(ys, nb, nkp, jA + 1, b, i);
          const int pos = toks[8 + b];  // column b's position in this step
          if (hh <= P.G) {  // RoPE on q and k
            const float cs = P.rope[(int64_t)pos * half + jj];
            const float sn = P.rope[(int64_t)P.max_ctx * half + (int64_t)pos * half + jj];
            const float a2 = a * cs - c * sn, c2 = c * cs + a * sn;
            a = a2; c = c2;
          }
          if (hh < P.G) {
            float *qd = P.q + vec_off(P, l, b, P.Hq * P.d) + (int64_t)(g * P.G + hh) * P.d;
            st_sc1(qd + jj, a);
            st_sc1(qd + jj + half, c);
          } else if (toks[16 + b]) {  // the layer's K or V cache of every sequence under one descriptor each
            // (a padding column of a ragged chunk appends nothing)
            const int64_t lbase = (int64_t)l * P.Bc * P.Hkv * P.max_ctx * P.d;
            const uint32_t bytes = (uint32_t)((int64_t)P.Bc * P.Hkv * P.max_ctx * P.d * 2);
            const int cs = P.chunk ? 0 : b;  // the column's sequence in the cache
            const uint32_t o0 = (uint32_t)((((int64_t)cs * P.Hkv + g) * P.max_ctx + pos) * P.d + jj) * 2;
            if (hh == P.G) {
              const Rsrc rr = mkbuf(P.kc + lbase, bytes);
              st16<CP_SC1>(rr, o0, f2bf(a));
              st16<CP_SC1>(rr, o0 + (uint32_t)half * 2, f2bf(c));
            } else {
              const Rsrc rv = mkbuf(P.vc + lbase, bytes);
              st16<CP_SC1>(rv, o0, f2bf(a));
              st16<CP_SC1>(rv, o0 + (uint32_t)half * 2, f2bf(c));
            }
          }
        }
        break;
      }
      case OP_GU: {
        for (int e = tid; e < (nb >> 1) * 2 * B; e += T) {
          const int b = e % B, o = (e / B) & 1, k = e / (2 * B), jA = 2 * k;
          const int r0 = t.r0 + 16 * ((j0 + jA) >> 1) + 8 * o;
          if (j0 + jA >= nrg || r0 >= t.r1) continue;
          const float r = M.rs[b];
          float u[8];
#pragma unroll
          for (int i = 0; i < 8; ++i)
            u[i] = silu(r * mb_y(ys, nb, nkp, jA, b, 8 * o + i)) * (r * mb_y(ys, nb, nkp, jA + 1, b, 8 * o + i));
          pk_store8(pk_u(P, l), P.ffn, r0 >> 3, b, u);
        }
        break;
      }
      case OP_OPROJ:
      case OP_DOWN: {
        const bool down = op == OP_DOWN;
        const uint16_t *gain = !down ? (const uint16_t *)P.layers[l].ffn_norm
                               : l + 1 < P.L ? (const uint16_t *)P.layers[l + 1].attn_norm : P.final_norm;
        uint8_t *dst = down ? pk_x(P, l + 1) : pk_m(P, l);
        const int ne = nb * 2 * B;
        for (int e = tid; e < ne; e += T) {
          const int b = e % B, o = (e / B) & 1, j = e / (2 * B);
          const int r0 = t.r0 + 16 * (j0 + j) + 8 * o;
          float sq = 0.f;
          if (j0 + j < nrg && r0 < t.r1) {
            float x[8], g[8];
            if (down) ld8_vec(P, P.xmid + vec_off(P, l, 0, P.h), b, r0, x);
            else mb_x_in(P, l, b, r0, toks, x);
            mb_gain8(P, gain, r0, g);
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] += mb_y(ys, nb, nkp, j, b, 8 * o + i);
            st8_vec(P, (down ? P.x_out : P.xmid) + vec_off(P, l, 0, P.h), b, r0, x);
            if (down && P.chk_hidden && l == P.L - 1 && toks[16 + b]) {
              float *hd = P.chk_hidden + ((int64_t)step * P.B + b) * P.h + r0;
#pragma unroll
              for (int i = 0; i < 8; ++i) hd[i] = x[i];
            }
            float xg[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) { sq = fmaf(x[i], x[i], sq); xg[i] = x[i] * g[i]; }
            pk_store8(dst, P.h, r0 >> 3, b, xg);
          }
          M.ep[e] = sq;
        }
        __syncthreads();
        if (tid < B) {  // this batch's sums of squares, in row order
          float s = M.ssq[tid];
          for (int e = tid; e < ne; e += B) s += M.ep[e];
          M.ssq[tid] = s;
        }
        break;
      }
      default: {  // OP_LM: wavefront b keeps sequence b's best
        const int wave = wave_task(), lane = tid & 63;
        if (wave < B) {
          const int b = wave;
          for (int e = lane; e < nb * 16; e += 64) {
            const int j = e >> 4, i = e & 15, row = t.r0 + 16 * (j0 + j) + i;
            if (j0 + j >= nrg || row >= t.r1) continue;
            const float y = M.rs[b] * mb_y(ys, nb, nkp, j, b, i);
            if (y != y) nan = true;
            else argmax_merge(bv, bi, y, row);
            if (P.chk_logits && toks[16 + b]) P.chk_logits[((int64_t)step * P.B + b) * P.V + row] = y;
          }
        }
        break;
      }
    }
    __syncthreads();  // ys is rewritten by the next batch
  }
  if (op == OP_LM) {
    const int wave = wave_task(), lane = tid & 63;
    if (wave < B) {
      wave_argmax_l63(bv, bi);
      const bool wn = __any(nan);
      if (lane == 63) {
        st_sc1(P.lmp + 2 * ((int64_t)lam * B + wave), wn ? __builtin_nanf("") : bv);
        st_flag(reinterpret_cast<uint32_t *>(P.lmp) + 2 * ((int64_t)lam * B + wave) + 1, (uint32_t)bi);
      }
    }
  } else if (op == OP_OPROJ || op == OP_DOWN) {
    if (tid < B) st_sc1(ssq_at(P, op == OP_DOWN ? 2 * (l + 1) : 2 * l + 1, lam) + tid, M.ssq[tid]);
  }
  return true;
}

// Embedding rows [r0, r1) of every sequence's token, packed (times the
// first layer's attention-norm gains) for the first QKV stage, with their
// sums of squares.
__device__ __forceinline__ bool mb_embed(const KP &P, const Task &t, int lam, const int *toks, float *lds) {
  const int tid = tid_task(), B = P.B;
  const MbLds M = mb_lds(P, lds);
  const uint16_t *gain = (const uint16_t *)P.layers[0].attn_norm;
  const int n8 = (t.r1 - t.r0) >> 3;
  if (tid < 8) M.ssq[tid] = 0.f;
  __syncthreads();
  for (int e0 = 0; e0 < n8 * B; e0 += P.nthr) {
    const int e = e0 + tid;
    float sq = 0.f;
    if (e < n8 * B) {
      const int b = e % B, r0 = t.r0 + 8 * (e / B);
      float x[8], g[8], xg[8];
      mb_x_in(P, 0, b, r0, toks, x);
      mb_gain8(P, gain, r0, g);
#pragma unroll
      for (int i = 0; i < 8; ++i) { sq = fmaf(x[i], x[i], sq); xg[i] = x[i] * g[i]; }
      pk_store8(pk_x(P, 0), P.h, r0 >> 3, b, xg);
    }
    M.ep[tid] = sq;
    __syncthreads();
    if (tid < B) {  // the threads whose element e0 + k belongs to sequence tid
      float s = M.ssq[tid];
      for (int k = (tid - e0 % B + B) % B; k < P.nthr; k += B) s += M.ep[k];
      M.ssq[tid] = s;
    }
    __syncthreads();
  }
  if (tid < B) st_sc1(ssq_at(P, 0, lam) + tid, M.ssq[tid]);
  return true;
}

// ---------------------------------------------------------------------------
// Attention: this workgroup's share of KV head g over all sequences.
//
// Step positions: sequence b attends n_b = pos_b + 1 positions.  KV head g's
// pairs (b, t) are numbered f = pre_b + t (pre_b = n_0 + .. + n_{b-1}) up to
// N = sum n_b; workgroup i of the head's Tw takes f in
// [i * N / Tw, (i + 1) * N / Tw).  Its piece of sequence b leaves a record
// (m, l, -, -, o[d]) per query head at ((l * W + lambda) * B + b).

__device__ __forceinline__ int64_t mb_share(int64_t N, int Tw, int i) { return (int64_t)i * N / Tw; }

// Positions [t0, t0 + cnt) of sequence b (at most cmax of them), merged into
// the running (max, sum, output) state of the piece kept in LDS; the last
// sub-piece writes the piece's record.  (The scheme of attn_core, the
// batch-1 chunk task's attention, kept as its own copy: instantiating that
// shared template in this register-bound kernel moved its register
// allocation and made the step about 2% slower.)  Both products run on the
// matrix cores (NQ = d / 32 column quarters of a head; NS = sets of 16 / NQ query
// heads in the score columns):
//  * Scores, with the same diagonal operand mapping as the GEMM stream: A
//    row i = (position i / NQ, quarter i % NQ) of 16 / NQ consecutive cached
//    K rows -- one 16-byte load per lane reads them whole, 1 KB contiguous
//    -- and B column j = (query head j / NQ, quarter j % NQ), the scaled q
//    as hi + lo bf16 parts.  The diagonal entries, added over the quarters,
//    are the scores; they go to LDS.
//  * After the softmax, o = sum_t p_t V_t in chunks of 32 positions: A rows
//    (head, hi/lo part of p), B column j = one of the head's dimensions, the
//    8 positions of a k-group packed from 8 V loads (each lane loads its own
//    8-dimension slice of 8 consecutive rows, so the packing stays in the
//    lane).
template <int NQ, int NS>
__device__ __forceinline__ void mb_attn_sub(const KP &P, int l, int lam, int b, int g, int t0, int cnt, int pos,
                                            int pnew, float *lds, const MbWaiter *wait, bool first, bool last,
                                            bool &ok) {
  constexpr int D = 32 * NQ;  // head dimension
  constexpr int PL = 16 / NQ;  // positions per K load
  constexpr int RA = 8;  // K loads in flight per wavefront
  constexpr uint32_t OOB = 0x80000000u;
  const int G = P.G, tid = tid_task(), T = P.nthr;
  const int wave = wave_task(), nw = P.nw, lane = tid & 63, ii = lane & 15, qg = lane >> 4;
  const int cpad = ((P.cmax + 63) / 64) * 64;
  float *qs = lds, *sc = qs + G * D, *ored = sc + G * cpad, *st = ored + nw * G * D;
  float *Or = st + 2 * G, *Mr = Or + G * D, *Lr = Mr + G;
  const int64_t cbase = (((int64_t)l * P.Bc + (P.chunk ? 0 : b)) * P.Hkv + g) * P.max_ctx * D;
  const Rsrc kr = mkbuf(P.kc + cbase, (uint32_t)P.max_ctx * D * 2);
  const Rsrc vr = mkbuf(P.vc + cbase, (uint32_t)P.max_ctx * D * 2);
  // K load u: positions u * PL ..; this lane's row and 16 bytes.  Before the
  // wait the rows this step's QKV stage writes (pnew .. pos: the newest one,
  // or a chunk's rows up to this column) are left out (reloaded after).
  auto koff = [&](int u, bool pre) -> uint32_t {
    const int tt = u * PL + ii / NQ;
    const bool in = tt < cnt && !(pre && t0 + tt >= pnew);
    return in ? (uint32_t)(t0 + tt) * (uint32_t)(D * 2) + (uint32_t)((ii % NQ) * 64 + qg * 16) : OOB;
  };
  const int nL = (cnt + PL - 1) / PL;
  const int nk = nL > wave ? (nL - wave + nw - 1) / nw : 0;  // this wavefront's loads u = wave + nw * k
  v4i ka[RA];
#pragma unroll
  for (int s = 0; s < RA; ++s) ka[s] = ld128<CP_SC1>(kr, koff(wave + nw * s, true));
  if (wait && !(*wait)(P)) { ok = false; return; }
  if (t0 <= pos && pnew < t0 + cnt) {  // the rows written this step, now complete
    const int ulo = (max(pnew, t0) - t0) / PL, uhi = (pos - t0) / PL;
#pragma unroll
    for (int s = 0; s < RA; ++s) {
      const int u = wave + nw * s;
      if (u >= ulo && u <= uhi) ka[s] = ld128<CP_SC1>(kr, koff(u, false));
    }
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
  // scores of K load u (positions u * PL ..) into sc
  auto scores = [&](const v4i &a, int u) {
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
      ka[s] = ld128<CP_SC1>(kr, koff(wave + nw * (k0 + s + RA), false));
    }
  }
  // V chunk c (positions c * 32 ..): load r of this lane = position
  // c * 32 + 8 qg + r, dimensions 8 (ii % (D / 8)) ..
  const uint32_t vcol = (uint32_t)(ii % (D / 8)) * 16u;
  auto vload = [&](v4i (&x)[8], int c) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int tt = c * 32 + 8 * qg + r;
      x[r] = ld128<CP_SC1>(vr, tt < cnt ? (uint32_t)(t0 + tt) * (uint32_t)(D * 2) + vcol : OOB);
    }
  };
  const int nC = (cnt + 31) >> 5;
  const int nkc = nC > wave ? (nC - wave + nw - 1) / nw : 0;  // this wavefront's chunks c = wave + nw * k
  v4i va[8], vn[8];
  vload(va, wave);  // the first V chunk, during the softmax
  __syncthreads();
  for (int hh = wave; hh < G; hh += nw) {
    float m = -INFINITY;
    for (int i = lane; i < cnt; i += 64) m = fmaxf(m, sc[hh * cpad + i]);
    m = wave_max(m);
    float sm = 0.f;
    for (int i = lane; i < cnt; i += 64) {
      const float e = expf(sc[hh * cpad + i] - m);
      sc[hh * cpad + i] = e;
      sm += e;
    }
    for (int i = cnt + lane; i < nC * 32; i += 64) sc[hh * cpad + i] = 0.f;  // whole chunks
    sm = wave_sum(sm);
    if (lane == 0) { st[2 * hh] = m; st[2 * hh + 1] = sm; }
  }
  __syncthreads();
  f32x4_t acc[D / 16];
#pragma unroll
  for (int m = 0; m < D / 16; ++m) acc[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  auto pv = [&](const v4i (&x)[8], int c) {
    // A: row ii = (head ii / 2, part ii % 2) of p, positions c * 32 + 8 qg ..
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
    vload(vn, wave + nw * (k + 1));
    pv(va, wave + nw * k);
    if (k + 1 >= nkc) break;
    vload(va, wave + nw * (k + 2));
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
  const int rec = D + PREC_O;
  float *pdst = P.part + (((int64_t)l * P.W + lam) * P.B + b) * G * rec;
  for (int i = tid; i < G * D; i += T) {
    const int hh = i / D, j = i % D;
    float s = 0.f;
    float ov[MAXW];
#pragma unroll
    for (int w = 0; w < MAXW; ++w) ov[w] = w < nw ? ored[(w * G + hh) * D + j] : 0.f;
#pragma unroll
    for (int w = 0; w < MAXW; ++w) s += ov[w];
    if (!first) {
      const float m = st[2 * hh], M = fmaxf(Mr[hh], m);
      s = Or[i] * expf(Mr[hh] - M) + s * expf(m - M);
    }
    Or[i] = s;
    if (last) st_sc1(pdst + hh * rec + PREC_O + j, s);
  }
  __syncthreads();
  for (int hh = tid; hh < G; hh += T) {
    float m = st[2 * hh], ls = st[2 * hh + 1];
    if (!first) {
      const float M = fmaxf(Mr[hh], m);
      ls = Lr[hh] * expf(Mr[hh] - M) + ls * expf(m - M);
      m = M;
    }
    Mr[hh] = m;
    Lr[hh] = ls;
    if (last) {
      st_sc1(pdst + hh * rec, m);
      st_sc1(pdst + hh * rec + 1, ls);
    }
  }
  __syncthreads();  // the LDS is reused by the next sub-piece
}

__device__ __forceinline__ bool mb_attn(const KP &P, const Task &t, int lam, int step, const int *toks, float *lds,
                                        const MbWaiter &wait) {
  const int g = t.aux, i = t.r0, Tw = t.r1;
  const int *posv = toks + 8;  // each column's position in this step
  int64_t N = 0;
  for (int b = 0; b < P.B; ++b) N += posv[b] + 1;
  const int64_t f0 = mb_share(N, Tw, i), f1 = mb_share(N, Tw, i + 1);
  bool ok = true, first = true;
  int64_t pre = 0;
  for (int b = 0; b < P.B && ok; ++b) {
    const int pos = posv[b];
    const int pnew = P.chunk ? posv[0] : pos;  // a chunk's rows of this step start at column 0's
    const int64_t lo = max(f0, pre), hi = min(f1, pre + pos + 1);
    // the piece in sub-pieces of at most cmax positions
    for (int64_t c0 = lo; c0 < hi && ok; c0 += P.cmax) {
      const int n = (int)min((int64_t)P.cmax, hi - c0);
      const MbWaiter *wp = first ? &wait : nullptr;
      if (P.d == 64)
        mb_attn_sub<2, 1>(P, t.layer, lam, b, g, (int)(c0 - pre), n, pos, pnew, lds, wp, c0 == lo, c0 + n == hi,
                          ok);
      else if (P.G <= 4)
        mb_attn_sub<4, 1>(P, t.layer, lam, b, g, (int)(c0 - pre), n, pos, pnew, lds, wp, c0 == lo, c0 + n == hi,
                          ok);
      else
        mb_attn_sub<4, 2>(P, t.layer, lam, b, g, (int)(c0 - pre), n, pos, pnew, lds, wp, c0 == lo, c0 + n == hi,
                          ok);
      first = false;
    }
    pre += pos + 1;
  }
  if (first && ok) ok = wait(P);  // no piece: still ordered after the producers
  return ok;
}

// Combine: elements [r0, r1) of KV head g's (sequence, query head, dim)
// space, 8 dims per group of 32 lanes.  The lanes of a group take the
// records of the sequence's workgroups (lane r: the r-th, r + 32-th, ...),
// merge them pairwise with the running-max rescaling, and reduce across the
// group; lane 0 packs the 8 outputs for the O projection.
__device__ __forceinline__ bool mb_comb(const KP &P, const Task &t, int step, const int *toks, const MbWaiter &wait) {
  if (!wait(P)) return false;
  const int g = t.aux, Tw = P.Tg, G = P.G, d = P.d, l = t.layer, tid = tid_task();
  const int *posv = toks + 8;
  const int rec = d + PREC_O, gd = G * d;
  const int ngr = (t.r1 - t.r0) >> 3, gpp = P.nthr >> 5;
  int64_t N = 0;
  for (int b = 0; b < P.B; ++b) N += posv[b] + 1;
  for (int q0 = 0; q0 < ngr; q0 += gpp) {
    const int grp = q0 + (tid >> 5), sub = tid & 31;
    const bool act = grp < ngr;
    const int e = t.r0 + 8 * grp, b = act ? e / gd : 0, k = e % gd, hh = k / d, j0 = k % d;
    int64_t pre = 0;
    for (int bb = 0; bb < b; ++bb) pre += posv[bb] + 1;
    const int64_t nb = posv[b] + 1;
    // workgroups holding f = pre and f = pre + nb - 1
    const int i_lo = (int)(((pre + 1) * Tw - 1) / N), i_hi = (int)(((pre + nb) * Tw - 1) / N);
    // the layer's records under one descriptor; record (wg, b, hh) at a per-lane offset
    const Rsrc rr = mkbuf(P.part + (int64_t)l * P.W * P.B * G * rec, (uint32_t)P.W * P.B * G * rec * 4);
    float M = -INFINITY, Ls = 0.f, O[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int i = i_lo + sub; act && i <= i_hi; i += 32) {
      if (mb_share(N, Tw, i) >= mb_share(N, Tw, i + 1)) continue;  // empty share: no record
      const uint32_t ro = (uint32_t)((((g * Tw + i) * P.B + b) * G + hh) * rec) * 4;
      const float4 ml = __builtin_bit_cast(float4, ld128<CP_SC1>(rr, ro));
      const float4 oa = __builtin_bit_cast(float4, ld128<CP_SC1>(rr, ro + (PREC_O + j0) * 4));
      const float4 ob = __builtin_bit_cast(float4, ld128<CP_SC1>(rr, ro + (PREC_O + j0 + 4) * 4));
      const float m = ml.x, ls = ml.y;
      const float o[8] = {oa.x, oa.y, oa.z, oa.w, ob.x, ob.y, ob.z, ob.w};
      const float Mn = fmaxf(M, m);
      const float a = M == -INFINITY ? 0.f : expf(M - Mn), c = expf(m - Mn);
      Ls = Ls * a + ls * c;
#pragma unroll
      for (int q = 0; q < 8; ++q) O[q] = O[q] * a + o[q] * c;
      M = Mn;
    }
#pragma unroll
    for (int x = 16; x >= 1; x >>= 1) {  // across the 32 lanes of the group
      const float Mo = __shfl_xor(M, x), Lo = __shfl_xor(Ls, x);
      float Oo[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) Oo[q] = __shfl_xor(O[q], x);
      const float Mn = fmaxf(M, Mo);
      const float a = M == -INFINITY ? 0.f : expf(M - Mn), c = Mo == -INFINITY ? 0.f : expf(Mo - Mn);
      Ls = Ls * a + Lo * c;
#pragma unroll
      for (int q = 0; q < 8; ++q) O[q] = O[q] * a + Oo[q] * c;
      M = Mn;
    }
    if (act && sub == 0) {
      float v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] = O[q] / Ls;
      pk_store8(pk_o(P, l), P.Hq * d, ((g * G + hh) * d + j0) >> 3, b, v);
    }
  }
  return true;
}

// Each sequence's greedy token from the W partials (wavefront b reads
// sequence b's); toks[b] = -1 on NaN.
__device__ __forceinline__ void mb_reduce(const KP &P, int *toks) {
  const int wave = wave_task(), lane = tid_task() & 63;
  __syncthreads();
  if (wave < P.B) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    bool nan = false;
    for (int i = lane; i < P.W; i += 64) {
      const int64_t o = 2 * ((int64_t)i * P.B + wave);
      const float v = ld_sc1(P.lmp + o);
      const int ix = (int)ld_flag(reinterpret_cast<const uint32_t *>(P.lmp) + o + 1);
      if (v != v) nan = true;
      else argmax_merge(bv, bi, v, ix);
    }
    wave_argmax_l63(bv, bi);
    const bool anynan = __any(nan);
    if (lane == 63) toks[wave] = anynan ? -1 : bi;
  }
  __syncthreads();
}

__device__ __forceinline__ bool mb_run_task(const Task &t, int lam, int step, const int *toks, float *lds,
                                            const MbWaiter &wait) {
  const KP &P = kp_fresh();
  switch (t.op) {
    case OP_EMBED: return mb_embed(P, t, lam, toks, lds);
    case OP_ATTN: return mb_attn(P, t, lam, step, toks, lds, wait);
    case OP_COMB: return mb_comb(P, t, step, toks, wait);
    default: return mb_gemm(P, t, lam, step, toks, lds, wait);
  }
}

// The micro-batch resident kernel (and, with P.persistent = 0, its
// per-operator baseline: one stage of one step per launch).
extern "C" __global__ void __launch_bounds__(512) pre_persistent_mb(KP P) {
  extern __shared__ __attribute__((aligned(16))) float lds[];
  __shared__ int sh[8];
  // [0, 8): each column's token of this step; [8, 16): its position in this
  // step; [16, 24): 1 if the column is a real token (0: padding of a ragged
  // chunk); [24, 32): the columns' positions at the call's start
  __shared__ int toks[32];
  const bool res = P.persistent != 0;
  const int lam = res ? lambda_of_block(blockIdx.x, P.W, P.X) : blockIdx.x;
  const int tid = tid_task();
  if (res && tid == 0) {
    const uint32_t x = xcc_id();
    P.xcc[lam] = x;
    if (P.W % P.X == 0 && (int)x != (int)(blockIdx.x % P.X))
      __hip_atomic_fetch_add(&P.status->xcc_mismatch, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  const int s_begin = res ? 0 : P.b_step, s_end = res ? P.n_steps : P.b_step + 1;
  const int si0 = res ? 0 : P.b_si, si1 = res ? P.n_si : P.b_si + 1;
  if (tid < P.B && !P.chunk)  // the first step's tokens (the baseline: its step's)
    toks[tid] = P.forced ? P.forced[(int64_t)s_begin * P.B + tid]
                         : (s_begin == 0 ? P.in_tok[tid] : P.tok_slot[tid]);
  // every sequence's start position (workgroup 0 advances them after the
  // last step; a chunk of one sequence has one); all workgroups see the same
  // values and leave together on an error
  for (int b = 0; b < (P.chunk ? 1 : P.B); ++b) {
    const int p = call_position(P, b);
    if (p < 0) return;
    if (tid == 0) toks[24 + b] = p;
  }
  __syncthreads();
  for (int s = s_begin; s < s_end; ++s) {
    const uint32_t ep = P.epoch_base + (uint32_t)s + 1u;
    if (tid < P.B) {
      if (P.chunk) {
        // column b is token j = s * B + b of the chunked sequence; past the
        // last token the padding repeats it and appends nothing
        const int j = s * P.B + tid, jj = min(j, P.chunk_n - 1);
        toks[tid] = P.forced[jj];
        toks[8 + tid] = toks[24] + jj;
        toks[16 + tid] = j < P.chunk_n;
      } else {
        if (res && P.forced) toks[tid] = P.forced[(int64_t)s * P.B + tid];
        toks[8 + tid] = toks[24 + tid] + s;
        toks[16 + tid] = 1;
      }
    }
    __syncthreads();
    int bad = 0, badtok = 0;
    for (int b = 0; b < P.B; ++b)
      if (toks[b] < 0 || toks[b] >= P.V) { bad = 1; badtok = toks[b]; }
    if (bad) {
      if (tid == 0) latch_error(P, PRE_DEV_BAD_TOKEN, s, -1, -1, (uint32_t)badtok, 0);
      return;
    }
    for (int si = si0; si < si1; ++si) {
      const Task t = P.tasks[(int64_t)si * P.W + lam];
      const int tr = res && P.trace != nullptr;
      const uint32_t tw = tr ? (uint32_t)now_ticks() : 0u;
      const MbWaiter wait{res ? 1 : 0, t.wait_lo, t.wait_hi, s, si, ep, sh, tr};
      if (!mb_run_task(t, lam, s, toks, lds, wait)) return;
      if (res) {
        signal_slot(P, t.signal, ep, false);
        if (tr) trace_rec(P, s, si, lam, tw, (uint32_t)sh[3], (uint32_t)now_ticks(), sh);
      }
    }
    if (!res) return;
    const bool need = (!P.forced && s + 1 < P.n_steps) || lam == 0;
    if (need) {
      const int s_lm = P.n_si - 1;
      if (!wait_slots(P, s_lm * P.W, (s_lm + 1) * P.W, ep, s, s_lm, sh)) return;
      const int act = toks[16 + min(tid, P.B - 1)];
      mb_reduce(P, toks);
      for (int b = 0; b < P.B; ++b)
        if (toks[b] < 0) {
          if (tid == 0) latch_error(P, PRE_DEV_NAN, s, s_lm, -1, 0, 0);
          return;
        }
      if (lam == 0 && tid < P.B && act) P.out_tok[(int64_t)s * P.B + tid] = toks[tid];
      __syncthreads();
    }
  }
  if (!res || lam != 0) return;
  // Workgroup 0 has seen every workgroup's LM flag of the last step: every
  // workgroup has read the start positions.  Commit the call's tokens.
  if (!P.chunk) {
    if (tid < P.B) st_flag(reinterpret_cast<uint32_t *>(P.ctx_len) + tid, (uint32_t)(toks[24 + tid] + P.n_steps));
  } else if (tid == 0) {
    int keep = P.chunk_n;
    if (P.verify) {
      // speculative verify (one step): column 0 is the current token and
      // columns 1..k the drafts; column b's greedy token (toks[b]) is the
      // model's successor of columns 0..b.  The drafts are accepted while each
      // equals the greedy successor of the one before; the accepted tokens and
      // the current one stay in the cache, the next input is the greedy
      // token after the last accepted draft.
      int a = 0;
      while (a + 1 < P.chunk_n && P.forced[a + 1] == toks[a]) ++a;
      P.v_accept[0] = a;
      keep = a + 1;
    }
    st_flag(reinterpret_cast<uint32_t *>(P.ctx_len), (uint32_t)(toks[24] + keep));
  }
}

// Baseline: each sequence's greedy token of step `step` (one workgroup).
extern "C" __global__ void __launch_bounds__(512) pre_k_argmax_mb(KP P, int step) {
  __shared__ int toks[8];
  mb_reduce(P, toks);
  if (threadIdx.x < P.B) {
    const int nt = toks[threadIdx.x];
    if (nt < 0) latch_error(P, PRE_DEV_NAN, step, P.n_si - 1, -1, 0, 0);
    P.tok_slot[threadIdx.x] = nt < 0 ? 0 : nt;
    P.out_tok[(int64_t)step * P.B + threadIdx.x] = nt;
  }
}

// Debug: D = A (16 x 32) * B (32 x 16) through mfma_16x16x32 with the lane
// layout the GEMM stream assumes (A, B row-major bf16; D row-major fp32).
extern "C" __global__ void pre_k_mfma_probe(const uint16_t *A, const uint16_t *Bm, float *Dm) {
  const int l = threadIdx.x & 63, r = l & 15, kq = l >> 4;
  v4i a, b;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = (int)((uint32_t)A[r * 32 + kq * 8 + 2 * i] | ((uint32_t)A[r * 32 + kq * 8 + 2 * i + 1] << 16));
    b[i] = (int)((uint32_t)Bm[(kq * 8 + 2 * i) * 16 + r] | ((uint32_t)Bm[(kq * 8 + 2 * i + 1) * 16 + r] << 16));
  }
  const f32x4_t d = mfma_16x16x32(a, b, f32x4_t{0.f, 0.f, 0.f, 0.f});
#pragma unroll
  for (int i = 0; i < 4; ++i) Dm[(4 * kq + i) * 16 + r] = d[i];
}
