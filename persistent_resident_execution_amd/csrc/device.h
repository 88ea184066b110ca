// Device-side primitives for gfx950 (CDNA4): buffer loads/stores with
// explicit cache-scope bits, device-scope flag access, DPP wavefront
// reductions and bf16 / fp8 unpacking.
//
// Visibility between workgroups inside one resident kernel.  The eight XCDs
// of the chip each have a private L2 that is not kept coherent with the
// others (persistent-execution survey, section 1; Fleet's two-level event
// sync relies on CDNA cache-scope modifiers, section 7.2).  Everything one
// workgroup hands to another therefore goes through device-scope ("sc1")
// accesses: producers write activations with sc1 stores (written through
// past the private L2), wait for those stores to complete (s_waitcnt), and
// only then store the ready flag with an sc1 store; consumers poll the flag
// with sc1 loads and read the activations with sc1 loads, which are not
// served from a stale private line.  No cache-wide write-back or invalidate
// is issued on the hot path.  Weights are only read, so they use ordinary
// (or streaming) loads.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pre {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef int v2i __attribute__((ext_vector_type(2)));

// Cache-policy operand of the buffer intrinsics on gfx94x/gfx950:
// bit 0 = sc0, bit 1 = nt, bit 4 = sc1.
constexpr int CP_DEF = 0;
constexpr int CP_SC0 = 1;
constexpr int CP_NT = 2;
constexpr int CP_SC1 = 16;

typedef __amdgpu_buffer_rsrc_t Rsrc;
// LDS addresses as 32-bit byte offsets (what ds_* instructions and M0 take)
typedef __attribute__((address_space(3))) void *LdsPtr;
__device__ __forceinline__ LdsPtr lds_ptr(uint32_t a) { return (LdsPtr)(uintptr_t)a; }
__device__ __forceinline__ uint32_t lds_u32(const void *p) { return (uint32_t)(uintptr_t)(LdsPtr)(void *)p; }

// A pointer every lane holds the same value of, as a scalar.  Buffer
// descriptors must live in scalar registers; when the compiler cannot prove
// a base pointer uniform (values merged across branches, pointers read from
// memory) it would otherwise loop over the lanes' copies at every access.
template <class T>
__device__ __forceinline__ T *uni_ptr(T *p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
  return (T *)(((uint64_t)hi << 32) | lo);
}

// Raw buffer over [p, p + bytes): loads past the end return 0, stores past
// the end are dropped.  Word 3 is the gfx9 data-format default.
__device__ __forceinline__ Rsrc mkbuf(const void *p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes,
                                           0x00020000);
}

template <int CP>
__device__ __forceinline__ v4i ld128(Rsrc r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, CP);
}
template <int CP>
__device__ __forceinline__ v2i ld64(Rsrc r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, CP);
}
template <int CP>
__device__ __forceinline__ float ldf(Rsrc r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, CP));
}
template <int CP>
__device__ __forceinline__ void stf(Rsrc r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, off, 0, CP);
}
template <int CP>
__device__ __forceinline__ void st128(Rsrc r, uint32_t off, v4i v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, CP);
}
template <int CP>
__device__ __forceinline__ void st16(Rsrc r, uint32_t off, uint16_t v) {
  __builtin_amdgcn_raw_buffer_store_b16(v, r, off, 0, CP);
}

// Device-scope 32-bit accesses at per-lane addresses (global_load/store sc1).
__device__ __forceinline__ uint32_t ld_flag(const uint32_t *p) {
  return __hip_atomic_load(const_cast<uint32_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_flag(uint32_t *p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_sc1(const float *p) {
  return __builtin_bit_cast(float, ld_flag(reinterpret_cast<const uint32_t *>(p)));
}
__device__ __forceinline__ void st_sc1(float *p, float v) {
  st_flag(reinterpret_cast<uint32_t *>(p), __builtin_bit_cast(uint32_t, v));
}

// Wait until every memory operation this thread issued has completed.
__device__ __forceinline__ void drain() { __builtin_amdgcn_s_waitcnt(0); }

// ---- wavefront reductions (DPP) ------------------------------------------
template <int CTRL, int ROWMASK = 0xf>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                               ROWMASK, 0xf, false));
}
// Sum over each group of 8 lanes, result in every lane of the group.
__device__ __forceinline__ float sum8(float v) {
  v += dpp<0xb1>(v);   // quad_perm [1,0,3,2]
  v += dpp<0x4e>(v);   // quad_perm [2,3,0,1]
  v += dpp<0x141>(v);  // row_half_mirror
  return v;
}
// Sum over each row of 16 lanes, result in every lane of the row.
__device__ __forceinline__ float sum16(float v) {
  v = sum8(v);
  v += dpp<0x140>(v);  // row_mirror
  return v;
}
// Sum over the 64 lanes, wave-uniform result.  Fixed order: deterministic.
__device__ __forceinline__ float wave_sum(float v) {
  v = sum16(v);
  v += dpp<0x142, 0xa>(v);  // row_bcast:15
  v += dpp<0x143, 0xc>(v);  // row_bcast:31
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}
// Two sums over the 64 lanes at once (same order as wave_sum); the totals
// are valid in lane 63 only, which saves the final readlane.
__device__ __forceinline__ float2 wave_sum2_l63(float a, float b) {
  a += dpp<0xb1>(a); b += dpp<0xb1>(b);
  a += dpp<0x4e>(a); b += dpp<0x4e>(b);
  a += dpp<0x141>(a); b += dpp<0x141>(b);
  a += dpp<0x140>(a); b += dpp<0x140>(b);
  a += dpp<0x142, 0xa>(a); b += dpp<0x142, 0xa>(b);
  a += dpp<0x143, 0xc>(a); b += dpp<0x143, 0xc>(b);
  return float2{a, b};
}
// DPP move where lanes the row mask excludes keep their own value.
template <int CTRL, int ROWMASK = 0xf>
__device__ __forceinline__ float dpp_keep(float v) {
  const int b = __builtin_bit_cast(int, v);
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(b, b, CTRL, ROWMASK, 0xf, false));
}
// Maximum over the 64 lanes, wave-uniform result.
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_keep<0xb1>(v));
  v = fmaxf(v, dpp_keep<0x4e>(v));
  v = fmaxf(v, dpp_keep<0x141>(v));
  v = fmaxf(v, dpp_keep<0x140>(v));
  v = fmaxf(v, dpp_keep<0x142, 0xa>(v));
  v = fmaxf(v, dpp_keep<0x143, 0xc>(v));
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}
// Sum of the four 16-lane rows, lane by lane (lane i gets x[i%16] + x[i%16+16]
// + x[i%16+32] + x[i%16+48]), with the gfx950 row-swap permutes.  Both
// registers of a swap are results (v_permlane16_swap exchanges the odd rows of
// the first with the even rows of the second; v_permlane32_swap the upper half
// of the first with the lower half of the second), so they are written as
// in/out asm operands; the builtins' second result is not usable with this
// compiler.  The s_nop pads cover the VALU-write / permlane-read hazard.
__device__ __forceinline__ float xrow_sum(float v) {
  float a = v, b = v;
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
  v = a + b;  // rows (0+1), (0+1), (2+3), (2+3)
  float c = v, e = v;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(c), "+v"(e));
  return c + e;
}

// ---- unpacking -----------------------------------------------------------
__device__ __forceinline__ float bf_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }
__device__ __forceinline__ float bf16f(uint16_t b) { return __builtin_bit_cast(float, (uint32_t)b << 16); }

// fp32 -> bf16, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x7fffffu)) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Eight bf16 weights (one 16-byte load) dotted with eight fp32 activations.
__device__ __forceinline__ float dot8_bf16(v4i w, const float4 a, const float4 b, float acc) {
  acc = fmaf(bf_lo(w.x), a.x, acc);
  acc = fmaf(bf_hi(w.x), a.y, acc);
  acc = fmaf(bf_lo(w.y), a.z, acc);
  acc = fmaf(bf_hi(w.y), a.w, acc);
  acc = fmaf(bf_lo(w.z), b.x, acc);
  acc = fmaf(bf_hi(w.z), b.y, acc);
  acc = fmaf(bf_lo(w.w), b.z, acc);
  acc = fmaf(bf_hi(w.w), b.w, acc);
  return acc;
}

// Four OCP e4m3 codes (one dword, byte 0 first) to fp32, exactly.
__device__ __forceinline__ void fp8x4(uint32_t w, float (&o)[4]) {
  v2f lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
  v2f hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
  o[0] = lo.x; o[1] = lo.y; o[2] = hi.x; o[3] = hi.y;
}

// fp32 -> OCP e4m3 code, round to nearest (ties to even), magnitudes at or
// above 448 saturate to +-448.  Below 2^-6 the codes are multiples of 2^-9
// (x * 512 rounded to an integer; 8 is the smallest normal); above, the
// mantissa is x scaled into [8, 16) and rounded, carrying into the exponent
// at 16.  Finite inputs only.
__device__ __forceinline__ uint32_t f2e4m3(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const uint32_t s = (u >> 24) & 0x80u;
  const float a = __builtin_fabsf(x);
  if (a >= 448.0f) return s | 0x7Eu;
  if (a < 0.015625f) return s | (uint32_t)__builtin_rintf(a * 512.0f);
  int E = (int)((__builtin_bit_cast(uint32_t, a) >> 23) & 0xffu) - 127;  // a in [2^E, 2^(E+1))
  float m = __builtin_rintf(a * __builtin_bit_cast(float, (uint32_t)(127 + 3 - E) << 23));
  if (m == 16.0f) { m = 8.0f; E += 1; }
  if (E > 8 || (E == 8 && m > 14.0f)) return s | 0x7Eu;
  return s | ((uint32_t)(E + 7) << 3) | ((uint32_t)m - 8u);
}

// Eight e4m3 codes (byte e = element e) as eight bf16 (exact: every e4m3
// value is a bf16 value) in the layout of one 16-byte bf16 load.
__device__ __forceinline__ v4i fp8x8_bf16(v2i w) {
  v4i r;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int wi = w[i];
    // gfx950's scaled conversion with scale 1: e4m3 values are bf16 values,
    // so it is exact (checked against the f32 route on every code)
    const auto lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wi, 1.0f, false);
    const auto hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wi, 1.0f, true);
    r[2 * i] = (int)__builtin_bit_cast(uint32_t, lo);
    r[2 * i + 1] = (int)__builtin_bit_cast(uint32_t, hi);
  }
  return r;
}

// Sixteen fp8 weights (one 16-byte load) dotted with sixteen activations.
__device__ __forceinline__ float dot16_fp8(v4i w, const float *x) {
  float acc = 0.f, f[4];
  const float4 *x4 = reinterpret_cast<const float4 *>(x);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    fp8x4((uint32_t)w[q], f);
    const float4 a = x4[q];
    acc = fmaf(f[0], a.x, acc);
    acc = fmaf(f[1], a.y, acc);
    acc = fmaf(f[2], a.z, acc);
    acc = fmaf(f[3], a.w, acc);
  }
  return acc;
}

// Wavefront index inside the workgroup and the number of wavefronts, as
// wave-uniform (scalar) values: read through readfirstlane so that the
// compiler keeps everything derived from them in scalar registers.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }
__device__ __forceinline__ int nwaves() { return __builtin_amdgcn_readfirstlane(blockDim.x >> 6); }

// The thread index behind an empty asm statement, for code inlined into a
// resident kernel's task loop.  Nothing derived from it can be hoisted out of
// the loop: with the plain index the compiler computes dozens of lane
// offsets once before the loop and keeps them live across every task, in
// registers the heaviest task then lacks, or spilled to scratch.
__device__ __forceinline__ int tid_task() {
  int t = (int)threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}
__device__ __forceinline__ int wave_task() { return __builtin_amdgcn_readfirstlane(tid_task() >> 6); }

__device__ __forceinline__ uint64_t now_ticks() { return __builtin_amdgcn_s_memrealtime(); }

__device__ __forceinline__ uint32_t xcc_id() {
  uint32_t v;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(v));
  return v & 0xf;
}

}  // namespace pre
