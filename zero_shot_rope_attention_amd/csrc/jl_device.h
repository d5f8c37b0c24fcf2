// Device-side building blocks shared by the prefill and decode kernels (gfx950).
//
// Matrix products use v_mfma_f32_32x32x16_bf16 (32x32 output tile, K = 16 per
// instruction).  Lane layout of that instruction on a 64-wide wave, with
// h = lane / 32 and n = lane % 32:
//   A (32 x 16): lane holds A[n][8h + e], e = 0..7
//   B (16 x 32): lane holds B[8h + e][n], e = 0..7
//   D (32 x 32): lane holds D[8(i/4) + 4h + (i%4)][n], i = 0..15
// Only the pairing of A's and B's k index matters for the sum, so the kernels
// are free to choose which key each k index stands for.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace jl {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kD = 128;     // head size
constexpr int kHalfD = 64;  // rotate-half pairs (d, d + 64)
constexpr int kBN = 64;     // keys per tile
constexpr float kNegBig = -1.0e30f;  // finite "minus infinity" for running maxima
constexpr float kLn2 = 0.69314718055994530942f;

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& u) { return __builtin_bit_cast(bf16x8, u); }

// bf16 halves of a packed dword -> fp32
__device__ __forceinline__ float bf_lo(uint32_t u) { return __builtin_bit_cast(float, u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __builtin_bit_cast(float, u & 0xffff0000u); }

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  f32x2 f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

// cos/sin of the angle c * theta_d, where theta_rev = theta_d / (2 pi).
// The product is reduced to [-1/2, 1/2] revolutions in fp64 (|c| theta_d can
// reach ~1e5 rad, where an fp32 angle would already be off by ~1e-2 rad); the
// reduced angle is then evaluated by the hardware sine/cosine, which take
// revolutions.  The reduction is one fused multiply-add, c theta - rint(c theta)
// with the product unrounded, written out so that every kernel computes the
// same bits whatever the compiler would contract on its own.
__device__ __forceinline__ f32x2 rot_cs(long long c, double theta_rev) {
  const double cd = (double)c;
  const double r = cd * theta_rev;
  const float f = (float)__builtin_fma(cd, theta_rev, -__builtin_rint(r));
  return f32x2{__builtin_amdgcn_cosf(f), __builtin_amdgcn_sinf(f)};
}

// The reduced angle of rot_cs alone, c theta_d in [-1/2, 1/2] revolutions, for
// a count known to fit 32 bits (both conversions to double are exact).
__device__ __forceinline__ float rev_reduce(int c, double theta_rev) {
  const double cd = (double)c;
  const double r = cd * theta_rev;
  return (float)__builtin_fma(cd, theta_rev, -__builtin_rint(r));
}

// rot_cs for a count known to fit 32 bits: the same bits, one conversion
// instead of the 64-bit sequence.
__device__ __forceinline__ f32x2 rot_cs(int c, double theta_rev) {
  const float f = rev_reduce(c, theta_rev);
  return f32x2{__builtin_amdgcn_cosf(f), __builtin_amdgcn_sinf(f)};
}

// acc + lo + hi of a packed bf16 pair, in one v_dot2 against (1, 1).
__device__ __forceinline__ float add_bf16_pair(uint32_t pair, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pair), __builtin_bit_cast(bf16x2, 0x3f803f80u),
                                         acc, false);
}

// Rotation of the rotate-half pair (x1, x2) by the angle with cosine c and sine
// s: (x1 c - x2 s, x2 c + x1 s).  Each component is one explicit fused
// multiply-add over one rounded product, so every kernel rounds it the same way
// whatever the compiler would contract on its own.
__device__ __forceinline__ f32x2 rot_pair(float x1, float x2, float c, float s) {
  return f32x2{__builtin_fmaf(x1, c, -(x2 * s)), __builtin_fmaf(x2, c, x1 * s)};
}

// Complex product (a.x + i a.y)(b.x + i b.y), rounded as rot_pair (the same
// rotation written on the first factor).
__device__ __forceinline__ f32x2 cmul(f32x2 a, f32x2 b) { return rot_pair(a.x, a.y, b.x, b.y); }

// Direct HBM -> LDS copy of 16 bytes per lane (gfx950 global_load_lds_dwordx4):
// lane l's 16 bytes land at lds_wave_base + 16 l; lds_wave_base must be the
// same for the whole wave.  Completion is tracked by vmcnt.
__device__ __forceinline__ void lds_dma16(const void* src, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(src, lds_wave_base, 16, 0, 0);
}

// Wait until every global load of this wave, including LDS DMA, has landed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

// LDS byte pointer.  lds_opaque() pins a per-lane LDS address in a VGPR as an
// opaque value, so that the reads made from it keep their constant parts in
// the instructions' offset field instead of re-adding the lane part per read.
typedef __attribute__((address_space(3))) uint8_t lds_byte;
__device__ __forceinline__ const lds_byte* lds_ptr(const void* generic) { return (const lds_byte*)generic; }
__device__ __forceinline__ const lds_byte* lds_opaque(const lds_byte* p) {
  asm volatile("" : "+v"(p));
  return p;
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
// ds_read_b64_tr_b16: within each group of 16 lanes, lane i receives element
// (i % 4) of the 8 bytes read by lanes 4e + i / 4 of the group, e = 0..3.
__device__ __forceinline__ u32x2 lds_read_tr16(const void* p) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}
__device__ __forceinline__ u32x2 lds_read_tr16(const lds_byte* p) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

// Combine a value with the one held by the lane 32 positions away (the other
// half-wave) through v_permlane32_swap, without an LDS round trip.  After the
// swap one register holds the lower half's values in every lane and the other
// the upper half's, so both halves compute op(lower, upper) identically.
__device__ __forceinline__ f32x2 half_pair(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return f32x2{__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1])};
}
__device__ __forceinline__ float half_max(float x) {
  const f32x2 p = half_pair(x);
  return fmaxf(p.x, p.y);
}
__device__ __forceinline__ float half_sum(float x) {
  const f32x2 p = half_pair(x);
  return p.x + p.y;
}

// floor(n / g) for 0 <= n < 2^22 and 1 <= g, using a float reciprocal plus an
// exact integer correction.
__device__ __forceinline__ int small_div(int n, int g, float inv_g) {
  int q = (int)((float)n * inv_g);
  if ((q + 1) * g <= n) ++q;
  if (q * g > n) --q;
  return q;
}

}  // namespace jl
