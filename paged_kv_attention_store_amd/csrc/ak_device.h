// Device-side helpers for the gfx950 kernels: vector types, number-format
// conversions, MFMA wrappers and wavefront reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ak_internal.h"

namespace ak {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ------------------------------------------------------------ conversions

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;

// binary32 -> bfloat16 bits, round to nearest even (gfx950 converts in hardware,
// v_cvt_pk_bf16_f32, in the default round-to-nearest-even mode).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Two bf16 values (lo, hi) packed in one dword, one conversion instruction.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 r;
  r[0] = (__bf16)lo;
  r[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, r);
}

// 2^x on the transcendental unit without the library's denormal-range fix-up:
// callers pass x <= 0, where results below 2^-126 do not matter.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// binary32 value (already divided by the scale) -> E4M3 code: nearest, ties to
// even, saturating at +-448, sign kept.
__device__ __forceinline__ uint32_t f32_to_e4m3(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  uint32_t mag;
  if (a > 0x7f800000u) {
    mag = 0x7f;                                          // NaN stays NaN
  } else if (a >= 0x43e00000u) {                         // |y| >= 448
    mag = 0x7e;
  } else if (a < 0x3c800000u) {                          // |y| < 2^-6: subnormal grid m * 2^-9
    mag = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);   // 0..8, ties to even
  } else {
    const uint32_t e = (a >> 23) - 127u + 7u;           // biased E4M3 exponent, 1..15
    const uint32_t keep = (a >> 20) & 7u;
    const uint32_t rem = a & 0xfffffu;
    mag = (e << 3) | keep;
    if (rem > 0x80000u || (rem == 0x80000u && (keep & 1u))) mag += 1;
    if (mag > 0x7e) mag = 0x7e;
  }
  return mag | sign;
}

// Eight consecutive E4M3 codes (two dwords, code 0 in the low byte) -> eight
// bf16 values, exact.  gfx950 converts two codes per instruction
// (v_cvt_scalef32_pk_bf16_fp8, OCP E4M3, scale 1).
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// ------------------------------------------------------------------ MFMA

// D(16x16) += A(16x32) * B(32x16), bf16 inputs, fp32 accumulate.
// Lane l holds A[l%16][8*(l/16) .. +8], B[8*(l/16) .. +8][l%16];
// D: lane l, element i -> row 4*(l/16) + i, column l%16.
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// D(32x32) += A(32x16) * B(16x32), bf16 inputs, fp32 accumulate.
// Lane l holds A[l%32][8*(l/32) .. +8], B[8*(l/32) .. +8][l%32];
// D: lane l, element i -> row 8*(i/4) + 4*(l/32) + i%4, column l%32.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// ------------------------------------------------------------ reductions

__device__ __forceinline__ float shfl_xor_f(float v, int mask) { return __shfl_xor(v, mask, 64); }

// Combine a value with the one held 32 lanes away (lanes n and n+32 both get the
// result) through v_permlane32_swap: a VALU op, no LDS round trip.
__device__ __forceinline__ float halves_max(float v) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float halves_sum(float v) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// --------------------------------------------------------- kernel arguments

struct AttnArgs {
  const Item* items;
  const Req* reqs;
  const int32_t* kv_indices;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  void* out;
  float* lse;          // may be null
  float* part_o;       // [partial_rows, D]
  float* part_lse;     // [partial_rows], log2 domain
  const MergeJob* merges;  // split small units' merge jobs (Item::merge0 indexes them)
  int32_t* counters;   // arrival counter per split small unit, at Item::merge0
  const int32_t* wg_first;   // stream-K: workgroup g runs small items wg_first[g] .. wg_first[g+1]-1
  int64_t q_st, q_sh;  // q strides (elements): token, head
  int64_t o_st, o_sh;
  int64_t l_st, l_sh;
  int64_t k_sp, k_sb, k_sh;  // cache strides (elements): page, slot, head
  int64_t v_sp, v_sb, v_sh;
  int64_t num_pages;   // pages in the pool (page ids are clamped to it)
  int32_t G, log2B, causal, window;
  float score_scale;   // sm_scale * log2(e) * k_scale
  float v_scale;
};

struct Merge2Args {          // two (out, lse) states of the same rows
  const void* oa;
  const void* ob;
  const float* la;
  const float* lb;
  void* out;
  float* lse;                // may be null
  int64_t a_st, a_sh, b_st, b_sh, o_st, o_sh;   // o_a, o_b, out strides (elements)
  int64_t la_st, la_sh, lb_st, lb_sh, l_st, l_sh;
  int32_t T, H;
};

struct MergeArgs {
  const MergeJob* jobs;
  const float* part_o;
  const float* part_lse;
  void* out;
  float* lse;
  int64_t o_st, o_sh, l_st, l_sh;
  int32_t n_jobs;
};

}  // namespace ak
