// Device-side helpers for the gfx950 kernels: vector types, the bf16 MFMA
// wrapper and its lane layout, RNE conversion, 3D-RoPE positions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_launch.h"

namespace mla {

typedef __bf16 bf16_t;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16_t;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// v_mfma_f32_32x32x16_bf16, D = A * B + C, lane l of a 64-wide wave holds
//   A[m = l % 32][k = 8 * (l / 32) + t]      (t = 0..7)
//   B[k = 8 * (l / 32) + t][n = l % 32]
//   D[m = 8 * (r / 4) + 4 * (l / 32) + r % 4][n = l % 32]   (r = 0..15)
// (checked on gfx950 hardware against a host matmul).
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// v_mfma_f32_16x16x32_{f16,bf16} (Elem<E>::mfma16), lane l holds
//   A[m = l % 16][k = 8 * (l / 16) + t]      (t = 0..7)
//   B[k = 8 * (l / 16) + t][n = l % 16]
//   D[m = 4 * (l / 16) + i][n = l % 16]      (i = 0..3)
// (checked on gfx950 hardware against a host matmul).

// Row of the 32x32 accumulator held in register r by lane half `hi`.
__device__ __forceinline__ int acc_row(int r, int hi) { return 8 * (r >> 2) + 4 * hi + (r & 3); }

__device__ __forceinline__ bf16x8 ld_bf16x8(const bf16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}
__device__ __forceinline__ void st_bf16x8(bf16_t* p, bf16x8 v) { *reinterpret_cast<bf16x8*>(p) = v; }
__device__ __forceinline__ void st_bf16x4(bf16_t* p, bf16x4 v) { *reinterpret_cast<bf16x4*>(p) = v; }

__device__ __forceinline__ bf16x8 zero_bf16x8() {
  bf16x8 z;
#pragma unroll
  for (int t = 0; t < 8; ++t) z[t] = (bf16_t)0.0f;
  return z;
}

// float -> bf16, round to nearest even (the compiler's fptrunc lowers to the
// hardware RNE conversion on gfx950).
__device__ __forceinline__ bf16_t to_bf16(float f) { return (bf16_t)f; }

// Element types of the cache, prepared queries and probabilities.  Both are
// 2-byte types fed to 32x32x16 or 16x16x32 MFMA with fp32 accumulation; the
// operand lane layouts are the same for both.
template <typename E>
struct Elem;

template <>
struct Elem<bf16_t> {
  typedef bf16x8 v8;
  typedef bf16x4 v4;
  static __device__ __forceinline__ f32x16 mfma(v8 a, v8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mfma16(v8 a, v8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ bf16_t from(float f) { return (bf16_t)f; }
};

template <>
struct Elem<f16_t> {
  typedef f16x8 v8;
  typedef f16x4 v4;
  static __device__ __forceinline__ f32x16 mfma(v8 a, v8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mfma16(v8 a, v8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f16_t from(float f) { return (f16_t)f; }
};

template <typename E>
__device__ __forceinline__ typename Elem<E>::v8 ld8(const E* p) {
  return *reinterpret_cast<const typename Elem<E>::v8*>(p);
}
template <typename E>
__device__ __forceinline__ typename Elem<E>::v8 zero8() {
  typename Elem<E>::v8 z;
#pragma unroll
  for (int t = 0; t < 8; ++t) z[t] = (E)0.0f;
  return z;
}

// OCP 8-bit float E4M3 ('fn' variant: exponent bias 7, no infinities, largest
// finite magnitude 448, smallest normal 2^-6, subnormal quantum 2^-9): the
// one-byte cache scalar.  Storage only: the attention core widens it to fp16,
// which holds every E4M3 value exactly.
struct e4m3_t {
  uint8_t bits;
};

// float -> E4M3 code, round to nearest even, saturating: magnitudes that
// round past 448 (infinities included) store 448; NaN stores the NaN code.
// Below 2^-6 a value is a multiple of 2^-9, so the code is rint(|f| * 2^9)
// (0 .. 8; 8 is the smallest normal's code).  Above, the code is the float's
// exponent and top three fraction bits, rounded half to even at bit 20 and
// rebased from exponent bias 127 to 7.
__device__ __forceinline__ uint32_t e4m3_code(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t mag = u & 0x7fffffffu;
  uint32_t m;
  if (mag >= 0x43e00000u)                          // 448.0f
    m = mag > 0x7f800000u ? 0x7fu : 0x7eu;
  else if (mag < 0x3c800000u)                      // 2^-6
    m = (uint32_t)__builtin_rintf(__uint_as_float(mag) * 512.0f);
  else
    m = ((mag + 0x7ffffu + ((mag >> 20) & 1u)) >> 20) - (120u << 3);
  return sign | m;
}

// Four floats -> four E4M3 codes, element i in byte i.
__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c, float d) {
  return e4m3_code(a) | (e4m3_code(b) << 8) | (e4m3_code(c) << 16) | (e4m3_code(d) << 24);
}

// Eight E4M3 codes (byte i of w0 = element i, byte i of w1 = element 4 + i) ->
// fp16, with gfx950's conversion instruction (unit scale: exact).
__device__ __forceinline__ f16x8 e4m3x8_to_f16(uint32_t w0, uint32_t w1) {
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  const f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, false);
  const f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, true);
  const f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, false);
  const f16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, true);
  f16x8 r = {a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  return r;
}

// 2^x on the hardware exponential unit (v_exp_f32) without the library's
// denormal-range fix-up: results below 2^-126 flush to zero, which softmax
// weights tolerate (they are summed against a maximum weight of at least 1).
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Position (frame, row, column) of global token g.
struct TokPos {
  int64_t f;
  int y, x;
};
__device__ __forceinline__ TokPos token_pos(int64_t g, int T, int grid_w) {
  TokPos p;
  p.f = g / T;
  int tau = (int)(g - p.f * T);
  p.y = tau / grid_w;
  p.x = tau - p.y * grid_w;
  return p;
}

__device__ __forceinline__ double pos_axis(const TokPos& p, int axis) {
  return axis == 0 ? (double)p.f : (axis == 1 ? (double)p.y : (double)p.x);
}

// cos and sin of an angle given in double: the angle is reduced to [-pi, pi]
// in double (exact to ~1e-16 for any frame index), then evaluated in fp32.
__device__ __forceinline__ void rope_cos_sin(double ang, float& c, float& s) {
  const double two_pi = 6.283185307179586476925286766559;
  const double k = rint(ang * (1.0 / two_pi));
  const float r = (float)fma(-k, two_pi, ang);
  sincosf(r, &s, &c);
}

// Rotate the pair (a, b) of rotary pair `pair` at position p.
__device__ __forceinline__ void rope_pair(const RopeTable& rt, int pair, const TokPos& p, float& a,
                                          float& b) {
  float c, s;
  rope_cos_sin(pos_axis(p, rt.axis[pair]) * rt.inv_freq[pair], c, s);
  const float ra = a * c - b * s;
  const float rb = a * s + b * c;
  a = ra;
  b = rb;
}

}  // namespace mla
