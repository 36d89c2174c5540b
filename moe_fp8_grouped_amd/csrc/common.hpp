// Shared device helpers of libmoefp8: number formats, wave reductions and
// the launch plumbing.  gfx950 (CDNA4) only: wave64, fp8 = OCP e4m3fn.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe_fp8.h"

#define MOE_WAVE 64

namespace moe {

// ---------------------------------------------------------------- bfloat16
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// float32 -> bfloat16, round to nearest, ties to even; NaN stays a quiet NaN.
// Branch-free (a select, not a divergent branch, handles NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  const uint32_t b = __float_as_uint(f);
  const uint32_t rounded = (b + 0x7fffu + ((b >> 16) & 1u)) >> 16;
  const uint32_t quiet = (b >> 16) | 0x0040u;
  return static_cast<uint16_t>((b & 0x7fffffffu) > 0x7f800000u ? quiet : rounded);
}

// ---------------------------------------------------------------- e4m3fn
// Encode a finite float already clipped to [-448, 448] as OCP e4m3fn,
// rounding to nearest, ties to even, keeping the sign of zero.
//  * |v| >= 2^-6 (normal e4m3): keep the float32 exponent and round the
//    23-bit mantissa to 3 bits on the bit pattern (adding 0x7ffff plus the
//    kept LSB rounds half to even; a carry ripples into the exponent), then
//    rebias the exponent from 127 to 7.
//  * |v| < 2^-6 (subnormal e4m3, spacing 2^-9): scale by 2^9 (exact) and
//    round to an integer 0..8 with the hardware round-half-even; 8 is the
//    code of 2^-6, the smallest normal, so the encoding stays continuous.
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
  const uint32_t b = __float_as_uint(v);
  const uint32_t sign = (b >> 24) & 0x80u;
  const uint32_t a = b & 0x7fffffffu;
  uint32_t code;
  if (a >= 0x3c800000u) {
    const uint32_t r = a + 0x7ffffu + ((a >> 20) & 1u);
    code = (r >> 20) - (120u << 3);
  } else {
    code = static_cast<uint32_t>(__builtin_rintf(__uint_as_float(a) * 512.0f));
  }
  return sign | code;
}

// x / s, clipped to the e4m3 range, encoded.  The divide is the IEEE
// correctly rounded float32 division (this library is built without fast
// math).
__device__ __forceinline__ uint32_t quantize_one(float x, float s) {
  float v = x / s;
  v = fminf(fmaxf(v, -448.0f), 448.0f);
  return e4m3_encode(v);
}

// x / s rounded to the nearest integer (ties to even) and saturated to the
// symmetric int8 range [-127, 127]; the quotient is the IEEE float32 divide.
// Returns the code's byte.
__device__ __forceinline__ uint32_t quantize_one_i8(float x, float s) {
  float v = __builtin_rintf(x / s);
  v = fminf(fmaxf(v, -127.0f), 127.0f);
  return static_cast<uint32_t>(static_cast<int>(v)) & 0xffu;
}

// ---------------------------------------------------------------- pinned exp
// float32 exp by Cody & Waite's two-constant argument reduction and the
// degree-7 Taylor polynomial of exp(r) in Horner form, every multiply and add
// rounded on its own (contraction into FMA is disabled here).  The input is
// clamped to [-87, 88] so the result is a finite normal float.
//   C1 = ln 2 cut to 16 significant bits   = 0x3f317200
//   C2 = float32(ln 2 - C1)                = 0x35bfbe8e
//   log2(e) as float32                     = 0x3fb8aa3b
//   coefficients float32(1/i!), i = 0..7
__device__ __forceinline__ float pinned_exp(float x) {
#pragma clang fp contract(off)
  x = fminf(fmaxf(x, -87.0f), 88.0f);
  const float n = __builtin_rintf(x * __uint_as_float(0x3fb8aa3bu));
  const float r = (x - n * __uint_as_float(0x3f317200u)) - n * __uint_as_float(0x35bfbe8eu);
  const float c7 = 1.0f / 5040.0f, c6 = 1.0f / 720.0f, c5 = 1.0f / 120.0f, c4 = 1.0f / 24.0f;
  const float c3 = 1.0f / 6.0f, c2 = 0.5f, c1 = 1.0f, c0 = 1.0f;
  float p = c7;
  p = p * r + c6;
  p = p * r + c5;
  p = p * r + c4;
  p = p * r + c3;
  p = p * r + c2;
  p = p * r + c1;
  p = p * r + c0;
  return ldexpf(p, static_cast<int>(n));
}

// The correctly rounded quotient a / d for d = 1 + e(-a) with d <= 2^126
// (so 1/d is a normal float; a a finite bfloat16 value): a reciprocal
// estimate, one Newton step y = y0 + y0 (1 - d y0), then Markstein's
// correction q = q0 + y (a - d q0) with q0 = a y.  Equal to the IEEE
// float32 quotient for every such a (checked on the device over all finite
// bfloat16 values); a zero quotient keeps the sign of a.
__device__ __forceinline__ float silu_quotient(float a, float d) {
  const float y0 = __builtin_amdgcn_rcpf(d);
  const float y = fmaf(fmaf(-d, y0, 1.0f), y0, y0);
  const float q0 = a * y;
  const float q = fmaf(fmaf(-d, q0, a), y, q0);
  return q0 == 0.0f ? q0 : q;
}

// h[i] = f32(silu(a[i]) * b[i]), silu(a) = f32(a / f32(1 + e(-a))), for eight
// values.  One branch for the group: the reciprocal path unless some
// denominator exceeds 2^126 (gates below about -87.3), then the IEEE divide.
__device__ __forceinline__ void silu_mul8(const float a[8], const float b[8], float h[8]) {
#pragma clang fp contract(off)
  float den[8];
  float dmax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    den[i] = 1.0f + pinned_exp(-a[i]);
    dmax = fmaxf(dmax, den[i]);
  }
  if (dmax <= 0x1p126f) {
#pragma unroll
    for (int i = 0; i < 8; ++i) h[i] = silu_quotient(a[i], den[i]) * b[i];
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) h[i] = (a[i] / den[i]) * b[i];
  }
}

// ---------------------------------------------------------------- reductions
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, MOE_WAVE));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, MOE_WAVE);
  return v;
}

// Sticky device-error word: OR a bit into the first int32 of a workspace.
__device__ __forceinline__ void raise_error(int32_t* err, int32_t bit) {
  if (err) atomicOr(err, bit);
}

}  // namespace moe

// ---------------------------------------------------------------- host side
#define MOE_CHECK_LAUNCH()                                   \
  do {                                                       \
    if (hipGetLastError() != hipSuccess) return MOE_ERR_HIP; \
  } while (0)

static inline int64_t moe_cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
