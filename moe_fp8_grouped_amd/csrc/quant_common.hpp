// Row quantization pieces shared by the row quantizer and the fused
// quantize-and-scatter of the sort: the bf16 unpacking, the correctly rounded
// division by a row scale and the e4m3fn encoding of eight values.  Both
// kernels use these functions, so they produce the same bytes.
#pragma once

#include "common.hpp"

namespace moe {

struct Bf16x8 {
  uint4 raw;
  __device__ __forceinline__ float get(int i) const {
    const uint32_t w = (&raw.x)[i >> 1];
    return (i & 1) ? __uint_as_float(w & 0xffff0000u) : __uint_as_float(w << 16);
  }
};

// x / s for one row's scale s, correctly rounded.  For s in [2^-64, 2^64]
// the quotient comes from the row's reciprocal y = RN(1/s) and one
// correction, q = RN(q0 + RN(x - s*q0) * y) with q0 = RN(x*y): Markstein's
// theorem (a correctly rounded reciprocal and a quotient within one ulp give
// the correctly rounded quotient after one FMA correction), which needs the
// residual x - s*q0 to be exact -- true in this range for every quotient of
// magnitude at least 2^-10, and smaller ones encode to a signed zero either
// way.  Zeros keep their sign and infinities or NaN pass through; other
// scales use the division.
struct RowDiv {
  float s, y;
  bool fast;
  __device__ __forceinline__ explicit RowDiv(float s_) : s(s_), y(1.0f / s_),
      fast(s_ >= 0x1p-64f && s_ <= 0x1p64f) {}
  __device__ __forceinline__ float quick(float x) const {
    const float q0 = x * y;
    const float r = fmaf(-s, q0, x);
    const float q = fmaf(r, y, q0);
    return (q0 == 0.0f || !(fabsf(q0) <= 3.0e38f)) ? q0 : q;
  }
};

// Eight values to e4m3fn codes: clip to [-448, 448], then the gfx950 fp8
// conversion (round to nearest even; on this clipped range it is the
// encoder in common.hpp, bit for bit).  The division takes one branch for
// all eight values (a select per value would compute both quotients).
__device__ __forceinline__ uint2 codes8(const float v[8], const RowDiv& d) {
  float c[8];
  if (d.fast) {
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = d.quick(v[i]);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = v[i] / d.s;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) c[i] = fminf(fmaxf(c[i], -448.0f), 448.0f);
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(c[0], c[1], 0, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(c[2], c[3], lo, true);
  int hi = __builtin_amdgcn_cvt_pk_fp8_f32(c[4], c[5], 0, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(c[6], c[7], hi, true);
  return make_uint2(static_cast<uint32_t>(lo), static_cast<uint32_t>(hi));
}

__device__ __forceinline__ void store_codes(uint8_t* __restrict__ q, int64_t off, const float v[8], const RowDiv& d) {
  *reinterpret_cast<uint2*>(q + off) = codes8(v, d);
}

__device__ __forceinline__ float scale_from_amax(float amax) {
  return amax == 0.0f ? 1.0f : amax / 448.0f;
}

namespace {
// The tensor scale from caller-given row maxima (MOE_SCALE_TENSOR_FROM_ROW_AMAX):
// one workgroup of 16 waves, eight independent loads per thread and round,
// then a wave and an LDS reduction (max is exact in any order).
__global__ __launch_bounds__(1024) void amax_scale_kernel(const float* __restrict__ v, int64_t n,
                                                          float* __restrict__ scale) {
  __shared__ float red[16];
  float m = 0.0f;
  for (int64_t i = threadIdx.x; i < n; i += 1024 * 8) {
    float t[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t j = i + 1024 * u;
      t[u] = j < n ? v[j] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) m = fmaxf(m, t[u]);
  }
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float r = red[0];
    for (int w = 1; w < 16; ++w) r = fmaxf(r, red[w]);
    *scale = scale_from_amax(r);
  }
}

}  // namespace

}  // namespace moe
