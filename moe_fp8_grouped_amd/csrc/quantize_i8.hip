// moe_quantize_rows_i8: absmax quantization of activations to symmetric int8
// codes, the activation side of the int8 variant ("Keep qwix out of
// tpu-inference's fused MoE kernel and pre-quantize weights", "Changes in
// this PR": weights pre-quantized to e4m3fn or to int8; no matrix core
// multiplies fp8 by int8, so int8 weights pair with int8 activations).
// Per-token scales as in "Quantize activations before EP all gather" (the
// activations are quantized per token before the sort), or one tensor scale
// (static, from the whole tensor's absmax, or from caller-given row maxima).
//   s = f32(amax / 127) (1.0 for an all-zero row), q = clip(rint(f32(x / s)),
//   -127, 127) with IEEE float32 divides and ties to even.
// One wave per row: the row's absmax by 16-byte loads and a wave reduction,
// then its codes, eight per lane per 16-byte load, written as 8 bytes.
#include "common.hpp"

namespace moe {
namespace {

__device__ __forceinline__ void unpack8(const uint4 raw, float v[8]) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

// ROW: per-row scales (and optionally the rows' maxima); otherwise one scale
// read from tscale[0] (written before this kernel on the same stream).
// AMAX_ONLY: only the rows' maxima (the first pass of a dynamic tensor scale).
template <bool ROW, bool AMAX_ONLY = false>
__global__ __launch_bounds__(256) void quantize_rows_i8_kernel(const uint16_t* __restrict__ x, int64_t R, int64_t C,
                                                               const float* __restrict__ tscale,
                                                               uint8_t* __restrict__ q, float* __restrict__ scale,
                                                               float* __restrict__ row_amax) {
  const int lane = threadIdx.x & 63;
  const int64_t nw = static_cast<int64_t>(gridDim.x) * 4;
  const int64_t nch = C >> 3;                      // 16-byte chunks (8 values) per row
  for (int64_t r = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6); r < R; r += nw) {
    const uint4* row = reinterpret_cast<const uint4*>(x + r * C);
    float s;
    if (ROW) {
      float m = 0.0f;
      for (int64_t c = lane; c < nch; c += 64) {
        float v[8];
        unpack8(row[c], v);
#pragma unroll
        for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
      }
      m = wave_max(m);
      s = m == 0.0f ? 1.0f : m / 127.0f;
      if (lane == 0) {
        if (!AMAX_ONLY) scale[r] = s;
        if (row_amax) row_amax[r] = m;
      }
      if (AMAX_ONLY) continue;
    } else {
      s = tscale[0];
    }
    uint2* qrow = reinterpret_cast<uint2*>(q + r * C);
    for (int64_t c = lane; c < nch; c += 64) {
      float v[8];
      unpack8(row[c], v);
      uint32_t b[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) b[i] = quantize_one_i8(v[i], s);
      qrow[c] = make_uint2(b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24), b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24));
    }
  }
}

// scale[0] = a static value, or f32(max(row_amax) / 127) (1.0 when 0).
__global__ __launch_bounds__(1024) void tensor_scale_i8_kernel(const float* __restrict__ row_amax, int64_t n,
                                                               float static_scale, float* __restrict__ scale) {
  __shared__ float red[16];
  if (!row_amax) {
    if (threadIdx.x == 0) scale[0] = static_scale;
    return;
  }
  float m = 0.0f;
  for (int64_t i = threadIdx.x; i < n; i += 1024) m = fmaxf(m, row_amax[i]);
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float r = red[0];
    for (int w = 1; w < 16; ++w) r = fmaxf(r, red[w]);
    scale[0] = r == 0.0f ? 1.0f : r / 127.0f;
  }
}

}  // namespace
}  // namespace moe

extern "C" int moe_quantize_rows_i8(const void* x, int64_t R, int64_t C, int scale_mode, float static_scale,
                                    int8_t* q, float* scale, float* row_amax, void* stream) {
  if (R < 0 || C <= 0 || C % 16) return MOE_ERR_SHAPE;
  if (scale_mode != MOE_SCALE_ROW_DYNAMIC && scale_mode != MOE_SCALE_TENSOR_DYNAMIC &&
      scale_mode != MOE_SCALE_TENSOR_STATIC && scale_mode != MOE_SCALE_TENSOR_FROM_ROW_AMAX)
    return MOE_ERR_UNSUPPORTED;
  if (scale_mode == MOE_SCALE_TENSOR_STATIC && !(static_scale > 0.0f && static_scale < 3.0e38f)) return MOE_ERR_SHAPE;
  if (!scale) return MOE_ERR_NULL;
  if (R > 0 && (!x || !q)) return MOE_ERR_NULL;
  const bool needs_amax = scale_mode == MOE_SCALE_TENSOR_DYNAMIC || scale_mode == MOE_SCALE_TENSOR_FROM_ROW_AMAX;
  if (needs_amax && R > 0 && !row_amax) return MOE_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(x) % 16 != 0 || reinterpret_cast<uintptr_t>(q) % 8 != 0) return MOE_ERR_SHAPE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  uint8_t* qb = reinterpret_cast<uint8_t*>(q);
  int64_t blocks = moe_cdiv(R, 4);
  if (blocks > 65536) blocks = 65536;
  const unsigned g = static_cast<unsigned>(blocks);
  if (scale_mode == MOE_SCALE_TENSOR_DYNAMIC && R > 0) {      // the rows' maxima first, into row_amax
    moe::quantize_rows_i8_kernel<true, true><<<g, 256, 0, st>>>(xb, R, C, nullptr, qb, nullptr, row_amax);
    MOE_CHECK_LAUNCH();
  }
  if (scale_mode != MOE_SCALE_ROW_DYNAMIC) {
    moe::tensor_scale_i8_kernel<<<1, 1024, 0, st>>>(scale_mode == MOE_SCALE_TENSOR_STATIC ? nullptr : row_amax, R,
                                                    static_scale, scale);
    MOE_CHECK_LAUNCH();
  }
  if (R == 0) return MOE_OK;
  if (scale_mode == MOE_SCALE_ROW_DYNAMIC)
    moe::quantize_rows_i8_kernel<true><<<g, 256, 0, st>>>(xb, R, C, nullptr, qb, scale, row_amax);
  else
    moe::quantize_rows_i8_kernel<false><<<g, 256, 0, st>>>(xb, R, C, scale, qb, nullptr, nullptr);
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}
