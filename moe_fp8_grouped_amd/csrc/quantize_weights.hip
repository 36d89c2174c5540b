// moe_quantize_weights / moe_quantize_weights_i8: offline blockwise absmax
// quantization of expert weights to e4m3fn (or int8) with [E, kb, 1, nb]
// scales ("Keep qwix out of tpu-inference's fused MoE kernel and pre-quantize
// weights", "Changes in this PR": either code type is allowed).  Setup-time
// work, run once per weight; the output can be laid out [E, K, N] or, for the
// matmul's preferred operand layout, [E, N, K].  The scale is amax / 448
// (e4m3fn) or amax / 127 (int8, symmetric codes).
#include "common.hpp"

namespace moe {
namespace {

// Per-output-channel case (block = bk rows x 1 column): one thread per
// (e, b, column), columns contiguous across threads so loads coalesce.
__global__ __launch_bounds__(256) void colmax_scale_kernel(const uint16_t* __restrict__ w, int64_t E,
                                                           int64_t K, int64_t N, int kb, int nb, float qmax,
                                                           float* __restrict__ scale) {
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t total = E * kb * N;
  if (gid >= total) return;
  const int64_t n = gid % N;
  const int64_t b = (gid / N) % kb;
  const int64_t e = gid / (N * kb);
  const int64_t bk = K / kb;
  const uint16_t* p = w + (e * K + b * bk) * N + n;
  float m = 0.0f;
  for (int64_t k = 0; k < bk; ++k) m = fmaxf(m, fabsf(bf16_to_f32(p[k * N])));
  scale[(e * kb + b) * nb + n] = m == 0.0f ? 1.0f : m / qmax;
}

// General blocks (bn > 1 columns): one workgroup per (e, b, c) block.
__global__ __launch_bounds__(256) void blockmax_scale_kernel(const uint16_t* __restrict__ w, int64_t K,
                                                             int64_t N, int kb, int nb, float qmax,
                                                             float* __restrict__ scale) {
  __shared__ float red[4];
  const int64_t blk = blockIdx.x;
  const int64_t c = blk % nb, b = (blk / nb) % kb, e = blk / (static_cast<int64_t>(nb) * kb);
  const int64_t bk = K / kb, bn = N / nb;
  float m = 0.0f;
  for (int64_t i = threadIdx.x; i < bk * bn; i += 256) {
    const int64_t r = i / bn, col = i % bn;
    m = fmaxf(m, fabsf(bf16_to_f32(w[(e * K + b * bk + r) * N + c * bn + col])));
  }
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    scale[blk] = m == 0.0f ? 1.0f : m / qmax;
  }
}

__global__ __launch_bounds__(256) void fill_kernel(float* __restrict__ p, int64_t n, float v) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < n) p[i] = v;
}

// Quantize a 64 x 64 tile (rows k, columns n) of one expert, writing either
// the same layout or the transposed one (through LDS, so both the read and
// the write are coalesced).  Grid: (N/64, K/64, E), 256 threads.
template <bool TRANSPOSE, bool I8>
__global__ __launch_bounds__(256) void quantize_tile_kernel(const uint16_t* __restrict__ w, int64_t K,
                                                            int64_t N, int kb, int nb,
                                                            const float* __restrict__ scale,
                                                            uint8_t* __restrict__ q) {
  __shared__ uint8_t tile[64][64 + 4];
  const int64_t e = blockIdx.z, k0 = static_cast<int64_t>(blockIdx.y) * 64, n0 = static_cast<int64_t>(blockIdx.x) * 64;
  const int64_t bk = K / kb, bn = N / nb;
  const float* sc = scale + e * kb * nb;
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int r = i / 64, c = i % 64;
    const int64_t k = k0 + r, n = n0 + c;
    uint32_t code = 0;
    if (k < K && n < N) {
      const float s = sc[(k / bk) * nb + n / bn];
      const float x = bf16_to_f32(w[(e * K + k) * N + n]);
      code = I8 ? quantize_one_i8(x, s) : quantize_one(x, s);
    }
    if (TRANSPOSE)
      tile[r][c] = static_cast<uint8_t>(code);
    else if (k < K && n < N)
      q[(e * K + k) * N + n] = static_cast<uint8_t>(code);
  }
  if (TRANSPOSE) {
    __syncthreads();
    for (int i = threadIdx.x; i < 64 * 64; i += 256) {
      const int c = i / 64, r = i % 64;     // output row = n, column = k
      const int64_t k = k0 + r, n = n0 + c;
      if (k < K && n < N) q[(e * N + n) * K + k] = tile[r][c];
    }
  }
}

}  // namespace
}  // namespace moe

namespace moe {
namespace {
int quantize_weights_entry(bool i8, const void* w, int64_t E, int64_t K, int64_t N, int32_t kb, int32_t nb,
                           int scale_mode, float static_scale, int transpose_out, uint8_t* q, float* scale,
                           void* stream) {
  if (E < 0 || K <= 0 || N <= 0 || K % 16 || N % 16) return MOE_ERR_SHAPE;
  if (kb <= 0 || nb <= 0 || K % kb || N % nb) return MOE_ERR_SHAPE;
  if (scale_mode != MOE_SCALE_ROW_DYNAMIC && scale_mode != MOE_SCALE_TENSOR_STATIC) return MOE_ERR_UNSUPPORTED;
  if (scale_mode == MOE_SCALE_TENSOR_STATIC && !(static_scale > 0.0f && static_scale < 3.0e38f))
    return MOE_ERR_SHAPE;
  if (transpose_out != 0 && transpose_out != 1) return MOE_ERR_UNSUPPORTED;
  if (E == 0) return MOE_OK;
  if (!w || !q || !scale) return MOE_ERR_NULL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const uint16_t* wb = static_cast<const uint16_t*>(w);
  const int64_t nscale = E * kb * nb;
  const float qmax = i8 ? 127.0f : 448.0f;
  if (scale_mode == MOE_SCALE_TENSOR_STATIC) {
    fill_kernel<<<static_cast<unsigned>(moe_cdiv(nscale, 256)), 256, 0, st>>>(scale, nscale, static_scale);
  } else if (nb == N) {
    colmax_scale_kernel<<<static_cast<unsigned>(moe_cdiv(E * kb * N, 256)), 256, 0, st>>>(wb, E, K, N, kb, nb, qmax,
                                                                                       scale);
  } else {
    blockmax_scale_kernel<<<static_cast<unsigned>(nscale), 256, 0, st>>>(wb, K, N, kb, nb, qmax, scale);
  }
  MOE_CHECK_LAUNCH();
  const dim3 grid(static_cast<unsigned>(moe_cdiv(N, 64)), static_cast<unsigned>(moe_cdiv(K, 64)),
                  static_cast<unsigned>(E));
  if (transpose_out)
    i8 ? quantize_tile_kernel<true, true><<<grid, 256, 0, st>>>(wb, K, N, kb, nb, scale, q)
       : quantize_tile_kernel<true, false><<<grid, 256, 0, st>>>(wb, K, N, kb, nb, scale, q);
  else
    i8 ? quantize_tile_kernel<false, true><<<grid, 256, 0, st>>>(wb, K, N, kb, nb, scale, q)
       : quantize_tile_kernel<false, false><<<grid, 256, 0, st>>>(wb, K, N, kb, nb, scale, q);
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}
}  // namespace
}  // namespace moe

extern "C" int moe_quantize_weights(const void* w, int64_t E, int64_t K, int64_t N, int32_t kb,
                                    int32_t nb, int scale_mode, float static_scale, int transpose_out,
                                    uint8_t* q, float* scale, void* stream) {
  return moe::quantize_weights_entry(false, w, E, K, N, kb, nb, scale_mode, static_scale, transpose_out, q, scale,
                                     stream);
}

extern "C" int moe_quantize_weights_i8(const void* w, int64_t E, int64_t K, int64_t N, int32_t kb,
                                       int32_t nb, int scale_mode, float static_scale, int transpose_out,
                                       int8_t* q, float* scale, void* stream) {
  return moe::quantize_weights_entry(true, w, E, K, N, kb, nb, scale_mode, static_scale, transpose_out,
                                     reinterpret_cast<uint8_t*>(q), scale, stream);
}
