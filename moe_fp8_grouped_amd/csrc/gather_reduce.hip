// moe_gather_reduce: un-sort plus top-k weighted combine ("Quantize
// activations before EP all gather", review comments on
// ragged_gather_reduce_v2.py: reduce the sorted expert outputs back to token
// rows over the valid rows; bf16 output when the dtype is unset or fp8).
//
// One wave per token row: the lanes read the token's k slot entries
// (inverse position, router weight), then sweep the row in 16-byte chunks,
// loading the k expert-output rows and accumulating in float32 in slot order.
// HBM-bound: reads n*N*2 (each sorted row once) + T*k*8, writes T*N*2 bytes.
#include "quant_common.hpp"

namespace moe {
namespace {

// Weighted sum of 8 values (one 16-byte chunk of a y row) into acc.
template <int YBF16>
__device__ __forceinline__ void fma_chunk(float acc[8], float wj, const uint4 lo, const uint4 hi) {
  if (YBF16) {
    const uint32_t wv[4] = {lo.x, lo.y, lo.z, lo.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] = fmaf(wj, __uint_as_float(wv[i] << 16), acc[2 * i]);
      acc[2 * i + 1] = fmaf(wj, __uint_as_float(wv[i] & 0xffff0000u), acc[2 * i + 1]);
    }
  } else {
    const float v[8] = {__uint_as_float(lo.x), __uint_as_float(lo.y), __uint_as_float(lo.z), __uint_as_float(lo.w),
                        __uint_as_float(hi.x), __uint_as_float(hi.y), __uint_as_float(hi.z), __uint_as_float(hi.w)};
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = fmaf(wj, v[i], acc[i]);
  }
}

template <int OBF16>
__device__ __forceinline__ void store_chunk(void* __restrict__ out, int64_t t, int64_t N, int64_t ch, const float acc[8]) {
  if (OBF16) {
    uint4 o;
    o.x = f32_to_bf16(acc[0]) | (static_cast<uint32_t>(f32_to_bf16(acc[1])) << 16);
    o.y = f32_to_bf16(acc[2]) | (static_cast<uint32_t>(f32_to_bf16(acc[3])) << 16);
    o.z = f32_to_bf16(acc[4]) | (static_cast<uint32_t>(f32_to_bf16(acc[5])) << 16);
    o.w = f32_to_bf16(acc[6]) | (static_cast<uint32_t>(f32_to_bf16(acc[7])) << 16);
    reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + t * N)[ch] = o;
  } else {
    float4* p = reinterpret_cast<float4*>(static_cast<float*>(out) + t * N) + 2 * ch;
    p[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    p[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
  }
}

// k <= 8: every slot's row chunk for two chunks per lane is loaded before any
// is summed (16 loads in flight per lane), then summed in slot order.
template <int YBF16, int OBF16>
__global__ __launch_bounds__(256) void gather_reduce_k8_kernel(const void* __restrict__ y,
                                                               const int32_t* __restrict__ inv,
                                                               const float* __restrict__ wts, int64_t T, int k,
                                                               int64_t N, void* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  int my_r = -1;
  float my_w = 0.0f;
  if (lane < k) {
    my_r = inv[t * k + lane];
    my_w = wts[t * k + lane];
  }
  const uint64_t m = __ballot(my_r >= 0);
  int r[8];
  float w[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    r[j] = __builtin_amdgcn_readlane(my_r, j);
    w[j] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_w), j));
  }
  const int64_t chunks = N >> 3;            // 8 elements per chunk
  const int64_t rowb = YBF16 ? N * 2 : N * 4;
  const uint8_t* yb = static_cast<const uint8_t*>(y);
  for (int64_t c0 = lane; c0 < chunks; c0 += 128) {
    const int64_t c1 = c0 + 64;
    const bool two = c1 < chunks;
    uint4 lo[2][8], hi[2][8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if ((m >> j) & 1ull) {                // uniform across the wave
        const uint8_t* row = yb + static_cast<int64_t>(r[j]) * rowb;
        if (YBF16) {
          lo[0][j] = reinterpret_cast<const uint4*>(row)[c0];
          if (two) lo[1][j] = reinterpret_cast<const uint4*>(row)[c1];
        } else {
          lo[0][j] = reinterpret_cast<const uint4*>(row)[2 * c0];
          hi[0][j] = reinterpret_cast<const uint4*>(row)[2 * c0 + 1];
          if (two) {
            lo[1][j] = reinterpret_cast<const uint4*>(row)[2 * c1];
            hi[1][j] = reinterpret_cast<const uint4*>(row)[2 * c1 + 1];
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if (u == 1 && !two) break;
      float acc[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j)            // slot order
        if ((m >> j) & 1ull) fma_chunk<YBF16>(acc, w[j], lo[u][j], hi[u][j]);
      store_chunk<OBF16>(out, t, N, u ? c1 : c0, acc);
    }
  }
}

template <int YBF16, int OBF16>
__global__ __launch_bounds__(256) void gather_reduce_kernel(const void* __restrict__ y, const int32_t* __restrict__ inv,
                                                            const float* __restrict__ wts, int64_t T, int k,
                                                            int64_t N, void* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  int my_r = -1;
  float my_w = 0.0f;
  if (lane < k) {
    my_r = inv[t * k + lane];
    my_w = wts[t * k + lane];
  }
  const uint64_t m = __ballot(my_r >= 0);
  const int64_t chunks = N >> 3;            // 8 elements per chunk
  for (int64_t ch = lane; ch < chunks; ch += 64) {
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
    for (int j = 0; j < k; ++j) {            // slot order, uniform across the wave
      if (!((m >> j) & 1ull)) continue;
      const int r = __builtin_amdgcn_readlane(my_r, j);
      const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_w), j));
      if (YBF16) {
        const uint4 v = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(y) + static_cast<int64_t>(r) * N)[ch];
        const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] = fmaf(wj, __uint_as_float(wv[i] << 16), acc[2 * i]);
          acc[2 * i + 1] = fmaf(wj, __uint_as_float(wv[i] & 0xffff0000u), acc[2 * i + 1]);
        }
      } else {
        const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(y) + static_cast<int64_t>(r) * N) + 2 * ch;
        const float4 a = p[0], b = p[1];
        const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = fmaf(wj, v[i], acc[i]);
      }
    }
    if (OBF16) {
      uint4 o;
      o.x = f32_to_bf16(acc[0]) | (static_cast<uint32_t>(f32_to_bf16(acc[1])) << 16);
      o.y = f32_to_bf16(acc[2]) | (static_cast<uint32_t>(f32_to_bf16(acc[3])) << 16);
      o.z = f32_to_bf16(acc[4]) | (static_cast<uint32_t>(f32_to_bf16(acc[5])) << 16);
      o.w = f32_to_bf16(acc[6]) | (static_cast<uint32_t>(f32_to_bf16(acc[7])) << 16);
      reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + t * N)[ch] = o;
    } else {
      float4* p = reinterpret_cast<float4*>(static_cast<float*>(out) + t * N) + 2 * ch;
      p[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
      p[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
    }
  }
}

// ---------------------------------------------------------------- backward
// One 16-byte chunk of the backward: dy = bf16(w * d) for its eight values
// (one float32 product, one rounding) and the chunk's share of dout . y as an
// FMA chain.
__device__ __forceinline__ float bwd_chunk(const uint4 d, const uint4 yv, float w, uint4& out) {
  const uint32_t dd[4] = {d.x, d.y, d.z, d.w}, yy[4] = {yv.x, yv.y, yv.z, yv.w};
  uint32_t o[4];
  float p = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float d0 = __uint_as_float(dd[i] << 16), d1 = __uint_as_float(dd[i] & 0xffff0000u);
    const float y0 = __uint_as_float(yy[i] << 16), y1 = __uint_as_float(yy[i] & 0xffff0000u);
    p = fmaf(d0, y0, p);
    p = fmaf(d1, y1, p);
    o[i] = f32_to_bf16(w * d0) | (static_cast<uint32_t>(f32_to_bf16(w * d1)) << 16);
  }
  out = make_uint4(o[0], o[1], o[2], o[3]);
  return p;
}

// The combine's backward, one wave per routed slot f = t*k + j: the token's
// upstream-gradient row and the slot's expert-output row are loaded together
// (CPL 16-byte chunks per lane, index clamped into the row; CPL = 0 streams
// longer rows), dy[r] = bf16(w * dout[t]) is written to the slot's sorted row
// r, and dw[f] = dout[t] . y[r] is summed in float32 -- eight-term FMA chains
// per chunk, the chunks of a lane, then a wave tree: at most
// (8 + chunks per lane + 6) float32 roundings deep.  A token's k waves are
// neighbours, so its dout row comes from HBM once.  Slots without a local row
// get dw = 0; extra waves zero dy's rows [n, M_cap), n = the local rows.
// QUANT (CPL > 0 only): the wave holds the whole dy row, so it also writes the
// row's e4m3fn codes, scale and absmax with the row quantizer's own functions
// (the bytes moe_quantize_rows gives for dy in row mode); zero rows get codes
// 0, scale 1 and absmax 0.
template <int CPL, bool QUANT>
__global__ __launch_bounds__(256) void gather_reduce_bwd_kernel(
    const uint16_t* __restrict__ dout, const uint16_t* __restrict__ y, const int32_t* __restrict__ inv,
    const float* __restrict__ wts, int64_t S, int k, int64_t N, int64_t M_cap, const int32_t* __restrict__ gs,
    int g0, int El, uint16_t* __restrict__ dy, float* __restrict__ dw, uint8_t* __restrict__ dyq,
    float* __restrict__ dys, float* __restrict__ dyamax) {
  static_assert(!QUANT || CPL > 0, "row quantization keeps the row in registers");
  const int lane = threadIdx.x & 63;
  const int64_t nw = static_cast<int64_t>(gridDim.x) * 4;
  const int64_t wid = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int64_t nch = N >> 3;
  for (int64_t f = wid; f < S; f += nw) {
    int r = inv[f];
    const float w = wts[f];
    if (r >= M_cap) r = -1;
    if (r < 0) {
      if (lane == 0) dw[f] = 0.0f;
      continue;
    }
    const uint4* drow = reinterpret_cast<const uint4*>(dout + (f / k) * N);
    const uint4* yrow = reinterpret_cast<const uint4*>(y + static_cast<int64_t>(r) * N);
    uint4* dyrow = reinterpret_cast<uint4*>(dy + static_cast<int64_t>(r) * N);
    float part = 0.0f;
    if constexpr (CPL > 0) {
      uint4 dv[CPL], yv[CPL], ov[CPL];
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const int64_t ch = lane + 64 * c;
        const int64_t cl = ch < nch ? ch : nch - 1;
        dv[c] = drow[cl];
        yv[c] = yrow[cl];
      }
      float amax = 0.0f;
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const int64_t ch = lane + 64 * c;
        if (ch < nch) {
          part += bwd_chunk(dv[c], yv[c], w, ov[c]);
          dyrow[ch] = ov[c];
          if constexpr (QUANT) {
            Bf16x8 o;
            o.raw = ov[c];
#pragma unroll
            for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(o.get(i)));
          }
        }
      }
      if constexpr (QUANT) {
        amax = wave_max(amax);
        const float sc = scale_from_amax(amax);
        const RowDiv div(sc);
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          const int64_t ch = lane + 64 * c;
          if (ch < nch) {
            Bf16x8 o;
            o.raw = ov[c];
            float v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = o.get(i);
            store_codes(dyq, static_cast<int64_t>(r) * N + ch * 8, v, div);
          }
        }
        if (lane == 0) {
          dys[r] = sc;
          dyamax[r] = amax;
        }
      }
    } else {
      for (int64_t ch = lane; ch < nch; ch += 64) {
        uint4 o;
        part += bwd_chunk(drow[ch], yrow[ch], w, o);
        dyrow[ch] = o;
      }
    }
    part = wave_sum(part);
    if (lane == 0) dw[f] = part;
  }
  // rows [n, M_cap) of dy are zero (n from the local group sizes; negative ones count as 0; summed in
  // 64 bits, so sizes adding up past 2^31 cannot wrap n below 0)
  int64_t own = 0;
  for (int g = lane; g < El; g += 64) own += max(gs[g0 + g], 0);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) own += __shfl_xor(own, o, 64);
  const int64_t n = own < M_cap ? own : M_cap;
  for (int64_t r = n + wid; r < M_cap; r += nw) {
    uint4* row = reinterpret_cast<uint4*>(dy + r * N);
    for (int64_t ch = lane; ch < nch; ch += 64) row[ch] = make_uint4(0, 0, 0, 0);
    if constexpr (QUANT) {
      uint2* qrow = reinterpret_cast<uint2*>(dyq + r * N);
      for (int64_t ch = lane; ch < nch; ch += 64) qrow[ch] = make_uint2(0, 0);
      if (lane == 0) {
        dys[r] = 1.0f;
        dyamax[r] = 0.0f;
      }
    }
  }
}

}  // namespace
}  // namespace moe

extern "C" int moe_gather_reduce(const void* y, int y_dtype, const int32_t* inv_pos, const float* topk_weights,
                                 int64_t T, int32_t k, int64_t N, int out_dtype, void* out, void* stream) {
  if (T < 0 || k <= 0 || k > 64 || N <= 0 || N % 8) return MOE_ERR_SHAPE;
  if (y_dtype != MOE_BF16 && y_dtype != MOE_F32) return MOE_ERR_UNSUPPORTED;
  if (out_dtype == MOE_DTYPE_DEFAULT || out_dtype == MOE_E4M3FN) out_dtype = MOE_BF16;
  if (out_dtype != MOE_BF16 && out_dtype != MOE_F32) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!y || !inv_pos || !topk_weights || !out) return MOE_ERR_NULL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 grid(static_cast<unsigned>(moe_cdiv(T, 4))), block(256);
  if (y_dtype == MOE_BF16 && out_dtype == MOE_BF16)
    k <= 8 ? moe::gather_reduce_k8_kernel<1, 1><<<grid, block, 0, st>>>(y, inv_pos, topk_weights, T, k, N, out)
           : moe::gather_reduce_kernel<1, 1><<<grid, block, 0, st>>>(y, inv_pos, topk_weights, T, k, N, out);
  else if (y_dtype == MOE_BF16)
    k <= 8 ? moe::gather_reduce_k8_kernel<1, 0><<<grid, block, 0, st>>>(y, inv_pos, topk_weights, T, k, N, out)
           : moe::gather_reduce_kernel<1, 0><<<grid, block, 0, st>>>(y, inv_pos, topk_weights, T, k, N, out);
  else if (out_dtype == MOE_BF16)
    k <= 8 ? moe::gather_reduce_k8_kernel<0, 1><<<grid, block, 0, st>>>(y, inv_pos, topk_weights, T, k, N, out)
           : moe::gather_reduce_kernel<0, 1><<<grid, block, 0, st>>>(y, inv_pos, topk_weights, T, k, N, out);
  else
    k <= 8 ? moe::gather_reduce_k8_kernel<0, 0><<<grid, block, 0, st>>>(y, inv_pos, topk_weights, T, k, N, out)
           : moe::gather_reduce_kernel<0, 0><<<grid, block, 0, st>>>(y, inv_pos, topk_weights, T, k, N, out);
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}

extern "C" int moe_gather_reduce_backward(const void* dout, const void* y, const int32_t* inv_pos,
                                          const float* topk_weights, int64_t T, int32_t k, int64_t N,
                                          const int32_t* group_sizes, int32_t E, int32_t group_offset,
                                          int32_t num_local_experts, int64_t M_cap, void* dy, float* dw,
                                          uint8_t* dy_q, float* dy_scale, float* dy_amax, void* stream) {
  if (T < 0 || k <= 0 || k > 64 || N <= 0 || N % 8 || M_cap < 0) return MOE_ERR_SHAPE;
  if (E <= 0 || E > 1024 || group_offset < 0 || num_local_experts < 0 || group_offset + num_local_experts > E)
    return MOE_ERR_SHAPE;
  if (T * k > INT32_MAX - 1) return MOE_ERR_SHAPE;
  if (T == 0 && M_cap == 0) return MOE_OK;
  if (!group_sizes) return MOE_ERR_NULL;
  if (T > 0 && (!dout || !inv_pos || !topk_weights || !dw)) return MOE_ERR_NULL;
  if (M_cap > 0 && (!y || !dy)) return MOE_ERR_NULL;
  const bool quant = dy_q != nullptr;
  if (quant && (!dy_scale || !dy_amax)) return MOE_ERR_NULL;
  if (quant && N / 8 > 16 * 64) return MOE_ERR_UNSUPPORTED;      // rows above 8192 elements
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t S = T * k;
  int64_t waves = S > M_cap / 4 ? S : M_cap / 4;
  if (waves < 4) waves = 4;
  if (waves > 262144) waves = 262144;
  const unsigned grid = static_cast<unsigned>(moe_cdiv(waves, 4));
  const int64_t cpl = moe_cdiv(N / 8, 64);
  const uint16_t* d = static_cast<const uint16_t*>(dout);
  const uint16_t* yy = static_cast<const uint16_t*>(y);
  uint16_t* o = static_cast<uint16_t*>(dy);
#define MOE_GRB(CPL, Q)                                                                                      \
  moe::gather_reduce_bwd_kernel<CPL, Q><<<grid, 256, 0, st>>>(d, yy, inv_pos, topk_weights, S, k, N, M_cap,  \
                                                                group_sizes, group_offset, num_local_experts, o, \
                                                                dw, dy_q, dy_scale, dy_amax)
#define MOE_GRB_Q(CPL) do { if (quant) MOE_GRB(CPL, true); else MOE_GRB(CPL, false); } while (0)
  if (cpl <= 1) MOE_GRB_Q(1);
  else if (cpl <= 2) MOE_GRB_Q(2);
  else if (cpl <= 4) MOE_GRB_Q(4);
  else if (cpl <= 8) MOE_GRB_Q(8);
  else if (cpl <= 16) MOE_GRB_Q(16);
  else MOE_GRB(0, false);
#undef MOE_GRB_Q
#undef MOE_GRB
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}
