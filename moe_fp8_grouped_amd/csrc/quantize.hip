// moe_quantize_rows: absmax quantization of bf16 activations to e4m3fn.
//
// Per-token dynamic absmax ("Quantize activations before EP all gather",
// description: quantize before the all-gather and the sort) and the fixed
// activation scale of fp8_static_wa ("Support quantization for tokamax gmm
// v2", tolerance discussion).  HBM-bound: 2 bytes read, 1 byte written per
// element (3 for the SiLU*mul variant), plus 4 bytes per row.
//
// Layout: one wave per row.  A lane owns 16-byte chunks (8 bf16) at chunk
// indices lane, lane + 64, ...; with CPL chunks per lane a row of up to
// CPL * 512 elements stays in registers between the absmax pass and the
// quantize pass, so each input byte is read once.  Longer rows use the
// streaming variant (CPL = 0), which reads the row twice (the second time
// from L2).
#include "quant_common.hpp"

namespace moe {
namespace {

template <int ACT>
__device__ __forceinline__ void load_vals(const uint16_t* __restrict__ x, const uint16_t* __restrict__ xu,
                                          int64_t off, float v[8]) {
  Bf16x8 a;
  a.raw = *reinterpret_cast<const uint4*>(x + off);
  if constexpr (ACT == MOE_ACT_SILU_MUL) {
    Bf16x8 b;
    b.raw = *reinterpret_cast<const uint4*>(xu + off);
    float av[8], bv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      av[i] = a.get(i);
      bv[i] = b.get(i);
    }
    silu_mul8(av, bv, v);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = a.get(i);
  }
}

// The raw 16-byte chunks lane + LPR * c of a row (x, and x_up for SiLU*mul),
// all loads issued before any is used; chunks past the row's end re-read its
// last chunk and are ignored by the caller.
template <int CPL, int ACT, int LPR>
__device__ __forceinline__ void load_row_share(const uint16_t* __restrict__ x, const uint16_t* __restrict__ xu,
                                               int64_t xbase, int64_t nchunks, int lane, Bf16x8 (&ra)[CPL],
                                               Bf16x8 (&rb)[CPL]) {
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int64_t ch = lane + LPR * c;
    const int64_t cl = ch < nchunks ? ch : nchunks - 1;
    ra[c].raw = *reinterpret_cast<const uint4*>(x + xbase + cl * 8);
    if constexpr (ACT == MOE_ACT_SILU_MUL) rb[c].raw = *reinterpret_cast<const uint4*>(xu + xbase + cl * 8);
  }
}

// Absolute maximum of one chunk's values; for SiLU*mul the values
// h = silu(a) * b are formed here and kept in h.
template <int ACT>
__device__ __forceinline__ float chunk_absmax(const Bf16x8& a, const Bf16x8& b, float (&h)[8]) {
  float m = 0.0f;
  if constexpr (ACT == MOE_ACT_SILU_MUL) {
    float av[8], bv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      av[i] = a.get(i);
      bv[i] = b.get(i);
    }
    silu_mul8(av, bv, h);
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(h[i]));
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(a.get(i)));
  }
  return m;
}

// The e4m3fn codes of one chunk (from h for SiLU*mul, else from the bf16 words).
template <int ACT>
__device__ __forceinline__ void store_chunk(uint8_t* __restrict__ q, int64_t off, const Bf16x8& a, const float (&h)[8],
                                            const RowDiv& div) {
  if constexpr (ACT == MOE_ACT_SILU_MUL) {
    store_codes(q, off, h, div);
  } else {
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = a.get(i);
    store_codes(q, off, v, div);
  }
}

// MODE_ROW: compute each row's scale; MODE_GIVEN: use *given_scale (tensor
// modes; computed by the first pass for the dynamic one).
constexpr int MODE_ROW = 0;
constexpr int MODE_GIVEN = 1;

// LPR lanes per row (64: one row per wave; 32: two rows per wave, for rows
// whose chunk count is an odd multiple of 32, e.g. 768 elements = 96 chunks).
template <int LPR>
__device__ __forceinline__ float row_max(float v) {
#pragma unroll
  for (int o = LPR / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, MOE_WAVE));
  return v;
}

template <int CPL, int ACT, int MODE, int LPR = 64>
__global__ __launch_bounds__(256) void quantize_rows_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ xu, int64_t R, int64_t C, int64_t ldx,
    const float* __restrict__ given_scale, uint8_t* __restrict__ q, float* __restrict__ scale,
    float* __restrict__ row_amax) {
  const int lane = threadIdx.x % LPR;
  const int64_t row = (static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6)) * (64 / LPR) + (threadIdx.x & 63) / LPR;
  if (row >= R) return;     // (a half-wave's partner rows never read this half's lanes)
  const int64_t nchunks = C >> 3;
  const int64_t base = row * C, xbase = row * ldx;
  float amax = 0.0f;
  if constexpr (CPL > 0) {
    // every load of the lane's share first (chunk index clamped into the
    // row), so one memory latency covers the whole share; the bf16 words
    // stay packed until used (the SiLU values are kept as float32)
    Bf16x8 ra[CPL], rb[CPL];
    load_row_share<CPL, ACT, LPR>(x, xu, xbase, nchunks, lane, ra, rb);
    float h[ACT == MOE_ACT_SILU_MUL ? CPL : 1][8];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      if (lane + LPR * c < nchunks) amax = fmaxf(amax, chunk_absmax<ACT>(ra[c], rb[c], h[ACT == MOE_ACT_SILU_MUL ? c : 0]));
    }
    amax = row_max<LPR>(amax);
    const float s = (MODE == MODE_ROW) ? scale_from_amax(amax) : *given_scale;
    const RowDiv div(s);
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int64_t ch = lane + LPR * c;
      if (ch < nchunks) store_chunk<ACT>(q, base + ch * 8, ra[c], h[ACT == MOE_ACT_SILU_MUL ? c : 0], div);
    }
    if (lane == 0) {
      if (MODE == MODE_ROW) scale[row] = s;
      if (row_amax) row_amax[row] = amax;
    }
  } else {
    for (int64_t ch = lane; ch < nchunks; ch += 64) {
      float v[8];
      load_vals<ACT>(x, xu, xbase + ch * 8, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    }
    amax = wave_max(amax);
    const float s = (MODE == MODE_ROW) ? scale_from_amax(amax) : *given_scale;
    const RowDiv div(s);
    for (int64_t ch = lane; ch < nchunks; ch += 64) {
      float v[8];
      load_vals<ACT>(x, xu, xbase + ch * 8, v);
      store_codes(q, base + ch * 8, v, div);
    }
    if (lane == 0) {
      if (MODE == MODE_ROW) scale[row] = s;
      if (row_amax) row_amax[row] = amax;
    }
  }
}

// Few long rows (up to 2048 rows of 2056..8192 elements, e.g. one GPU's own
// tokens of an expert-parallel layer): one workgroup of four waves per row,
// so that four times as many waves hide the memory latency.  Thread t owns
// chunks t, t + 256, ...; the row absmax is a wave reduction and a max over
// the four waves' results through LDS (max is exact in any order, so the
// scale and the codes equal the one-wave kernel's).
template <int CPL, int ACT, int MODE>
__global__ __launch_bounds__(256) void quantize_row_wg_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ xu, int64_t C, int64_t ldx,
    const float* __restrict__ given_scale, uint8_t* __restrict__ q, float* __restrict__ scale,
    float* __restrict__ row_amax) {
  __shared__ float wmax[4];
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int64_t nchunks = C >> 3;
  const int64_t base = row * C, xbase = row * ldx;
  Bf16x8 ra[CPL], rb[CPL];
  load_row_share<CPL, ACT, 256>(x, xu, xbase, nchunks, tid, ra, rb);
  float h[ACT == MOE_ACT_SILU_MUL ? CPL : 1][8];
  float amax = 0.0f;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    if (tid + 256 * c < nchunks) amax = fmaxf(amax, chunk_absmax<ACT>(ra[c], rb[c], h[ACT == MOE_ACT_SILU_MUL ? c : 0]));
  }
  amax = wave_max(amax);
  if ((tid & 63) == 0) wmax[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const float s = (MODE == MODE_ROW) ? scale_from_amax(amax) : *given_scale;
  const RowDiv div(s);
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int64_t ch = tid + 256 * c;
    if (ch < nchunks) store_chunk<ACT>(q, base + ch * 8, ra[c], h[ACT == MOE_ACT_SILU_MUL ? c : 0], div);
  }
  if (tid == 0) {
    if (MODE == MODE_ROW) scale[row] = s;
    if (row_amax) row_amax[row] = amax;
  }
}

// First pass of the tensor-dynamic mode: each block reduces the absmax of a
// grid-strided set of rows into partial[blockIdx.x] (no atomics, so the
// result does not depend on scheduling; max is exact in any order).
template <int ACT>
__global__ __launch_bounds__(256) void tensor_amax_kernel(const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ xu, int64_t R,
                                                          int64_t C, int64_t ldx, float* __restrict__ partial,
                                                          float* __restrict__ row_amax) {
  __shared__ float red[4];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t nchunks = C >> 3;
  float bmax = 0.0f;
  for (int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + w; row < R; row += static_cast<int64_t>(gridDim.x) * 4) {
    float amax = 0.0f;
    for (int64_t ch = lane; ch < nchunks; ch += 64) {
      float v[8];
      load_vals<ACT>(x, xu, row * ldx + ch * 8, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    }
    amax = wave_max(amax);
    if (lane == 0 && row_amax) row_amax[row] = amax;
    bmax = fmaxf(bmax, amax);
  }
  if (lane == 0) red[w] = bmax;
  __syncthreads();
  if (threadIdx.x == 0) partial[blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// Reduce the per-block partial maxima to the tensor scale.
__global__ __launch_bounds__(256) void tensor_scale_kernel(const float* __restrict__ partial, int n,
                                                           float* __restrict__ scale) {
  __shared__ float red[4];
  float m = 0.0f;
  for (int i = threadIdx.x; i < n; i += 256) m = fmaxf(m, partial[i]);
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) *scale = scale_from_amax(fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])));
}

__global__ void fill_scale_kernel(float* scale, float v) { *scale = v; }

constexpr int64_t kWgRowsMax = 2048;   // up to here a row gets a workgroup when it is long

template <int ACT, int MODE>
hipError_t launch_rows(const uint16_t* x, const uint16_t* xu, int64_t R, int64_t C, int64_t ldx, const float* given,
                       uint8_t* q, float* scale, float* row_amax, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(moe_cdiv(R, 4))), block(256);
  const int64_t chunks_per_lane = moe_cdiv(C / 8, 64);
  // rows of 96 + 64j chunks: two rows per wave, 32 lanes each, no idle lanes
  const int64_t nch = C / 8;
  if (nch % 64 == 32 && nch <= 32 * 5) {
    const dim3 grid2(static_cast<unsigned>(moe_cdiv(R, 8)));
    if (nch == 32)
      quantize_rows_kernel<1, ACT, MODE, 32><<<grid2, block, 0, st>>>(x, xu, R, C, ldx, given, q, scale, row_amax);
    else if (nch == 96)
      quantize_rows_kernel<3, ACT, MODE, 32><<<grid2, block, 0, st>>>(x, xu, R, C, ldx, given, q, scale, row_amax);
    else
      quantize_rows_kernel<5, ACT, MODE, 32><<<grid2, block, 0, st>>>(x, xu, R, C, ldx, given, q, scale, row_amax);
    return hipGetLastError();
  }
  // few long rows: a workgroup per row (at 1024 rows of 7168, 4 waves per SIMD instead of 1)
  if (R <= kWgRowsMax && nch > 256 && nch <= 1024) {
    const dim3 gridr(static_cast<unsigned>(R));
    if (nch <= 512)
      quantize_row_wg_kernel<2, ACT, MODE><<<gridr, block, 0, st>>>(x, xu, C, ldx, given, q, scale, row_amax);
    else
      quantize_row_wg_kernel<4, ACT, MODE><<<gridr, block, 0, st>>>(x, xu, C, ldx, given, q, scale, row_amax);
    return hipGetLastError();
  }
  // Keep the row in registers when it fits (the SiLU variant holds float32).
  const int max_cpl = (ACT == MOE_ACT_SILU_MUL) ? 8 : 16;
  if (chunks_per_lane <= 1)
    quantize_rows_kernel<1, ACT, MODE><<<grid, block, 0, st>>>(x, xu, R, C, ldx, given, q, scale, row_amax);
  else if (chunks_per_lane <= 2)
    quantize_rows_kernel<2, ACT, MODE><<<grid, block, 0, st>>>(x, xu, R, C, ldx, given, q, scale, row_amax);
  else if (chunks_per_lane <= 4)
    quantize_rows_kernel<4, ACT, MODE><<<grid, block, 0, st>>>(x, xu, R, C, ldx, given, q, scale, row_amax);
  else if (chunks_per_lane <= 8)
    quantize_rows_kernel<8, ACT, MODE><<<grid, block, 0, st>>>(x, xu, R, C, ldx, given, q, scale, row_amax);
  else if (chunks_per_lane <= max_cpl)
    quantize_rows_kernel<(ACT == MOE_ACT_SILU_MUL ? 8 : 16), ACT, MODE>
        <<<grid, block, 0, st>>>(x, xu, R, C, ldx, given, q, scale, row_amax);
  else
    quantize_rows_kernel<0, ACT, MODE><<<grid, block, 0, st>>>(x, xu, R, C, ldx, given, q, scale, row_amax);
  return hipGetLastError();
}

constexpr int kTensorBlocks = 1024;

template <int ACT>
int quantize_rows_impl(const uint16_t* x, const uint16_t* xu, int64_t R, int64_t C, int64_t ldx, int mode,
                       float static_scale, uint8_t* q, float* scale, float* row_amax, void* ws,
                       hipStream_t st) {
  if (mode == MOE_SCALE_ROW_DYNAMIC) {
    if (R == 0) return MOE_OK;
    return launch_rows<ACT, MODE_ROW>(x, xu, R, C, ldx, nullptr, q, scale, row_amax, st) == hipSuccess
               ? MOE_OK : MOE_ERR_HIP;
  }
  if (mode == MOE_SCALE_TENSOR_STATIC) {
    fill_scale_kernel<<<1, 1, 0, st>>>(scale, static_scale);
    MOE_CHECK_LAUNCH();
    if (R == 0) return MOE_OK;
    return launch_rows<ACT, MODE_GIVEN>(x, xu, R, C, ldx, scale, q, scale, row_amax, st) == hipSuccess
               ? MOE_OK : MOE_ERR_HIP;
  }
  if (mode == MOE_SCALE_TENSOR_FROM_ROW_AMAX) {
    // the maximum of the caller's row maxima, then the quantize pass (row_amax is an input here)
    if (R == 0) {
      fill_scale_kernel<<<1, 1, 0, st>>>(scale, 1.0f);
      MOE_CHECK_LAUNCH();
      return MOE_OK;
    }
    amax_scale_kernel<<<1, 1024, 0, st>>>(row_amax, R, scale);
    MOE_CHECK_LAUNCH();
    return launch_rows<ACT, MODE_GIVEN>(x, xu, R, C, ldx, scale, q, scale, nullptr, st) == hipSuccess
               ? MOE_OK : MOE_ERR_HIP;
  }
  // tensor dynamic: partial maxima in the workspace after the error word
  float* partial = reinterpret_cast<float*>(static_cast<char*>(ws) + 256);
  const int nblk = static_cast<int>(R == 0 ? 1 : (moe_cdiv(R, 4) < kTensorBlocks ? moe_cdiv(R, 4) : kTensorBlocks));
  if (R == 0) {
    fill_scale_kernel<<<1, 1, 0, st>>>(scale, 1.0f);
    MOE_CHECK_LAUNCH();
    return MOE_OK;
  }
  tensor_amax_kernel<ACT><<<nblk, 256, 0, st>>>(x, xu, R, C, ldx, partial, row_amax);
  MOE_CHECK_LAUNCH();
  tensor_scale_kernel<<<1, 256, 0, st>>>(partial, nblk, scale);
  MOE_CHECK_LAUNCH();
  return launch_rows<ACT, MODE_GIVEN>(x, xu, R, C, ldx, scale, q, scale, nullptr, st) == hipSuccess
             ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace

size_t quantize_rows_ws_bytes(int64_t R, int64_t C, int mode) {
  (void)R; (void)C;
  return mode == MOE_SCALE_TENSOR_DYNAMIC ? 256 + kTensorBlocks * sizeof(float) : 256;
}

}  // namespace moe

extern "C" int moe_quantize_rows_strided(const void* x, const void* x_up, int64_t ldx, int act, int64_t R,
                                         int64_t C, int scale_mode, float static_scale, uint8_t* q, float* scale,
                                         float* row_amax, void* ws, size_t ws_bytes, void* stream) {
  if (R < 0 || C <= 0 || C % 16 != 0) return MOE_ERR_SHAPE;
  if (ldx < C || ldx % 8 != 0) return MOE_ERR_SHAPE;
  if (act != MOE_ACT_NONE && act != MOE_ACT_SILU_MUL) return MOE_ERR_UNSUPPORTED;
  if (scale_mode != MOE_SCALE_ROW_DYNAMIC && scale_mode != MOE_SCALE_TENSOR_DYNAMIC &&
      scale_mode != MOE_SCALE_TENSOR_STATIC && scale_mode != MOE_SCALE_TENSOR_FROM_ROW_AMAX)
    return MOE_ERR_UNSUPPORTED;
  if (scale_mode == MOE_SCALE_TENSOR_STATIC && !(static_scale > 0.0f && static_scale < 3.0e38f))
    return MOE_ERR_SHAPE;
  if (!scale || (R > 0 && (!x || !q))) return MOE_ERR_NULL;
  if (scale_mode == MOE_SCALE_TENSOR_FROM_ROW_AMAX && R > 0 && !row_amax) return MOE_ERR_NULL;
  if (act == MOE_ACT_SILU_MUL && R > 0 && !x_up) return MOE_ERR_NULL;
  if (act == MOE_ACT_NONE && x_up) return MOE_ERR_UNSUPPORTED;
  if (scale_mode == MOE_SCALE_TENSOR_DYNAMIC) {
    if (!ws) return MOE_ERR_WORKSPACE;
    if (ws_bytes < moe::quantize_rows_ws_bytes(R, C, scale_mode)) return MOE_ERR_WORKSPACE;
  }
  // 16-byte loads: every row start must stay 16-byte aligned
  if ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(x_up)) % 16 != 0) return MOE_ERR_SHAPE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  const uint16_t* ub = static_cast<const uint16_t*>(x_up);
  if (act == MOE_ACT_SILU_MUL)
    return moe::quantize_rows_impl<MOE_ACT_SILU_MUL>(xb, ub, R, C, ldx, scale_mode, static_scale, q, scale,
                                                     row_amax, ws, st);
  return moe::quantize_rows_impl<MOE_ACT_NONE>(xb, nullptr, R, C, ldx, scale_mode, static_scale, q, scale,
                                               row_amax, ws, st);
}

extern "C" int moe_quantize_rows(const void* x, const void* x_up, int act, int64_t R, int64_t C,
                                 int scale_mode, float static_scale, uint8_t* q, float* scale,
                                 float* row_amax, void* ws, size_t ws_bytes, void* stream) {
  return moe_quantize_rows_strided(x, x_up, C, act, R, C, scale_mode, static_scale, q, scale, row_amax, ws,
                                   ws_bytes, stream);
}
