// The grouped matmuls for contraction or output sizes that are multiples of
// 16 but not of 128 ("Quantize activations before EP all gather": the gmm_v2
// call; "Support quantization for tokamax gmm v2": tgmm2), which the tiled
// kernels in gmm.hip and tgmm.hip cannot take: their direct-to-LDS stages and
// 128-column tiles need multiples of 128.  Both kernels here stage 64 x 128
// byte operand tiles through LDS with plain 16-byte loads, zero-filling the
// contraction tail, the columns past N and (tgmm) the rows past a group's end
// -- a zero operand adds nothing to an fp8 matrix-core product -- and compute
// 64 x 64 output tiles with v_mfma_f32_16x16x128_f8f6f4 (four waves of 32 x 32,
// 2 x 2 blocks each).  Every size being a multiple of 16, a 16-byte chunk (and
// a lane's four output columns) is either wholly inside the matrix or wholly
// outside.  These are correctness paths for unusual shapes; the workloads'
// shapes all take the tiled kernels.
#include "tile_common.hpp"

namespace moe {
namespace {
using namespace tile;

constexpr int ET = 64;                      // output tile edge
constexpr int EK = 128;                     // contraction bytes per step
constexpr int ES = EK + 16;                 // staged row stride (bytes)

__device__ __forceinline__ uint32_t pack_bf16x2_rne(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

// Scatter the 16 bytes of v into column `col` of a [row][k]-staged tile at
// rows r0 .. r0+15 (a transpose of 16 consecutive elements along the
// source's contiguous axis).
__device__ __forceinline__ void scatter16(uint8_t* base, int r0, int col, const uint4 v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int b = 0; b < 16; ++b) base[(r0 + b) * ES + col] = static_cast<uint8_t>(w[b >> 2] >> (8 * (b & 3)));
}

// gmm for K or N not multiples of 128: out[r, c] = ls[r] * sum_b rs[g, b, c] *
// sum_{k in b} X[r, k] W_g[k, c], f32 accumulate; rows [n, M) zero.  Blockwise
// K scales need K / Kb a multiple of 128 (the host rejects the rest), so every
// 128-byte step lies in one scale block.
template <bool TRANS, bool OUT_BF16, bool I8>
__global__ __launch_bounds__(256) void gmm_edge_kernel(const uint8_t* __restrict__ lhs, const float* __restrict__ ls,
                                                       int ls_per_row, const uint8_t* __restrict__ rhs,
                                                       const float* __restrict__ rs, int Kb, int Nb,
                                                       const int32_t* __restrict__ group_sizes, int g0, int El,
                                                       int64_t M, int64_t K, int64_t N, void* __restrict__ out,
                                                       int32_t* __restrict__ err) {
  __shared__ __attribute__((aligned(16))) uint8_t As[ET * ES];
  __shared__ __attribute__((aligned(16))) uint8_t Bs[ET * ES];
  __shared__ GroupTable gt;
  __shared__ int tmp[kMaxLocal];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int NT = static_cast<int>((N + ET - 1) / ET);
  build_groups(group_sizes, g0, El, M, NT, ET, err, gt, tmp, 0);
  const int total = gt.tiles_off[El];
  const int n_rows = gt.rows_off[El];
  const int KT = static_cast<int>((K + EK - 1) / EK);
  const int64_t kblk = K / Kb;                  // contraction bytes per scale block
  const int64_t ncb = N / Nb;                   // columns per scale block
  const int rbase = (wave >> 1) * 32, cbase = (wave & 1) * 32;
  for (int t = blockIdx.x; t < total; t += gridDim.x) {
    const int g = find_group(gt, El, t);
    const int local = t - gt.tiles_off[g];
    const int m_g = gt.rows_off[g + 1] - gt.rows_off[g];
    const int per = (m_g + ET - 1) / ET;
    const int nt = local / per, mt = local - nt * per;
    const int64_t row0 = gt.rows_off[g] + static_cast<int64_t>(mt) * ET;
    const int rows_here = min(ET, m_g - mt * ET);
    const int64_t col0 = static_cast<int64_t>(nt) * ET;
    const uint8_t* wg = rhs + static_cast<int64_t>(g) * K * N;
    const float* rs_g = rs + static_cast<int64_t>(g) * Kb * Nb;
    v4f acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
    for (int kt = 0; kt < KT; ++kt) {
      const int64_t k0 = static_cast<int64_t>(kt) * EK;
      __syncthreads();                           // the previous step's fragment reads are done
#pragma unroll
      for (int u = 0; u < 2; ++u) {               // A: 64 rows x 8 chunks of 16 bytes
        const int c = tid + 256 * u, r = c >> 3, kc = (c & 7) * 16;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (r < rows_here && k0 + kc < K) v = *reinterpret_cast<const uint4*>(lhs + (row0 + r) * K + k0 + kc);
        *reinterpret_cast<uint4*>(As + r * ES + kc) = v;
      }
      if (TRANS) {                                // W stored [N, K]: rows are output columns
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int c = tid + 256 * u, r = c >> 3, kc = (c & 7) * 16;
          uint4 v = make_uint4(0, 0, 0, 0);
          if (col0 + r < N && k0 + kc < K) v = *reinterpret_cast<const uint4*>(wg + (col0 + r) * K + k0 + kc);
          *reinterpret_cast<uint4*>(Bs + r * ES + kc) = v;
        }
      } else {                                    // W stored [K, N]: 128 k-rows x 4 chunks of 16 columns
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int c = tid + 256 * u, kk = c >> 2, nc = (c & 3) * 16;
          uint4 v = make_uint4(0, 0, 0, 0);
          if (k0 + kk < K && col0 + nc < N) v = *reinterpret_cast<const uint4*>(wg + (k0 + kk) * N + col0 + nc);
          scatter16(Bs, nc, kk, v);
        }
      }
      __syncthreads();
      v8i a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) a[i] = frag_rows(As, rbase + 16 * i + (lane & 15), lane >> 4);
#pragma unroll
      for (int j = 0; j < 2; ++j) b[j] = frag_rows(Bs, cbase + 16 * j + (lane & 15), lane >> 4);
      if (Kb > 1) {                               // fold this step's product with its block's column scales
        const int64_t kb = k0 / kblk;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int64_t c = col0 + cbase + 16 * j + 4 * (lane >> 4);
          float s[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) s[q] = c + q < N ? rs_g[kb * Nb + (c + q) / ncb] : 0.f;
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            v4f p;
            if constexpr (I8)
              p = __builtin_convertvector(mfma_i8x2(b[j], a[i], v4i32{0, 0, 0, 0}), v4f);
            else
              p = mfma_f8(b[j], a[i], v4f{0.f, 0.f, 0.f, 0.f});
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[i][j][q] = fmaf(s[q], p[q], acc[i][j][q]);
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            if constexpr (I8)
              acc[i][j] = __builtin_bit_cast(v4f, mfma_i8x2(b[j], a[i], __builtin_bit_cast(v4i32, acc[i][j])));
            else
              acc[i][j] = mfma_f8(b[j], a[i], acc[i][j]);
          }
      }
    }
    if constexpr (I8) {
      if (Kb == 1) {                              // the int32 sums to float32
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_convertvector(__builtin_bit_cast(v4i32, acc[i][j]), v4f);
      }
    }
    // epilogue: lane l holds row rbase + 16 i + l%16 and columns cbase + 16 j + 4 (l/16) .. +3
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t c = col0 + cbase + 16 * j + 4 * (lane >> 4);
      if (c >= N) continue;
      float s[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) s[q] = Kb > 1 ? 1.f : rs_g[(c + q) / ncb];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = rbase + 16 * i + (lane & 15);
        if (r >= rows_here) continue;
        const float l = ls[ls_per_row ? row0 + r : 0];
        const float o0 = l * (acc[i][j][0] * s[0]), o1 = l * (acc[i][j][1] * s[1]);
        const float o2 = l * (acc[i][j][2] * s[2]), o3 = l * (acc[i][j][3] * s[3]);
        const int64_t idx = (row0 + r) * N + c;
        if (OUT_BF16)
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + idx) =
              make_uint2(pack_bf16x2_rne(o0, o1), pack_bf16x2_rne(o2, o3));
        else
          *reinterpret_cast<float4*>(static_cast<float*>(out) + idx) = make_float4(o0, o1, o2, o3);
      }
    }
  }
  // rows [n, M) are zero (N is a multiple of 16: whole 16-byte chunks)
  const int64_t per16 = OUT_BF16 ? 8 : 4;
  const int64_t total_chunks = (M - n_rows) * N / per16;
  uint4* base = OUT_BF16 ? reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + n_rows * N)
                         : reinterpret_cast<uint4*>(static_cast<float*>(out) + n_rows * N);
  for (int64_t c = static_cast<int64_t>(blockIdx.x) * 256 + tid; c < total_chunks; c += static_cast<int64_t>(gridDim.x) * 256)
    base[c] = make_uint4(0, 0, 0, 0);
}

// tgmm for K or N not multiples of 128: out[g, k, c] = ls[k] * rs[c] *
// sum_{r in group g} X[r, k] dY[r, c]; an empty group gives zeros.  A step
// stages 128 rows of the group: X's 64 k-columns and dY's 64 c-columns,
// transposed into [column][row] so the group's rows are the contraction.
template <bool OUT_BF16>
__global__ __launch_bounds__(256) void tgmm_edge_kernel(const uint8_t* __restrict__ lhs, const float* __restrict__ ls,
                                                        int ls_len, const uint8_t* __restrict__ rhs,
                                                        const float* __restrict__ rs, int rs_len,
                                                        const int32_t* __restrict__ group_sizes, int g0, int El,
                                                        int64_t M, int64_t K, int64_t N, void* __restrict__ out,
                                                        int32_t* __restrict__ err) {
  __shared__ __attribute__((aligned(16))) uint8_t Xs[ET * ES];
  __shared__ __attribute__((aligned(16))) uint8_t Ds[ET * ES];
  __shared__ GroupTable gt;
  __shared__ int tmp[kMaxLocal];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  build_groups(group_sizes, g0, El, M, 0, EK, err, gt, tmp, 0);
  const int KTo = static_cast<int>((K + ET - 1) / ET), NTo = static_cast<int>((N + ET - 1) / ET);
  const int per_group = KTo * NTo;
  const int64_t total = static_cast<int64_t>(El) * per_group;
  const int rbase = (wave >> 1) * 32, cbase = (wave & 1) * 32;
  for (int64_t t = blockIdx.x; t < total; t += gridDim.x) {
    const int g = static_cast<int>(t / per_group);
    const int local = static_cast<int>(t - static_cast<int64_t>(g) * per_group);
    const int64_t k0 = static_cast<int64_t>(local % KTo) * ET, n0 = static_cast<int64_t>(local / KTo) * ET;
    const int64_t r0 = gt.rows_off[g];
    const int m_g = gt.rows_off[g + 1] - gt.rows_off[g];
    v4f acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
    for (int rt = 0; rt * EK < m_g; ++rt) {
      __syncthreads();
#pragma unroll
      for (int u = 0; u < 2; ++u) {               // 128 rows x 4 chunks of 16 columns, each operand
        const int c = tid + 256 * u, rr = c >> 2, cc = (c & 3) * 16;
        const int row = rt * EK + rr;
        uint4 x = make_uint4(0, 0, 0, 0), d = make_uint4(0, 0, 0, 0);
        if (row < m_g && k0 + cc < K) x = *reinterpret_cast<const uint4*>(lhs + (r0 + row) * K + k0 + cc);
        if (row < m_g && n0 + cc < N) d = *reinterpret_cast<const uint4*>(rhs + (r0 + row) * N + n0 + cc);
        scatter16(Xs, cc, rr, x);
        scatter16(Ds, cc, rr, d);
      }
      __syncthreads();
      v8i a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) a[i] = frag_rows(Xs, rbase + 16 * i + (lane & 15), lane >> 4);
#pragma unroll
      for (int j = 0; j < 2; ++j) b[j] = frag_rows(Ds, cbase + 16 * j + (lane & 15), lane >> 4);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma_f8(b[j], a[i], acc[i][j]);
    }
    // lane l holds k = k0 + rbase + 16 i + l%16 and c = n0 + cbase + 16 j + 4 (l/16) .. +3
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t c = n0 + cbase + 16 * j + 4 * (lane >> 4);
      if (c >= N) continue;
      float s[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) s[q] = rs[rs_len == 1 ? 0 : c + q];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int64_t k = k0 + rbase + 16 * i + (lane & 15);
        if (k >= K) continue;
        const float l = m_g > 0 ? ls[ls_len == 1 ? 0 : k] : 0.f;      // an empty group writes exact zeros
        const float o0 = l * (acc[i][j][0] * s[0]), o1 = l * (acc[i][j][1] * s[1]);
        const float o2 = l * (acc[i][j][2] * s[2]), o3 = l * (acc[i][j][3] * s[3]);
        const int64_t idx = (static_cast<int64_t>(g) * K + k) * N + c;
        if (OUT_BF16)
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + idx) =
              make_uint2(pack_bf16x2_rne(o0, o1), pack_bf16x2_rne(o2, o3));
        else
          *reinterpret_cast<float4*>(static_cast<float*>(out) + idx) = make_float4(o0, o1, o2, o3);
      }
    }
  }
}

}  // namespace

hipError_t gmm_edge_launch(const uint8_t* lhs, const float* ls, int per_row, const uint8_t* rhs, const float* rs,
                           int Kb, int Nb, bool trans, const int32_t* gs, int g0, int El, int64_t M, int64_t K,
                           int64_t N, bool bf16, bool i8, void* out, int32_t* err, hipStream_t st) {
  const int64_t ub = (moe_cdiv(M, ET) + El) * moe_cdiv(N, ET);
  int64_t grid = 4LL * tile::num_cus();
  if (ub < grid) grid = ub;
  if (grid < 1) grid = 1;
  const unsigned gx = static_cast<unsigned>(grid);
#define MOE_EDGE(TR, BF, I) \
  gmm_edge_kernel<TR, BF, I><<<gx, 256, 0, st>>>(lhs, ls, per_row, rhs, rs, Kb, Nb, gs, g0, El, M, K, N, out, err)
#define MOE_EDGE_I(TR, BF) do { if (i8) MOE_EDGE(TR, BF, true); else MOE_EDGE(TR, BF, false); } while (0)
  if (trans) {
    if (bf16) MOE_EDGE_I(true, true); else MOE_EDGE_I(true, false);
  } else {
    if (bf16) MOE_EDGE_I(false, true); else MOE_EDGE_I(false, false);
  }
#undef MOE_EDGE_I
#undef MOE_EDGE
  return hipGetLastError();
}

hipError_t tgmm_edge_launch(const uint8_t* lhs, const float* ls, int ls_len, const uint8_t* rhs, const float* rs,
                            int rs_len, const int32_t* gs, int g0, int El, int64_t M, int64_t K, int64_t N, bool bf16,
                            void* out, int32_t* err, hipStream_t st) {
  const int64_t ub = static_cast<int64_t>(El) * moe_cdiv(K, ET) * moe_cdiv(N, ET);
  int64_t grid = 4LL * tile::num_cus();
  if (ub < grid) grid = ub;
  if (grid < 1) grid = 1;
  const unsigned gx = static_cast<unsigned>(grid);
  if (bf16)
    tgmm_edge_kernel<true><<<gx, 256, 0, st>>>(lhs, ls, ls_len, rhs, rs, rs_len, gs, g0, El, M, K, N, out, err);
  else
    tgmm_edge_kernel<false><<<gx, 256, 0, st>>>(lhs, ls, ls_len, rhs, rs, rs_len, gs, g0, El, M, K, N, out, err);
  return hipGetLastError();
}

}  // namespace moe
