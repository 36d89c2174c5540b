// moe_gmm_fp8 / moe_tgmm_fp8: grouped matmul of e4m3fn operands on the
// gfx950 fp8 matrix cores (v_mfma_f32_16x16x128_f8f6f4, float32 accumulate).
//
//  gmm  ("Quantize activations before EP all gather", the prequantized
//       gmm_v2 call; "Keep qwix out of tpu-inference's fused MoE kernel ...":
//       32-bit accumulator, [E, blocks, 1, N] weight scales):
//         out[r, c] = ls[r] * sum_b rs[g, b, c] * sum_{k in block b} X[r, k] W_g[k, c]
//  tgmm ("Support quantization for tokamax gmm v2", gmm2 / tgmm2):
//         out[g, k, c] = ls[k] * rs[c] * sum_{r in group g} X[r, k] dY[r, c]
//
// Tiling: a 256-thread workgroup computes a 128 x 128 output tile in steps
// of 128 along the contraction; its four waves each own a 64 x 64 quarter,
// i.e. 4 x 4 MFMA tiles of 16 x 16 (acc: 64 floats per lane).  Operands are
// staged through LDS, rows padded to 144 bytes so that the 16-byte fragment
// reads of 8 consecutive rows hit distinct banks.  An MFMA lane l supplies
// row (l % 16) and contraction bytes 32*(l/16) .. +31 of each operand:
//   * K-contiguous operands (lhs rows; rhs stored [E, N, K]) are read with
//     two 16-byte LDS reads per fragment;
//   * N- or row-contiguous operands (rhs stored [E, K, N]; both tgmm
//     operands, whose contraction runs over rows) are read with the gfx950
//     LDS transpose load ds_read_b64_tr_b8: within each 16-lane group, lane
//     i receives byte i%8 of the 8-byte chunks addressed by lanes 2j + i/8,
//     j = 0..7, so lane L addresses row 8q + L/2, column 8*(L%2) of the
//     stored [contraction][column] tile for read q of four.
// The byte order inside a lane (byte b <-> contraction index 32*(l/16) + b)
// is the same for both operands, which is all the dot product needs.
//
// Scheduling: persistent workgroups.  Each workgroup derives the local group
// offsets and the tile count from group_sizes itself (no host sync, empty
// groups own no tiles), then the tile range is split into eight contiguous
// parts, one per XCD (the hardware deals workgroups round-robin over the
// eight XCDs), so that tiles sharing an expert's weights run under one L2.
// Inside a group, m-tiles vary fastest, so consecutive tiles reuse the same
// weight tile.
#include "common.hpp"

namespace moe {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v2i lds_v2i;
// four 16-byte chunks held in registers between a global load and an LDS store
typedef uint32_t stage_t __attribute__((ext_vector_type(16)));

constexpr int BM = 128, BN = 128, BK = 128;
constexpr int LDS_STRIDE = BK + 16;         // bytes per staged row
constexpr int TILE_BYTES = 128 * LDS_STRIDE;
constexpr int kHdr = 256;                   // workspace header (error word)
constexpr int kMaxLocal = 1024;

__device__ __forceinline__ v4f mfma_f8(const v8i& a, const v8i& b, const v4f& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Fragment of a K-contiguous staged tile: 32 bytes at row `row`, byte 32*grp.
__device__ __forceinline__ v8i frag_rows(const uint8_t* lds, int row, int grp) {
  const uint4* p = reinterpret_cast<const uint4*>(lds + row * LDS_STRIDE + 32 * grp);
  const uint4 lo = p[0], hi = p[1];
  v8i r;
  r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
  r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
  return r;
}

// Fragment of a [contraction][column] staged tile for columns col0..col0+15,
// through four transpose loads.
__device__ __forceinline__ v8i frag_tr(const uint8_t* lds, int col0, int lane) {
  const int grp = lane >> 4, L = lane & 15;
  v8i r;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int row = 32 * grp + 8 * q + (L >> 1);
    const uint8_t* p = lds + row * LDS_STRIDE + col0 + 8 * (L & 1);
    const v2i t = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(p));
    r[2 * q] = t[0];
    r[2 * q + 1] = t[1];
  }
  return r;
}

// Local group table, computed by every workgroup from group_sizes.
struct GroupTable {
  int rows_off[kMaxLocal + 1];   // first compact row of each local group
  int tiles_off[kMaxLocal + 1];  // first tile of each local group
};

// Exclusive scan of v[0..n) into out[0..n] (out[n] = total) by wave 0.
__device__ void wave0_scan(const int* v, int* out, int n) {
  if (threadIdx.x >= 64) return;
  const int lane = threadIdx.x;
  int carry = 0;
  for (int b = 0; b < n; b += 64) {
    const int i = b + lane;
    const int x = i < n ? v[i] : 0;
    int incl = x;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(incl, o, 64);
      if (lane >= o) incl += t;
    }
    if (i < n) out[i] = carry + incl - x;
    carry += __shfl(incl, 63, 64);
  }
  if (lane == 0) out[n] = carry;
}

// Fill the table: clamps negative sizes and rows past max_rows (flagging
// the error word) so that every tile stays inside the buffers.
__device__ void build_groups(const int32_t* __restrict__ group_sizes, int g0, int El, int64_t max_rows,
                             int tiles_per_mrow, int32_t* err, GroupTable& gt, int* tmp) {
  for (int g = threadIdx.x; g < El; g += blockDim.x) {
    int m = group_sizes[g0 + g];
    if (m < 0) {
      if (blockIdx.x == 0) raise_error(err, MOE_DEVERR_GROUP_SIZE);
      m = 0;
    }
    tmp[g] = m;
  }
  __syncthreads();
  wave0_scan(tmp, gt.rows_off, El);
  __syncthreads();
  for (int g = threadIdx.x; g < El; g += blockDim.x) {
    int64_t lo = gt.rows_off[g], hi = gt.rows_off[g + 1];
    if (hi > max_rows) {
      if (blockIdx.x == 0) raise_error(err, MOE_DEVERR_ROWS);
      hi = max_rows;
      if (lo > hi) lo = hi;
    }
    tmp[g] = static_cast<int>(hi - lo);   // clamped rows
  }
  __syncthreads();
  // recompute offsets from clamped sizes; then tiles
  wave0_scan(tmp, gt.rows_off, El);
  __syncthreads();
  for (int g = threadIdx.x; g < El; g += blockDim.x) {
    const int m = gt.rows_off[g + 1] - gt.rows_off[g];
    tmp[g] = tiles_per_mrow > 0 ? ((m + BM - 1) / BM) * tiles_per_mrow : 1;
  }
  __syncthreads();
  wave0_scan(tmp, gt.tiles_off, El);
  __syncthreads();
}

__device__ __forceinline__ int find_group(const GroupTable& gt, int El, int t) {
  int lo = 0, hi = El - 1;             // last g with tiles_off[g] <= t
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (gt.tiles_off[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// The XCD-contiguous share of [0, total) for this workgroup: tiles
// first, first + step, ... < last.
__device__ __forceinline__ void xcd_share(int total, int& first, int& last, int& step) {
  const int nxcd = 8;
  const int x = blockIdx.x % nxcd;
  const int nb = gridDim.x;
  const int in_x = (nb - x + nxcd - 1) / nxcd;     // workgroups on this XCD
  const int lo = static_cast<int>((static_cast<int64_t>(total) * x) / nxcd);
  const int hi = static_cast<int>((static_cast<int64_t>(total) * (x + 1)) / nxcd);
  first = lo + static_cast<int>(blockIdx.x / nxcd);
  last = hi;
  step = in_x;
}

__device__ __forceinline__ void put4(stage_t& s, int i, const uint4& v) {
  s[4 * i] = v.x; s[4 * i + 1] = v.y; s[4 * i + 2] = v.z; s[4 * i + 3] = v.w;
}
__device__ __forceinline__ uint4 get4(const stage_t& s, int i) {
  return make_uint4(s[4 * i], s[4 * i + 1], s[4 * i + 2], s[4 * i + 3]);
}

// Global -> register staging of one 128 x 128-byte tile per operand: thread
// tid moves 16-byte chunks tid + 256*i (row chunk/8, byte 16*(chunk%8)).
template <bool TRANS>
__device__ __forceinline__ void gmm_load(const uint8_t* __restrict__ lhs, const uint8_t* __restrict__ wg, int64_t K,
                                         int64_t N, int64_t row0, int rows_here, int64_t col0, int kt, int tid,
                                         stage_t& ra, stage_t& rb) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + 256 * i;
    const int r = c >> 3, cb = (c & 7) * 16;
    const int64_t grow = row0 + (r < rows_here ? r : 0);   // rows past the group: any valid row
    const uint4 a = *reinterpret_cast<const uint4*>(lhs + grow * K + static_cast<int64_t>(kt) * BK + cb);
    uint4 b;
    if (TRANS)   // rhs [N, K]: staged row = column n
      b = *reinterpret_cast<const uint4*>(wg + (col0 + r) * K + static_cast<int64_t>(kt) * BK + cb);
    else         // rhs [K, N]: staged row = contraction index k
      b = *reinterpret_cast<const uint4*>(wg + (static_cast<int64_t>(kt) * BK + r) * N + col0 + cb);
    put4(ra, i, a);
    put4(rb, i, b);
  }
}

// tgmm staging: rows of the group (past its end: zeros, they must not add).
__device__ __forceinline__ void tgmm_load(const uint8_t* __restrict__ lhs, const uint8_t* __restrict__ rhs, int64_t K,
                                          int64_t N, int64_t r0, int m_g, int64_t k0, int64_t n0, int rt, int tid,
                                          stage_t& rx, stage_t& rd) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + 256 * i;
    const int r = c >> 3, cb = (c & 7) * 16;
    const int rr = rt * BK + r;
    uint4 x = make_uint4(0, 0, 0, 0), d = make_uint4(0, 0, 0, 0);
    if (rr < m_g) {
      x = *reinterpret_cast<const uint4*>(lhs + (r0 + rr) * K + k0 + cb);
      d = *reinterpret_cast<const uint4*>(rhs + (r0 + rr) * N + n0 + cb);
    }
    put4(rx, i, x);
    put4(rd, i, d);
  }
}

__device__ __forceinline__ void stash_tiles(uint8_t* As, uint8_t* Bs, int tid, const stage_t& ra,
                                            const stage_t& rb) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + 256 * i;
    const int r = c >> 3, cb = (c & 7) * 16;
    *reinterpret_cast<uint4*>(As + r * LDS_STRIDE + cb) = get4(ra, i);
    *reinterpret_cast<uint4*>(Bs + r * LDS_STRIDE + cb) = get4(rb, i);
  }
}

// ------------------------------------------------------------------ gmm
template <bool TRANS, bool KBLOCKS, bool OUT_BF16>
__global__ __launch_bounds__(256) void gmm_kernel(const uint8_t* __restrict__ lhs, const float* __restrict__ ls,
                                                  int ls_per_row, const uint8_t* __restrict__ rhs,
                                                  const float* __restrict__ rs, int Kb, int Nb,
                                                  const int32_t* __restrict__ group_sizes, int g0, int El,
                                                  int64_t M, int64_t K, int64_t N, void* __restrict__ out,
                                                  int32_t* __restrict__ err) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * TILE_BYTES];
  __shared__ GroupTable gt;
  __shared__ int tmp[kMaxLocal];
  uint8_t* As = smem;
  uint8_t* Bs = smem + TILE_BYTES;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int NT = static_cast<int>(N / BN);
  build_groups(group_sizes, g0, El, M, NT, err, gt, tmp);
  const int total = gt.tiles_off[El];
  const int n_rows = gt.rows_off[El];
  const int KT = static_cast<int>(K / BK);
  const int kblk_steps = static_cast<int>(K / Kb / BK);   // K steps per scale block
  const int64_t ncol_blk = N / Nb;
  int first, last, step;
  xcd_share(total, first, last, step);

  for (int t = first; t < last; t += step) {
    const int g = find_group(gt, El, t);
    const int local = t - gt.tiles_off[g];
    const int m_g = gt.rows_off[g + 1] - gt.rows_off[g];
    const int mtiles = (m_g + BM - 1) / BM;
    const int nt = local / mtiles, mt = local % mtiles;
    const int64_t row0 = gt.rows_off[g] + static_cast<int64_t>(mt) * BM;   // first compact row
    const int rows_here = min(BM, m_g - mt * BM);
    const int64_t col0 = static_cast<int64_t>(nt) * BN;
    const uint8_t* wg = rhs + static_cast<int64_t>(g) * K * N;

    // global -> register staging: 4 x 16 bytes per thread per operand
    stage_t ra, rb;
    v4f acc[4][4], tot[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
        tot[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
      }

    gmm_load<TRANS>(lhs, wg, K, N, row0, rows_here, col0, 0, tid, ra, rb);
    __syncthreads();     // previous tile's readers are done with the LDS
    stash_tiles(As, Bs, tid, ra, rb);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
      if (kt + 1 < KT) gmm_load<TRANS>(lhs, wg, K, N, row0, rows_here, col0, kt + 1, tid, ra, rb);
      v8i a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = frag_rows(As, wm * 64 + i * 16 + (lane & 15), lane >> 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (TRANS)
          b[j] = frag_rows(Bs, wn * 64 + j * 16 + (lane & 15), lane >> 4);
        else
          b[j] = frag_tr(Bs, wn * 64 + j * 16, lane);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma_f8(a[i], b[j], acc[i][j]);
      if (KBLOCKS && ((kt + 1) % kblk_steps == 0)) {
        // fold this K block: tot += rs[g, b, col] * acc
        const int bidx = kt / kblk_steps;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int64_t col = col0 + wn * 64 + j * 16 + (lane & 15);
          const float s = rs[(static_cast<int64_t>(g) * Kb + bidx) * Nb + col / ncol_blk];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int v = 0; v < 4; ++v) tot[i][j][v] = fmaf(s, acc[i][j][v], tot[i][j][v]);
            acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
          }
        }
      }
      __syncthreads();
      if (kt + 1 < KT) {
        stash_tiles(As, Bs, tid, ra, rb);
        __syncthreads();
      }
    }

    // epilogue: lane holds rows 4*(lane/16) + v, column lane % 16 of each 16x16 tile
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t col = col0 + wn * 64 + j * 16 + (lane & 15);
      const float s_col = KBLOCKS ? 1.0f : rs[static_cast<int64_t>(g) * Nb + col / ncol_blk];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int r = wm * 64 + i * 16 + 4 * (lane >> 4) + v;
          if (r >= rows_here) continue;
          const int64_t grow = row0 + r;
          const float lsr = ls_per_row ? ls[grow] : ls[0];
          const float val = KBLOCKS ? tot[i][j][v] : acc[i][j][v] * s_col;
          const float o = lsr * val;
          if (OUT_BF16)
            static_cast<uint16_t*>(out)[grow * N + col] = f32_to_bf16(o);
          else
            static_cast<float*>(out)[grow * N + col] = o;
        }
      }
    }
  }

  // rows [n, M) are zero
  const int64_t elems_per_row = N;
  const int64_t zero_rows = M - n_rows;
  if (zero_rows > 0) {
    const int64_t chunk = OUT_BF16 ? 8 : 4;    // elements per 16 bytes
    const int64_t total_chunks = zero_rows * elems_per_row / chunk;
    for (int64_t c = static_cast<int64_t>(blockIdx.x) * 256 + tid; c < total_chunks;
         c += static_cast<int64_t>(gridDim.x) * 256) {
      if (OUT_BF16)
        reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + n_rows * N)[c] = make_uint4(0, 0, 0, 0);
      else
        reinterpret_cast<uint4*>(static_cast<float*>(out) + n_rows * N)[c] = make_uint4(0, 0, 0, 0);
    }
  }
}

// ------------------------------------------------------------------ tgmm
template <bool OUT_BF16>
__global__ __launch_bounds__(256) void tgmm_kernel(const uint8_t* __restrict__ lhs, const float* __restrict__ ls,
                                                   int ls_len, const uint8_t* __restrict__ rhs,
                                                   const float* __restrict__ rs, int rs_len,
                                                   const int32_t* __restrict__ group_sizes, int g0, int El,
                                                   int64_t M, int64_t K, int64_t N, void* __restrict__ out,
                                                   int32_t* __restrict__ err) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * TILE_BYTES];
  __shared__ GroupTable gt;
  __shared__ int tmp[kMaxLocal];
  uint8_t* Xs = smem;                 // [row][k]
  uint8_t* Ds = smem + TILE_BYTES;    // [row][n]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  build_groups(group_sizes, g0, El, M, 0, err, gt, tmp);
  const int KTo = static_cast<int>(K / BM), NT = static_cast<int>(N / BN);
  const int per_group = KTo * NT;
  const int total = El * per_group;
  int first, last, step;
  xcd_share(total, first, last, step);

  for (int t = first; t < last; t += step) {
    const int g = t / per_group;
    const int local = t % per_group;
    const int kt_o = local % KTo, nt = local / KTo;   // k-tiles fastest: they share the dY tile
    const int64_t k0 = static_cast<int64_t>(kt_o) * BM, n0 = static_cast<int64_t>(nt) * BN;
    const int64_t r0 = gt.rows_off[g];
    const int m_g = gt.rows_off[g + 1] - gt.rows_off[g];
    const int RT = (m_g + BK - 1) / BK;

    stage_t rx, rd;
    v4f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
    if (RT > 0) {
      tgmm_load(lhs, rhs, K, N, r0, m_g, k0, n0, 0, tid, rx, rd);
      __syncthreads();
      stash_tiles(Xs, Ds, tid, rx, rd);
      __syncthreads();
      for (int rt = 0; rt < RT; ++rt) {
        if (rt + 1 < RT) tgmm_load(lhs, rhs, K, N, r0, m_g, k0, n0, rt + 1, tid, rx, rd);
        v8i a[4], b[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = frag_tr(Xs, wm * 64 + i * 16, lane);
#pragma unroll
        for (int j = 0; j < 4; ++j) b[j] = frag_tr(Ds, wn * 64 + j * 16, lane);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = mfma_f8(a[i], b[j], acc[i][j]);
        __syncthreads();
        if (rt + 1 < RT) {
          stash_tiles(Xs, Ds, tid, rx, rd);
          __syncthreads();
        }
      }
    }
    // epilogue: out[g, k, n] = ls[k] * rs[n] * acc
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t n = n0 + wn * 64 + j * 16 + (lane & 15);
      const float rsn = rs_len == 1 ? rs[0] : rs[n];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int64_t k = k0 + wm * 64 + i * 16 + 4 * (lane >> 4) + v;
          const float lsk = ls_len == 1 ? ls[0] : ls[k];
          const float o = (lsk * rsn) * acc[i][j][v];
          const int64_t idx = (static_cast<int64_t>(g) * K + k) * N + n;
          if (OUT_BF16)
            static_cast<uint16_t*>(out)[idx] = f32_to_bf16(o);
          else
            static_cast<float*>(out)[idx] = o;
        }
      }
    }
  }
}

int g_num_cus = 0;

int num_cus() {
  if (g_num_cus <= 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      g_num_cus = n;
    else
      g_num_cus = 256;
  }
  return g_num_cus;
}

}  // namespace

size_t gmm_ws_bytes() { return kHdr; }

}  // namespace moe

extern "C" int moe_gmm_fp8(const uint8_t* lhs, const float* lhs_scale, int lhs_scale_mode, const uint8_t* rhs,
                           const float* rhs_scale, int32_t Kb, int32_t Nb, int transpose_rhs,
                           const int32_t* group_sizes, int32_t E, int32_t group_offset,
                           int32_t num_local_experts, int64_t M, int64_t K, int64_t N, int out_dtype,
                           void* out, void* ws, size_t ws_bytes, void* stream) {
  if (M < 0 || K <= 0 || N <= 0 || K % 128 || N % 128) return MOE_ERR_SHAPE;
  if (E <= 0 || E > 1024 || group_offset < 0 || num_local_experts < 0 ||
      num_local_experts > moe::kMaxLocal || group_offset + num_local_experts > E)
    return MOE_ERR_SHAPE;
  if (M > INT32_MAX - 1) return MOE_ERR_SHAPE;
  if (Kb <= 0 || Nb <= 0 || K % Kb || N % Nb) return MOE_ERR_SHAPE;
  if (Kb > 1 && (K / Kb) % 128) return MOE_ERR_UNSUPPORTED;
  if (lhs_scale_mode != MOE_SCALE_ROW_DYNAMIC && lhs_scale_mode != MOE_SCALE_TENSOR_DYNAMIC &&
      lhs_scale_mode != MOE_SCALE_TENSOR_STATIC)
    return MOE_ERR_UNSUPPORTED;
  if (transpose_rhs != 0 && transpose_rhs != 1) return MOE_ERR_UNSUPPORTED;
  if (out_dtype == MOE_DTYPE_DEFAULT || out_dtype == MOE_E4M3FN) out_dtype = MOE_BF16;
  if (out_dtype != MOE_BF16 && out_dtype != MOE_F32) return MOE_ERR_UNSUPPORTED;
  if (M == 0) return MOE_OK;
  if (!out || !group_sizes) return MOE_ERR_NULL;
  if (num_local_experts > 0 && (!lhs || !lhs_scale || !rhs || !rhs_scale)) return MOE_ERR_NULL;
  if (!ws) return MOE_ERR_WORKSPACE;
  if (ws_bytes < moe::gmm_ws_bytes()) return MOE_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  int32_t* err = static_cast<int32_t*>(ws);
  const int El = num_local_experts;
  // upper bound of the tile count; the grid is at most two workgroups per CU
  const int64_t ub = (moe_cdiv(M, moe::BM) + El) * (N / moe::BN);
  int64_t grid = 2LL * moe::num_cus();
  if (ub < grid) grid = ub;
  if (grid < 8) grid = 8;
  const int per_row = lhs_scale_mode == MOE_SCALE_ROW_DYNAMIC ? 1 : 0;
  const bool kblocks = Kb > 1;
  const bool bf16 = out_dtype == MOE_BF16;
#define MOE_GMM_LAUNCH(T, KB, BF)                                                                      \
  moe::gmm_kernel<T, KB, BF><<<static_cast<unsigned>(grid), 256, 0, st>>>(                             \
      lhs, lhs_scale, per_row, rhs, rhs_scale, Kb, Nb, group_sizes, group_offset, El, M, K, N, out, err)
  if (transpose_rhs) {
    if (kblocks) { if (bf16) MOE_GMM_LAUNCH(true, true, true); else MOE_GMM_LAUNCH(true, true, false); }
    else         { if (bf16) MOE_GMM_LAUNCH(true, false, true); else MOE_GMM_LAUNCH(true, false, false); }
  } else {
    if (kblocks) { if (bf16) MOE_GMM_LAUNCH(false, true, true); else MOE_GMM_LAUNCH(false, true, false); }
    else         { if (bf16) MOE_GMM_LAUNCH(false, false, true); else MOE_GMM_LAUNCH(false, false, false); }
  }
#undef MOE_GMM_LAUNCH
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}

extern "C" int moe_tgmm_fp8(const uint8_t* lhs, const float* lhs_scale, int32_t lhs_scale_len,
                            const uint8_t* rhs, const float* rhs_scale, int32_t rhs_scale_len,
                            const int32_t* group_sizes, int32_t E, int32_t group_offset,
                            int32_t num_local_experts, int64_t M, int64_t K, int64_t N, int out_dtype,
                            void* out, void* ws, size_t ws_bytes, void* stream) {
  if (M < 0 || K <= 0 || N <= 0 || K % 128 || N % 128) return MOE_ERR_SHAPE;
  if (E <= 0 || E > 1024 || group_offset < 0 || num_local_experts < 0 ||
      num_local_experts > moe::kMaxLocal || group_offset + num_local_experts > E)
    return MOE_ERR_SHAPE;
  if (M > INT32_MAX - 1) return MOE_ERR_SHAPE;
  if (lhs_scale_len != 1 && lhs_scale_len != K) return MOE_ERR_UNSUPPORTED;
  if (rhs_scale_len != 1 && rhs_scale_len != N) return MOE_ERR_UNSUPPORTED;
  if (out_dtype == MOE_DTYPE_DEFAULT) out_dtype = MOE_F32;
  if (out_dtype != MOE_BF16 && out_dtype != MOE_F32) return MOE_ERR_UNSUPPORTED;
  const int El = num_local_experts;
  if (El == 0) return MOE_OK;
  if (!out || !group_sizes || !lhs_scale || !rhs_scale) return MOE_ERR_NULL;
  if (M > 0 && (!lhs || !rhs)) return MOE_ERR_NULL;
  if (!ws) return MOE_ERR_WORKSPACE;
  if (ws_bytes < moe::gmm_ws_bytes()) return MOE_ERR_WORKSPACE;
  if (static_cast<int64_t>(El) * (K / 128) * (N / 128) > INT32_MAX) return MOE_ERR_SHAPE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  int32_t* err = static_cast<int32_t*>(ws);
  const int64_t ub = static_cast<int64_t>(El) * (K / moe::BM) * (N / moe::BN);
  int64_t grid = 2LL * moe::num_cus();
  if (ub < grid) grid = ub;
  if (grid < 8) grid = 8;
  if (out_dtype == MOE_BF16)
    moe::tgmm_kernel<true><<<static_cast<unsigned>(grid), 256, 0, st>>>(
        lhs, lhs_scale, lhs_scale_len, rhs, rhs_scale, rhs_scale_len, group_sizes, group_offset, El, M, K, N, out, err);
  else
    moe::tgmm_kernel<false><<<static_cast<unsigned>(grid), 256, 0, st>>>(
        lhs, lhs_scale, lhs_scale_len, rhs, rhs_scale, rhs_scale_len, group_sizes, group_offset, El, M, K, N, out, err);
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}
