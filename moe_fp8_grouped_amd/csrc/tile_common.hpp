// Shared pieces of the grouped-matmul kernels: the fp8 MFMA, the local group
// table every workgroup builds from group_sizes, the XCD-aware split of a tile
// range, and the LDS fragment readers of the 144-byte-padded staging layout.
#pragma once

#include "common.hpp"

namespace moe {
namespace tile {

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
constexpr int kAbsMaxLocal = 512;           // group table of the kernels with absorbing tiles (LDS budget)
// Split last round of the grouped matmul: workspace layout after the header --
// one counter per leftover tile (kSplitPerXcd per XCD), then one float32 slot
// of kSplitSlot elements (a 144 x 256 tile) per workgroup
constexpr int kSplitPerXcd = 128;
constexpr int kSplitMinSteps = 4;           // K steps per part at least
constexpr int kSplitSlot = 144 * 256;
constexpr int64_t kSplitCntOff = 256;       // bytes
constexpr int64_t kSplitSlotOff = 8192;     // bytes

// The split parts' sums travel between workgroups that may sit on different
// XCDs, each behind its own L2.  They are written and read with the
// device-scope cache policy (sc1, bit 4 of the buffer access's cache field):
// the coding the compiler itself uses for relaxed device-scope atomic loads
// and stores, so each 4-byte element is such an atomic and is coherent across
// the XCDs without the whole-L2 writeback and invalidate of a device-scope
// fence.  Ordering comes from waiting for the stores' completion before the
// counting atomic, and from issuing the reads only after its result is known.
constexpr int kCachePolicyDevice = 16;
typedef uint32_t v4u32 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t slot_rsrc(float* slot) {   // slot: uniform over the workgroup
  const uint64_t b = reinterpret_cast<uint64_t>(slot);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b >> 32));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo), 0,
                                           kSplitSlot * static_cast<int>(sizeof(float)), 0x00020000);
}
__device__ __forceinline__ void slot_store(__amdgpu_buffer_rsrc_t r, int byte_off, v4f v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u32, v), r, byte_off, 0, kCachePolicyDevice);
}
__device__ __forceinline__ v4f slot_load(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, kCachePolicyDevice));
}

__device__ __forceinline__ v4f mfma_f8(const v8i& a, const v8i& b, const v4f& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

typedef int v4i32 __attribute__((ext_vector_type(4)));

// The int8 counterpart of mfma_f8 on the same 32-byte fragments: two
// v_mfma_i32_16x16x64_i8, the first on bytes 0..15 of every lane's share of
// the contraction, the second on bytes 16..31.  Both operands split their
// fragments the same way, so the pair sums every product exactly once, in
// int32 (exact for |codes| <= 127 below 2^17 terms).
__device__ __forceinline__ v4i32 mfma_i8x2(const v8i& a, const v8i& b, v4i32 c) {
  c = __builtin_amdgcn_mfma_i32_16x16x64_i8(v4i32{a[0], a[1], a[2], a[3]}, v4i32{b[0], b[1], b[2], b[3]}, c, 0, 0, 0);
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(v4i32{a[4], a[5], a[6], a[7]}, v4i32{b[4], b[5], b[6], b[7]}, c, 0, 0,
                                               0);
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

// Local group table of up to NMAX groups, computed by every workgroup from
// group_sizes.
template <int NMAX>
struct GroupTableN {
  int rows_off[NMAX + 1];   // first compact row of each local group
  int tiles_off[NMAX + 1];  // first tile of each local group
};
typedef GroupTableN<kMaxLocal> GroupTable;

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

// Exclusive scan of v[0..n) (every v >= 0) into out[0..n] by wave 0,
// saturating at cap: out[i] = min(v[0] + ... + v[i-1], cap), out[n] =
// min(total, cap).  The running sums are 64-bit (n <= 1024 values below 2^31
// stay below 2^41), so sizes that add up past 2^31 cannot wrap; cap < 2^31.
// Returns (in lane 0 of wave 0) whether the total exceeded cap.
__device__ bool wave0_scan_sat(const int* v, int* out, int n, int64_t cap) {
  if (threadIdx.x >= 64) return false;
  const int lane = threadIdx.x;
  int64_t carry = 0;
  for (int b = 0; b < n; b += 64) {
    const int i = b + lane;
    const int64_t x = i < n ? v[i] : 0;
    int64_t incl = x;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int64_t t = __shfl_up(incl, o, 64);
      if (lane >= o) incl += t;
    }
    if (i < n) out[i] = static_cast<int>(min(carry + incl - x, cap));
    carry += __shfl(incl, 63, 64);
  }
  if (lane == 0) out[n] = static_cast<int>(min(carry, cap));
  return carry > cap;
}

// Tiles of a group of m rows.  tail_mode 0 (plain): ceil(m / bm) m-tiles per
// n-tile.  1 (wide tails, gmm): full m-tiles of bm rows, and a remainder of at
// most bm/2 rows is covered by tiles of bm/2 rows x two n-tiles (an odd last
// n-tile keeps a plain tail tile).  2 (all wide): every tile is bm/2 rows x
// two n-tiles, ceil(m / (bm/2)) of them per n-tile pair (an odd last n-tile
// keeps plain tiles).
// 3 (all wide, absorbing): as 2, but ceil(m / (bm/2 + 16)) row blocks per
// n-tile pair, each of at most bm/2 + 16 rows (the first blocks take the rows
// past bm/2 per block, up to 16 each).
__device__ __forceinline__ int group_tiles(int m, int bm, int nt, int tail_mode) {
  if (nt <= 0) return 1;
  if (tail_mode == 2) return ((m + bm / 2 - 1) / (bm / 2)) * (nt / 2) + (nt & 1) * ((m + bm - 1) / bm);
  if (tail_mode == 3) return ((m + bm / 2 + 15) / (bm / 2 + 16)) * (nt / 2) + (nt & 1) * ((m + bm - 1) / bm);
  const int full = m / bm, rem = m - full * bm;
  if (tail_mode == 0 || rem == 0 || rem > bm / 2) return (full + (rem ? 1 : 0)) * nt;
  return (nt / 2) * (2 * full + 1) + (nt & 1) * (full + 1);
}

// Fill the table: clamps negative sizes to 0 and the row offsets to
// max_rows (flagging the error word) so that every tile stays inside the
// buffers -- the offsets are a saturating 64-bit scan, so group sizes whose
// sum passes 2^31 cannot wrap into a table that points outside the buffer;
// a group of m rows owns group_tiles(m, bm, tiles_per_mrow, tail_mode) tiles
// (tiles_per_mrow = 0: one entry per group).  The host bounds the tile count
// of max_rows rows below 2^31.
template <class GT>
__device__ void build_groups(const int32_t* __restrict__ group_sizes, int g0, int El, int64_t max_rows,
                             int tiles_per_mrow, int bm, int32_t* err, GT& gt, int* tmp,
                             int tail_mode = 0) {
  for (int g = threadIdx.x; g < El; g += blockDim.x) {
    int m = group_sizes[g0 + g];
    if (m < 0) {
      if (blockIdx.x == 0) raise_error(err, MOE_DEVERR_GROUP_SIZE);
      m = 0;
    }
    tmp[g] = m;
  }
  __syncthreads();
  const bool over = wave0_scan_sat(tmp, gt.rows_off, El, max_rows);
  if (over && threadIdx.x == 0 && blockIdx.x == 0) raise_error(err, MOE_DEVERR_ROWS);
  __syncthreads();
  for (int g = threadIdx.x; g < El; g += blockDim.x) {
    const int m = gt.rows_off[g + 1] - gt.rows_off[g];
    tmp[g] = group_tiles(m, bm, tiles_per_mrow, tail_mode);
  }
  __syncthreads();
  wave0_scan(tmp, gt.tiles_off, El);
  __syncthreads();
}

template <class GT>
__device__ __forceinline__ int find_group(const GT& gt, int El, int t) {
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

inline int num_cus() {
  static int g_num_cus = 0;
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

}  // namespace tile
}  // namespace moe
