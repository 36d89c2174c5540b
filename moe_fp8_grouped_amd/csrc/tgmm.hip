// moe_tgmm_fp8: transposed grouped matmul for weight gradients on the gfx950
// fp8 matrix cores ("Support quantization for tokamax gmm v2": quantized
// gmm2 / tgmm2, backward split into an input-gradient gmm and a per-group
//   out[g, k, c] = ls[k] * rs[c] * sum_{r in group g} X[r, k] dY[r, c]
// weight-gradient tgmm).  The contraction runs over each group's rows, so
// both operands are row-contiguous: 128 x 128-byte row tiles are staged
// through LDS (rows padded to 144 bytes) and read with ds_read_b64_tr_b8;
// rows past the group's end are staged as zeros.  A 256-thread workgroup
// owns a 128 x 128 output tile (four 64 x 64 wave quarters of 16 x 16 MFMA
// tiles); persistent workgroups take tiles from an XCD-contiguous range.
// Bound by the float32 output write (E_loc * K * N * 4 bytes).
#include "tile_common.hpp"
#include "quant_common.hpp"

namespace moe {
namespace {
using namespace tile;

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
  build_groups(group_sizes, g0, El, M, 0, BM, err, gt, tmp);
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
          for (int j = 0; j < 4; ++j) acc[i][j] = mfma_f8(b[j], a[i], acc[i][j]);
        __syncthreads();
        if (rt + 1 < RT) {
          stash_tiles(Xs, Ds, tid, rx, rd);
          __syncthreads();
        }
      }
    }
    // epilogue: out[g, k, n] = ls[k] * rs[n] * acc.  The block product is
    // formed transposed (dY fragment first), so lane l holds row
    // k0 + 64 wm + 16 i + l%16 and the four consecutive columns
    // n0 + 64 wn + 16 j + 4 (l/16) .. +3: one 16-byte (f32) or 8-byte (bf16)
    // store per block.
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t n = n0 + wn * 64 + j * 16 + 4 * (lane >> 4);
      const float4 rsn = rs_len == 1 ? make_float4(rs[0], rs[0], rs[0], rs[0])
                                     : make_float4(rs[n], rs[n + 1], rs[n + 2], rs[n + 3]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t k = k0 + wm * 64 + i * 16 + (lane & 15);
        const float lsk = ls_len == 1 ? ls[0] : ls[k];
        const float o0 = (lsk * rsn.x) * acc[i][j][0], o1 = (lsk * rsn.y) * acc[i][j][1];
        const float o2 = (lsk * rsn.z) * acc[i][j][2], o3 = (lsk * rsn.w) * acc[i][j][3];
        const int64_t idx = (static_cast<int64_t>(g) * K + k) * N + n;
        if (OUT_BF16) {
          const uint32_t lo = f32_to_bf16(o0) | (static_cast<uint32_t>(f32_to_bf16(o1)) << 16);
          const uint32_t hi = f32_to_bf16(o2) | (static_cast<uint32_t>(f32_to_bf16(o3)) << 16);
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + idx) = make_uint2(lo, hi);
        } else {
          *reinterpret_cast<float4*>(static_cast<float*>(out) + idx) = make_float4(o0, o1, o2, o3);
        }
      }
    }
  }
}

// ------------------------------------------------------------------ transpose
// AT[c, 128 * tiles_off[g] + i] = A[rows_off[g] + i, c] for i < m_g and 0 for
// m_g <= i < the group's padded length (a multiple of 128): the rows of each
// group become a contraction axis of its own, contiguous per column.  An
// item is a 128-row block (inside one group, as padded lengths are multiples
// of 128) and up to two 64-column blocks, so every store instruction writes
// whole 128-byte lines: eight lanes cover the 128 rows of one column.  A
// workgroup walks its items with two register buffers: the four 16-byte
// loads of its next item are in flight while the current one goes through
// LDS and out, behind bare barriers that do not wait for those loads.  The
// staged rows are 128 bytes with 16-byte piece p of row r at slot
// p ^ ((r / 16) & 7), which keeps the dword reads of the transpose (16 rows
// x 4 columns per thread, 4 x 4 byte blocks transposed in registers with
// v_perm_b32) at the minimum two LDS cycles per instruction.
__device__ __forceinline__ void transpose4x4(const uint32_t* d, uint32_t* e) {
  // d[i]: row i's four column bytes; e[c]: column c's four row bytes
  const uint32_t lo01 = __builtin_amdgcn_perm(d[1], d[0], 0x05010400u);
  const uint32_t hi01 = __builtin_amdgcn_perm(d[1], d[0], 0x07030602u);
  const uint32_t lo23 = __builtin_amdgcn_perm(d[3], d[2], 0x05010400u);
  const uint32_t hi23 = __builtin_amdgcn_perm(d[3], d[2], 0x07030602u);
  e[0] = __builtin_amdgcn_perm(lo23, lo01, 0x05040100u);
  e[1] = __builtin_amdgcn_perm(lo23, lo01, 0x07060302u);
  e[2] = __builtin_amdgcn_perm(hi23, hi01, 0x05040100u);
  e[3] = __builtin_amdgcn_perm(hi23, hi01, 0x07060302u);
}

// LDS-only barrier: waits for this wave's LDS operations, not its global loads.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

struct TItem {
  int64_t p0, cb0;   // first padded row, first 64-column block
  int nb;            // column blocks in this item (1..2)
  int keep;          // bit u: this thread's load u holds data (else the piece is zero)
};

// GATHER: where row i of local group g comes from.
//   0  A holds the sorted rows: row rows_off[g] + i of A [rows, C] (e4m3 codes).
//   1  The sort's gather in this layout: the row is source token
//      perm[start + rows_off[g] + i] / k of A = xq [T, C] (e4m3 codes), start
//      = the group sizes before g0 (the window's first slot).
//   2  As 1 from bf16 rows A = x [T, C], quantized on the way with the static
//      scale s: e4m3(clip(x / s)), the row quantizer's codes.
// Token indices outside [0, T) and slots outside perm are clamped (their
// columns are those of a valid row; no access leaves a buffer).
template <int GATHER>
__global__ __launch_bounds__(256) void transpose_groups_kernel(const uint8_t* __restrict__ A, int64_t C,
                                                               const int32_t* __restrict__ group_sizes, int g0,
                                                               int El, int64_t max_rows, int64_t Mpad,
                                                               uint8_t* __restrict__ AT, int32_t* __restrict__ err,
                                                               const int32_t* __restrict__ perm, int k, int64_t T,
                                                               float static_scale) {
  constexpr int IR = 128;                     // rows per item
  constexpr int ES = GATHER == 2 ? 2 : 1;     // source bytes per element
  constexpr int NV = GATHER == 2 ? 8 : 4;     // 16-byte loads per thread and item
  __shared__ GroupTable gt;
  __shared__ int tmp[kMaxLocal];
  __shared__ __attribute__((aligned(16))) uint8_t tl[IR * 128];
  __shared__ long long start_s;
  build_groups(group_sizes, g0, El, max_rows, 1, 128, err, gt, tmp, false);
  if (GATHER) {   // the window's first slot: the sizes of the groups before g0 (negative ones count as 0)
    if (threadIdx.x < 64) {
      long long sum = 0;
      for (int e = threadIdx.x; e < g0; e += 64) sum += max(group_sizes[e], 0);
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o, 64);
      if (threadIdx.x == 0) start_s = sum;
    }
    __syncthreads();
  }
  const long long start = GATHER ? start_s : 0;
  const long long nslots = static_cast<long long>(T) * k;
  const int64_t P = static_cast<int64_t>(gt.tiles_off[El]) * 128;    // padded rows
  const int64_t cblocks = C / 64;
  const int64_t cq = (cblocks + 1) / 2;
  const int64_t items = (P / IR) * cq;
  const int tid = threadIdx.x;
  const int lr = tid >> 3, pc = tid & 7;       // load: rows lr + 32 u, 16-byte piece pc of 128 bytes
  const int rg = tid & 7, cg = tid >> 3;       // transpose: 16-row group rg, 4-column group cg
  const RowDiv div(static_scale);

  // item `it`: its first padded row and column block, and where its rows sit
  struct Loc { int64_t p0, cb0, i0; int nb, row0, m_g; };
  auto locate = [&](int64_t it) {
    Loc L;
    const int64_t pb = it / cq, q = it - pb * cq;
    L.p0 = pb * IR;
    L.cb0 = q * 2;
    L.nb = static_cast<int>(cblocks - L.cb0 < 2 ? cblocks - L.cb0 : 2);
    // the group holding padded rows p0 .. p0 + 127; the item is the
    // workgroup's, so the search runs on scalars
    int lo = 0, hi = El - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (static_cast<int64_t>(__builtin_amdgcn_readfirstlane(gt.tiles_off[mid])) * 128 <= L.p0) lo = mid;
      else hi = mid - 1;
    }
    L.row0 = __builtin_amdgcn_readfirstlane(gt.rows_off[lo]);
    L.i0 = L.p0 - static_cast<int64_t>(__builtin_amdgcn_readfirstlane(gt.tiles_off[lo])) * 128;
    L.m_g = __builtin_amdgcn_readfirstlane(gt.rows_off[lo + 1]) - L.row0;
    return L;
  };
  // GATHER: the source tokens of the thread's four rows of item `it` (-1: past the group), loaded one item
  // ahead of their use so that the row loads do not wait for them
  auto load_tok = [&](int64_t it, int (&tk)[4]) {
    if (!GATHER) return;
    const Loc L = locate(it);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t r = L.i0 + lr + 32 * u;
      long long slot = start + L.row0 + r;
      slot = slot < nslots ? slot : nslots - 1;
      tk[u] = r < L.m_g ? perm[slot] : -1;
    }
  };
  // issue the loads of item `it`; every load is issued (a piece with no data
  // reads A's first bytes and is zeroed when staged), so the loads carry no
  // branches and stay in flight
  auto fetch = [&](int64_t it, TItem& I, const int (&tk)[4], uint4 (&v)[NV]) {
    const Loc L = locate(it);
    I.p0 = L.p0;
    I.cb0 = L.cb0;
    I.nb = L.nb;
    const bool col_ok = (pc >> 2) < I.nb;
    I.keep = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t r = L.i0 + lr + 32 * u;
      const bool ok = col_ok && r < L.m_g;
      int64_t src_row = L.row0 + r;
      if (GATHER) {
        const int64_t tok = tk[u] >= 0 ? tk[u] / k : 0;
        src_row = tok < T ? tok : T - 1;
      }
      I.keep |= ok ? 1 << u : 0;
      const uint8_t* src = A + (src_row * C + I.cb0 * 64 + 16 * pc) * ES;
      if (ES == 1) {
        v[u] = *reinterpret_cast<const uint4*>(ok ? src : A);
      } else {
        v[2 * u] = *reinterpret_cast<const uint4*>(ok ? src : A);
        v[2 * u + 1] = *reinterpret_cast<const uint4*>(ok ? src + 16 : A);
      }
    }
  };
  // stage item I's rows in LDS, transpose, store its columns
  auto put = [&](const TItem& I, const uint4 (&v)[NV]) {
    lds_barrier();                            // the previous item's reads of tl are done
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int r = lr + 32 * u;
      uint4 w;
      if (ES == 1) {
        w = v[u];
      } else {   // 16 bf16 values to 16 codes
        float f[16];
        const uint32_t ww[8] = {v[2 * u].x, v[2 * u].y, v[2 * u].z, v[2 * u].w,
                                v[2 * u + 1].x, v[2 * u + 1].y, v[2 * u + 1].z, v[2 * u + 1].w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          f[2 * i] = __uint_as_float(ww[i] << 16);
          f[2 * i + 1] = __uint_as_float(ww[i] & 0xffff0000u);
        }
        const uint2 c0 = codes8(f, div), c1 = codes8(f + 8, div);
        w = make_uint4(c0.x, c0.y, c1.x, c1.y);
      }
      w = (I.keep >> u) & 1 ? w : make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4*>(tl + r * 128 + 16 * (pc ^ ((r >> 4) & 7))) = w;
    }
    lds_barrier();
    if ((cg >> 4) < I.nb) {
      const uint8_t* t = tl + (16 * rg) * 128 + 16 * ((cg >> 2) ^ rg) + 4 * (cg & 3);
      uint32_t d[16], e[4][4];
#pragma unroll
      for (int j = 0; j < 16; ++j) d[j] = *reinterpret_cast<const uint32_t*>(t + j * 128);
#pragma unroll
      for (int b = 0; b < 4; ++b) transpose4x4(d + 4 * b, e[b]);
      uint8_t* dst = AT + (I.cb0 * 64 + 4 * cg) * Mpad + I.p0 + 16 * rg;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        *reinterpret_cast<uint4*>(dst + kk * Mpad) = make_uint4(e[0][kk], e[1][kk], e[2][kk], e[3][kk]);
    }
  };

  // The fetch of the item after the last one re-reads the last item (never
  // staged): every fetch is unconditional, so no register buffer is merged
  // across a branch and the loads are never waited for early.
  const int64_t G = gridDim.x;
  int64_t it = blockIdx.x;
  if (it >= items) return;
  auto next = [&](int64_t i) { return i + G < items ? i + G : items - 1; };
  TItem ia, ib;
  uint4 va[NV], vb[NV];
  int ta[4] = {0, 0, 0, 0}, tb[4] = {0, 0, 0, 0};
  load_tok(it, ta);
  fetch(it, ia, ta, va);
  load_tok(next(it), tb);
  for (;;) {
    fetch(next(it), ib, tb, vb);
    load_tok(next(next(it)), ta);
    put(ia, va);
    it += G;
    if (it >= items) break;
    fetch(next(it), ia, ta, va);
    load_tok(next(next(it)), tb);
    put(ib, vb);
    it += G;
    if (it >= items) break;
  }
}

__global__ void write_scale_kernel(float* scale, float v) { *scale = v; }

}  // namespace

// Transposed-operand staging of the weight-gradient product: padded row
// capacity (a multiple of 256) and workspace bytes.
int64_t tgmm_mpad(int64_t M, int E) { return moe_cdiv(M + 128 * static_cast<int64_t>(E), 256) * 256; }
size_t tgmm_ws_bytes(int64_t M, int64_t K, int64_t N, int E) {
  return tile::kHdr + static_cast<size_t>((K + N) * tgmm_mpad(M, E));
}
hipError_t tgmm_edge_launch(const uint8_t* lhs, const float* ls, int ls_len, const uint8_t* rhs, const float* rs,
                            int rs_len, const int32_t* gs, int g0, int El, int64_t M, int64_t K, int64_t N, bool bf16,
                            void* out, int32_t* err, hipStream_t st);
hipError_t gmm_batched_launch(const uint8_t* A, const float* ls, int ls_len, const uint8_t* B, const float* rs,
                              int rs_len, const int32_t* group_sizes, int g0, int El, int64_t max_rows, int64_t M,
                              int64_t K, int64_t N, bool bf16, void* out, int32_t* err, hipStream_t st);
}  // namespace moe

extern "C" int moe_tgmm_fp8(const uint8_t* lhs, const float* lhs_scale, int32_t lhs_scale_len,
                            const uint8_t* rhs, const float* rhs_scale, int32_t rhs_scale_len,
                            const int32_t* group_sizes, int32_t E, int32_t group_offset,
                            int32_t num_local_experts, int64_t M, int64_t K, int64_t N, int out_dtype,
                            void* out, void* ws, size_t ws_bytes, void* stream) {
  if (M < 0 || K <= 0 || N <= 0 || K % 16 || N % 16) return MOE_ERR_SHAPE;
  if (E <= 0 || E > 1024 || group_offset < 0 || num_local_experts < 0 ||
      num_local_experts > moe::tile::kMaxLocal || group_offset + num_local_experts > E)
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
  if (ws_bytes < moe::tile::kHdr) return MOE_ERR_WORKSPACE;
  if (static_cast<int64_t>(El) * moe_cdiv(K, 64) * moe_cdiv(N, 64) > INT32_MAX) return MOE_ERR_SHAPE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  int32_t* err = static_cast<int32_t*>(ws);
  if (K % 128 || N % 128)        // multiples of 16 only: the edge kernel
    return moe::tgmm_edge_launch(lhs, lhs_scale, lhs_scale_len, rhs, rhs_scale, rhs_scale_len, group_sizes,
                                 group_offset, El, M, K, N, out_dtype == MOE_BF16, out, err, st) == hipSuccess
               ? MOE_OK : MOE_ERR_HIP;
  // Main path: both operands transposed into the workspace (each group's rows
  // become a contraction axis of their own), then the gmm pipeline per group.
  // The one-kernel path (transposing in LDS while multiplying) serves smaller
  // workspaces and K not a multiple of 256.
  if (K % 256 == 0 && ws_bytes >= moe::tgmm_ws_bytes(M, K, N, E)) {
    const int64_t Mpad = moe::tgmm_mpad(M, E);
    uint8_t* XT = static_cast<uint8_t*>(ws) + moe::tile::kHdr;
    uint8_t* DT = XT + K * Mpad;
    const unsigned tgrid = static_cast<unsigned>(4 * moe::tile::num_cus());
    if (M > 0) {
      moe::transpose_groups_kernel<0><<<tgrid, 256, 0, st>>>(lhs, K, group_sizes, group_offset, El, M, Mpad, XT, err,
                                                             nullptr, 1, 0, 1.0f);
      MOE_CHECK_LAUNCH();
      moe::transpose_groups_kernel<0><<<tgrid, 256, 0, st>>>(rhs, N, group_sizes, group_offset, El, M, Mpad, DT, err,
                                                             nullptr, 1, 0, 1.0f);
      MOE_CHECK_LAUNCH();
    }
    return moe::gmm_batched_launch(XT, lhs_scale, lhs_scale_len, DT, rhs_scale, rhs_scale_len, group_sizes,
                                   group_offset, El, M, K, Mpad, N, out_dtype == MOE_BF16, out, err, st) == hipSuccess
               ? MOE_OK : MOE_ERR_HIP;
  }
  const int64_t ub = static_cast<int64_t>(El) * (K / moe::tile::BM) * (N / moe::tile::BN);
  int64_t grid = 2LL * moe::tile::num_cus();
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

extern "C" int moe_tgmm_xt_cols(int64_t M, int32_t E, int64_t* cols) {
  if (!cols) return MOE_ERR_NULL;
  if (M < 0 || E <= 0 || E > 1024) return MOE_ERR_SHAPE;
  *cols = moe::tgmm_mpad(M, E);
  return MOE_OK;
}

extern "C" int moe_sort_gather_transposed(const void* x, int x_dtype, float static_scale, int64_t T, int32_t k,
                                          int64_t H, const int32_t* perm, const int32_t* group_sizes, int32_t E,
                                          int32_t group_offset, int32_t num_local_experts, int64_t M, uint8_t* xt,
                                          float* scale_out, void* ws, size_t ws_bytes, void* stream) {
  if (T < 0 || k <= 0 || k > 64 || H <= 0 || M < 0) return MOE_ERR_SHAPE;
  if (H % 256) return MOE_ERR_UNSUPPORTED;
  if (E <= 0 || E > 1024 || group_offset < 0 || num_local_experts < 0 ||
      num_local_experts > moe::tile::kMaxLocal || group_offset + num_local_experts > E)
    return MOE_ERR_SHAPE;
  if (T * k > INT32_MAX - 1 || M > INT32_MAX - 1) return MOE_ERR_SHAPE;
  if (x_dtype != MOE_E4M3FN && x_dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (x_dtype == MOE_BF16 && !(static_scale > 0.0f && static_scale < 3.0e38f)) return MOE_ERR_SHAPE;
  if (!group_sizes) return MOE_ERR_NULL;
  if (!ws) return MOE_ERR_WORKSPACE;
  if (ws_bytes < moe::tile::kHdr) return MOE_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  int32_t* err = static_cast<int32_t*>(ws);
  if (scale_out && x_dtype == MOE_BF16) {
    moe::write_scale_kernel<<<1, 1, 0, st>>>(scale_out, static_scale);
    MOE_CHECK_LAUNCH();
  }
  const int El = num_local_experts;
  if (El == 0 || M == 0 || T == 0) return MOE_OK;
  if (!x || !perm || !xt) return MOE_ERR_NULL;
  const int64_t Mpad = moe::tgmm_mpad(M, E);
  const unsigned tgrid = static_cast<unsigned>(4 * moe::tile::num_cus());
  const uint8_t* src = static_cast<const uint8_t*>(x);
  if (x_dtype == MOE_E4M3FN)
    moe::transpose_groups_kernel<1><<<tgrid, 256, 0, st>>>(src, H, group_sizes, group_offset, El, M, Mpad, xt, err,
                                                           perm, k, T, 1.0f);
  else
    moe::transpose_groups_kernel<2><<<tgrid, 256, 0, st>>>(src, H, group_sizes, group_offset, El, M, Mpad, xt, err,
                                                           perm, k, T, static_scale);
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}

extern "C" int moe_tgmm_fp8_xt(const uint8_t* xt, const float* lhs_scale, int32_t lhs_scale_len, const uint8_t* rhs,
                               const float* rhs_scale, int32_t rhs_scale_len, const int32_t* group_sizes, int32_t E,
                               int32_t group_offset, int32_t num_local_experts, int64_t M, int64_t K, int64_t N,
                               int out_dtype, void* out, void* ws, size_t ws_bytes, void* stream) {
  if (M < 0 || K <= 0 || N <= 0) return MOE_ERR_SHAPE;
  if (K % 256 || N % 128) return MOE_ERR_UNSUPPORTED;
  if (E <= 0 || E > 1024 || group_offset < 0 || num_local_experts < 0 ||
      num_local_experts > moe::tile::kMaxLocal || group_offset + num_local_experts > E)
    return MOE_ERR_SHAPE;
  if (M > INT32_MAX - 1) return MOE_ERR_SHAPE;
  if (lhs_scale_len != 1 && lhs_scale_len != K) return MOE_ERR_UNSUPPORTED;
  if (rhs_scale_len != 1 && rhs_scale_len != N) return MOE_ERR_UNSUPPORTED;
  if (out_dtype == MOE_DTYPE_DEFAULT) out_dtype = MOE_F32;
  if (out_dtype != MOE_BF16 && out_dtype != MOE_F32) return MOE_ERR_UNSUPPORTED;
  const int El = num_local_experts;
  if (El == 0) return MOE_OK;
  if (!out || !group_sizes || !lhs_scale || !rhs_scale) return MOE_ERR_NULL;
  if (M > 0 && (!xt || !rhs)) return MOE_ERR_NULL;
  if (!ws) return MOE_ERR_WORKSPACE;
  const int64_t Mpad = moe::tgmm_mpad(M, E);
  if (ws_bytes < static_cast<size_t>(moe::tile::kHdr + N * Mpad)) return MOE_ERR_WORKSPACE;
  if (static_cast<int64_t>(El) * moe_cdiv(K, 64) * moe_cdiv(N, 64) > INT32_MAX) return MOE_ERR_SHAPE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  int32_t* err = static_cast<int32_t*>(ws);
  uint8_t* DT = static_cast<uint8_t*>(ws) + moe::tile::kHdr;
  if (M > 0) {
    const unsigned tgrid = static_cast<unsigned>(4 * moe::tile::num_cus());
    moe::transpose_groups_kernel<0><<<tgrid, 256, 0, st>>>(rhs, N, group_sizes, group_offset, El, M, Mpad, DT, err,
                                                           nullptr, 1, 0, 1.0f);
    MOE_CHECK_LAUNCH();
  }
  return moe::gmm_batched_launch(xt, lhs_scale, lhs_scale_len, DT, rhs_scale, rhs_scale_len, group_sizes,
                                 group_offset, El, M, K, Mpad, N, out_dtype == MOE_BF16, out, err, st) == hipSuccess
             ? MOE_OK : MOE_ERR_HIP;
}
