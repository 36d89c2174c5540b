// moe_sort_by_expert: stable ragged sort of the routed rows by expert and the
// gather of the quantized token rows into that order ("Quantize activations
// before EP all gather": review comments on ragged_sort.py -- fp8 rows are
// gathered by the sorted token indices into this shard's window, the scale
// follows only when it is per token).
//
// Three or four launches on the caller's stream:
//  1. hist   one block per tile of 512 routed slots (2048 for inputs whose
//            tile table would not fit in LDS): per-tile expert counts.
//  2. scan   per-expert exclusive scan over tiles, the expert bases,
//            group_sizes, and this shard's window (start, n).  When the tile
//            table fits in LDS every rank block does this itself (no launch);
//            otherwise one block does it in global memory.
//  3. rank   one block per tile: the stable rank of every slot inside its
//            tile (a wave ranks 64 slots at a time: ballots over the bits of
//            the expert id give each lane the set of lanes holding the same
//            expert -- the warp-level multisplit of Ashkiani et al., 2016 --
//            and a per-wave running count per expert in LDS carries the order
//            across chunks); writes perm and inv_pos.
//  4. scatter one wave per token: reads the token's fp8 row once and writes
//            it to each of its local destinations; extra waves zero rows
//            [n, M_cap).  Coalesced 16-byte loads and stores.
// No float atomics and no order-dependent steps: the result is deterministic.
#include <mutex>

#include "quant_common.hpp"

namespace moe {
namespace {

constexpr int kTile = 2048;          // routed slots per tile (256 threads x 8), large inputs
constexpr int kTileSmall = 512;      // routed slots per tile when the tile table fits in LDS
constexpr int kScanLds = 15104;      // int32 entries of the tile table the scan keeps in LDS (59 KiB: with a
                                     // row of counts and the kernel's own 68 bytes it stays within 64 KiB)
constexpr int kHdr = 256;            // workspace header bytes
// header int32 slots
constexpr int kErr = 0, kStart = 1, kN = 2, kValid = 3;

__device__ __forceinline__ int key_of(int32_t id, int E, int32_t* err) {
  if (id < 0 || id >= E) {
    raise_error(err, MOE_DEVERR_EXPERT_ID);
    return E;                         // invalid ids form a bucket after every expert
  }
  return id;
}

template <int TILE>
__global__ __launch_bounds__(256) void sort_hist_kernel(const int32_t* __restrict__ ids, int64_t M, int E,
                                                        int32_t* __restrict__ err, int32_t* __restrict__ tile_hist) {
  extern __shared__ int hist[];
  // every load of the thread's ids goes out before the first is used (one memory latency, not one per id)
  const int64_t base = static_cast<int64_t>(blockIdx.x) * TILE;
  int idv[TILE / 256];
#pragma unroll
  for (int i = 0; i < TILE / 256; ++i) {
    const int64_t f = base + i * 256 + threadIdx.x;
    idv[i] = f < M ? ids[f] : -1;
  }
  for (int e = threadIdx.x; e <= E; e += 256) hist[e] = 0;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < TILE / 256; ++i) {
    const int64_t f = base + i * 256 + threadIdx.x;
    if (f < M) atomicAdd(&hist[key_of(idv[i], E, err)], 1);
  }
  __syncthreads();
  int32_t* out = tile_hist + static_cast<int64_t>(blockIdx.x) * (E + 1);
  for (int e = threadIdx.x; e <= E; e += 256) out[e] = hist[e];
}

// Copy n ints from global memory to LDS with `nthreads` threads: each thread
// issues up to 32 independent loads before their LDS stores, so a table of
// up to 32 cells per thread costs one memory latency instead of one per cell.
__device__ __forceinline__ void copy_to_lds(const int32_t* __restrict__ src, int* dst, int n, int nthreads) {
  constexpr int U = 32;
  for (int i0 = threadIdx.x; i0 < n; i0 += U * nthreads) {
    int v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u * nthreads;
      v[u] = i < n ? src[i] : 0;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u * nthreads;
      if (i < n) dst[i] = v[u];
    }
  }
}

// Exclusive prefix sum of a[0..n) in LDS by every wave of the block: each
// 64-entry chunk is scanned by one wave with lane shuffles, then every entry
// adds the totals of the chunks before it (wt: at least ceil(n / 64) ints).
__device__ void block_exclusive_scan(int* a, int n, int* wt) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int nch = (n + 63) / 64;
  for (int c = w; c < nch; c += nw) {
    const int i = c * 64 + lane;
    const int v = i < n ? a[i] : 0;
    int incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(incl, o, 64);
      if (lane >= o) incl += t;
    }
    if (i < n) a[i] = incl - v;
    if (lane == 63) wt[c] = incl;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    int s = 0;
    for (int c = 0; c < i / 64; ++c) s += wt[c];
    a[i] += s;
  }
}

// in_lds: the whole [ntiles][E + 1] table is read into LDS with coalesced
// loads, scanned there and written back (small tables); otherwise each
// thread walks its experts' column in global memory.
__global__ __launch_bounds__(1024) void sort_scan_kernel(int32_t* __restrict__ tile_hist, int ntiles, int E,
                                                         int g0, int El, int32_t* __restrict__ group_sizes,
                                                         int32_t* __restrict__ hdr, int in_lds) {
  extern __shared__ int tot[];        // [E + 1], then the table when in_lds
  __shared__ int wt[17];              // chunk totals of the expert scan (E + 1 <= 1025)
  int* tab = tot + (E + 1);
  const int64_t cells = static_cast<int64_t>(ntiles) * (E + 1);
  int32_t* col = in_lds ? tab : tile_hist;
  if (in_lds) {
    copy_to_lds(tile_hist, tab, static_cast<int>(cells), blockDim.x);
    __syncthreads();
  }
  for (int e = threadIdx.x; e <= E; e += blockDim.x) {
    int run = 0;
    for (int t = 0; t < ntiles; ++t) {
      const int c = col[static_cast<int64_t>(t) * (E + 1) + e];
      col[static_cast<int64_t>(t) * (E + 1) + e] = run;
      run += c;
    }
    tot[e] = run;
    if (e < E) group_sizes[e] = run;
  }
  __syncthreads();
  block_exclusive_scan(tot, E + 1, wt);
  __syncthreads();
  if (in_lds) {
    for (int64_t i = threadIdx.x; i < cells; i += blockDim.x) tile_hist[i] = tab[i] + tot[i % (E + 1)];
  } else {
    for (int e = threadIdx.x; e <= E; e += blockDim.x) {
      const int b = tot[e];
      for (int t = 0; t < ntiles; ++t) tile_hist[static_cast<int64_t>(t) * (E + 1) + e] += b;
    }
  }
  if (threadIdx.x == 0) {
    const int start = tot[g0];
    hdr[kStart] = start;
    hdr[kN] = tot[g0 + El] - start;
    hdr[kValid] = tot[E];
  }
}

// FUSED_SCAN: tile_off holds the per-tile counts (no scan kernel ran); every
// block reads the whole [ntiles][E + 1] table into LDS and derives its own
// tile's offsets -- the counts of the earlier tiles plus the expert bases --
// and block 0 writes group_sizes and the window header.  Otherwise tile_off
// holds the offsets the scan kernel wrote.  NWV waves per block, each ranking
// TILE / NWV slots: the phases are latency chains, so more waves per tile
// shorten every one of them.
template <int TILE, bool FUSED_SCAN, int NWV>
__global__ __launch_bounds__(64 * NWV) void sort_rank_kernel(const int32_t* __restrict__ ids, int64_t M, int E,
                                                             int nbits, int64_t M_cap, int32_t* __restrict__ hdr,
                                                             int32_t* __restrict__ err,
                                                             const int32_t* __restrict__ tile_off, int ntiles, int g0,
                                                             int El, int32_t* __restrict__ group_sizes,
                                                             int32_t* __restrict__ perm, int32_t* __restrict__ inv_pos) {
  constexpr int NT = 64 * NWV, CH = TILE / NT;   // threads; 64-slot chunks per wave
  static_assert(CH >= 1 && TILE % NT == 0, "whole chunks per wave");
  extern __shared__ int lds[];
  int* cnt = lds;                      // [NWV][E + 1] running counts per wave
  int* off = lds + NWV * (E + 1);      // [E + 1] global base of this tile
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  __shared__ int win[2];               // start, n of the local window
  __shared__ int wt[17];               // chunk totals of the expert scan (E + 1 <= 1025)
  // the thread's ids, loaded first: their latency overlaps the offsets' set-up, and the ranking below
  // never waits for memory chunk by chunk
  const int64_t wbase = static_cast<int64_t>(blockIdx.x) * TILE + w * (TILE / NWV);
  int idv[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int64_t f = wbase + c * 64 + lane;
    idv[c] = f < M ? ids[f] : 0;
  }
  if constexpr (FUSED_SCAN) {
    int* tab = off + (E + 1);          // [ntiles][E + 1] counts
    int* tot = tab + ntiles * (E + 1); // [E + 1] totals, then their exclusive scan
    const int cells = ntiles * (E + 1);
    copy_to_lds(tile_off, tab, cells, NT);
    __syncthreads();
    // each expert's counts over the earlier tiles and over all tiles, P threads per expert (P a power of
    // two, so a group of P lanes sits in one wave), combined with lane shuffles
    int P = 1;
    while (P < 16 && 2 * P * (E + 1) <= NT) P *= 2;
    const int part = threadIdx.x & (P - 1);
    for (int e0 = 0; e0 <= E; e0 += NT / P) {
      const int e = e0 + static_cast<int>(threadIdx.x) / P;
      int before = 0, all = 0;
      if (e <= E) {
        for (int t = part; t < ntiles; t += P) {
          const int c = tab[t * (E + 1) + e];
          before += t < static_cast<int>(blockIdx.x) ? c : 0;
          all += c;
        }
      }
      for (int o = 1; o < P; o <<= 1) {
        before += __shfl_xor(before, o, 64);
        all += __shfl_xor(all, o, 64);
      }
      if (e <= E && part == 0) {
        off[e] = before;
        tot[e] = all;
        if (blockIdx.x == 0 && e < E) group_sizes[e] = all;
      }
    }
    __syncthreads();
    block_exclusive_scan(tot, E + 1, wt);
    __syncthreads();
    for (int e = threadIdx.x; e <= E; e += NT) off[e] += tot[e];
    if (threadIdx.x == 0) {
      win[0] = tot[g0];
      win[1] = tot[g0 + El] - tot[g0];
      if (blockIdx.x == 0) {
        hdr[kStart] = win[0];
        hdr[kN] = win[1];
        hdr[kValid] = tot[E];
      }
    }
  } else {
    for (int e = threadIdx.x; e <= E; e += NT) off[e] = tile_off[static_cast<int64_t>(blockIdx.x) * (E + 1) + e];
    if (threadIdx.x == 0) {
      win[0] = hdr[kStart];
      win[1] = hdr[kN];
    }
  }
  for (int i = threadIdx.x; i < NWV * (E + 1); i += NT) cnt[i] = 0;
  __syncthreads();
  const uint64_t lt_mask = (1ull << lane) - 1ull;
  int keys[CH], rank[CH];
  int* my = cnt + w * (E + 1);
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int64_t f = wbase + c * 64 + lane;
    const bool valid = f < M;
    const int key = valid ? key_of(idv[c], E, nullptr) : 0;
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (key >> b) & 1;
      const uint64_t bb = __ballot(bit);
      peers &= bit ? bb : ~bb;
    }
    const int r = __popcll(peers & lt_mask);
    int prior = 0;
    if (valid) prior = my[key];
    __builtin_amdgcn_wave_barrier();
    if (valid && r == 0) my[key] = prior + __popcll(peers);
    __builtin_amdgcn_wave_barrier();
    keys[c] = valid ? key : -1;
    rank[c] = prior + r;
  }
  __syncthreads();
  for (int e = threadIdx.x; e <= E; e += NT) {   // each wave's base: the counts of the waves before it
    int s = 0;
#pragma unroll
    for (int ww = 0; ww < NWV; ++ww) {
      const int t = cnt[ww * (E + 1) + e];
      cnt[ww * (E + 1) + e] = s;
      s += t;
    }
  }
  __syncthreads();
  const int start = win[0], n = win[1];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int key = keys[c];
    if (key < 0) continue;
    const int64_t f = wbase + c * 64 + lane;
    const int pos = off[key] + my[key] + rank[c];
    perm[pos] = static_cast<int32_t>(f);
    int ip = -1;
    if (key < E && pos >= start && pos < start + n) {
      ip = pos - start;
      if (ip >= M_cap) {
        raise_error(err, MOE_DEVERR_ROWS);
        ip = -1;
      }
    }
    inv_pos[f] = ip;
  }
}

// One wave per token row (grid-strided), then the zero tail of xs / ss.
__global__ __launch_bounds__(256) void sort_scatter_kernel(const uint8_t* __restrict__ xq, const float* __restrict__ xscale,
                                                           int row_scale, const int32_t* __restrict__ inv_pos, int64_t T,
                                                           int k, int64_t H, int64_t M_cap,
                                                           const int32_t* __restrict__ hdr, uint8_t* __restrict__ xs,
                                                           float* __restrict__ ss) {
  const int lane = threadIdx.x & 63;
  const int64_t nw = static_cast<int64_t>(gridDim.x) * 4;
  const int64_t wid = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int64_t segs = H >> 4;
  if (xq) {
    for (int64_t t = wid; t < T; t += nw) {
      int my_r = -1;
      if (lane < k) my_r = inv_pos[t * k + lane];
      if (my_r >= M_cap) my_r = -1;
      if (my_r >= 0 && row_scale && ss) ss[my_r] = xscale[t];
      uint64_t m = __ballot(my_r >= 0);
      if (m == 0) continue;
      const uint4* src = reinterpret_cast<const uint4*>(xq + t * H);
      for (int64_t s = lane; s < segs; s += 64) {
        const uint4 v = src[s];
        uint64_t mm = m;
        while (mm) {
          const int j = __builtin_ctzll(mm);
          mm &= mm - 1;
          const int r = __builtin_amdgcn_readlane(my_r, j);
          reinterpret_cast<uint4*>(xs + static_cast<int64_t>(r) * H)[s] = v;
        }
      }
    }
  } else if (row_scale && ss) {
    for (int64_t t = wid; t < T; t += nw) {
      if (lane < k) {
        const int r = inv_pos[t * k + lane];
        if (r >= 0 && r < M_cap) ss[r] = xscale[t];
      }
    }
  }
  int64_t n = hdr[kN];
  if (n > M_cap) n = M_cap;
  for (int64_t r = n + wid; r < M_cap; r += nw) {
    if (xs) {
      uint4* dst = reinterpret_cast<uint4*>(xs + r * H);
      for (int64_t s = lane; s < segs; s += 64) dst[s] = make_uint4(0, 0, 0, 0);
    }
    if (ss && row_scale && lane == 0) ss[r] = 0.0f;
  }
}

// The fused quantize-and-gather (one GPU): one wave per token reads the
// token's bf16 row once, forms its absmax and e4m3fn codes in registers with
// the row quantizer's own functions (same bytes as moe_quantize_rows), and
// writes each 16-byte group of codes to every local destination row of the
// token; a token without one is skipped unless its scale is asked for.
// GPL 16-element groups per lane keep rows of up to GPL * 1024 elements in
// registers; GPL = 0 reads the row twice (absmax pass, then codes).  Rows
// [n, M_cap) get zeros.
template <int GPL>
__device__ __forceinline__ void load_group16(const uint16_t* __restrict__ row, int64_t gi, float v[16]) {
  Bf16x8 a, b;
  a.raw = *reinterpret_cast<const uint4*>(row + gi * 16);
  b.raw = *reinterpret_cast<const uint4*>(row + gi * 16 + 8);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[i] = a.get(i);
    v[8 + i] = b.get(i);
  }
}

__device__ __forceinline__ void scatter_codes(uint8_t* __restrict__ xs, int64_t H, int64_t gi, uint64_t m, int my_r,
                                              const float v[16], const RowDiv& d) {
  const uint2 lo = codes8(v, d), hi = codes8(v + 8, d);
  const uint4 code = make_uint4(lo.x, lo.y, hi.x, hi.y);
  while (m) {
    const int j = __builtin_ctzll(m);
    m &= m - 1;
    const int r = __builtin_amdgcn_readlane(my_r, j);
    *reinterpret_cast<uint4*>(xs + static_cast<int64_t>(r) * H + gi * 16) = code;
  }
}

// given_scale (device [1], the tensor scale from row maxima) or static_mode
// make it a tensor mode: one scale, no per-row scales; in row mode row_amax
// (optional) receives every token's absmax.
template <int GPL>
__global__ __launch_bounds__(256) void quantize_scatter_kernel(const uint16_t* __restrict__ x, int static_mode,
                                                               float static_scale, const float* __restrict__ given_scale,
                                                               const int32_t* __restrict__ inv_pos,
                                                               int64_t T, int k, int64_t H, int64_t M_cap,
                                                               const int32_t* __restrict__ hdr, uint8_t* __restrict__ xs,
                                                               float* __restrict__ ss, float* __restrict__ tok_scale,
                                                               float* __restrict__ row_amax) {
  const int lane = threadIdx.x & 63;
  const int64_t nw = static_cast<int64_t>(gridDim.x) * 4;
  const int64_t wid = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int64_t G = H >> 4;
  const bool tensor = static_mode || given_scale;
  const bool every = !tensor && (tok_scale || row_amax);   // every token's scale or absmax is asked for
  if (static_mode && tok_scale && wid == 0 && lane == 0) tok_scale[0] = static_scale;
  for (int64_t t = wid; t < T; t += nw) {
    const uint16_t* row = x + t * H;
    // the row's groups (index clamped into the row) are loaded together
    // with the token's destinations: one memory latency, not one per load
    Bf16x8 ra[GPL > 0 ? GPL : 1][2];
    if constexpr (GPL > 0) {
#pragma unroll
      for (int c = 0; c < GPL; ++c) {
        const int64_t gi = lane + 64 * c;
        const int64_t gl = gi < G ? gi : G - 1;
        ra[c][0].raw = *reinterpret_cast<const uint4*>(row + gl * 16);
        ra[c][1].raw = *reinterpret_cast<const uint4*>(row + gl * 16 + 8);
      }
    }
    int my_r = -1;
    if (lane < k) my_r = inv_pos[t * k + lane];
    if (my_r >= M_cap) my_r = -1;
    const uint64_t m = __ballot(my_r >= 0);
    if (m == 0 && !every) continue;
    float amax = 0.0f;
    if constexpr (GPL > 0) {
      float v[GPL][16];
#pragma unroll
      for (int c = 0; c < GPL; ++c) {
        const int64_t gi = lane + 64 * c;
        if (gi < G) {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            v[c][i] = ra[c][0].get(i);
            v[c][8 + i] = ra[c][1].get(i);
          }
#pragma unroll
          for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[c][i]));
        }
      }
      amax = wave_max(amax);
      const float s = given_scale ? *given_scale : static_mode ? static_scale : scale_from_amax(amax);
      const RowDiv d(s);
#pragma unroll
      for (int c = 0; c < GPL; ++c) {
        const int64_t gi = lane + 64 * c;
        if (gi < G) scatter_codes(xs, H, gi, m, my_r, v[c], d);
      }
      if (!tensor) {
        if (my_r >= 0 && ss) ss[my_r] = s;
        if (tok_scale && lane == 0) tok_scale[t] = s;
        if (row_amax && lane == 0) row_amax[t] = amax;
      }
    } else {
      for (int64_t gi = lane; gi < G; gi += 64) {
        float v[16];
        load_group16<0>(row, gi, v);
#pragma unroll
        for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
      }
      amax = wave_max(amax);
      const float s = given_scale ? *given_scale : static_mode ? static_scale : scale_from_amax(amax);
      const RowDiv d(s);
      for (int64_t gi = lane; gi < G; gi += 64) {
        float v[16];
        load_group16<0>(row, gi, v);
        scatter_codes(xs, H, gi, m, my_r, v, d);
      }
      if (!tensor) {
        if (my_r >= 0 && ss) ss[my_r] = s;
        if (tok_scale && lane == 0) tok_scale[t] = s;
        if (row_amax && lane == 0) row_amax[t] = amax;
      }
    }
  }
  int64_t n = hdr[kN];
  if (n > M_cap) n = M_cap;
  for (int64_t r = n + wid; r < M_cap; r += nw) {
    uint4* dst = reinterpret_cast<uint4*>(xs + r * H);
    for (int64_t c = lane; c < (H >> 4); c += 64) dst[c] = make_uint4(0, 0, 0, 0);
    if (ss && !tensor && lane == 0) ss[r] = 0.0f;
  }
}

}  // namespace

size_t sort_ws_bytes(int64_t M, int E) {
  const int64_t ntiles = moe_cdiv(M, kTileSmall);      // enough for either tile size
  return kHdr + static_cast<size_t>(moe_cdiv(ntiles * (E + 1) * 4, 256) * 256);
}

}  // namespace moe

namespace moe {
namespace {
// The sort's metadata stages (histogram, scan, stable rank) into perm,
// inv_pos, group_sizes and the window header hdr; tile_hist holds
// sort_ws_bytes(M, E) - kHdr bytes; device-data errors are OR'ed into err
// (may be NULL).
int sort_metadata(const int32_t* expert_ids, int64_t T, int32_t k, int32_t E, int32_t group_offset,
                  int32_t num_local_experts, int64_t M_cap, int32_t* perm, int32_t* inv_pos, int32_t* group_sizes,
                  int32_t* hdr, int32_t* tile_hist, int32_t* err, hipStream_t st) {
  const int64_t M = T * k;
  // small tiles (more workgroups) whenever their table fits the scan's LDS
  const bool small = moe_cdiv(M, kTileSmall) * (E + 1) <= kScanLds;
  const int tile = small ? kTileSmall : kTile;
  const int ntiles = static_cast<int>(moe_cdiv(M, tile));
  const bool scan_in_lds = static_cast<int64_t>(ntiles) * (E + 1) <= kScanLds;
  int nbits = 0;
  while ((1 << nbits) < E + 1) ++nbits;
  const size_t hist_lds = (E + 1) * sizeof(int);
  if (ntiles > 0) {
    if (small)
      sort_hist_kernel<kTileSmall><<<ntiles, 256, hist_lds, st>>>(expert_ids, M, E, err, tile_hist);
    else
      sort_hist_kernel<kTile><<<ntiles, 256, hist_lds, st>>>(expert_ids, M, E, err, tile_hist);
    MOE_CHECK_LAUNCH();
  }
  // hist -> rank with the scan fused into every rank block when the tile
  // table fits in LDS; hist -> scan -> rank otherwise.  Rank blocks: 16 waves
  // on a 2048-slot tile, 8 on a 512-slot tile (two and one 64-slot chunks per
  // wave) with a row of per-wave counts each in LDS; 4 waves where that would
  // not fit in 64 KiB (many experts).
  const size_t table_lds = static_cast<size_t>(ntiles) * (E + 1) * sizeof(int);
  auto rank_lds = [&](int nwv, bool fused) { return (nwv + (fused ? 2 : 1)) * hist_lds + (fused ? table_lds : 0); };
  constexpr size_t kMaxLds = 64 * 1024 - 256;    // dynamic LDS, leaving room for the kernel's own arrays
  const bool fused = ntiles > 0 && scan_in_lds && rank_lds(4, true) <= kMaxLds;
  const bool wide = rank_lds(small ? 8 : 16, fused) <= kMaxLds;
  const size_t lds = rank_lds(wide ? (small ? 8 : 16) : 4, fused);
  if (!fused) {
    const size_t scan_lds = hist_lds + (scan_in_lds ? table_lds : 0);
    sort_scan_kernel<<<1, 1024, scan_lds, st>>>(tile_hist, ntiles, E, group_offset, num_local_experts,
                                                     group_sizes, hdr, scan_in_lds ? 1 : 0);
    MOE_CHECK_LAUNCH();
  }
  if (ntiles > 0) {
#define MOE_RANK(TILE, FUSED, NWV)                                                                              \
  sort_rank_kernel<TILE, FUSED, NWV><<<ntiles, 64 * NWV, lds, st>>>(expert_ids, M, E, nbits, M_cap, hdr, err,   \
                                                                     tile_hist, ntiles, group_offset,          \
                                                                     num_local_experts, group_sizes, perm, inv_pos)
    if (small) {
      if (fused) { if (wide) MOE_RANK(kTileSmall, true, 8); else MOE_RANK(kTileSmall, true, 4); }
      else { if (wide) MOE_RANK(kTileSmall, false, 8); else MOE_RANK(kTileSmall, false, 4); }
    } else {
      if (fused) { if (wide) MOE_RANK(kTile, true, 16); else MOE_RANK(kTile, true, 4); }
      else { if (wide) MOE_RANK(kTile, false, 16); else MOE_RANK(kTile, false, 4); }
    }
#undef MOE_RANK
    MOE_CHECK_LAUNCH();
  }
  return MOE_OK;
}

// Argument checks of moe_sort_by_expert that do not involve the workspace.
int sort_check(const int32_t* expert_ids, int64_t T, int32_t k, int32_t E, int32_t group_offset,
               int32_t num_local_experts, const uint8_t* xq, const float* xscale, int xscale_mode, int64_t H,
               int64_t M_cap, const int32_t* perm, const int32_t* inv_pos, const int32_t* group_sizes,
               const uint8_t* xs, const float* ss) {
  if (T < 0 || k <= 0 || k > 64 || E <= 0 || E > 1024) return MOE_ERR_SHAPE;
  if (group_offset < 0 || num_local_experts < 0 || group_offset + num_local_experts > E) return MOE_ERR_SHAPE;
  if (M_cap < 0 || T * k > INT32_MAX - 1) return MOE_ERR_SHAPE;
  if (xscale_mode != MOE_SCALE_ROW_DYNAMIC && xscale_mode != MOE_SCALE_TENSOR_DYNAMIC &&
      xscale_mode != MOE_SCALE_TENSOR_STATIC)
    return MOE_ERR_UNSUPPORTED;
  if (xq && (H <= 0 || H % 16)) return MOE_ERR_SHAPE;
  const int64_t M = T * k;
  if (!group_sizes || (M > 0 && (!expert_ids || !perm || !inv_pos))) return MOE_ERR_NULL;
  if (xq && M_cap > 0 && !xs) return MOE_ERR_NULL;
  const bool row_scale = xscale_mode == MOE_SCALE_ROW_DYNAMIC;
  if (row_scale && xscale && M_cap > 0 && !ss) return MOE_ERR_NULL;
  if (row_scale && ss && T > 0 && !xscale) return MOE_ERR_NULL;
  return MOE_OK;
}

// The whole sort on the given header, table and error word: metadata, then
// the gather of the token rows (and per-token scales) when asked for.
int sort_run(const int32_t* expert_ids, int64_t T, int32_t k, int32_t E, int32_t group_offset,
             int32_t num_local_experts, const uint8_t* xq, const float* xscale, int xscale_mode, int64_t H,
             int64_t M_cap, int32_t* perm, int32_t* inv_pos, int32_t* group_sizes, uint8_t* xs, float* ss,
             int32_t* hdr, int32_t* tile_hist, int32_t* err, hipStream_t st) {
  const int rc = sort_metadata(expert_ids, T, k, E, group_offset, num_local_experts, M_cap, perm, inv_pos,
                               group_sizes, hdr, tile_hist, err, st);
  if (rc != MOE_OK) return rc;
  if (xs || ss) {
    int64_t waves = T > M_cap / 4 ? T : M_cap / 4;
    if (waves < 4) waves = 4;
    if (waves > 65536) waves = 65536;
    sort_scatter_kernel<<<static_cast<unsigned>(moe_cdiv(waves, 4)), 256, 0, st>>>(
        xq, xscale, xscale_mode == MOE_SCALE_ROW_DYNAMIC ? 1 : 0, inv_pos, T, k, H, M_cap, hdr, xs, ss);
    MOE_CHECK_LAUNCH();
  }
  return MOE_OK;
}
}  // namespace
}  // namespace moe

extern "C" int moe_sort_by_expert(const int32_t* expert_ids, int64_t T, int32_t k, int32_t E,
                                  int32_t group_offset, int32_t num_local_experts, const uint8_t* xq,
                                  const float* xscale, int xscale_mode, int64_t H, int64_t M_cap,
                                  int32_t* perm, int32_t* inv_pos, int32_t* group_sizes, uint8_t* xs,
                                  float* ss, void* ws, size_t ws_bytes, void* stream) {
  const int rc = moe::sort_check(expert_ids, T, k, E, group_offset, num_local_experts, xq, xscale, xscale_mode, H,
                                 M_cap, perm, inv_pos, group_sizes, xs, ss);
  if (rc != MOE_OK) return rc;
  if (!ws) return MOE_ERR_NULL;
  if (ws_bytes < moe::sort_ws_bytes(T * k, E)) return MOE_ERR_WORKSPACE;
  int32_t* hdr = static_cast<int32_t*>(ws);
  int32_t* tile_hist = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + moe::kHdr);
  return moe::sort_run(expert_ids, T, k, E, group_offset, num_local_experts, xq, xscale, xscale_mode, H, M_cap,
                       perm, inv_pos, group_sizes, xs, ss, hdr, tile_hist, hdr + moe::kErr,
                       static_cast<hipStream_t>(stream));
}

extern "C" int moe_quantize_sort_by_expert(const void* x, int64_t T, int64_t H, int scale_mode, float static_scale,
                                           const int32_t* expert_ids, int32_t k, int32_t E, int32_t group_offset,
                                           int32_t num_local_experts, int64_t M_cap, int32_t* perm, int32_t* inv_pos,
                                           int32_t* group_sizes, uint8_t* xs, float* ss, float* scale,
                                           float* row_amax, void* ws, size_t ws_bytes, void* stream) {
  if (T < 0 || k <= 0 || k > 64 || E <= 0 || E > 1024) return MOE_ERR_SHAPE;
  if (group_offset < 0 || num_local_experts < 0 || group_offset + num_local_experts > E) return MOE_ERR_SHAPE;
  if (M_cap < 0 || T * k > INT32_MAX - 1) return MOE_ERR_SHAPE;
  if (H <= 0 || H % 16) return MOE_ERR_SHAPE;
  if (scale_mode == MOE_SCALE_TENSOR_DYNAMIC) return MOE_ERR_UNSUPPORTED;   // needs the whole tensor first
  if (scale_mode != MOE_SCALE_ROW_DYNAMIC && scale_mode != MOE_SCALE_TENSOR_STATIC &&
      scale_mode != MOE_SCALE_TENSOR_FROM_ROW_AMAX)
    return MOE_ERR_UNSUPPORTED;
  const bool static_mode = scale_mode == MOE_SCALE_TENSOR_STATIC;
  const bool from_rows = scale_mode == MOE_SCALE_TENSOR_FROM_ROW_AMAX;
  const bool tensor = static_mode || from_rows;
  if (static_mode && !(static_scale > 0.0f && static_scale < 3.0e38f)) return MOE_ERR_SHAPE;
  const int64_t M = T * k;
  if (!group_sizes || !ws || (M > 0 && (!expert_ids || !perm || !inv_pos))) return MOE_ERR_NULL;
  if (T > 0 && !x) return MOE_ERR_NULL;
  if (M_cap > 0 && (!xs || (!tensor && !ss))) return MOE_ERR_NULL;
  if (from_rows && (!scale || (T > 0 && !row_amax))) return MOE_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(x) % 16 != 0) return MOE_ERR_SHAPE;
  if (ws_bytes < moe::sort_ws_bytes(M, E)) return MOE_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  int32_t* hdr = static_cast<int32_t*>(ws);
  int32_t* tile_hist = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + moe::kHdr);
  const int rc = moe::sort_metadata(expert_ids, T, k, E, group_offset, num_local_experts, M_cap, perm, inv_pos,
                                    group_sizes, hdr, tile_hist, hdr + moe::kErr, st);
  if (rc != MOE_OK) return rc;
  int64_t waves = T > M_cap / 4 ? T : M_cap / 4;
  if (waves < 4) waves = 4;
  if (waves > 65536) waves = 65536;
  const dim3 grid(static_cast<unsigned>(moe_cdiv(waves, 4))), block(256);
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  const int sm = static_mode ? 1 : 0;
  const int64_t G = H / 16, gpl = moe_cdiv(G, 64);
  if (from_rows) {        // the tensor scale from the given token maxima, into scale[0]
    moe::amax_scale_kernel<<<1, 1024, 0, st>>>(row_amax, T, scale);
    MOE_CHECK_LAUNCH();
  }
  const float* given = from_rows ? scale : nullptr;
  float* tok = from_rows ? nullptr : scale;
  float* amax_out = tensor ? nullptr : row_amax;
#define MOE_QS(GPL) \
  moe::quantize_scatter_kernel<GPL><<<grid, block, 0, st>>>(xb, sm, static_scale, given, inv_pos, T, k, H, M_cap, \
                                                             hdr, xs, ss, tok, amax_out)
  if (gpl <= 1) MOE_QS(1);
  else if (gpl <= 2) MOE_QS(2);
  else if (gpl <= 4) MOE_QS(4);
  else if (gpl <= 8) MOE_QS(8);
  else MOE_QS(0);
#undef MOE_QS
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}

// ---------------------------------------------------------------- no workspace
// moe_sort_by_expert_noalloc keeps the window header and the histogram table
// in this library-owned array instead of a caller workspace: one copy per GPU,
// held until the process ends.  In host code the array's name is only a
// stand-in for the device symbol, so it is never passed to a kernel; each
// device's address comes from hipGetSymbolAddress, looked up once per device
// (with that device current) on the entry point's first call there.
static __device__ __align__(256) uint8_t scratch[MOE_SORT_NOALLOC_SCRATCH_BYTES];

namespace moe {
namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

int scratch_on_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}
}  // namespace
}  // namespace moe

extern "C" int moe_sort_by_expert_noalloc(const int32_t* expert_ids, int64_t T, int32_t k, int32_t E,
                                          int32_t group_offset, int32_t num_local_experts, const uint8_t* xq,
                                          const float* xscale, int xscale_mode, int64_t H, int64_t M_cap,
                                          int32_t* perm, int32_t* inv_pos, int32_t* group_sizes, uint8_t* xs,
                                          float* ss, int32_t* device_error, void* stream) {
  int rc = moe::sort_check(expert_ids, T, k, E, group_offset, num_local_experts, xq, xscale, xscale_mode, H, M_cap,
                           perm, inv_pos, group_sizes, xs, ss);
  if (rc != MOE_OK) return rc;
  if (moe::sort_ws_bytes(T * k, E) > MOE_SORT_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
  void* p = nullptr;
  rc = moe::scratch_on_current_device(&p);
  if (rc != MOE_OK) return rc;
  // every word of the header and the table that the kernels read is written
  // by this call's own kernels first, so nothing is cleared between calls
  int32_t* hdr = static_cast<int32_t*>(p);
  int32_t* tile_hist = reinterpret_cast<int32_t*>(static_cast<char*>(p) + moe::kHdr);
  return moe::sort_run(expert_ids, T, k, E, group_offset, num_local_experts, xq, xscale, xscale_mode, H, M_cap,
                       perm, inv_pos, group_sizes, xs, ss, hdr, tile_hist, device_error,
                       static_cast<hipStream_t>(stream));
}

// The row gather alone, on the metadata a moe_sort_by_expert call without
// rows left in the same workspace (its window header) and in inv_pos.
extern "C" int moe_sort_gather_rows(const uint8_t* xq, const float* xscale, int xscale_mode, const int32_t* inv_pos,
                                    int64_t T, int32_t k, int64_t H, int64_t M_cap, uint8_t* xs, float* ss, void* ws,
                                    size_t ws_bytes, void* stream) {
  if (T < 0 || k <= 0 || k > 64 || M_cap < 0 || T * k > INT32_MAX - 1) return MOE_ERR_SHAPE;
  if (xscale_mode != MOE_SCALE_ROW_DYNAMIC && xscale_mode != MOE_SCALE_TENSOR_DYNAMIC &&
      xscale_mode != MOE_SCALE_TENSOR_STATIC)
    return MOE_ERR_UNSUPPORTED;
  if (H <= 0 || H % 16) return MOE_ERR_SHAPE;
  const bool row_scale = xscale_mode == MOE_SCALE_ROW_DYNAMIC;
  if (!xs && !(row_scale && ss)) return MOE_ERR_NULL;           // nothing to gather into
  if (T > 0 && (!xq || !inv_pos)) return MOE_ERR_NULL;
  if (row_scale && ss && T > 0 && !xscale) return MOE_ERR_NULL;
  if (!ws) return MOE_ERR_NULL;
  if (ws_bytes < static_cast<size_t>(moe::kHdr)) return MOE_ERR_WORKSPACE;
  if (M_cap == 0 && T == 0) return MOE_OK;
  int64_t waves = T > M_cap / 4 ? T : M_cap / 4;
  if (waves < 4) waves = 4;
  if (waves > 65536) waves = 65536;
  hipStream_t st = static_cast<hipStream_t>(stream);
  moe::sort_scatter_kernel<<<static_cast<unsigned>(moe_cdiv(waves, 4)), 256, 0, st>>>(
      xq, xscale, row_scale ? 1 : 0, inv_pos, T, k, H, M_cap, static_cast<const int32_t*>(ws), xs, ss);
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}
