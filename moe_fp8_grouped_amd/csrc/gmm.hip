// moe_gmm_fp8: grouped matmul of e4m3fn operands on the gfx950 fp8 matrix
// cores (v_mfma_f32_16x16x128_f8f6f4, float32 accumulate):
//     out[r, c] = ls[r] * sum_b rs[g, b, c] * sum_{k in block b} X[r, k] W_g[k, c]
// for the rows r of local group g ("Quantize activations before EP all
// gather": the prequantized gmm_v2 call with rhs_scale and group_offset;
// "Keep qwix out of tpu-inference's fused MoE kernel and pre-quantize
// weights": 32-bit accumulator, [E, blocks, 1, N] weight scales).
//
// Workgroup tile BM x BN x (K step 128) with NW waves (the shipped
// configuration: BM = 256, BN = 128, three LDS stages, 8 waves = two per
// SIMD).  The waves form a 4 x 2 grid of 64 x 64 wave tiles, 4 x 4 MFMA
// tiles of 16 x 16 each, whose float accumulators stay in registers.  Two
// waves per SIMD: direct-to-LDS loads are issue-limited per wave, and a
// second wave keeps the matrix core busy while the other issues its loads.
// An MFMA lane l supplies row l%16 and contraction bytes 32*(l/16) .. +31 of
// each operand.
//
// Staging: NST LDS stages (A: BM rows, B: BN rows, 128 bytes each, plus a
// 1 KiB slot for the step's blockwise weight scales), filled straight from
// global memory by global_load_lds (each lane moves 16 bytes; a wave
// instruction fills 1 KiB = 8 staged rows lane-linearly).  NST-1 steps are
// in flight while the waves multiply one; a wave waits only for its own
// loads of the step it needs (vmcnt counts the later stages' loads, which
// complete in order), then one barrier per K step.  The loads of a step are
// spread over the MFMA rounds of the previous ones so a stalled load issue
// never holds a long run of MFMAs.  Inside a staged row the 16-byte chunk c
// sits at slot c ^ f(row), f(r) = (r & 7) ^ (((r >> 3) ^ (r >> 5)) & 1):
// the 16-byte fragment reads of 8 (or 16) consecutive rows per lane group
// and the 8-byte transpose reads (8 rows from each of two 32-row bands) then
// touch distinct banks.  (An earlier f, ((r >> 1) & 7) ^ 4((r >> 5) & 1),
// measured 0.94 bank-conflict cycles per LDS access on this target: it
// serves a 16-byte read 8 lanes at a time.)
//  * K-contiguous operands (lhs rows; rhs stored [E, N, K]) are read as two
//    16-byte chunks per fragment;
//  * rhs stored [E, K, N] is staged as [128 k][128 n] halves and read with
//    ds_read_b64_tr_b8 (within a 16-lane group, lane i gets byte i%8 of the
//    chunks addressed by lanes 2j + i/8, j = 0..7).
// The product is formed transposed per 16 x 16 block (the MFMA gets the
// weight fragment as its first operand), so output lane l holds one output
// row and four consecutive output columns.
// Scales: per-channel weight scales multiply at the end; blockwise K scales
// (K/Kb a multiple of 128) are folded every K step, tot += rs * P_step,
// which is the same sum as rs * (sum of the block's steps) up to rounding.
// The lhs row scale is applied in float32 before the single rounding to
// bfloat16 (round to nearest even, the hardware's packed conversion); each
// lane writes its four columns as one 8-byte LDS store, and the staged tile
// goes out with full 16-byte stores per output row segment.
//
// Short groups: a group's last m-tile often holds only a few rows.  When the
// remainder is at most BM/2 rows it is covered by wide tiles of BM/2 rows x
// 2*BN columns (two n-tiles at once): the stage holds 128 A rows and 256 B
// rows -- the same bytes and the same loads per wave as a plain tile --
// and the waves split it into the same 64 x 64 wave tiles, so such a tail costs
// half a plain tile per n-tile (the wide tile's wave grid is 2 x 4).
//
// Absorbing tiles (all-wide mode, [E, N, K] weights, at most 512 local
// groups): a group of m rows gets ceil(m / 144) row blocks instead of
// ceil(m / 128); block b starts at row 128 b + min(16 b, x), x = m - 128 *
// blocks, so the first blocks carry up to 16 rows past their 128.  Those rows
// are staged in a 2 KiB region after the stage's scale slot (each wave's
// lanes 0..15 fill two of the 16 rows: every wave issues one more load per
// step, so the wait counts stay uniform) and each wave multiplies them with
// its own weight fragments, two more 16 x 16 blocks per step.  A group of
// 257..288 rows then takes two row blocks instead of three: with routing
// that fills experts to about 256 rows, the leftover rows of the fuller
// experts no longer cost a third pass over their weights.
//
// Split last round: when an XCD's share of tiles leaves a last round that
// occupies few of its workgroups, each of those tiles is split along K into
// up to workgroups / tiles parts (at least four K steps each).  A part writes
// its raw float32 sums to its workgroup's slot in the workspace with
// device-coherent stores, waits for them to complete and counts itself in
// with an integer atomic; the part that finishes last reads the slots back
// with device-coherent loads, adds them up in part order and writes the
// output -- no waiting, the same sums in the same order on every run, and no
// device-scope fence (on this chip one writes back and invalidates a whole
// L2, which cost more than the split saves).  The counters return to zero
// after each use.
//
// Scheduling: persistent workgroups (as many per CU as the LDS allows).
// Each derives the local group table (row and tile offsets) from
// group_sizes in LDS -- empty groups
// own no tiles, no host synchronisation -- splits the tile range into eight
// contiguous parts, one per XCD (workgroups are dealt round-robin over the
// XCDs), and walks its part with m-tiles fastest inside a group so that
// consecutive tiles reuse the expert's weight tile from that XCD's L2.
// Rows [n, M) are zeroed after the tiles.
#include <type_traits>

#include "tile_common.hpp"

#ifndef MOE_GMM_CFG
#define MOE_GMM_CFG 256, 128, 3, 8     // BM, BN, stages, waves
#endif
// Which pipeline each entry uses (0: per-tile, 1: streaming).  Measured: the
// per-tile kernel is faster on the grouped forward product with ragged
// groups; the streaming kernel on the weight-gradient product, whose tiles
// have only a few K steps each.
#ifndef MOE_GMM_STREAM
#define MOE_GMM_STREAM 0
#endif
// Every forward tile of the 256 x 128 kernel as BM/2 rows x 2 BN columns (two
// weight column blocks per stage, the two 128-row halves of a group's rows on
// neighbouring workgroups): the same stage bytes and loads per wave, each
// weight block fetched from HBM once and reread from L2 by the other half.
// Measured on the expert slice's launches (interleaved A/B, medians): down
// projection 222 -> 205 us, fused input projections 351 -> 347 us.
#ifndef MOE_GMM_WIDE_ALL
#define MOE_GMM_WIDE_ALL 1
#endif
// Absorbing tiles in the all-wide mode (see the header comment; [E, N, K]
// weights, at most 512 local groups).
#ifndef MOE_GMM_ABSORB
#define MOE_GMM_ABSORB 1
#endif
#ifndef MOE_GMM_STREAM_BATCH
#define MOE_GMM_STREAM_BATCH 1
#endif
// Cache policy of the batched (weight-gradient) product's output stores: 2 is
// the non-temporal hint, so the float32 output, several times larger than an
// XCD's L2, streams past the L2 instead of evicting the operand tiles that the
// group's other output tiles still read.
#ifndef MOE_GMM_BATCH_STORE_POLICY
#define MOE_GMM_BATCH_STORE_POLICY 2
#endif

namespace moe {
namespace {
using namespace tile;

constexpr int G_BK = 128;
typedef __attribute__((address_space(3))) void lds_void;

// Chunk slot swizzle of staged row r: any 8 consecutive rows from a multiple
// of 8 use 8 distinct 16-byte slots, and rows r and r + 8 (and r and r + 32)
// differ in slot parity, so a 16-byte read of 8 (or 16) consecutive rows per
// lane group and the 8-byte transpose reads of 8 rows from each of two 32-row
// bands meet distinct banks.
__device__ __forceinline__ int swz(int row) { return (row & 7) ^ (((row >> 3) ^ (row >> 5)) & 1); }
constexpr int SWZ_FLIP = 1;      // the slot bit the per-instruction bit flips

// Per-lane pieces of the staging addresses.  A load instruction fills staged
// rows R .. R+7 (R a multiple of 8); lane l fetches row R + l/8 into slot l%8,
// i.e. logical chunk (l%8) ^ swz(R + l/8).  For the R a wave issues, that
// chunk is c0 ^ SWZ_FLIP*p with c0 = (l%8) ^ (the lane's part of the swizzle)
// and p a per-instruction bit, so a lane needs only two offsets per operand;
// the rest of the address is uniform (scalar registers).
struct LaneOff {
  uint32_t v0, v1;
  // arithmetic select: keeps the pair in registers
  __device__ __forceinline__ uint32_t pick(int bit) const { return v0 ^ ((v0 ^ v1) & (0u - static_cast<uint32_t>(bit))); }
};

__device__ __forceinline__ LaneOff stage_lane_off(int lane, int64_t stride) {
  const int sub = lane >> 3, c0 = (lane & 7) ^ sub;
  LaneOff o;
  o.v0 = static_cast<uint32_t>(sub * stride + 16 * c0);
  o.v1 = static_cast<uint32_t>(sub * stride + 16 * (c0 ^ SWZ_FLIP));
  return o;
}

// Swizzle bit of the instruction that fills rows R .. R+7 (R % 8 == 0).
__device__ __forceinline__ int stage_bit(int R) { return ((R >> 3) & 1) ^ ((R >> 5) & 1); }

// Slot S of a wave's 48/NW loads per K step loads A (lhs) rows: a wave's
// first slots load A.
template <int NW, int S>
__device__ __forceinline__ bool slot_is_a(bool wide) { return S < (wide ? 16 / NW : 32 / NW); }

// Staged row of slot S's first row inside its operand, and the slot's LDS
// byte offset inside a stage.
template <int NW, int S>
__device__ __forceinline__ int slot_row(bool wide, int wave) {
  return slot_is_a<NW, S>(wide) ? wave * (wide ? 128 / NW : 256 / NW) + 8 * S
                                : wave * (wide ? 256 / NW : 128 / NW) + 8 * (S - (wide ? 16 / NW : 32 / NW));
}
template <int NW, int S>
__device__ __forceinline__ int slot_dst(bool wide, int wave) {
  return slot_is_a<NW, S>(wide) ? slot_row<NW, S>(wide, wave) * G_BK
                                : (wide ? 128 : 256) * G_BK + slot_row<NW, S>(wide, wave) * G_BK;
}

// This lane's source of slot S at contraction offset 0; step kb reads
// src0 + kb (lhs rows, rhs [E, N, K]) or src0 + kb * N (rhs [E, K, N]).
template <bool TRANS, int NW, int S>
__device__ __forceinline__ const uint8_t* slot_src0(bool wide, const uint8_t* __restrict__ lhs,
                                                    const uint8_t* __restrict__ wg, int64_t K, int64_t N, int64_t row0,
                                                    int64_t col0, int64_t M, bool tail, int wave, int lane,
                                                    const LaneOff offK, const LaneOff offN) {
  const int R = slot_row<NW, S>(wide, wave);
  if (slot_is_a<NW, S>(wide)) {
    // the lane's row, clamped into the buffer (a no-op unless the tile reaches past row M - 1); always
    // clamped rather than branching on `tail`, so the per-tile source set-up stays free of branches
    const uint32_t off = offK.pick(stage_bit(R));
    const int sub = lane >> 3;
    const int64_t r = min(row0 + R + sub, M - 1);
    return lhs + r * K + (off - static_cast<uint32_t>(sub * K));
  }
  if (TRANS)      // staged row r = output column col0 + r
    return wg + (col0 + R) * K + offK.pick(stage_bit(R));
  // staged half R / 128 holds columns 128h.., staged row = contraction index
  return wg + static_cast<int64_t>(R & 127) * N + col0 + 128 * (R >> 7) + offN.pick(stage_bit(R));
}

// A 16-byte direct-to-LDS load (wave-uniform destination, lane-linear).
__device__ __forceinline__ void issue_from_dst(const uint8_t* __restrict__ src, uint8_t* dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)dst, 16, 0, 0);
}

// Slot S's direct-to-LDS load from a computed source.
template <int NW, int S>
__device__ __forceinline__ void issue_from(const uint8_t* src, bool wide, uint8_t* stage, int wave) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)(stage + slot_dst<NW, S>(wide, wave)), 16, 0, 0);
}

// Load slot S (0 .. 48/NW - 1) of one K step for wave `wave` of NW: one
// direct-to-LDS instruction filling 8 staged rows.  A plain tile stages 256
// A rows and 128 B rows; a wide tile 128 A rows and 256 B rows -- the same
// 48 KiB and the same 48/NW loads per wave, so the pipeline's wait counts do
// not depend on the tile kind.  Each wave fills 1/NW of either operand; its
// first slots load A.  tail: the tile reaches past the last lhs row,
// so lhs rows are clamped.
template <bool TRANS, int NW, int S>
__device__ __forceinline__ void issue_slot(bool wide, uint8_t* stage, const uint8_t* __restrict__ lhs,
                                           const uint8_t* __restrict__ wg, int64_t K, int64_t N, int64_t row0,
                                           int64_t col0, int64_t M, bool tail, int64_t kb, int wave, int lane,
                                           const LaneOff offK, const LaneOff offN) {
  const uint8_t* src = slot_src0<TRANS, NW, S>(wide, lhs, wg, K, N, row0, col0, M, tail, wave, lane, offK, offN);
  src += (TRANS || slot_is_a<NW, S>(wide)) ? kb : kb * N;
  __builtin_amdgcn_global_load_lds(src, (lds_void*)(stage + slot_dst<NW, S>(wide, wave)), 16, 0, 0);
}

// Two floats to packed bfloat16 (low half from lo), rounding to nearest even
// with the gfx950 conversion instruction.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  typedef float f2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2{lo, hi}), bf2));
}

// Four 16-byte LDS reads at p + {0, 16, 32, 48} floats, completed before
// returning.  One asm block: the blockwise-scale slot is filled by direct
// loads whose completion the caller has already waited for, and the
// compiler's own tracking of those loads would add a wait for every load
// still in flight before a plain read of it.
__device__ __forceinline__ void lds_read_4x16f(const float* p, float4 (&r)[4]) {
  typedef const __attribute__((address_space(3))) float lds_f32;
  const uint32_t a = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_f32*)p));   // LDS byte offset
  v4f t0, t1, t2, t3;
  asm volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %4 offset:64\n\t"
      "ds_read_b128 %2, %4 offset:128\n\t"
      "ds_read_b128 %3, %4 offset:192\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(t0), "=&v"(t1), "=&v"(t2), "=&v"(t3)
      : "v"(a)
      : "memory");
  r[0] = make_float4(t0[0], t0[1], t0[2], t0[3]);
  r[1] = make_float4(t1[0], t1[1], t1[2], t1[3]);
  r[2] = make_float4(t2[0], t2[1], t2[2], t2[3]);
  r[3] = make_float4(t3[0], t3[1], t3[2], t3[3]);
}

// LDS byte offsets of the two 16-byte chunks of MFMA fragment rows
// base + 16*i + l%16 (base % 64 == 0): swz of those rows is
// f(l%16) ^ SWZ_FLIP*((i >> 1) & 1), so two variants cover every i.
struct FragOff {
  int lo[2], hi[2];
};

__device__ __forceinline__ FragOff frag_off(int base, int lane) {
  const int l15 = lane & 15, grp = lane >> 4;
  const int f = (l15 & 7) ^ (l15 >> 3);
  FragOff o;
  const int row = (base + l15) * G_BK;
  o.lo[0] = row + 16 * ((2 * grp) ^ f);
  o.hi[0] = row + 16 * ((2 * grp + 1) ^ f);
  o.lo[1] = row + 16 * ((2 * grp) ^ f ^ SWZ_FLIP);
  o.hi[1] = row + 16 * ((2 * grp + 1) ^ f ^ SWZ_FLIP);
  return o;
}

// Fragment 0 (rows 0 .. 15) of a K-contiguous staged region at `region`, as
// frag_i reads it, completed before returning.  One asm block, for the same
// reason as lds_read_4x16f: the region is filled by direct loads whose
// completion the caller has already waited for, and a plain read of it made
// the compiler wait for every direct load still in flight (vmcnt(0) inside
// the K loop, which drains the later stages' loads).
__device__ __forceinline__ v8i frag0_waited(const uint8_t* region, const FragOff& o) {
  typedef const __attribute__((address_space(3))) uint8_t lds_u8;
  const uint32_t base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_u8*)region));
  const uint32_t a0 = base + static_cast<uint32_t>(o.lo[0]), a1 = base + static_cast<uint32_t>(o.hi[0]);
  v4i32 lo, hi;
  asm volatile(
      "ds_read_b128 %0, %2\n\t"
      "ds_read_b128 %1, %3\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(lo), "=&v"(hi)
      : "v"(a0), "v"(a1)
      : "memory");
  v8i r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
  r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
  return r;
}

// Fragment i (rows base + 16 i ..) of a K-contiguous staged operand.
__device__ __forceinline__ v8i frag_i(const uint8_t* stage, const FragOff& o, int i) {
  const int b = (i >> 1) & 1;
  const uint4 lo = *reinterpret_cast<const uint4*>(stage + o.lo[b] + i * 16 * G_BK);
  const uint4 hi = *reinterpret_cast<const uint4*>(stage + o.hi[b] + i * 16 * G_BK);
  v8i r;
  r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
  r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
  return r;
}

// Fragment of columns n0 .. n0+15 of a [128 k][128 n] staged half.
__device__ __forceinline__ v8i frag_tr_swz(const uint8_t* half, int n0, int lane) {
  const int grp = lane >> 4, L = lane & 15;
  const int chunk = n0 >> 4;
  v8i r;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int row = 32 * grp + 8 * q + (L >> 1);
    const uint8_t* p = half + row * G_BK + 16 * (chunk ^ swz(row)) + 8 * (L & 1);
    const v2i t = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(p));
    r[2 * q] = t[0];
    r[2 * q + 1] = t[1];
  }
  return r;
}

// s_waitcnt immediate for vmcnt(n) with the other counters left open (gfx9
// encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Workgroup barrier between K steps.  __syncthreads() would add a release
// fence, which on this target waits for every outstanding vector-memory
// operation -- including the later stages' loads the pipeline keeps in
// flight.  The caller waits for exactly what it needs first; the asm is a
// compiler memory barrier so no LDS access moves across it.
__device__ __forceinline__ void step_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Tile configuration: BM x BN output tile, NST LDS stages, NW waves.  A
// plain tile is split over a (BM/WM) x (BN/WN) wave grid, a wide tile
// (BM/2 x 2BN) over (BM/2WM) x (2BN/WN); both use WM x WN wave tiles (NW = 4:
// 128 x 64, NW = 8: 64 x 64).  A stage holds the A rows, the B rows and 1 KiB
// for the step's blockwise weight scales (one float per tile column).
// The last part of a split tile: the parts' raw sums, read back from their
// slots with device-coherent loads, added up in part order, then scaled like
// the ordinary epilogue (out = ls[row] * (rs[col] *) sum).  Kept out of line so
// that its registers (every part's loads of a thread's share go out together:
// one memory round trip per part) do not count against the tile loop's.
// Slot of part p: xcd + 8 * (ul + p * lft) (workgroup ul + p * lft of the XCD).
// INT_SUMS (int8 codes, one scale per column): the slots hold int32 sums,
// added as integers and converted to float32 once, as without the split.
template <int THREADS, int EPT, bool KBLOCKS, bool OUT_BF16, bool INT_SUMS>
__device__ __attribute__((noinline)) void split_fixup(const float* __restrict__ part, int xcd, int ul, int lft,
                                                      int parts, int rows, int cols, const float* ls_tile,
                                                      const float* __restrict__ rs_g, uint32_t ncol_blk,
                                                      int64_t row0, int64_t col0, int64_t N, void* out_t) {
  const int tid = threadIdx.x;
  const int q4 = cols / 4, nel = rows * q4;
  v4f tot[EPT];
#pragma unroll
  for (int u = 0; u < EPT; ++u) tot[u] = v4f{0.f, 0.f, 0.f, 0.f};
  for (int pp = 0; pp < parts; ++pp) {
    const __amdgpu_buffer_rsrc_t sp = slot_rsrc(const_cast<float*>(part) +
                                                static_cast<int64_t>(xcd + 8 * (ul + pp * lft)) * kSplitSlot);
    v4f v[EPT];
#pragma unroll
    for (int u = 0; u < EPT; ++u) {
      const int e = min(tid + u * THREADS, nel - 1);
      v[u] = slot_load(sp, 4 * ((e / q4) * cols + 4 * (e % q4)));
    }
#pragma unroll
    for (int u = 0; u < EPT; ++u)
      tot[u] = INT_SUMS ? __builtin_bit_cast(v4f, __builtin_bit_cast(v4i32, tot[u]) + __builtin_bit_cast(v4i32, v[u]))
                        : tot[u] + v[u];
  }
  if (INT_SUMS) {
#pragma unroll
    for (int u = 0; u < EPT; ++u) tot[u] = __builtin_convertvector(__builtin_bit_cast(v4i32, tot[u]), v4f);
  }
#pragma unroll
  for (int u = 0; u < EPT; ++u) {
    const int e = tid + u * THREADS;
    if (e >= nel) break;
    const int r = e / q4, c = 4 * (e % q4);
    const int64_t gc = col0 + c;
    float4 sc = make_float4(1.f, 1.f, 1.f, 1.f);
    if (!KBLOCKS)
      sc = make_float4(rs_g[static_cast<uint32_t>(gc) / ncol_blk], rs_g[static_cast<uint32_t>(gc + 1) / ncol_blk],
                       rs_g[static_cast<uint32_t>(gc + 2) / ncol_blk], rs_g[static_cast<uint32_t>(gc + 3) / ncol_blk]);
    const float lsr = ls_tile[r];
    const float o0 = lsr * (tot[u][0] * sc.x), o1 = lsr * (tot[u][1] * sc.y), o2 = lsr * (tot[u][2] * sc.z),
                o3 = lsr * (tot[u][3] * sc.w);
    if (OUT_BF16)
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out_t) + (row0 + r) * N + gc) =
          make_uint2(pack_bf16x2(o0, o1), pack_bf16x2(o2, o3));
    else
      *reinterpret_cast<float4*>(static_cast<float*>(out_t) + (row0 + r) * N + gc) = make_float4(o0, o1, o2, o3);
  }
}

template <int BM_, int BN_, int NST_, int NW_ = 4>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, NST = NST_, NW = NW_, THREADS = 64 * NW;
  static constexpr int WN = 64, WM = BM * BN / (NW * WN);  // wave tile
  static constexpr int SLOTS = 48 / NW;                    // direct loads per wave per K step
  static constexpr int MI = WM / 16, JN = WN / 16;         // 16 x 16 MFMA tiles per wave
  static constexpr int SC_OFF = (BM + BN) * G_BK;          // scale slot inside a stage
  static constexpr int STAGE = SC_OFF + 1024;
  static constexpr int OUT_STRIDE = BN + 8;                // bf16 elements per staged output row
  static constexpr int LDS_OUT = BM * OUT_STRIDE * 2;
  static constexpr int LDS = NST * STAGE > LDS_OUT ? NST * STAGE : LDS_OUT;
};

template <class C, bool KBLOCKS>
constexpr int loads_per_step() { return C::SLOTS + (KBLOCKS ? 1 : 0); }   // per wave

// BATCH (the weight-gradient product): one independent matmul per local
// group g, out[g] (M x N) = A_g B_g^T with A and B stored contraction-
// contiguous, row stride K, group g's contraction at columns
// 128 * tiles_off[g] .. of both (its rows, zero-padded to a multiple of 128);
// rows = the group table's row bound (max_rows).  Empty groups get zeros.
// I8: int8 operands (v_mfma_i32_16x16x64_i8 pairs, int32 accumulation; with
// blockwise scales each step's exact int32 product is folded in float32).
// ABS: absorbing tiles in the all-wide mode (see the header comment).
template <class C, bool TRANS, bool KBLOCKS, bool OUT_BF16, bool BATCH = false, bool I8 = false, bool ABS = false>
__global__ __launch_bounds__(C::THREADS) void gmm_kernel(const uint8_t* __restrict__ lhs, const float* __restrict__ ls,
                                                       int ls_per_row, const uint8_t* __restrict__ rhs,
                                                       const float* __restrict__ rs, int Kb, int Nb,
                                                       const int32_t* __restrict__ group_sizes, int g0, int El,
                                                       int64_t M, int64_t K, int64_t N, void* __restrict__ out,
                                                       int32_t* __restrict__ err, int64_t max_rows = 0,
                                                       int wide_all = 0, float* __restrict__ part = nullptr,
                                                       int32_t* __restrict__ cnt = nullptr, int nslots = 0) {
  constexpr int BM = C::BM, BN = C::BN, NST = C::NST, WM = C::WM, WN = C::WN, MI = C::MI, JN = C::JN;
  constexpr int XROWS = 16;                                   // ABS: rows a block may carry past BM/2
  constexpr int X_OFF = C::SC_OFF + 1024;                     // ABS: their staging region in a stage
  constexpr int STAGE = C::STAGE + (ABS ? XROWS * G_BK : 0);
  constexpr int LDS_BYTES = ABS && NST * STAGE > C::LDS ? NST * STAGE : C::LDS;
  static_assert(!ABS || (TRANS && !BATCH && BM == 256 && BN == 128), "absorbing tiles: forward, [E, N, K] weights");
  static_assert(!ABS || (BM / 2 + XROWS) * (2 * BN + 8) * 2 <= LDS_BYTES, "absorbing tile's output staging");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[LDS_BYTES];
  __shared__ GroupTableN<ABS ? kAbsMaxLocal : kMaxLocal> gt;
  __shared__ float ls_tile[BM];
  __shared__ int split_last;                                  // ABS: this part finished its split tile last
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);    // uniform: keeps staging addresses scalar
  constexpr int NW = C::NW, G_THREADS = C::THREADS;
  const int NT = static_cast<int>(N / BN);
  static_assert(BM == 256 && BN == 128 && JN == 4 && (NW == 4 || NW == 8),
                "wide tail tiles are BM/2 x 2BN with the same wave tiles");
  const int MTb = static_cast<int>(M / BM);          // BATCH: m-tiles per group
  if constexpr (BATCH)   // tiles_off = the groups' padded row offsets in 128-row blocks
    build_groups(group_sizes, g0, El, max_rows, 1, G_BK, err, gt, reinterpret_cast<int*>(smem), false);
  else
    build_groups(group_sizes, g0, El, M, NT, BM, err, gt, reinterpret_cast<int*>(smem),
                 wide_all ? (ABS ? 3 : 2) : 1);
  // ABS: absorbing row blocks only where they take fewer rounds of tiles over the workgroups of an
  // XCD than the plain all-wide layout; otherwise they only make a few tiles heavier.  Every
  // workgroup takes the same decision from the same group sizes.
  int use_abs = 0;
  if constexpr (ABS && !BATCH) {
    int* plain = reinterpret_cast<int*>(smem);                // per-group plain tile counts, then their scan
    int* plain_off = plain + kAbsMaxLocal + 1;
    for (int g = threadIdx.x; g < El; g += blockDim.x)
      plain[g] = group_tiles(gt.rows_off[g + 1] - gt.rows_off[g], BM, NT, 2);
    __syncthreads();
    wave0_scan(plain, plain_off, El);
    __syncthreads();
    const int per_xcd = max(static_cast<int>(gridDim.x) / 8, 1);
    const int r_abs = ((gt.tiles_off[El] + 7) / 8 + per_xcd - 1) / per_xcd;
    const int r_plain = ((plain_off[El] + 7) / 8 + per_xcd - 1) / per_xcd;
    use_abs = __builtin_amdgcn_readfirstlane(r_abs < r_plain ? 1 : 0);
    if (!use_abs)
      for (int g = threadIdx.x; g <= El; g += blockDim.x) gt.tiles_off[g] = plain_off[g];
    __syncthreads();
  }
  const int total = BATCH ? El * MTb * NT : gt.tiles_off[El];
  const int n_rows = gt.rows_off[El];
  const int KT = static_cast<int>(K / G_BK);
  const int steps_per_block = static_cast<int>(K / Kb / G_BK);
  const uint32_t ncol_blk = static_cast<uint32_t>(N / Nb);
  int first, last, step;
  xcd_share(total, first, last, step);
  const LaneOff offK = stage_lane_off(lane, K);
  const LaneOff offN = stage_lane_off(lane, N);
  // ABS: the last, partial round of this XCD's tiles may be split along K: its `lft` tiles go to
  // `split_s` workgroups each (part p of tile l: workgroup l + p * lft on the XCD)
  const int xj = static_cast<int>(blockIdx.x) / 8;            // this workgroup's index on its XCD
  int n_full, split_s = 1, lft = 0, lbase = 0;
  {
    const int x = static_cast<int>(blockIdx.x) % 8;
    const int lo = static_cast<int>((static_cast<int64_t>(total) * x) / 8);
    const int hi = static_cast<int>((static_cast<int64_t>(total) * (x + 1)) / 8);
    const int rounds = (hi - lo) / step;
    lft = hi - lo - rounds * step;
    lbase = lo + rounds * step;
    if constexpr (ABS) {
      if (part != nullptr && lft > 0 && static_cast<int>(gridDim.x) <= nslots && lft <= kSplitPerXcd)
        split_s = max(min(step / lft, KT / kSplitMinSteps), 1);
    }
    n_full = split_s >= 2 ? rounds : (first < last ? (last - first + step - 1) / step : 0);
  }
  const int ul = lft > 0 ? xj % lft : 0, up = lft > 0 ? xj / lft : 0;   // this workgroup's leftover tile, part
  const int n_items = n_full + (split_s >= 2 && xj < lft * split_s ? 1 : 0);

  // decode tile t of the group table: its group, n-tile, first row, rows and kind (tiles of a group:
  // n-tile major, m-tiles fastest; a short remainder of at most BM/2 rows is covered by wide tiles of two
  // n-tiles each, placed after the two n-tiles' full m-tiles so they reuse the same weight columns from L2)
  auto decode = [&](int t, int& g, int& nt, int64_t& row0, int& rows_here, bool& wide, int& m_g) {
    g = BATCH ? t / (MTb * NT) : find_group(gt, El, t);
    const int local = BATCH ? t - g * (MTb * NT) : t - gt.tiles_off[g];
    m_g = gt.rows_off[g + 1] - gt.rows_off[g];
    const int full = m_g / BM, rem = m_g - full * BM;
    int roff;                     // the tile's first row inside the group
    int wrows = BM / 2;           // rows of a wide tile (ABS: up to BM/2 + XROWS)
    wide = false;
    if (BATCH) {
      nt = local / MTb;
      roff = (local - nt * MTb) * BM;
    } else if (wide_all) {        // every tile BM/2 rows x two n-tiles, m-tiles fastest within a pair
      const int half = BM / 2, npair = NT / 2;
      const int mtw = use_abs ? (m_g + half + XROWS - 1) / (half + XROWS) : (m_g + half - 1) / half;
      const int xr = use_abs ? max(m_g - half * mtw, 0) : 0;  // rows past half * blocks, spread over the first blocks
      if (local < npair * mtw) {
        const int pr = local / mtw, mb = local - pr * mtw;
        nt = 2 * pr;
        roff = mb * half + (ABS ? min(XROWS * mb, xr) : 0);
        if (ABS) wrows = (mb + 1 < mtw ? (mb + 1) * half + min(XROWS * (mb + 1), xr) : min(m_g, roff + half + XROWS)) - roff;
        wide = true;
      } else {
        nt = NT - 1;
        roff = (local - npair * mtw) * BM;
      }
    } else if (rem == 0 || rem > BM / 2) {
      const int per = full + (rem ? 1 : 0);
      nt = local / per;
      roff = (local - nt * per) * BM;
    } else {
      const int pairblk = 2 * full + 1, npair = NT / 2;
      if (local < npair * pairblk) {
        const int pr = local / pairblk, w = local - pr * pairblk;
        if (w < 2 * full) {
          const int h = w >= full ? 1 : 0;
          nt = 2 * pr + h;
          roff = (w - h * full) * BM;
        } else {
          nt = 2 * pr;
          roff = full * BM;
          wide = true;
        }
      } else {
        nt = NT - 1;
        roff = (local - npair * pairblk) * BM;
      }
    }
    row0 = BATCH ? static_cast<int64_t>(roff) : gt.rows_off[g] + static_cast<int64_t>(roff);
    rows_here = BATCH ? BM : min(wide ? wrows : BM, m_g - roff);
  };
  // ABS: the tiles this workgroup runs, decoded up front into LDS by one thread each (a search of the
  // group table and a few integer divisions that would otherwise sit between every two tiles); items past
  // the table's end decode inline
  constexpr int kDesc = ABS ? 96 : 1;
  __shared__ int4 tdesc[kDesc];       // {first row, n-tile, group, rows | wide << 16}
  if constexpr (ABS) {
    for (int i = tid; i < min(n_items, kDesc); i += G_THREADS) {
      const int t = split_s >= 2 && i == n_full ? lbase + ul : first + i * step;
      int g, nt, rh, mg;
      int64_t r0;
      bool wd;
      decode(t, g, nt, r0, rh, wd, mg);
      tdesc[i] = make_int4(static_cast<int>(r0), nt, g, rh | (wd ? 1 << 16 : 0));
    }
    __syncthreads();
  }

  // the tile loop, compiled once with a split part and once without, so the
  // workgroups of an XCD without a split round run a loop that holds none of
  // the split's state
  auto tile_loop = [&](auto split_c) {
  constexpr bool SPLIT = decltype(split_c)::value;
  for (int item = 0; item < n_items; ++item) {
    const bool psplit = SPLIT && item == n_full;               // a part of a split tile
    const int t = psplit ? lbase + ul : first + item * step;
    const int kbeg = psplit ? (up * KT) / split_s : 0;
    const int kend = psplit ? ((up + 1) * KT) / split_s : KT;
    int g, nt, rows_here, m_g = 0;
    int64_t row0;
    bool wide;
    if (ABS && item < kDesc) {    // decoded up front
      const int4 dsc = tdesc[item];
      row0 = __builtin_amdgcn_readfirstlane(dsc.x);
      nt = __builtin_amdgcn_readfirstlane(dsc.y);
      g = __builtin_amdgcn_readfirstlane(dsc.z);
      const int f = __builtin_amdgcn_readfirstlane(dsc.w);
      rows_here = f & 0xffff;
      wide = (f >> 16) & 1;
    } else {
      decode(t, g, nt, row0, rows_here, wide, m_g);
    }
    // ABS: this tile carries rows past BM/2 (uniform: keeps its branches scalar)
    const bool ab = ABS && __builtin_amdgcn_readfirstlane(wide && rows_here > BM / 2 ? 1 : 0) != 0;
    const int64_t col0 = static_cast<int64_t>(nt) * BN;
    // BATCH: the group's contraction columns, its K steps and its output matrix
    const int64_t cofs = BATCH ? static_cast<int64_t>(gt.tiles_off[g]) * G_BK : 0;
    const int KTt = BATCH ? (m_g + G_BK - 1) / G_BK : kend - kbeg;
    const int kofs = BATCH ? 0 : kbeg;                          // the tile's first K step (split parts)
    const uint8_t* lhs_t = lhs + cofs;
    const uint8_t* wg = BATCH ? rhs + cofs : rhs + static_cast<int64_t>(g) * K * N;
    void* out_t = BATCH ? static_cast<void*>(static_cast<uint8_t*>(out) +
                                             static_cast<int64_t>(g) * M * N * (OUT_BF16 ? 2 : 4))
                        : out;
    const int bm_t = wide ? BM / 2 : BM, bn_t = wide ? 2 * BN : BN;     // this tile's shape
    const bool tail = row0 + bm_t > M;
    // this wave's output block: rows rbase .. +WM-1, columns cbase .. +63
    const int gn = wide ? 2 * BN / WN : BN / WN;          // wave-grid columns
    const int rbase = (wave / gn) * WM, cbase = (wave % gn) * WN;
    const FragOff fa = frag_off(rbase, lane);
    const FragOff fb = frag_off(cbase, lane);
    const FragOff fx = frag_off(0, lane);                  // ABS: the extra rows' staging region
    const float* rs_g = BATCH ? rs : rs + static_cast<int64_t>(g) * Kb * Nb;
    // blockwise scales ride the stages: lane l of wave w stages the scale of
    // tile column 64(w mod 4) + l (clamped to the tile; surplus lanes and the
    // upper four of eight waves repeat columns, writing the same values)
    const int w4 = wave & 3;
    const float* rs_lane = rs_g + static_cast<uint32_t>(col0 + min(w4 * 64 + lane, bn_t - 1)) / ncol_blk;
    // ABS: lanes 0..15 of wave w stage extra rows 2w and 2w + 1 (rows BM/2 + 2w.. of the tile, clamped
    // into the buffer; rows past the tile's are never stored), chunk c of a row at slot c ^ swz(row)
    const uint8_t* xsrc = nullptr;
    if constexpr (ABS) {
      const int xrow = 2 * wave + ((lane >> 3) & 1);
      xsrc = lhs + min(row0 + BM / 2 + xrow, M - 1) * K + 16 * ((lane & 7) ^ swz(xrow));
    }
#define MOE_XLOAD(stg, kbv)                                                                                 \
  do {                                                                                                      \
    if (lane < 16) __builtin_amdgcn_global_load_lds(xsrc + (kbv), (lds_void*)((stg) + X_OFF + 2 * wave * G_BK), 16, \
                                                    0, 0);                                                  \
  } while (0)

    // the tile body, compiled once for tiles that carry extra rows and once for
    // the rest, so the ordinary tiles' K loop has no branches on the tile kind
    auto tile_body = [=](auto ab_c) {
      constexpr bool AB = decltype(ab_c)::value;
      v4f acc[MI][JN];
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < JN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
      v4f acc_x[2] = {v4f{0.f, 0.f, 0.f, 0.f}, v4f{0.f, 0.f, 0.f, 0.f}};   // ABS: the two extra blocks

      // the previous tile's epilogue is done with the LDS (a bare barrier: its
      // output stores need not have completed)
      step_barrier();
      // prologue: stages 0 .. NST-2 in flight
#pragma unroll
      for (int s = 0; s < NST - 1; ++s) {
        if (s < KTt) {
          const int64_t kb = static_cast<int64_t>(kofs + s) * G_BK;
  #define MOE_SLOT(S, stg, kbv) \
    issue_slot<TRANS, NW, S>(wide, stg, lhs_t, wg, K, N, row0, col0, M, tail, kbv, wave, lane, offK, offN)
          MOE_SLOT(0, smem + s * STAGE, kb); MOE_SLOT(1, smem + s * STAGE, kb); MOE_SLOT(2, smem + s * STAGE, kb);
          MOE_SLOT(3, smem + s * STAGE, kb); MOE_SLOT(4, smem + s * STAGE, kb); MOE_SLOT(5, smem + s * STAGE, kb);
          if constexpr (C::SLOTS == 12) {
            MOE_SLOT(6, smem + s * STAGE, kb); MOE_SLOT(7, smem + s * STAGE, kb); MOE_SLOT(8, smem + s * STAGE, kb);
            MOE_SLOT(9, smem + s * STAGE, kb); MOE_SLOT(10, smem + s * STAGE, kb); MOE_SLOT(11, smem + s * STAGE, kb);
          }
          if (KBLOCKS)
            __builtin_amdgcn_global_load_lds(rs_lane + static_cast<int64_t>((kofs + s) / steps_per_block) * Nb,
                                             (lds_void*)(smem + s * STAGE + C::SC_OFF + w4 * 256), 4, 0, 0);
          if constexpr (AB) MOE_XLOAD(smem + s * STAGE, kb);
          if (s == 0) {   // the tile's lhs row scales ride its first stage (rows past the tile repeat its last)
            const int r = min(w4 * 64 + lane, rows_here - 1);
            __builtin_amdgcn_global_load_lds(ls + (ls_per_row ? row0 + r : 0), (lds_void*)(ls_tile + w4 * 64), 4, 0, 0);
          }
        }
      }

      for (int kt = 0; kt < KTt; ++kt) {
        // this wave's loads of step kt have landed once at most the loads of the
        // NST-2 later stages are outstanding (loads complete in order)
        if (kt + NST - 1 <= KTt) {
          if constexpr (AB)
            __builtin_amdgcn_s_waitcnt(waitcnt_vm((NST - 2) * (loads_per_step<C, KBLOCKS>() + 1)));
          else
            __builtin_amdgcn_s_waitcnt(waitcnt_vm((NST - 2) * loads_per_step<C, KBLOCKS>()));
        } else {
          __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        }
        step_barrier();                         // everyone's have, and step kt-1's readers are done
        const int ks = kt + NST - 1;            // the step whose loads are issued now
        const bool more = ks < KTt;
        const int64_t kb_next = static_cast<int64_t>(kofs + ks) * G_BK;
        uint8_t* nxt = smem + (ks % NST) * STAGE;
        const uint8_t* As = smem + (kt % NST) * STAGE;
        const uint8_t* Bs = As + bm_t * G_BK;
        float4 s_col[JN];    // scales of this lane's output columns 16j + 4(l/16) .. +3
        const float* sc = reinterpret_cast<const float*>(As + C::SC_OFF) + cbase + 4 * (lane >> 4);
        static_assert(JN == 4, "four column groups per scale read");
        v8i b[JN];
#pragma unroll
        for (int j = 0; j < JN; ++j) {
          const int n0 = cbase + j * 16;
          if (TRANS)
            b[j] = frag_i(Bs, fb, j);
          else
            b[j] = frag_tr_swz(Bs + (n0 >> 7) * (128 * G_BK), n0 & 127, lane);
        }
        v4f pp[JN];          // KBLOCKS: the previous round's block products
        // MI rounds: an A fragment, this round's share of the loads of step ks,
        // then the round's MFMAs -- so memory back-pressure on the loads never
        // holds up a long run of MFMA issue
        // (the step's SLOTS loads spread over the MI rounds, 1.5 per round)
#pragma unroll
        for (int i = 0; i < MI; ++i) {
          const v8i a = frag_i(As, fa, i);
          if (more) {
            if constexpr (C::SLOTS == 12) {
              if (i == 0) { MOE_SLOT(0, nxt, kb_next); }
              if (i == 1) { MOE_SLOT(1, nxt, kb_next); MOE_SLOT(2, nxt, kb_next); }
              if (i == 2) { MOE_SLOT(3, nxt, kb_next); }
              if (i == 3) { MOE_SLOT(4, nxt, kb_next); MOE_SLOT(5, nxt, kb_next); }
              if (i == 4) { MOE_SLOT(6, nxt, kb_next); }
              if (i == 5) { MOE_SLOT(7, nxt, kb_next); MOE_SLOT(8, nxt, kb_next); }
              if (i == 6) { MOE_SLOT(9, nxt, kb_next); }
              if (i == 7) { MOE_SLOT(10, nxt, kb_next); MOE_SLOT(11, nxt, kb_next); }
            } else {
              if (i == 0) { MOE_SLOT(0, nxt, kb_next); MOE_SLOT(1, nxt, kb_next); }
              if (i == 1) { MOE_SLOT(2, nxt, kb_next); if constexpr (AB) MOE_XLOAD(nxt, kb_next); }
              if (i == 2) { MOE_SLOT(3, nxt, kb_next); MOE_SLOT(4, nxt, kb_next); }
              if (i == 3) { MOE_SLOT(5, nxt, kb_next); }
            }
            if (KBLOCKS && i == 0)
              __builtin_amdgcn_global_load_lds(rs_lane + static_cast<int64_t>((kofs + ks) / steps_per_block) * Nb,
                                               (lds_void*)(nxt + C::SC_OFF + w4 * 256), 4, 0, 0);
          }
          v4f pc[JN];
#pragma unroll
          for (int j = 0; j < JN; ++j) {
            if (KBLOCKS) {
              if constexpr (I8)
                pc[j] = __builtin_convertvector(mfma_i8x2(b[j], a, v4i32{0, 0, 0, 0}), v4f);   // exact: |p| < 2^24
              else
                pc[j] = mfma_f8(b[j], a, v4f{0.f, 0.f, 0.f, 0.f});
            } else if constexpr (I8) {      // the int32 sums live in the accumulator's registers
              acc[i][j] = __builtin_bit_cast(v4f, mfma_i8x2(b[j], a, __builtin_bit_cast(v4i32, acc[i][j])));
            } else {
              acc[i][j] = mfma_f8(b[j], a, acc[i][j]);
            }
          }
          // Blockwise scales: the previous round's block products are folded while this round's MFMAs run.
          // The empty asm reads the folded accumulators, so the fold stays in this round (it is ordered
          // against the round's direct loads); left free, the compiler moves every fold to the end of the
          // step, which keeps all sixteen products live (a spill) and leaves the matrix cores idle there.
          // the scales are read once round 0's MFMAs are issued: the first fold needs them only in round 1,
          // so the step's start waits for one LDS round trip (the fragments), not two
          if (KBLOCKS && i == 0) {
            __builtin_amdgcn_sched_barrier(0);
            lds_read_4x16f(sc, s_col);
          }
          if (KBLOCKS) {
            if (i > 0) {
#pragma unroll
              for (int j = 0; j < JN; ++j) {
                acc[i - 1][j][0] = fmaf(s_col[j].x, pp[j][0], acc[i - 1][j][0]);
                acc[i - 1][j][1] = fmaf(s_col[j].y, pp[j][1], acc[i - 1][j][1]);
                acc[i - 1][j][2] = fmaf(s_col[j].z, pp[j][2], acc[i - 1][j][2]);
                acc[i - 1][j][3] = fmaf(s_col[j].w, pp[j][3], acc[i - 1][j][3]);
              }
              asm volatile("" ::"v"(acc[i - 1][0]), "v"(acc[i - 1][1]), "v"(acc[i - 1][2]), "v"(acc[i - 1][3]));
            }
#pragma unroll
            for (int j = 0; j < JN; ++j) pp[j] = pc[j];
          }
        }
        if (KBLOCKS) {
#pragma unroll
          for (int j = 0; j < JN; ++j) {
            acc[MI - 1][j][0] = fmaf(s_col[j].x, pp[j][0], acc[MI - 1][j][0]);
            acc[MI - 1][j][1] = fmaf(s_col[j].y, pp[j][1], acc[MI - 1][j][1]);
            acc[MI - 1][j][2] = fmaf(s_col[j].z, pp[j][2], acc[MI - 1][j][2]);
            acc[MI - 1][j][3] = fmaf(s_col[j].w, pp[j][3], acc[MI - 1][j][3]);
          }
        }
        if constexpr (AB) {
          {   // the extra rows: this wave's blocks at tile rows BM/2 .. +15, columns cbase + 32 (wave / 4) ..
            const v8i ax = frag0_waited(As + X_OFF, fx);
            auto xblock = [&](v4f& c, const v8i& bj, const float4& sj) {
              if (KBLOCKS) {
                v4f p;
                if constexpr (I8)
                  p = __builtin_convertvector(mfma_i8x2(bj, ax, v4i32{0, 0, 0, 0}), v4f);
                else
                  p = mfma_f8(bj, ax, v4f{0.f, 0.f, 0.f, 0.f});
                c[0] = fmaf(sj.x, p[0], c[0]);
                c[1] = fmaf(sj.y, p[1], c[1]);
                c[2] = fmaf(sj.z, p[2], c[2]);
                c[3] = fmaf(sj.w, p[3], c[3]);
              } else if constexpr (I8) {
                c = __builtin_bit_cast(v4f, mfma_i8x2(bj, ax, __builtin_bit_cast(v4i32, c)));
              } else {
                c = mfma_f8(bj, ax, c);
              }
            };
            if (wave < 4) {
              xblock(acc_x[0], b[0], s_col[0]);
              xblock(acc_x[1], b[1], s_col[1]);
            } else {
              xblock(acc_x[0], b[2], s_col[2]);
              xblock(acc_x[1], b[3], s_col[3]);
            }
          }
        }
      }
  #undef MOE_XLOAD

      if constexpr (SPLIT) {
        if (psplit) {   // a part of a split tile: its raw sums (int8 per column: int32) to this workgroup's slot
                        // ([row][bn_t columns])
          const __amdgpu_buffer_rsrc_t slot = slot_rsrc(part + static_cast<int64_t>(blockIdx.x) * kSplitSlot);
#pragma unroll
          for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < JN; ++j)
              slot_store(slot, 4 * ((rbase + 16 * i + (lane & 15)) * bn_t + cbase + 16 * j + 4 * (lane >> 4)), acc[i][j]);
          if constexpr (AB) {
            const int jx = wave < 4 ? 0 : 2;
#pragma unroll
            for (int q = 0; q < 2; ++q)
              slot_store(slot, 4 * ((BM / 2 + (lane & 15)) * bn_t + cbase + 16 * (jx + q) + 4 * (lane >> 4)), acc_x[q]);
          }
          __builtin_amdgcn_s_waitcnt(0);                           // this wave's sums have reached the coherent level
          __syncthreads();                                         // ... and every wave's
          int32_t* ctr = cnt + (static_cast<int>(blockIdx.x) % 8) * kSplitPerXcd + ul;
          if (tid == 0) {
            const int before = atomicAdd(ctr, 1);
            split_last = before == split_s - 1;
            if (split_last)                                        // every part has counted in: reset for the next call
              __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
          __syncthreads();
          if (split_last) {   // the parts' sums in part order, then the epilogue
            constexpr int EPT = ((BM / 2 + XROWS) * 2 * BN / 4 + G_THREADS - 1) / G_THREADS;
            static_assert(EPT * G_THREADS * 4 >= BM * BN, "plain tiles fit the same count");
            split_fixup<G_THREADS, EPT, KBLOCKS, OUT_BF16, I8 && !KBLOCKS>(
                part, static_cast<int>(blockIdx.x) % 8, ul, lft, split_s, rows_here, bn_t, ls_tile, rs_g, ncol_blk,
                row0, col0, N, out_t);
          }
          return;
        }
      }
      if constexpr (I8 && !KBLOCKS) {   // the int32 sums to float32 (rounded to nearest beyond 2^24)
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int j = 0; j < JN; ++j) acc[i][j] = __builtin_convertvector(__builtin_bit_cast(v4i32, acc[i][j]), v4f);
#pragma unroll
        for (int q = 0; q < 2; ++q) acc_x[q] = __builtin_convertvector(__builtin_bit_cast(v4i32, acc_x[q]), v4f);
      }
      // ---- epilogue: out = ls[row] * (rs[col] *) acc
      // The product is formed transposed per 16 x 16 block (D = B^T A^T), so
      // lane l holds output row rbase + 16i + l%16 and the four consecutive
      // columns cbase + 16j + 4(l/16) .. +3.
      float4 s_out[JN];
#pragma unroll
      for (int j = 0; j < JN; ++j) {
        const int64_t c = col0 + cbase + j * 16 + 4 * (lane >> 4);
        if (KBLOCKS)
          s_out[j] = make_float4(1.f, 1.f, 1.f, 1.f);
        else if (ncol_blk == 1)
          s_out[j] = *reinterpret_cast<const float4*>(rs_g + c);
        else
          s_out[j] = make_float4(rs_g[static_cast<uint32_t>(c) / ncol_blk], rs_g[static_cast<uint32_t>(c + 1) / ncol_blk],
                                 rs_g[static_cast<uint32_t>(c + 2) / ncol_blk], rs_g[static_cast<uint32_t>(c + 3) / ncol_blk]);
      }
      // BATCH: a group without rows writes exact zeros (its row scales were never loaded)
      const bool empty = BATCH && KTt == 0;
      if (empty) {
#pragma unroll
        for (int j = 0; j < JN; ++j) s_out[j] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
      if (OUT_BF16) {
        const int ch_log = wide ? 5 : 4;          // log2 of the 16-byte chunks per output row
        const int OS = bn_t + 8;
        __syncthreads();                          // all waves are done with the operand stages
        // [bm_t rows][bn_t cols] bf16 with rows padded to OS elements (OS/2 = 4 mod
        // 64 dwords): each half-wave's 8-byte writes (16 rows x two 8-byte
        // column steps) land on distinct bank pairs
        uint16_t* st = reinterpret_cast<uint16_t*>(smem);
        uint16_t* st_lane = st + (rbase + (lane & 15)) * OS + cbase + 4 * (lane >> 4);
#pragma unroll
        for (int i = 0; i < MI; ++i) {
          const float lsr = empty ? 0.f : ls_tile[rbase + i * 16 + (lane & 15)];
#pragma unroll
          for (int j = 0; j < JN; ++j) {
            const uint32_t lo = pack_bf16x2(lsr * (acc[i][j][0] * s_out[j].x), lsr * (acc[i][j][1] * s_out[j].y));
            const uint32_t hi = pack_bf16x2(lsr * (acc[i][j][2] * s_out[j].z), lsr * (acc[i][j][3] * s_out[j].w));
            *reinterpret_cast<uint2*>(st_lane + i * 16 * OS + j * 16) = make_uint2(lo, hi);
          }
        }
        if constexpr (AB) {         // the extra rows BM/2 .. +15 (a wide tile: OS = 2 BN + 8)
          const float lsr = ls_tile[BM / 2 + (lane & 15)];
          const int jx = wave < 4 ? 0 : 2;
          uint16_t* xl = st + (BM / 2 + (lane & 15)) * OS + cbase + 4 * (lane >> 4);
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const float4 so = jx == 0 ? s_out[q] : s_out[2 + q];
            const uint32_t lo = pack_bf16x2(lsr * (acc_x[q][0] * so.x), lsr * (acc_x[q][1] * so.y));
            const uint32_t hi = pack_bf16x2(lsr * (acc_x[q][2] * so.z), lsr * (acc_x[q][3] * so.w));
            *reinterpret_cast<uint2*>(xl + (jx + q) * 16) = make_uint2(lo, hi);
          }
        }
        __syncthreads();
        uint16_t* o = static_cast<uint16_t*>(out_t);
        // chunks: a plain tile BM x BN/8, a wide one BM/2 x 2BN/8 (ABS: plus XROWS rows)
        constexpr int OUT_IT = (BM * (BN / 8) + (ABS ? XROWS * (2 * BN / 8) : 0) + G_THREADS - 1) / G_THREADS;
#pragma unroll 4
        for (int it = 0; it < OUT_IT; ++it) {
          const int id = it * G_THREADS + tid;
          const int r = id >> ch_log, c = id & ((1 << ch_log) - 1);
          if (r < rows_here) {
            const uint4 v = *reinterpret_cast<const uint4*>(st + r * OS + c * 8);
            *reinterpret_cast<uint4*>(o + (row0 + r) * N + col0 + c * 8) = v;
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < MI; ++i) {
          const int r = rbase + i * 16 + (lane & 15);
          if (r >= rows_here) continue;
          const float lsr = empty ? 0.f : ls_tile[r];
          float* o = static_cast<float*>(out_t) + (row0 + r) * N + col0 + cbase + 4 * (lane >> 4);
#pragma unroll
          for (int j = 0; j < JN; ++j)
            *reinterpret_cast<float4*>(o + j * 16) =
                make_float4(lsr * (acc[i][j][0] * s_out[j].x), lsr * (acc[i][j][1] * s_out[j].y),
                            lsr * (acc[i][j][2] * s_out[j].z), lsr * (acc[i][j][3] * s_out[j].w));
        }
        if constexpr (AB) {
          const int r = BM / 2 + (lane & 15);
          if (r < rows_here) {
            const float lsr = ls_tile[r];
            const int jx = wave < 4 ? 0 : 2;
            float* o = static_cast<float*>(out_t) + (row0 + r) * N + col0 + cbase + 4 * (lane >> 4);
#pragma unroll
            for (int q = 0; q < 2; ++q) {
              const float4 so = jx == 0 ? s_out[q] : s_out[2 + q];
              *reinterpret_cast<float4*>(o + (jx + q) * 16) =
                  make_float4(lsr * (acc_x[q][0] * so.x), lsr * (acc_x[q][1] * so.y), lsr * (acc_x[q][2] * so.z),
                              lsr * (acc_x[q][3] * so.w));
            }
          }
        }
      }
    };
    if constexpr (ABS) {
      if (ab)
        tile_body(std::integral_constant<bool, true>{});
      else
        tile_body(std::integral_constant<bool, false>{});
    } else {
      tile_body(std::integral_constant<bool, false>{});
    }
  }
  };
  if constexpr (ABS) {
    if (split_s >= 2)
      tile_loop(std::integral_constant<bool, true>{});
    else
      tile_loop(std::integral_constant<bool, false>{});
  } else {
    tile_loop(std::integral_constant<bool, false>{});
  }
#undef MOE_SLOT
  // rows [n, M) are zero
  const int64_t zero_rows = BATCH ? 0 : M - n_rows;
  if (zero_rows > 0) {
    const int64_t per16 = OUT_BF16 ? 8 : 4;
    const int64_t total_chunks = zero_rows * N / per16;
    uint4* base = OUT_BF16 ? reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + n_rows * N)
                           : reinterpret_cast<uint4*>(static_cast<float*>(out) + n_rows * N);
    for (int64_t c = static_cast<int64_t>(blockIdx.x) * G_THREADS + tid; c < total_chunks;
         c += static_cast<int64_t>(gridDim.x) * G_THREADS)
      base[c] = make_uint4(0, 0, 0, 0);
  }
}

// ---------------------------------------------------------------- streaming
// gmm_stream_kernel: the same tiles, wave grid, staging and MFMA rounds as
// gmm_kernel, with one load pipeline through all of a workgroup's tiles.
// The loads that go out while the waves multiply step q belong to step
// q + NST - 1 of the workgroup's whole sequence of K steps, which near the
// end of a tile is a step of the next tile (or of the one after it, when
// tiles have a single step) -- so a tile starts with its first stages
// already landed, and short tiles (few K steps) no longer pay the load
// latency at every tile start.
//  * A tile's first step also stages its parameters into one of three LDS
//    parameter slots: the lhs scales of its rows and the weight scales of its
//    columns (one 4-byte direct load per wave).  The slot of tile j is read
//    by tile j's epilogue at the end of its last step and refilled by tile
//    j + 3's first step, which is issued at least one barrier later.
//  * The wait before step q counts exactly the loads issued after step q's:
//    the next step's SLOTS (+1 blockwise scale) loads, plus one when that
//    step starts a tile.
//  * The epilogue writes the output from registers, since the stages in
//    flight occupy the LDS: float32 as 16-byte stores per lane, after a DPP
//    row-mirror swap that makes each store cover whole 128-byte lines of 8
//    rows (store_rows_lines); bfloat16 after two lane swaps per dword pair
//    (v_permlane32_swap, then v_permlane16_swap), which turn a lane's two
//    blocks' four-column pieces into eight consecutive columns of its row --
//    again one 16-byte store.
constexpr int kStreamMaxLocal = 512;   // group table capacity (LDS budget)
constexpr int PRM = 512;               // floats per parameter slot: 256 row scales, 256 column scales
constexpr int PRM_SLOTS = 3;

struct TileDesc {
  int g, KT, rows_here, wide;
  int64_t row0, col0, cofs;
};

// Decode tile t exactly as gmm_kernel does (n-tile major, m-tiles fastest,
// wide tails after their two n-tiles' full m-tiles; BATCH: per-group m x n
// grid over the group's padded contraction columns).
template <class C, bool BATCH, class GT>
__device__ __forceinline__ TileDesc decode_tile(const GT& gt, int El, int MTb, int NT, int KT, int t) {
  constexpr int BM = C::BM, BN = C::BN;
  const int g = BATCH ? t / (MTb * NT) : find_group(gt, El, t);
  const int local = BATCH ? t - g * (MTb * NT) : t - gt.tiles_off[g];
  const int m_g = gt.rows_off[g + 1] - gt.rows_off[g];
  const int full = m_g / BM, rem = m_g - full * BM;
  int nt, mt, wide = 0;
  if (BATCH) {
    nt = local / MTb;
    mt = local - nt * MTb;
  } else if (rem == 0 || rem > BM / 2) {
    const int per = full + (rem ? 1 : 0);
    nt = local / per;
    mt = local - nt * per;
  } else {
    const int pairblk = 2 * full + 1, npair = NT / 2;
    if (local < npair * pairblk) {
      const int pr = local / pairblk, w = local - pr * pairblk;
      if (w < 2 * full) {
        const int h = w >= full ? 1 : 0;
        nt = 2 * pr + h;
        mt = w - h * full;
      } else {
        nt = 2 * pr;
        mt = full;
        wide = 1;
      }
    } else {
      nt = NT - 1;
      mt = local - npair * pairblk;
    }
  }
  TileDesc d;
  d.g = g;
  d.wide = wide;
  d.row0 = BATCH ? static_cast<int64_t>(mt) * BM : gt.rows_off[g] + static_cast<int64_t>(mt) * BM;
  d.rows_here = BATCH ? BM : min(BM, m_g - mt * BM);
  d.col0 = static_cast<int64_t>(nt) * BN;
  d.cofs = BATCH ? static_cast<int64_t>(gt.tiles_off[g]) * G_BK : 0;
  d.KT = BATCH ? (m_g + G_BK - 1) / G_BK : KT;
  return d;
}

// Four LDS floats at p + {0, 16, 32, 48}, completed before returning (one asm
// block, for the same reason as lds_read_4x16f).
__device__ __forceinline__ float4 lds_read_4x1f(const float* p) {
  typedef const __attribute__((address_space(3))) float lds_f32;
  const uint32_t a = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_f32*)p));
  float x, y, z, w;
  asm volatile(
      "ds_read_b32 %0, %4\n\t"
      "ds_read_b32 %1, %4 offset:64\n\t"
      "ds_read_b32 %2, %4 offset:128\n\t"
      "ds_read_b32 %3, %4 offset:192\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(x), "=&v"(y), "=&v"(z), "=&v"(w)
      : "v"(a)
      : "memory");
  return make_float4(x, y, z, w);
}

// Lane l = 16 g + r holds, for the blocks of columns 32p .. 32p+15 (P) and
// 32p+16 .. 32p+31 (Q) of its row r, the packed bfloat16 pairs of columns
// 4g .. 4g+3 of each.  Returns columns 32p + 8g .. 32p + 8g + 7 of the same
// row: the 32-lane swap exchanges P of lane groups 2, 3 with Q of groups 0, 1,
// the 16-lane swap then exchanges odd groups of the first operand with even
// groups of the second.
__device__ __forceinline__ uint4 row8_from_blocks(uint32_t p0, uint32_t p1, uint32_t q0, uint32_t q1) {
  const auto s0 = __builtin_amdgcn_permlane32_swap(p0, q0, false, false);
  const auto t0 = __builtin_amdgcn_permlane16_swap(s0[0], s0[1], false, false);
  const auto s1 = __builtin_amdgcn_permlane32_swap(p1, q1, false, false);
  const auto t1 = __builtin_amdgcn_permlane16_swap(s1[0], s1[1], false, false);
  return make_uint4(t0[0], t1[0], t0[1], t1[1]);
}

// One tile's output as it leaves the registers: 16-byte pieces of the lane's
// row (base + 16 i) at column offsets (elements) col_of(i, u).
template <class C, bool OUT_BF16>
struct OutPieces {
  static constexpr int U = OUT_BF16 ? C::JN / 2 : C::JN;   // pieces per row block
  uint4 v[C::MI][U];
};

// Scale and convert the accumulators: out = ls[row] * (acc * cs[col]).
template <class C, bool OUT_BF16>
__device__ __forceinline__ void convert_tile(const v4f (&acc)[C::MI][C::JN], const float4 lsr, const float4 (&cs)[C::JN],
                                             OutPieces<C, OUT_BF16>& o) {
#pragma unroll
  for (int i = 0; i < C::MI; ++i) {
    const float l = i == 0 ? lsr.x : i == 1 ? lsr.y : i == 2 ? lsr.z : lsr.w;
    if constexpr (OUT_BF16) {
#pragma unroll
      for (int p = 0; p < C::JN / 2; ++p) {
        const v4f& a = acc[i][2 * p];
        const v4f& b = acc[i][2 * p + 1];
        const float4 sa = cs[2 * p], sb = cs[2 * p + 1];
        const uint32_t p0 = pack_bf16x2(l * (a[0] * sa.x), l * (a[1] * sa.y));
        const uint32_t p1 = pack_bf16x2(l * (a[2] * sa.z), l * (a[3] * sa.w));
        const uint32_t q0 = pack_bf16x2(l * (b[0] * sb.x), l * (b[1] * sb.y));
        const uint32_t q1 = pack_bf16x2(l * (b[2] * sb.z), l * (b[3] * sb.w));
        o.v[i][p] = row8_from_blocks(p0, p1, q0, q1);
      }
    } else {
#pragma unroll
      for (int j = 0; j < C::JN; ++j) {
        const v4f& a = acc[i][j];
        o.v[i][j] = make_uint4(__float_as_uint(l * (a[0] * cs[j].x)), __float_as_uint(l * (a[1] * cs[j].y)),
                               __float_as_uint(l * (a[2] * cs[j].z)), __float_as_uint(l * (a[3] * cs[j].w)));
      }
    }
  }
}

// The buffer descriptor of a tile's output rows: base = its first row,
// range = its valid rows, so a piece of a row past the tile is dropped by
// the range check -- every wave issues the same number of stores, which
// keeps the pipeline's wait counts exact.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(uint8_t* base, uint32_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b >> 32));
  void* u = reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(u, 0, static_cast<int>(__builtin_amdgcn_readfirstlane(bytes)), 0x00020000);
}

// Row block i of a converted tile: voff = the byte offset of the lane's row
// of block 0 and its first column from the tile's first row.
template <class C, bool OUT_BF16, int POL = 0>
__device__ __forceinline__ void store_rows(const OutPieces<C, OUT_BF16>& o, int i, __amdgpu_buffer_rsrc_t r,
                                           uint32_t voff, uint32_t row_bytes) {
  typedef uint32_t u4 __attribute__((ext_vector_type(4)));
#pragma unroll
  for (int u = 0; u < OutPieces<C, OUT_BF16>::U; ++u) {   // bf16: 32 columns apart; f32: 16
    const uint4 v = o.v[i][u];
    __builtin_amdgcn_raw_buffer_store_b128(u4{v.x, v.y, v.z, v.w}, r, voff + 16 * i * row_bytes + u * 64, 0, POL);
  }
}

// Row block i of a converted float32 tile, written as whole 128-byte lines.
// A lane's pieces of column blocks 2p and 2p+1 lie 64 bytes apart in its
// row (row r = lane % 16), so storing them as they are fills each line of a
// row with two stores.  Lanes r and 15 - r (one in each half of the 16 rows)
// swap one piece over the DPP row mirror: lane r < 8 keeps block 2p of row r
// and receives block 2p of row 15 - r; lane r >= 8 keeps block 2p + 1 of row
// r and receives block 2p + 1 of row 15 - r.  The first store then covers
// rows 0..7 and the second rows 8..15, each row's 128 bytes whole.
// voff_a, voff_b = the byte offsets (from the tile's first row) of the
// lane's piece in row block 0 for the two stores: rows min(r, 15 - r) and
// max(r, 15 - r), at byte 64 (r / 8) + 16 (lane / 16) of the column range.
template <class C, int POL = 0>
__device__ __forceinline__ void store_rows_lines(const OutPieces<C, false>& o, int i, __amdgpu_buffer_rsrc_t r,
                                                 uint32_t voff_a, uint32_t voff_b, uint32_t row_bytes, bool upper) {
  typedef uint32_t u4 __attribute__((ext_vector_type(4)));
  static_assert(C::JN % 2 == 0, "pairs of column blocks");
#pragma unroll
  for (int p = 0; p < C::JN / 2; ++p) {
    const uint4 p0 = o.v[i][2 * p], p1 = o.v[i][2 * p + 1];
    const uint4 x = upper ? p0 : p1;              // the piece the mirrored lane stores
    uint4 y;
    y.x = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x.x), 0x140, 0xF, 0xF, false));
    y.y = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x.y), 0x140, 0xF, 0xF, false));
    y.z = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x.z), 0x140, 0xF, 0xF, false));
    y.w = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x.w), 0x140, 0xF, 0xF, false));
    const uint4 a = upper ? y : p0;               // rows 0..7
    const uint4 b = upper ? p1 : y;               // rows 8..15
    const uint32_t blk = 16 * i * row_bytes + p * 128;
    __builtin_amdgcn_raw_buffer_store_b128(u4{a.x, a.y, a.z, a.w}, r, voff_a + blk, 0, POL);
    __builtin_amdgcn_raw_buffer_store_b128(u4{b.x, b.y, b.z, b.w}, r, voff_b + blk, 0, POL);
  }
}

template <class C, bool TRANS, bool KBLOCKS, bool OUT_BF16, bool BATCH>
__global__ __launch_bounds__(C::THREADS) void gmm_stream_kernel(
    const uint8_t* __restrict__ lhs, const float* __restrict__ ls, int ls_per_row, const uint8_t* __restrict__ rhs,
    const float* __restrict__ rs, int Kb, int Nb, const int32_t* __restrict__ group_sizes, int g0, int El, int64_t M,
    int64_t K, int64_t N, void* __restrict__ out, int32_t* __restrict__ err, int64_t max_rows) {
  constexpr int BM = C::BM, BN = C::BN, NST = C::NST, WM = C::WM, WN = C::WN, MI = C::MI, JN = C::JN;
  constexpr int STAGE = C::STAGE, NW = C::NW;
  static_assert(BM == 256 && BN == 128 && NST == 3 && NW == 8 && JN == 4, "streaming layout");
  constexpr int LPS = loads_per_step<C, KBLOCKS>();
  constexpr int ESZ = OUT_BF16 ? 2 : 4;
  constexpr int SPOL = BATCH ? MOE_GMM_BATCH_STORE_POLICY : 0;   // output store cache policy
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NST * STAGE];
  __shared__ __attribute__((aligned(16))) float prm[PRM_SLOTS * PRM];
  __shared__ GroupTableN<kStreamMaxLocal> gt;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int w4 = wave & 3;
  const int NT = static_cast<int>(N / BN);
  const int MTb = static_cast<int>(M / BM);
  if constexpr (BATCH)
    build_groups(group_sizes, g0, El, max_rows, 1, G_BK, err, gt, reinterpret_cast<int*>(smem), false);
  else
    build_groups(group_sizes, g0, El, M, NT, BM, err, gt, reinterpret_cast<int*>(smem), true);
  const int total = BATCH ? El * MTb * NT : gt.tiles_off[El];
  const int n_rows = gt.rows_off[El];
  const int KT = static_cast<int>(K / G_BK);
  const int steps_per_block = static_cast<int>(K / Kb / G_BK);
  const uint32_t ncol_blk = static_cast<uint32_t>(N / Nb);
  int first, last, tstep;
  xcd_share(total, first, last, tstep);
  const LaneOff offK = stage_lane_off(lane, K);
  const LaneOff offN = stage_lane_off(lane, N);
  const int64_t row_bytes = N * ESZ;

  // ---- load cursor: tile lt (descriptor L), its step lk, its parameter slot
  int lt = first, lk = 0, lslot = 0;
  TileDesc L = {};
  while (lt < last) {
    L = decode_tile<C, BATCH>(gt, El, MTb, NT, KT, lt);
    if (L.KT > 0) break;
    lt += tstep;
  }

  // per load tile: this lane's six slot sources at contraction offset 0 and
  // its blockwise-scale source (first block)
  const uint8_t* lsrc[6];
  const float* lsc = rs;
#define MOE_SPLAN()                                                                                              \
  do {                                                                                                           \
    const bool tl = L.row0 + (L.wide ? BM / 2 : BM) > M;                                                         \
    const uint8_t* lh = lhs + L.cofs;                                                                            \
    const uint8_t* wgl = BATCH ? rhs + L.cofs : rhs + L.g * K * N;                                               \
    const bool wd = L.wide != 0;                                                                                 \
    lsrc[0] = slot_src0<TRANS, NW, 0>(wd, lh, wgl, K, N, L.row0, L.col0, M, tl, wave, lane, offK, offN);         \
    lsrc[1] = slot_src0<TRANS, NW, 1>(wd, lh, wgl, K, N, L.row0, L.col0, M, tl, wave, lane, offK, offN);         \
    lsrc[2] = slot_src0<TRANS, NW, 2>(wd, lh, wgl, K, N, L.row0, L.col0, M, tl, wave, lane, offK, offN);         \
    lsrc[3] = slot_src0<TRANS, NW, 3>(wd, lh, wgl, K, N, L.row0, L.col0, M, tl, wave, lane, offK, offN);         \
    lsrc[4] = slot_src0<TRANS, NW, 4>(wd, lh, wgl, K, N, L.row0, L.col0, M, tl, wave, lane, offK, offN);         \
    lsrc[5] = slot_src0<TRANS, NW, 5>(wd, lh, wgl, K, N, L.row0, L.col0, M, tl, wave, lane, offK, offN);         \
    if (KBLOCKS)                                                                                                 \
      lsc = (BATCH ? rs : rs + static_cast<int64_t>(L.g) * Kb * Nb) +                                            \
            static_cast<uint32_t>(L.col0 + min(w4 * 64 + lane, (L.wide ? 2 * BN : BN) - 1)) / ncol_blk;         \
  } while (0)
  if (lt < last) MOE_SPLAN();
#define MOE_SSLOT(S, stg, kbv)                                                                                   \
  issue_from<NW, S>(lsrc[S] + ((TRANS || slot_is_a<NW, S>(L.wide != 0)) ? (kbv) : (kbv) * N), L.wide != 0, stg, wave)
  // the step's extra loads: its blockwise weight scales, and on a tile's first
  // step the tile's parameters (waves 0-3 the row scales, 4-7 the column scales)
#define MOE_SEXTRA(stg)                                                                                          \
  do {                                                                                                           \
    const int bn_l = L.wide ? 2 * BN : BN;                                                                       \
    const float* rs_l = BATCH ? rs : rs + static_cast<int64_t>(L.g) * Kb * Nb;                                   \
    if (KBLOCKS)                                                                                                 \
      __builtin_amdgcn_global_load_lds(lsc + static_cast<int64_t>(lk / steps_per_block) * Nb,                     \
                                       (lds_void*)(stg + C::SC_OFF + w4 * 256), 4, 0, 0);                         \
    if (lk == 0) {                                                                                               \
      float* pslot = prm + lslot * PRM;                                                                          \
      if (wave < 4) {                                                                                            \
        const int r = min(w4 * 64 + lane, L.rows_here - 1);                                                      \
        __builtin_amdgcn_global_load_lds(ls + (ls_per_row ? L.row0 + r : 0), (lds_void*)(pslot + w4 * 64), 4, 0, \
                                         0);                                                                     \
      } else {                                                                                                   \
        const int c = min(w4 * 64 + lane, bn_l - 1);                                                             \
        __builtin_amdgcn_global_load_lds(rs_l + static_cast<uint32_t>(L.col0 + c) / ncol_blk,                    \
                                         (lds_void*)(pslot + 256 + w4 * 64), 4, 0, 0);                           \
      }                                                                                                          \
    }                                                                                                            \
  } while (0)
  // after a step's loads: next step, or the next tile with steps
#define MOE_SADVANCE()                                 \
  do {                                                 \
    if (++lk == L.KT) {                                \
      lk = 0;                                          \
      lslot = lslot == PRM_SLOTS - 1 ? 0 : lslot + 1;  \
      lt += tstep;                                     \
      while (lt < last) {                              \
        L = decode_tile<C, BATCH>(gt, El, MTb, NT, KT, lt); \
        if (L.KT > 0) break;                           \
        lt += tstep;                                   \
      }                                                \
      if (lt < last) MOE_SPLAN();                      \
    }                                                  \
  } while (0)

  // ---- prologue: steps 0 .. NST-2 of the sequence
  int issued = 0;
  bool next_starts = false;      // the step after the one computed next starts a tile
#pragma unroll
  for (int s = 0; s < NST - 1; ++s) {
    if (lt < last) {
      uint8_t* stg = smem + s * STAGE;
      const int64_t kb = static_cast<int64_t>(lk) * G_BK;
      MOE_SSLOT(0, stg, kb); MOE_SSLOT(1, stg, kb); MOE_SSLOT(2, stg, kb);
      MOE_SSLOT(3, stg, kb); MOE_SSLOT(4, stg, kb); MOE_SSLOT(5, stg, kb);
      if (s == 1) next_starts = lk == 0;
      MOE_SEXTRA(stg);
      ++issued;
      MOE_SADVANCE();
    }
  }

  // ---- compute cursor: tile ct (descriptor Cd), its step ck, its slot
  int ct = first, ck = 0, cslot = 0;
  TileDesc Cd = {};
  const int gn_plain = BN / WN;
  // the empty tiles of a BATCH sequence get zeros; then the first tile with steps
  OutPieces<C, OUT_BF16> po;
  __amdgpu_buffer_rsrc_t p_rsrc = tile_rsrc(static_cast<uint8_t*>(out), 0);   // the converted tile's rows
  uint32_t p_voff = 0;
  // stores issued after the loads of the steps in flight: st_prev = the
  // previous iteration's epilogue stores, st_tail2 = the one before it
  // (an epilogue's stores follow all of its iteration's loads); drain = zero
  // tiles were written (a variable count): wait for everything once
  constexpr int ST = MI * OutPieces<C, OUT_BF16>::U;   // stores per converted tile and wave
  bool st_prev = false, st_tail2 = false, drain = false;
#define MOE_ZERO_TILE(D)                                                                                         \
  do {                                                                                                           \
    const int rb = (wave / gn_plain) * WM, cb = (wave % gn_plain) * WN;                                          \
    const __amdgpu_buffer_rsrc_t zr = tile_rsrc(static_cast<uint8_t*>(out) + static_cast<int64_t>(D.g) * M * row_bytes + \
                                                D.row0 * row_bytes, static_cast<uint32_t>(D.rows_here * row_bytes)); \
    const uint32_t zo = static_cast<uint32_t>((rb + (lane & 15)) * row_bytes + (D.col0 + cb) * ESZ + 16 * (lane >> 4)); \
    OutPieces<C, OUT_BF16> z;                                                                                    \
    _Pragma("unroll") for (int i = 0; i < MI; ++i) _Pragma("unroll") for (int u = 0; u < OutPieces<C, OUT_BF16>::U; ++u) \
        z.v[i][u] = make_uint4(0, 0, 0, 0);                                                                      \
    _Pragma("unroll") for (int i = 0; i < MI; ++i) store_rows<C, OUT_BF16, SPOL>(z, i, zr, zo, static_cast<uint32_t>(row_bytes)); \
    drain = true;                                                                                                \
  } while (0)
  while (ct < last) {
    Cd = decode_tile<C, BATCH>(gt, El, MTb, NT, KT, ct);
    if (Cd.KT > 0) break;
    MOE_ZERO_TILE(Cd);
    ct += tstep;
  }
  int gn = Cd.wide ? 2 * BN / WN : BN / WN;
  int rbase = (wave / gn) * WM, cbase = (wave % gn) * WN;
  FragOff fa = frag_off(rbase, lane);
  FragOff fb = frag_off(cbase, lane);

  v4f acc[MI][JN];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < JN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  int q = 0, cur = 0;            // sequence step being computed, its stage
  while (ct < last) {
    // this wave's loads of step q have landed once at most the operations
    // issued after them are outstanding: the next step's loads and the stores
    // that went out since (vector-memory operations, loads and stores alike,
    // complete in issue order)
    if (issued > q + 1 && !drain) {
      const int code = (next_starts ? 1 : 0) | (st_prev ? 2 : 0) | (st_tail2 ? 4 : 0);
      switch (code) {
        case 0: __builtin_amdgcn_s_waitcnt(waitcnt_vm(LPS)); break;
        case 1: __builtin_amdgcn_s_waitcnt(waitcnt_vm(LPS + 1)); break;
        case 2: __builtin_amdgcn_s_waitcnt(waitcnt_vm(LPS + ST)); break;
        case 3: __builtin_amdgcn_s_waitcnt(waitcnt_vm(LPS + 1 + ST)); break;
        case 4: __builtin_amdgcn_s_waitcnt(waitcnt_vm(LPS + ST)); break;
        case 5: __builtin_amdgcn_s_waitcnt(waitcnt_vm(LPS + 1 + ST)); break;
        case 6: __builtin_amdgcn_s_waitcnt(waitcnt_vm(LPS + 2 * ST)); break;
        default: __builtin_amdgcn_s_waitcnt(waitcnt_vm(LPS + 1 + 2 * ST)); break;
      }
    } else {
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    }
    drain = false;
    step_barrier();                         // everyone's have, and step q-1's readers are done
    const bool more = lt < last;
    const int nxt_i = cur == 0 ? 2 : cur - 1;     // (cur + NST - 1) % NST
    uint8_t* nxt = smem + nxt_i * STAGE;
    const int64_t kb_next = static_cast<int64_t>(lk) * G_BK;
    const bool starts = lk == 0;
    const uint8_t* As = smem + cur * STAGE;
    const uint8_t* Bs = As + (Cd.wide ? BM / 2 : BM) * G_BK;
    float4 s_col[JN];
    if (KBLOCKS) {
      const float* sc = reinterpret_cast<const float*>(As + C::SC_OFF) + cbase + 4 * (lane >> 4);
      lds_read_4x16f(sc, s_col);
    }
    v8i b[JN];
#pragma unroll
    for (int j = 0; j < JN; ++j) {
      const int n0 = cbase + j * 16;
      if (TRANS)
        b[j] = frag_i(Bs, fb, j);
      else
        b[j] = frag_tr_swz(Bs + (n0 >> 7) * (128 * G_BK), n0 & 127, lane);
    }
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const v8i a = frag_i(As, fa, i);
      if (more) {
        if (i == 0) { MOE_SSLOT(0, nxt, kb_next); MOE_SSLOT(1, nxt, kb_next); MOE_SEXTRA(nxt); }
        if (i == 1) { MOE_SSLOT(2, nxt, kb_next); }
        if (i == 2) { MOE_SSLOT(3, nxt, kb_next); MOE_SSLOT(4, nxt, kb_next); }
        if (i == 3) { MOE_SSLOT(5, nxt, kb_next); }
      }
#pragma unroll
      for (int j = 0; j < JN; ++j) {
        if (KBLOCKS) {
          const v4f p = mfma_f8(b[j], a, v4f{0.f, 0.f, 0.f, 0.f});
          acc[i][j][0] = fmaf(s_col[j].x, p[0], acc[i][j][0]);
          acc[i][j][1] = fmaf(s_col[j].y, p[1], acc[i][j][1]);
          acc[i][j][2] = fmaf(s_col[j].z, p[2], acc[i][j][2]);
          acc[i][j][3] = fmaf(s_col[j].w, p[3], acc[i][j][3]);
        } else {
          acc[i][j] = mfma_f8(b[j], a, acc[i][j]);
        }
      }
    }
    bool st_now = false;    // this iteration ends a tile: its epilogue stores follow its loads
    if (more) {
      next_starts = starts;
      ++issued;
      MOE_SADVANCE();
    } else {
      next_starts = false;
    }
    ++q;
    cur = cur == NST - 1 ? 0 : cur + 1;

    if (++ck == Cd.KT) {
      // ---- epilogue of tile ct: scales from its parameter slot
      const float* pslot = prm + cslot * PRM;
      const float4 lsr = lds_read_4x1f(pslot + rbase + (lane & 15));
      float4 cs[JN];
      if (KBLOCKS) {
#pragma unroll
        for (int j = 0; j < JN; ++j) cs[j] = make_float4(1.f, 1.f, 1.f, 1.f);
      } else {
        lds_read_4x16f(pslot + 256 + cbase + 4 * (lane >> 4), cs);
      }
      convert_tile<C, OUT_BF16>(acc, lsr, cs, po);
      p_rsrc = tile_rsrc(static_cast<uint8_t*>(out) + (BATCH ? static_cast<int64_t>(Cd.g) * M * row_bytes : 0) +
                             Cd.row0 * row_bytes,
                         static_cast<uint32_t>(Cd.rows_here * row_bytes));
      if constexpr (!OUT_BF16) {
        const int r = lane & 15;
        const bool upper = r >= 8;
        const uint32_t colb = static_cast<uint32_t>((Cd.col0 + cbase) * ESZ + 64 * (upper ? 1 : 0) + 16 * (lane >> 4));
        const uint32_t va = static_cast<uint32_t>((rbase + (upper ? 15 - r : r)) * row_bytes) + colb;
        const uint32_t vb = static_cast<uint32_t>((rbase + (upper ? r : 15 - r)) * row_bytes) + colb;
#pragma unroll
        for (int i = 0; i < MI; ++i) store_rows_lines<C, SPOL>(po, i, p_rsrc, va, vb, static_cast<uint32_t>(row_bytes), upper);
      } else {
        p_voff = static_cast<uint32_t>((rbase + (lane & 15)) * row_bytes + (Cd.col0 + cbase) * ESZ + 16 * (lane >> 4));
#pragma unroll
        for (int i = 0; i < MI; ++i) store_rows<C, OUT_BF16, SPOL>(po, i, p_rsrc, p_voff, static_cast<uint32_t>(row_bytes));
      }
      st_now = true;
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < JN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
      ck = 0;
      cslot = cslot == PRM_SLOTS - 1 ? 0 : cslot + 1;
      ct += tstep;
      while (ct < last) {
        Cd = decode_tile<C, BATCH>(gt, El, MTb, NT, KT, ct);
        if (Cd.KT > 0) break;
        MOE_ZERO_TILE(Cd);
        ct += tstep;
      }
      gn = Cd.wide ? 2 * BN / WN : BN / WN;
      rbase = (wave / gn) * WM;
      cbase = (wave % gn) * WN;
      fa = frag_off(rbase, lane);
      fb = frag_off(cbase, lane);
    }
    st_tail2 = st_prev;
    st_prev = st_now;
  }
#undef MOE_SSLOT
#undef MOE_SPLAN
#undef MOE_SEXTRA
#undef MOE_SADVANCE
#undef MOE_ZERO_TILE
  // rows [n, M) are zero
  const int64_t zero_rows = BATCH ? 0 : M - n_rows;
  if (zero_rows > 0) {
    const int64_t total_chunks = zero_rows * row_bytes / 16;
    uint4* base = reinterpret_cast<uint4*>(static_cast<uint8_t*>(out) + n_rows * row_bytes);
    for (int64_t c = static_cast<int64_t>(blockIdx.x) * C::THREADS + tid; c < total_chunks;
         c += static_cast<int64_t>(gridDim.x) * C::THREADS)
      base[c] = make_uint4(0, 0, 0, 0);
  }
}

// Launch one configuration: persistent grid of (workgroups per CU) x CUs.
template <class C, bool TRANS, bool KBLOCKS, bool OUT_BF16, bool I8>
hipError_t launch_cfg(const uint8_t* lhs, const float* ls, int per_row, const uint8_t* rhs, const float* rs, int Kb,
                      int Nb, const int32_t* gs, int g0, int El, int64_t M, int64_t K, int64_t N, void* out,
                      int32_t* err, float* part, int32_t* cnt, int nslots, hipStream_t st) {
  constexpr int lds = C::LDS + static_cast<int>(sizeof(GroupTable)) + C::BM * 4;
  constexpr int per_cu = (160 * 1024) / lds > 0 ? (160 * 1024) / lds : 1;
  const int64_t ub = (moe_cdiv(M, C::BM) + El) * (N / C::BN);    // tile-count bound
  int64_t grid = static_cast<int64_t>(per_cu) * tile::num_cus();
  if (ub < grid) grid = ub;
  if (grid < 8) grid = 8;
  if constexpr (MOE_GMM_STREAM != 0 && !I8) {
    if (El <= kStreamMaxLocal) {
      gmm_stream_kernel<C, TRANS, KBLOCKS, OUT_BF16, false>
          <<<static_cast<unsigned>(grid), C::THREADS, 0, st>>>(lhs, ls, per_row, rhs, rs, Kb, Nb, gs, g0, El, M, K, N,
                                                              out, err, 0);
      return hipGetLastError();
    }
  }
  if constexpr (TRANS && MOE_GMM_WIDE_ALL != 0 && MOE_GMM_ABSORB != 0) {
    if (El <= kAbsMaxLocal) {
      gmm_kernel<C, TRANS, KBLOCKS, OUT_BF16, false, I8, true><<<static_cast<unsigned>(grid), C::THREADS, 0, st>>>(
          lhs, ls, per_row, rhs, rs, Kb, Nb, gs, g0, El, M, K, N, out, err, 0, 1, part, cnt, nslots);
      return hipGetLastError();
    }
  }
  gmm_kernel<C, TRANS, KBLOCKS, OUT_BF16, false, I8><<<static_cast<unsigned>(grid), C::THREADS, 0, st>>>(
      lhs, ls, per_row, rhs, rs, Kb, Nb, gs, g0, El, M, K, N, out, err, 0, MOE_GMM_WIDE_ALL);
  return hipGetLastError();
}

template <class C, bool TRANS, bool KBLOCKS, bool I8>
hipError_t launch_dtype(bool bf16, const uint8_t* lhs, const float* ls, int per_row, const uint8_t* rhs,
                        const float* rs, int Kb, int Nb, const int32_t* gs, int g0, int El, int64_t M, int64_t K,
                        int64_t N, void* out, int32_t* err, float* part, int32_t* cnt, int nslots, hipStream_t st) {
  return bf16 ? launch_cfg<C, TRANS, KBLOCKS, true, I8>(lhs, ls, per_row, rhs, rs, Kb, Nb, gs, g0, El, M, K, N, out,
                                                        err, part, cnt, nslots, st)
              : launch_cfg<C, TRANS, KBLOCKS, false, I8>(lhs, ls, per_row, rhs, rs, Kb, Nb, gs, g0, El, M, K, N, out,
                                                         err, part, cnt, nslots, st);
}

}  // namespace

// The header (error word), and for the split last round the counters and one
// float32 slot per workgroup of the persistent grid (one workgroup per CU).
size_t gmm_ws_bytes() {
  return static_cast<size_t>(tile::kSplitSlotOff) +
         static_cast<size_t>(tile::num_cus()) * tile::kSplitSlot * sizeof(float);
}

hipError_t gmm_edge_launch(const uint8_t* lhs, const float* ls, int per_row, const uint8_t* rhs, const float* rs,
                           int Kb, int Nb, bool trans, const int32_t* gs, int g0, int El, int64_t M, int64_t K,
                           int64_t N, bool bf16, bool i8, void* out, int32_t* err, hipStream_t st);

// The weight-gradient product on the gmm pipeline: for each local group g,
// out[g] (M x N, f32 or bf16) = ls[m] * rs[n] * sum_r A[m, c_g + r] B[n, c_g + r]
// with A [M, K] and B [N, K] contraction-contiguous (row stride K), c_g =
// 128 * (the group's padded row offset in 128-row blocks), the group's rows
// zero-padded to a multiple of 128; ls_len in {1, M}, rs_len in {1, N}.
// Requires M % 256 == 0 and N % 128 == 0.
hipError_t gmm_batched_launch(const uint8_t* A, const float* ls, int ls_len, const uint8_t* B, const float* rs,
                              int rs_len, const int32_t* group_sizes, int g0, int El, int64_t max_rows, int64_t M,
                              int64_t K, int64_t N, bool bf16, void* out, int32_t* err, hipStream_t st) {
  using C = Cfg<MOE_GMM_CFG>;
  const int64_t tiles = static_cast<int64_t>(El) * (M / C::BM) * (N / C::BN);
  int64_t grid = tile::num_cus();
  if (tiles < grid) grid = tiles;
  if (grid < 8) grid = 8;          // the XCD split gives each of the 8 parts its own workgroups
  const int per_row = ls_len == M ? 1 : 0;
  const int Nb = rs_len == 1 ? 1 : static_cast<int>(N);
  const unsigned gx = static_cast<unsigned>(grid);
  if (MOE_GMM_STREAM_BATCH != 0 && El <= kStreamMaxLocal) {
    if (bf16)
      gmm_stream_kernel<C, true, false, true, true><<<gx, C::THREADS, 0, st>>>(
          A, ls, per_row, B, rs, 1, Nb, group_sizes, g0, El, M, K, N, out, err, max_rows);
    else
      gmm_stream_kernel<C, true, false, false, true><<<gx, C::THREADS, 0, st>>>(
          A, ls, per_row, B, rs, 1, Nb, group_sizes, g0, El, M, K, N, out, err, max_rows);
  } else if (bf16) {
    gmm_kernel<C, true, false, true, true><<<gx, C::THREADS, 0, st>>>(A, ls, per_row, B, rs, 1, Nb, group_sizes, g0,
                                                                       El, M, K, N, out, err, max_rows);
  } else {
    gmm_kernel<C, true, false, false, true><<<gx, C::THREADS, 0, st>>>(A, ls, per_row, B, rs, 1, Nb, group_sizes, g0,
                                                                        El, M, K, N, out, err, max_rows);
  }
  return hipGetLastError();
}

}  // namespace moe

namespace moe {
namespace {
// Validation and dispatch shared by the e4m3fn and the int8 entry points.
template <bool I8>
int gmm_entry(const uint8_t* lhs, const float* lhs_scale, int lhs_scale_mode, const uint8_t* rhs,
              const float* rhs_scale, int32_t Kb, int32_t Nb, int transpose_rhs, const int32_t* group_sizes,
              int32_t E, int32_t group_offset, int32_t num_local_experts, int64_t M, int64_t K, int64_t N,
              int out_dtype, void* out, void* ws, size_t ws_bytes, void* stream) {
  using moe::tile::kMaxLocal;
  if (M < 0 || K <= 0 || N <= 0 || K % 16 || N % 16) return MOE_ERR_SHAPE;
  if (I8 && K > (int64_t{1} << 17)) return MOE_ERR_SHAPE;   // 127^2 * 2^17 < 2^31: the int32 sums stay exact
  if (E <= 0 || E > 1024 || group_offset < 0 || num_local_experts < 0 || num_local_experts > kMaxLocal ||
      group_offset + num_local_experts > E)
    return MOE_ERR_SHAPE;
  if (M > INT32_MAX - 1) return MOE_ERR_SHAPE;
  // the tile table of any split of M rows into El groups stays below 2^31 entries
  if ((moe_cdiv(M, 64) + num_local_experts + 1) * moe_cdiv(N, 64) > INT32_MAX) return MOE_ERR_SHAPE;
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
  if (ws_bytes < static_cast<size_t>(moe::tile::kHdr)) return MOE_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  int32_t* err = static_cast<int32_t*>(ws);
  // the split last round needs the counters and the slots: a workspace of the full size
  float* part = nullptr;
  int32_t* cnt = nullptr;
  int nslots = 0;
  if (ws_bytes >= moe::gmm_ws_bytes()) {
    cnt = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + moe::tile::kSplitCntOff);
    part = reinterpret_cast<float*>(static_cast<char*>(ws) + moe::tile::kSplitSlotOff);
    nslots = static_cast<int>((ws_bytes - moe::tile::kSplitSlotOff) / (moe::tile::kSplitSlot * sizeof(float)));
  }
  const int El = num_local_experts;
  const int per_row = lhs_scale_mode == MOE_SCALE_ROW_DYNAMIC ? 1 : 0;
  const bool bf16 = out_dtype == MOE_BF16;
  hipError_t e;
  if (K % 128 || N % 128)        // multiples of 16 only: the edge kernel
    return moe::gmm_edge_launch(lhs, lhs_scale, per_row, rhs, rhs_scale, Kb, Nb, transpose_rhs != 0, group_sizes,
                                group_offset, El, M, K, N, bf16, I8, out, err, st) == hipSuccess ? MOE_OK : MOE_ERR_HIP;
  using C = moe::Cfg<MOE_GMM_CFG>;
#define MOE_GMM_ARGS bf16, lhs, lhs_scale, per_row, rhs, rhs_scale, Kb, Nb, group_sizes, group_offset, El, M, K, N, out, err, \
                     part, cnt, nslots, st
  if (transpose_rhs)
    e = Kb > 1 ? moe::launch_dtype<C, true, true, I8>(MOE_GMM_ARGS) : moe::launch_dtype<C, true, false, I8>(MOE_GMM_ARGS);
  else
    e = Kb > 1 ? moe::launch_dtype<C, false, true, I8>(MOE_GMM_ARGS)
               : moe::launch_dtype<C, false, false, I8>(MOE_GMM_ARGS);
#undef MOE_GMM_ARGS
  return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}
}  // namespace
}  // namespace moe

extern "C" int moe_gmm_fp8(const uint8_t* lhs, const float* lhs_scale, int lhs_scale_mode, const uint8_t* rhs,
                           const float* rhs_scale, int32_t Kb, int32_t Nb, int transpose_rhs,
                           const int32_t* group_sizes, int32_t E, int32_t group_offset,
                           int32_t num_local_experts, int64_t M, int64_t K, int64_t N, int out_dtype,
                           void* out, void* ws, size_t ws_bytes, void* stream) {
  return moe::gmm_entry<false>(lhs, lhs_scale, lhs_scale_mode, rhs, rhs_scale, Kb, Nb, transpose_rhs, group_sizes, E,
                               group_offset, num_local_experts, M, K, N, out_dtype, out, ws, ws_bytes, stream);
}

extern "C" int moe_gmm_i8(const int8_t* lhs, const float* lhs_scale, int lhs_scale_mode, const int8_t* rhs,
                          const float* rhs_scale, int32_t Kb, int32_t Nb, int transpose_rhs,
                          const int32_t* group_sizes, int32_t E, int32_t group_offset,
                          int32_t num_local_experts, int64_t M, int64_t K, int64_t N, int out_dtype,
                          void* out, void* ws, size_t ws_bytes, void* stream) {
  return moe::gmm_entry<true>(reinterpret_cast<const uint8_t*>(lhs), lhs_scale, lhs_scale_mode,
                              reinterpret_cast<const uint8_t*>(rhs), rhs_scale, Kb, Nb, transpose_rhs, group_sizes, E,
                              group_offset, num_local_experts, M, K, N, out_dtype, out, ws, ws_bytes, stream);
}
