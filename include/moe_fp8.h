/*
 * moe_fp8.h -- C ABI of libmoefp8.so, the fp8 mixture-of-experts
 * grouped-matmul hot path for AMD Instinct MI355X (gfx950).
 *
 * The path, as the MaxText pull requests "Quantize activations before EP all
 * gather" (PR 4812), "Support quantization for tokamax gmm v2" (PR 4451) and
 * "Keep qwix out of tpu-inference's fused MoE kernel and pre-quantize
 * weights" (PR 5136) describe it:
 *   1. per-token absmax quantization of activations to float8_e4m3fn;
 *   2. a stable ragged sort of the routed rows into contiguous per-expert
 *      groups (group_sizes, group_offset), moving fp8 rows and their scales;
 *   3. the grouped matmul of fp8 operands with a 32-bit accumulator, a per-row
 *      lhs scale and per-channel or blockwise [E, blocks, 1, N] rhs scales
 *      (gmm), and its transposed form for weight gradients (tgmm);
 *   4. the un-sort plus top-k weighted gather-reduce back to token rows.
 *
 * Conventions shared by every call
 *   - Every tensor argument is caller-owned DEVICE memory, row-major and
 *     densely packed, unless a comment says "host".  The library allocates
 *     nothing, frees nothing and never synchronises (except
 *     moe_debug_check).  Scratch memory comes from the caller's workspace
 *     `ws` of `ws_bytes` bytes, sized by moe_workspace_bytes().  The first
 *     int32 of a workspace is a sticky device-error word: the caller zeroes a
 *     workspace once before its first use; kernels OR error bits into it
 *     (MOE_DEVERR_*) and never clear it.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL is the default
 *     stream).  The return value reports host-side validation and launch
 *     errors only; data-dependent problems (an expert id out of range, a
 *     negative group size, more local rows than the buffer holds) set the
 *     sticky error word, kernels clamp so that no access leaves its buffer,
 *     and the affected outputs are unspecified.
 *   - Unsupported combinations are rejected with MOE_ERR_UNSUPPORTED, never
 *     silently ignored.  Zero-sized problems return MOE_OK after writing
 *     whatever outputs are defined for them (zeros).
 *   - Element types: bf16 = bfloat16 bit patterns (uint16), f32 = IEEE
 *     binary32, e4m3fn = OCP float8 E4M3 (bias 7, max 448, no infinities,
 *     NaN = S.1111.111; not the "fnuz" variant).
 *   - Calls are stateless and may be issued from several host threads.
 */
#ifndef MOE_FP8_H
#define MOE_FP8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define MOE_OK 0
#define MOE_ERR_NULL 1          /* a required pointer is NULL */
#define MOE_ERR_SHAPE 2         /* sizes inconsistent or outside the supported range */
#define MOE_ERR_UNSUPPORTED 3   /* a valid but unsupported combination */
#define MOE_ERR_WORKSPACE 4     /* workspace missing or too small */
#define MOE_ERR_HIP 5           /* a HIP launch failed */

/* element types */
#define MOE_DTYPE_DEFAULT (-1)
#define MOE_BF16 0
#define MOE_F32 1
#define MOE_E4M3FN 2

/* activation-scale granularity */
#define MOE_SCALE_ROW_DYNAMIC 0     /* one scale per row, from the row's absmax: [R] */
#define MOE_SCALE_TENSOR_DYNAMIC 1  /* one scale from the whole tensor's absmax: [1] */
#define MOE_SCALE_TENSOR_STATIC 2   /* one fixed scale given by the caller: [1] */
#define MOE_SCALE_TENSOR_FROM_ROW_AMAX 3 /* one scale from caller-given row maxima: [1] */

/* activation applied before quantization */
#define MOE_ACT_NONE 0
#define MOE_ACT_SILU_MUL 1          /* quantize silu(x) * x_up (gated FFN) */

/* operation ids for moe_workspace_bytes */
#define MOE_OP_QUANTIZE_ROWS 0
#define MOE_OP_SORT_BY_EXPERT 1
#define MOE_OP_GMM 2
#define MOE_OP_TGMM 3
#define MOE_OP_GATHER_REDUCE 4
#define MOE_OP_QUANTIZE_WEIGHTS 5

/* bits of the sticky device-error word (first int32 of a workspace) */
#define MOE_DEVERR_EXPERT_ID 1      /* an expert id outside [0, E) */
#define MOE_DEVERR_GROUP_SIZE 2     /* a negative group size */
#define MOE_DEVERR_ROWS 4           /* local rows exceed the row capacity */

/*
 * moe_quantize_rows -- absmax quantization of activations to e4m3fn.
 * Defined by "Quantize activations before EP all gather" (description: the
 * activations are quantized before the expert-parallel all-gather and the
 * activation sort; review comments on ragged_sort.py: a per-token scale has
 * the token dimension first) and by the schemes of "Support quantization
 * for tokamax gmm v2" (fp8_dynamic = absmax, fp8_static_wa = fixed scale).
 *
 *   x        [R, C] bf16.  With act == MOE_ACT_SILU_MUL, x is the gate a and
 *            x_up [R, C] bf16 the up projection b, and the quantized matrix is
 *            h = f32(silu(a) * b), silu(a) = f32(a / f32(1 + exp(-a))), using
 *            the library's pinned float32 exp (Cody-Waite reduction, degree-7
 *            Taylor polynomial, no fused multiply-add).  x_up must be NULL
 *            otherwise.
 *   scale_mode, static_scale: see MOE_SCALE_*; static_scale must be a
 *            positive finite float for MOE_SCALE_TENSOR_STATIC.
 *   q        [R, C] e4m3fn out.  q = e4m3(clip(f32(v / s), -448, 448)) with an
 *            IEEE float32 divide and round-to-nearest-even (sign kept,
 *            subnormals kept).
 *   scale    out: [R] f32 (row mode) or [1] f32 (tensor modes);
 *            s = f32(amax / 448), or 1.0 when amax is 0.
 *   row_amax optional [R] f32 out (may be NULL): each row's absmax.  With
 *            MOE_SCALE_TENSOR_FROM_ROW_AMAX it is an INPUT instead (required):
 *            the rows' absmax as an earlier row-mode call on the same rows
 *            wrote it; the scale is then f32(max(row_amax) / 448) (1.0 when
 *            that is 0), which equals MOE_SCALE_TENSOR_DYNAMIC's result
 *            without its absmax pass over x.
 *   ws       needed only for MOE_SCALE_TENSOR_DYNAMIC (may be NULL otherwise).
 * R >= 0; C > 0 and a multiple of 16.  Inputs must be finite.
 */
int moe_quantize_rows(const void* x, const void* x_up, int act, int64_t R, int64_t C,
                      int scale_mode, float static_scale, uint8_t* q, float* scale,
                      float* row_amax, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_quantize_rows_strided -- moe_quantize_rows over inputs whose rows are
 * ldx elements apart (the same step, "Support quantization for tokamax gmm
 * v2" absmax scheme; for the gated FFN, the requantization of silu(a) * b
 * where a and b are the two column halves of one grouped-matmul output).
 *   ldx      row stride of x and x_up in elements; ldx >= C, a multiple of 8,
 *            and x, x_up 16-byte aligned (MOE_ERR_SHAPE otherwise).  q stays
 *            [R, C] contiguous.  Every other argument, the result and the
 *            errors are those of moe_quantize_rows, which is this call with
 *            ldx = C.
 */
int moe_quantize_rows_strided(const void* x, const void* x_up, int64_t ldx, int act, int64_t R, int64_t C,
                              int scale_mode, float static_scale, uint8_t* q, float* scale,
                              float* row_amax, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_quantize_weights -- offline blockwise absmax quantization of expert
 * weights, the pre-quantization of "Keep qwix out of tpu-inference's fused
 * MoE kernel and pre-quantize weights" ("Changes in this PR": float8_e4m3fn
 * weights with [E, blocks, 1, N] scales, blockwise or channelwise).
 *
 *   w        [E, K, N] bf16 (contraction dim K, output channels N).
 *   kb, nb   scale blocks: block (b, c) covers K rows b*K/kb.. and columns
 *            c*N/nb..; kb divides K, nb divides N.  kb = 1, nb = N is
 *            per-output-channel.
 *   scale_mode MOE_SCALE_ROW_DYNAMIC (absmax of each block) or
 *            MOE_SCALE_TENSOR_STATIC (every block gets static_scale).
 *   transpose_out 0: q is [E, K, N]; 1: q is [E, N, K] (contraction dim
 *            contiguous, the layout moe_gmm_fp8 reads with transpose_rhs = 1).
 *   q        e4m3fn out; scale [E, kb, 1, nb] f32 out (s = f32(amax/448), 1.0
 *            for an all-zero block), q = e4m3(clip(f32(w / s), -448, 448)).
 * K, N multiples of 16.  Setup-time call; needs no workspace.
 */
int moe_quantize_weights(const void* w, int64_t E, int64_t K, int64_t N, int32_t kb, int32_t nb,
                         int scale_mode, float static_scale, int transpose_out, uint8_t* q,
                         float* scale, void* stream);

/*
 * moe_quantize_rows_i8 -- absmax quantization of activations to symmetric
 * int8 codes, the activation side of the int8 variant: "Keep qwix out of
 * tpu-inference's fused MoE kernel and pre-quantize weights" ("Changes in
 * this PR") allows int8 weights beside e4m3fn ones, and no matrix core
 * multiplies int8 by fp8 codes, so int8 weights take int8 activations, with
 * the per-token scales of "Quantize activations before EP all gather".
 *
 *   x        [R, C] bf16, rows contiguous, 16-byte aligned; C a multiple
 *            of 16.
 *   scale_mode MOE_SCALE_ROW_DYNAMIC (scale [R]), MOE_SCALE_TENSOR_DYNAMIC
 *            (scale [1] from the whole tensor; row_amax [R] is required and
 *            receives the rows' maxima), MOE_SCALE_TENSOR_STATIC (scale[0] =
 *            static_scale, finite and > 0) or MOE_SCALE_TENSOR_FROM_ROW_AMAX
 *            (scale [1] from the caller's row_amax [R]).
 *   q        [R, C] int8 out, 8-byte aligned: q = clip(rint(f32(x / s)),
 *            -127, 127), ties to even; s = f32(amax / 127), 1.0 for an
 *            all-zero row or tensor.
 *   row_amax [R] f32, optional in row mode (the rows' absmax out).
 * Needs no workspace.  MOE_ERR_SHAPE for a bad size, alignment or static
 * scale, MOE_ERR_NULL for a missing buffer, MOE_ERR_UNSUPPORTED for an
 * unknown mode; R = 0 writes only the tensor scale.
 */
int moe_quantize_rows_i8(const void* x, int64_t R, int64_t C, int scale_mode, float static_scale, int8_t* q,
                         float* scale, float* row_amax, void* stream);

/*
 * moe_quantize_weights_i8 -- moe_quantize_weights with int8 codes (the same
 * passage allows int8 weights with the same [E, blocks, 1, N] scales):
 * s = f32(amax / 127) per block (1.0 for an all-zero block),
 * q = clip(rint(f32(w / s)), -127, 127) with ties to even.  Arguments,
 * layouts and errors as in moe_quantize_weights; q is int8.
 */
int moe_quantize_weights_i8(const void* w, int64_t E, int64_t K, int64_t N, int32_t kb, int32_t nb,
                            int scale_mode, float static_scale, int transpose_out, int8_t* q,
                            float* scale, void* stream);

/*
 * moe_sort_by_expert -- stable ragged sort of routed rows into per-expert
 * groups, and the gather of the quantized token rows into that order.
 * Defined by "Quantize activations before EP all gather" (review comments on
 * ragged_sort.py: qvalue rows are gathered by the sorted token indices into
 * this shard's window of sorted rows; the scale is gathered with them only
 * when it is per token, a per-tensor scale passes through).
 *
 *   expert_ids [T, k] int32: routed expert of slot j of token t; the flat
 *            routed index is f = t*k + j.
 *   E        number of experts (1 <= E <= 1024); group_offset, num_local_experts:
 *            this GPU's experts are [group_offset, group_offset + num_local_experts).
 *   perm     [T*k] int32 out: flat index f of each globally sorted row; the
 *            sort is stable (equal expert ids keep increasing f).
 *   inv_pos  [T*k] int32 out: local sorted row of f, or -1 when f routes to a
 *            non-local expert.  Local sorted row 0 is the first row of expert
 *            group_offset (compact window).
 *   group_sizes [E] int32 out: rows per expert (global histogram).
 *   xq       optional [T, H] e4m3fn token rows (NULL skips the row gather);
 *   xscale   their scale: [T] f32 when xscale_mode == MOE_SCALE_ROW_DYNAMIC,
 *            otherwise [1] and passed through (ss may then be NULL).
 *   xs       [M_cap, H] e4m3fn out: xs[r] = xq[perm[start + r] / k] for the n
 *            local rows, zero for rows [n, M_cap).
 *   ss       [M_cap] f32 out (row mode): the gathered scales, zero past n.
 *   ws       workspace of moe_workspace_bytes(MOE_OP_SORT_BY_EXPERT, T*k, 0, 0, E).
 * Invalid expert ids set MOE_DEVERR_EXPERT_ID and are sorted after every
 * valid row without entering any group; n > M_cap sets MOE_DEVERR_ROWS and
 * rows past M_cap are dropped.  H is a multiple of 16 (when xq is given).
 */
int moe_sort_by_expert(const int32_t* expert_ids, int64_t T, int32_t k, int32_t E,
                       int32_t group_offset, int32_t num_local_experts, const uint8_t* xq,
                       const float* xscale, int xscale_mode, int64_t H, int64_t M_cap,
                       int32_t* perm, int32_t* inv_pos, int32_t* group_sizes, uint8_t* xs,
                       float* ss, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_sort_gather_rows -- the row gather of moe_sort_by_expert alone, on the
 * metadata an earlier moe_sort_by_expert call (with xq NULL) wrote: its
 * inv_pos and the window header in its workspace ws.  The same bytes as the
 * one-call sort; lets the metadata run while the token rows are still being
 * quantized ("Quantize activations before EP all gather": the sort's order
 * depends on the routing only, the gathered rows on the quantized tokens).
 *   xq, xscale, xscale_mode, H, M_cap, xs, ss: as in moe_sort_by_expert.
 *   inv_pos  [T*k] from that call; ws: that call's workspace, unchanged
 *            since (the call must be ordered before this one on the device).
 * Errors: MOE_ERR_SHAPE, MOE_ERR_UNSUPPORTED, MOE_ERR_NULL, MOE_ERR_WORKSPACE.
 */
int moe_sort_gather_rows(const uint8_t* xq, const float* xscale, int xscale_mode, const int32_t* inv_pos,
                         int64_t T, int32_t k, int64_t H, int64_t M_cap, uint8_t* xs, float* ss, void* ws,
                         size_t ws_bytes, void* stream);

/* Bytes of the device array that moe_sort_by_expert_noalloc uses in place of
 * a workspace (one per GPU). */
#define MOE_SORT_NOALLOC_SCRATCH_BYTES (2u << 20)

/*
 * moe_sort_by_expert_noalloc -- moe_sort_by_expert that allocates nothing and
 * takes no workspace, for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid it.
 * The sort's scratch (the window header and the per-tile histogram table)
 * lives in a library-owned device array of MOE_SORT_NOALLOC_SCRATCH_BYTES
 * bytes, one per GPU, held from the first call on that GPU until the process
 * ends.  Every call on a GPU shares that GPU's array: calls that overlap on
 * one GPU (different streams, or several host threads) race and must be
 * ordered by the caller.
 *   device_error  optional [1] int32 device out (may be NULL, then dropped):
 *            the MOE_DEVERR_* bits of this call's device-data errors are
 *            OR'ed into it; the caller zeroes it.
 * Every other argument, the results and the errors are those of
 * moe_sort_by_expert.  Sizes whose workspace
 * (moe_workspace_bytes(MOE_OP_SORT_BY_EXPERT, T*k, 0, 0, E)) exceeds
 * MOE_SORT_NOALLOC_SCRATCH_BYTES return MOE_ERR_WORKSPACE before any launch:
 * T*k may be at most 4128768 with E = 64, 1043968 with E = 256 and 261632
 * with E = 1024.
 * No hipMalloc, hipFree or allocating call is made.
 */
int moe_sort_by_expert_noalloc(const int32_t* expert_ids, int64_t T, int32_t k, int32_t E,
                               int32_t group_offset, int32_t num_local_experts, const uint8_t* xq,
                               const float* xscale, int xscale_mode, int64_t H, int64_t M_cap,
                               int32_t* perm, int32_t* inv_pos, int32_t* group_sizes, uint8_t* xs,
                               float* ss, int32_t* device_error, void* stream);

/*
 * moe_quantize_sort_by_expert -- moe_quantize_rows followed by
 * moe_sort_by_expert in one pass over the activations, for the single-GPU
 * path where no all-gather sits between them (the quantized activation
 * sort of "Quantize activations before EP all gather"; the same per-token
 * absmax scheme of "Support quantization for tokamax gmm v2").  Each token's
 * bf16 row is read once and its e4m3fn codes go straight to its local
 * destination rows; a token with none is not quantized (unless `scale` asks
 * for its scale).
 *   x        [T, H] bf16, 16-byte aligned; H > 0, a multiple of 16.
 *   scale_mode MOE_SCALE_ROW_DYNAMIC, MOE_SCALE_TENSOR_STATIC (with
 *            static_scale as in moe_quantize_rows) or
 *            MOE_SCALE_TENSOR_FROM_ROW_AMAX (the tensor scale from the token
 *            maxima in row_amax, as in moe_quantize_rows);
 *            MOE_SCALE_TENSOR_DYNAMIC needs the whole tensor before any code
 *            and is MOE_ERR_UNSUPPORTED.
 *   expert_ids .. group_sizes, M_cap, ws, ws_bytes: as in moe_sort_by_expert
 *            (workspace of moe_workspace_bytes(MOE_OP_SORT_BY_EXPERT, ...)).
 *   xs       [M_cap, H] e4m3fn out: the bytes moe_quantize_rows then
 *            moe_sort_by_expert would write (rows [n, M_cap) zero).
 *   ss       row mode: [M_cap] f32 out, each local row's token scale (0 past
 *            n); static mode: unused, may be NULL.
 *   scale    optional: row mode [T] f32 out, every token's scale (then every
 *            token is quantized); static mode [1] f32 out = static_scale;
 *            required in MOE_SCALE_TENSOR_FROM_ROW_AMAX mode, [1] f32 out.
 *   row_amax row mode: optional [T] f32 out, every token's absmax (then every
 *            token is quantized); MOE_SCALE_TENSOR_FROM_ROW_AMAX: required
 *            [T] f32 input, the tokens' absmax as a row-mode pass wrote it;
 *            ignored in static mode.
 * Errors as in moe_sort_by_expert; device-data errors (bad expert ids, more
 * local rows than M_cap) set the same workspace error bits.
 */
int moe_quantize_sort_by_expert(const void* x, int64_t T, int64_t H, int scale_mode, float static_scale,
                                const int32_t* expert_ids, int32_t k, int32_t E, int32_t group_offset,
                                int32_t num_local_experts, int64_t M_cap, int32_t* perm, int32_t* inv_pos,
                                int32_t* group_sizes, uint8_t* xs, float* ss, float* scale, float* row_amax,
                                void* ws, size_t ws_bytes, void* stream);

/*
 * moe_gmm_fp8 -- grouped matmul of fp8 operands, the gmm_v2 call of "Quantize
 * activations before EP all gather" (review comment on the prequantized test:
 * lhs_q, rhs_q, group_sizes, rhs_scale, group_offset, no lhs quantization in
 * the kernel), with the 32-bit accumulator that "Keep qwix out of
 * tpu-inference's fused MoE kernel" shows fp8 x fp8 needs, and the
 * [E, blocks, 1, N] weight scales of its "Changes in this PR".
 *
 * For local group g (rows [o_g, o_g + m_g) of lhs, o_g = sum of
 * group_sizes[group_offset .. group_offset+g-1], m_g = group_sizes[group_offset+g]):
 *   out[r, c] = ls[r] * sum_b rs[g, b, 0, c*Nb/N] * sum_{k in block b} lhs[r, k] * W_g[k, c]
 * accumulated in float32 by the fp8 matrix cores, the lhs scale applied in
 * float32 before the single rounding to out_dtype; rows [n, M) are zero.
 *
 *   lhs      [M, K] e4m3fn; lhs_scale [M] (MOE_SCALE_ROW_DYNAMIC) or [1]
 *            (either tensor mode) f32.
 *   rhs      [E_loc, K, N] e4m3fn (transpose_rhs = 0), or [E_loc, N, K]
 *            (transpose_rhs = 1: W_g = rhs[g]^T, e.g. the input gradient
 *            against the forward weight).
 *   rhs_scale [E_loc, Kb, 1, Nb] f32; K/Kb and N/Nb must be multiples of 128
 *            unless Kb == 1 (resp. Nb == 1 or Nb == N).
 *   group_sizes [E] int32 device; E, group_offset, num_local_experts as in
 *            moe_sort_by_expert.
 *   out      [M, N], out_dtype MOE_BF16 (default) or MOE_F32.
 *   ws       workspace of moe_workspace_bytes(MOE_OP_GMM, M, K, N, E): the
 *            error word, one counter per tile of a split last round, and one
 *            float32 slot of 144 x 256 per workgroup (about 36 MiB on a
 *            256-CU GPU).  Zeroed once before its first use; the counters
 *            return to zero at the end of every call.  With it, when an XCD's
 *            share of tiles leaves a last round that fills few of its
 *            workgroups, each of those tiles is split along K over several
 *            workgroups and their float32 sums are added in a fixed order
 *            (int8 with one K block: int32 sums, added exactly).  Any smaller
 *            workspace of at least 256 bytes also works, without the split:
 *            the fp8 results may then differ in the last bits (another
 *            association of the same float32 sums); the same workspace size
 *            gives the same bits on every call.  Calls that share a workspace
 *            must not overlap (same stream, or ordered by events).
 * K and N multiples of 16 (MOE_ERR_SHAPE otherwise); multiples of 128 take
 * the tiled matrix-core kernels, other sizes a plainer edge kernel with the
 * same results.  M >= 0, 1 <= E <= 1024, num_local_experts <= 1024.
 */
int moe_gmm_fp8(const uint8_t* lhs, const float* lhs_scale, int lhs_scale_mode, const uint8_t* rhs,
                const float* rhs_scale, int32_t Kb, int32_t Nb, int transpose_rhs,
                const int32_t* group_sizes, int32_t E, int32_t group_offset,
                int32_t num_local_experts, int64_t M, int64_t K, int64_t N, int out_dtype,
                void* out, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_gmm_i8 -- moe_gmm_fp8 with int8 operands (codes in [-127, 127] from
 * moe_quantize_rows_i8 / moe_quantize_weights_i8), the int8 weights of "Keep
 * qwix out of tpu-inference's fused MoE kernel and pre-quantize weights"
 * ("Changes in this PR") with the 32-bit accumulator its description shows
 * quantized operands need.  The products are summed exactly in int32 by the
 * int8 matrix cores (exact for K up to 2^17); with one K block the sum is
 * converted to float32 once, with several each block's exact sum is scaled
 * and added in float32:
 *   out[r, c] = ls[r] * sum_b rs[g, b, 0, c*Nb/N] * P_b[r, c],
 *   P_b = sum_{k in block b} lhs[r, k] * W_g[k, c] (an integer).
 * Arguments, layouts, workspace, size rules and errors as in moe_gmm_fp8;
 * K <= 2^17 (MOE_ERR_SHAPE beyond).
 */
int moe_gmm_i8(const int8_t* lhs, const float* lhs_scale, int lhs_scale_mode, const int8_t* rhs,
               const float* rhs_scale, int32_t Kb, int32_t Nb, int transpose_rhs,
               const int32_t* group_sizes, int32_t E, int32_t group_offset,
               int32_t num_local_experts, int64_t M, int64_t K, int64_t N, int out_dtype,
               void* out, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_tgmm_fp8 -- transposed grouped matmul for weight gradients, the tgmm2
 * of "Support quantization for tokamax gmm v2" ("What this does": quantized
 * gmm2 / tgmm2, backward split into sub-functions):
 *   out[g, k, c] = (ls[k] * rs[c]) * sum_{r in group g} lhs[r, k] * rhs[r, c]
 * accumulated in float32; an empty local group gives zeros.
 *
 *   lhs      [M, K] e4m3fn with lhs_scale of lhs_scale_len 1 or K entries;
 *   rhs      [M, N] e4m3fn with rhs_scale of rhs_scale_len 1 or N entries.
 *            Scales must be constant along the contracted rows (a per-row
 *            scale does not factor out of the sum and is rejected).
 *   out      [E_loc, K, N], out_dtype MOE_F32 (default) or MOE_BF16.
 *   ws       workspace of moe_workspace_bytes(MOE_OP_TGMM, M, K, N, E).
 * K and N multiples of 16 (MOE_ERR_SHAPE otherwise); multiples of 128 take
 * the tiled kernels, other sizes a plainer edge kernel with the same results.
 */
int moe_tgmm_fp8(const uint8_t* lhs, const float* lhs_scale, int32_t lhs_scale_len,
                 const uint8_t* rhs, const float* rhs_scale, int32_t rhs_scale_len,
                 const int32_t* group_sizes, int32_t E, int32_t group_offset,
                 int32_t num_local_experts, int64_t M, int64_t K, int64_t N, int out_dtype,
                 void* out, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_tgmm_xt_cols -- columns (host out `cols`) of the transposed operand
 * layout that moe_sort_gather_transposed writes and moe_tgmm_fp8_xt reads,
 * for M local rows and E experts: 256 * ceil((M + 128 E) / 256).
 * MOE_ERR_SHAPE for M < 0 or E outside 1..1024.
 */
int moe_tgmm_xt_cols(int64_t M, int32_t E, int64_t* cols);

/*
 * moe_sort_gather_transposed -- the sort's row gather ("Quantize activations
 * before EP all gather": the fp8 token rows are gathered by the sorted token
 * indices into this shard's window) written straight into the layout the
 * weight-gradient product contracts over (tgmm2 of "Support quantization for
 * tokamax gmm v2"): the rows of each local group become a contraction axis
 * of their own.  For local group g with sorted rows rows_off[g] ..
 * rows_off[g] + m_g - 1 of the window and padded start P_g = 128 *
 * sum_{h<g} ceil(m_h / 128):
 *   xt[c, P_g + i] = code of x[perm[start + rows_off[g] + i] / k, c]   (i < m_g)
 *   xt[c, P_g + i] = 0                  (m_g <= i < 128 * ceil(m_g / 128))
 * with start = sum of group_sizes[0 .. group_offset-1] (the window's first
 * slot); columns past the last group's padded end are not written.
 *
 *   x        [T, H]: e4m3fn codes (x_dtype MOE_E4M3FN, e.g. from
 *            moe_quantize_rows with a tensor scale), or bf16 rows (MOE_BF16)
 *            quantized here with the static scale static_scale (> 0, finite)
 *            exactly as moe_quantize_rows(MOE_SCALE_TENSOR_STATIC) codes them.
 *   perm, group_sizes, E, group_offset, num_local_experts: as written by
 *            moe_sort_by_expert for the same routing (T*k slots, top-k = k).
 *   M        local rows of the weight-gradient call (rows of its dY).
 *   xt       [H, moe_tgmm_xt_cols(M, E)] bytes, row-major.
 *   scale_out optional device float [1]: receives static_scale (MOE_BF16).
 *   ws       workspace of at least 256 bytes (the error word).
 * H a multiple of 256 (MOE_ERR_UNSUPPORTED otherwise), 1 <= k <= 64.  A
 * source index outside the buffers is clamped (no access leaves them).
 * Errors: MOE_ERR_SHAPE, MOE_ERR_UNSUPPORTED, MOE_ERR_NULL, MOE_ERR_WORKSPACE.
 */
int moe_sort_gather_transposed(const void* x, int x_dtype, float static_scale, int64_t T, int32_t k,
                               int64_t H, const int32_t* perm, const int32_t* group_sizes, int32_t E,
                               int32_t group_offset, int32_t num_local_experts, int64_t M, uint8_t* xt,
                               float* scale_out, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_tgmm_fp8_xt -- moe_tgmm_fp8 with its lhs already in the transposed
 * layout of moe_sort_gather_transposed: xt [K, moe_tgmm_xt_cols(M, E)]
 * (column P_g + i = row rows_off[g] + i of the sorted lhs, zeros in each
 * group's padding).  Same result as moe_tgmm_fp8 on the sorted rows, bit for
 * bit.  rhs [M, N] as there.  K a multiple of 256 and N of 128
 * (MOE_ERR_UNSUPPORTED otherwise).  ws: at least 256 + N * cols bytes
 * (moe_workspace_bytes(MOE_OP_TGMM, M, K, N, E) is enough).  Other arguments
 * and errors as in moe_tgmm_fp8.
 */
int moe_tgmm_fp8_xt(const uint8_t* xt, const float* lhs_scale, int32_t lhs_scale_len, const uint8_t* rhs,
                    const float* rhs_scale, int32_t rhs_scale_len, const int32_t* group_sizes, int32_t E,
                    int32_t group_offset, int32_t num_local_experts, int64_t M, int64_t K, int64_t N,
                    int out_dtype, void* out, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_gather_reduce -- un-sort plus top-k weighted combine, the ragged
 * gather-reduce of "Quantize activations before EP all gather" (review
 * comments on ragged_gather_reduce_v2.py: rows are reduced over a valid-rows
 * mask; the output dtype is bf16 when unspecified or fp8):
 *   out[t, :] = sum_{j < k, inv_pos[t, j] >= 0} w[t, j] * y[inv_pos[t, j], :]
 * accumulated in float32 in slot order j = 0..k-1, one rounding at the end.
 *
 *   y        [rows, N], y_dtype MOE_BF16 or MOE_F32 (rows >= 1 + max inv_pos).
 *   inv_pos  [T, k] int32 (from moe_sort_by_expert); topk_weights [T, k] f32.
 *   out      [T, N]; out_dtype MOE_BF16 (also for MOE_DTYPE_DEFAULT and
 *            MOE_E4M3FN) or MOE_F32.
 * N a multiple of 8.  Needs no workspace.
 */
int moe_gather_reduce(const void* y, int y_dtype, const int32_t* inv_pos, const float* topk_weights,
                      int64_t T, int32_t k, int64_t N, int out_dtype, void* out, void* stream);

/*
 * moe_gather_reduce_backward -- the backward of moe_gather_reduce, for the
 * layer backward that "Support quantization for tokamax gmm v2" splits into
 * gmm / tgmm calls ("What this does"; its accuracy tables compare gradients
 * as well as outputs).  With out[t] = sum_j w[t, j] * y[inv_pos[t, j]]:
 *   dy[inv_pos[t, j], :] = bf16(w[t, j] * dout[t, :])   (one float32
 *                           product, rounded to nearest even)
 *   dw[t, j]             = sum_c dout[t, c] * y[inv_pos[t, j], c]  (float32)
 * for every slot whose inverse position is in [0, M_cap); other slots get
 * dw = 0.  Rows [n, M_cap) of dy are zero, n = sum of
 * group_sizes[group_offset .. group_offset + num_local_experts).
 *
 *   dout     [T, N] bf16, the gradient of the combined token rows.
 *   y        [M_cap, N] bf16, the expert outputs the forward combined.
 *   inv_pos  [T, k] int32 and group_sizes [E] int32, from moe_sort_by_expert
 *            (every local row is the image of exactly one slot).
 *   topk_weights [T, k] f32.
 *   dy       [M_cap, N] bf16 out; dw [T, k] f32 out.
 *   dy_q, dy_scale, dy_amax  optional (all NULL, or all set; N <= 8192):
 *            [M_cap, N] e4m3fn, [M_cap] f32, [M_cap] f32 out -- dy quantized
 *            per row exactly as moe_quantize_rows(dy, MOE_SCALE_ROW_DYNAMIC)
 *            would (codes, scales and row absmax), formed while the row is in
 *            registers instead of in a second pass over dy.
 * N a multiple of 8, k <= 64.  Needs no workspace.  Errors: MOE_ERR_SHAPE,
 * MOE_ERR_NULL, MOE_ERR_UNSUPPORTED (dy_q with N > 8192); T = 0 with
 * M_cap = 0 returns MOE_OK.
 */
int moe_gather_reduce_backward(const void* dout, const void* y, const int32_t* inv_pos,
                               const float* topk_weights, int64_t T, int32_t k, int64_t N,
                               const int32_t* group_sizes, int32_t E, int32_t group_offset,
                               int32_t num_local_experts, int64_t M_cap, void* dy, float* dw,
                               uint8_t* dy_q, float* dy_scale, float* dy_amax, void* stream);

/*
 * moe_silu_mul_backward -- gradients of the gated FFN's activation
 * h = silu(a) * b for an upstream gradient dh, the activation step of the
 * layer backward that "Support quantization for tokamax gmm v2" splits into
 * gmm / tgmm calls ("What this does").  A pinned float32 recipe, one
 * rounding per step, no fused multiply-add:
 *   den = 1 + e(-a) (the forward's pinned exp), s = 1 / den, q = a / den,
 *   db = dh * q,  da = (dh * b) * (s * (1 + a * (1 - s)))
 * each result rounded to bf16 (nearest even).
 *
 *   a, b     [R, C] bf16 with row stride lda elements (e.g. the two column
 *            halves of the fused input-projection output, lda = 2C).
 *   dh       [R, C] bf16, dense.
 *   da, db   [R, C] bf16 out with row stride ldo (e.g. the halves of one
 *            [R, 2C] buffer that the input-gradient gmm over [W0 | W1]^T
 *            reads as its lhs).
 * C, lda, ldo multiples of 8, lda >= C, ldo >= C.  Needs no workspace.
 * Errors: MOE_ERR_SHAPE, MOE_ERR_NULL; R = 0 returns MOE_OK.
 */
int moe_silu_mul_backward(const void* a, const void* b, int64_t lda, const void* dh, int64_t R, int64_t C,
                          void* da, void* db, int64_t ldo, void* stream);

/*
 * moe_workspace_bytes -- workspace size (host out `bytes`) for `op` with
 * problem sizes d0, d1, d2 and E:
 *   MOE_OP_QUANTIZE_ROWS   d0 = R, d1 = C, d2 = scale_mode
 *   MOE_OP_SORT_BY_EXPERT  d0 = T*k
 *   MOE_OP_GMM, MOE_OP_TGMM d0 = M, d1 = K, d2 = N
 *   others                 only the error word
 * Every size is a multiple of 256 bytes and at least 256.
 */
int moe_workspace_bytes(int op, int64_t d0, int64_t d1, int64_t d2, int32_t E, size_t* bytes);

/*
 * moe_debug_check -- synchronises `stream` and copies the sticky error word
 * of workspace `ws` into host *device_error.  Debug use only.
 */
int moe_debug_check(const void* ws, void* stream, int32_t* device_error);

/* moe_status_string -- static text for a status code. */
const char* moe_status_string(int status);

/* moe_version -- library version as 10000*major + 100*minor + patch. */
int moe_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_FP8_H */
