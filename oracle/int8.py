"""The int8 variant of the path: absmax quantization of activations and
weights to int8 and the grouped matmul with an int32 accumulator.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix:

* Weights are pre-quantized outside the kernel, to e4m3fn or to int8 codes,
  with [E, blocks, 1, N] scales, blockwise or channelwise ("Keep qwix out of
  tpu-inference's fused MoE kernel and pre-quantize weights", "Changes in
  this PR").
* The matmul of quantized operands needs a 32-bit accumulator (the Mosaic
  error in that page's description).
* Activations are quantized per token with a dynamic absmax scale, or with a
  fixed scale in the static scheme ("Quantize activations before EP all
  gather", description; "Support quantization for tokamax gmm v2", the
  fp8_dynamic and fp8_static_wa schemes), and a per-token scale follows its
  rows through the sort.

Readings where the pages are silent (each listed in the design notes):

* int8 codes are symmetric: [-127, 127], never -128;
* the scale is ``s = float32(amax / 127)`` with an IEEE float32 divide, 1.0
  for an all-zero row or block;
* an element is ``q = clip(rint(float32(x / s)), -127, 127)``: the IEEE
  float32 quotient, rounded to the nearest integer with ties to even, then
  saturated (reachable only with a static scale);
* no matrix core multiplies fp8 by int8 codes, so int8 weights pair with
  int8 activations: both operands int8, the products summed exactly in
  int32 (|q| <= 127, so a contraction below 2^17 terms cannot overflow).
"""

import numpy as np

from .codec import bf16_decode, bf16_rne_from_f64
from .gmm import local_group_offsets

I8_MAX = 127
_F127 = np.float32(I8_MAX)

SCALE_ROW_DYNAMIC = 0
SCALE_TENSOR_DYNAMIC = 1
SCALE_TENSOR_STATIC = 2
SCALE_TENSOR_FROM_ROW_AMAX = 3


def int8_rne(v) -> np.ndarray:
    """float32 values to int8 codes: round half to even, saturate to +-127."""
    v = np.asarray(v, dtype=np.float32)
    if not np.all(np.isfinite(v)):
        raise ValueError("int8_rne: non-finite input")
    return np.clip(np.rint(v), -I8_MAX, I8_MAX).astype(np.int8)


def _scale_from_amax(amax) -> np.ndarray:
    amax = np.asarray(amax, dtype=np.float32)
    s = amax / _F127                          # float32 / float32: IEEE divide
    return np.where(amax == np.float32(0.0), np.float32(1.0), s).astype(np.float32)


def _quantize_with_scale(xf, s_bcast) -> np.ndarray:
    return int8_rne((xf / s_bcast).astype(np.float32))


def quantize_rows_int8(x_bits, mode, static_scale=None, row_amax_in=None):
    """Quantize a [R, C] bf16 matrix to int8 codes.

    mode: SCALE_ROW_DYNAMIC (a scale per row, [R]), SCALE_TENSOR_DYNAMIC (one
    scale from the whole tensor's absmax), SCALE_TENSOR_STATIC (the given
    ``static_scale``) or SCALE_TENSOR_FROM_ROW_AMAX (one scale from the
    maximum of the given row maxima).  Returns (q int8 [R, C], scale float32,
    row_amax float32 [R])."""
    xf = bf16_decode(x_bits)
    if xf.ndim != 2:
        raise ValueError("quantize_rows_int8: expected a 2-D input")
    R = xf.shape[0]
    row_amax = (np.max(np.abs(xf), axis=1) if xf.shape[1] else np.zeros(R)).astype(np.float32)
    if mode == SCALE_ROW_DYNAMIC:
        s = _scale_from_amax(row_amax)
        return _quantize_with_scale(xf, s[:, None]), s, row_amax
    if mode == SCALE_TENSOR_DYNAMIC:
        s = _scale_from_amax(np.array([np.max(row_amax) if R else 0.0], np.float32))
    elif mode == SCALE_TENSOR_STATIC:
        s = np.array([static_scale], dtype=np.float32)
    elif mode == SCALE_TENSOR_FROM_ROW_AMAX:
        given = np.asarray(row_amax_in, dtype=np.float32)
        s = _scale_from_amax(np.array([np.max(given) if R else 0.0], np.float32))
    else:
        raise ValueError("quantize_rows_int8: unknown scale mode")
    return _quantize_with_scale(xf, s[0]), s, row_amax


def quantize_weights_int8(w_bits, kb, nb, static_scale=None):
    """Blockwise absmax quantization of expert weights [E, K, N] (bf16 bits)
    to int8 with [E, kb, 1, nb] scales (block (b, c) covers contraction rows
    b*K/kb .. and columns c*N/nb ..).  Returns (q int8 [E, K, N], s)."""
    w = bf16_decode(w_bits)
    E, K, N = w.shape
    if K % kb or N % nb:
        raise ValueError("quantize_weights_int8: blocks must tile the matrix")
    bk, bn = K // kb, N // nb
    wb = w.reshape(E, kb, bk, nb, bn)                 # [expert, K block, row in block, N block, column in block]
    if static_scale is None:
        s = _scale_from_amax(np.abs(wb).max(axis=(2, 4)))
    else:
        s = np.full((E, kb, nb), static_scale, dtype=np.float32)
    q = _quantize_with_scale(wb, s[:, :, None, :, None]).reshape(E, K, N)
    return q, s.reshape(E, kb, 1, nb).astype(np.float32)


def gmm_int8(lhs_q, lhs_scale, rhs_q, rhs_scale, group_sizes, group_offset, num_local_experts,
             transpose_rhs=False):
    """out[r, c] = ls[r] * sum_b rs[g, b, c] * P_b[r, c] for local group g,
    P_b = the exact integer dot product of int8 codes over K block b (int32
    accumulation is exact at these sizes, and so is a float64 matmul of
    them: |products| <= 127^2, sums far below 2^53); the scales multiply in
    float64, blocks in ascending order.  rhs_q is [E_loc, K, N] int8 (or
    [E_loc, N, K] with transpose_rhs); rows [n, M) are zero.  Returns the
    float64 result ``out``, the abs-sum ``abs_sum`` and ``bf16`` bits."""
    lhs_q = np.asarray(lhs_q, dtype=np.int8)
    rhs_q = np.asarray(rhs_q, dtype=np.int8)
    M, K = lhs_q.shape
    E_loc = num_local_experts
    N = rhs_q.shape[1] if transpose_rhs else rhs_q.shape[2]
    rs = np.asarray(rhs_scale, dtype=np.float64)
    kb, nb = rs.shape[1], rs.shape[3]
    bk = K // kb
    offs, sizes, n = local_group_offsets(group_sizes, group_offset, E_loc)
    if n > M:
        raise ValueError("local rows exceed M")
    ls = np.asarray(lhs_scale, dtype=np.float64).reshape(-1)
    ls = np.full(M, ls[0]) if ls.size == 1 else ls
    o = np.zeros((M, N))
    a = np.zeros((M, N))
    for g in range(E_loc):
        m = sizes[g]
        if m == 0:
            continue
        rows = slice(offs[g], offs[g] + m)
        X = lhs_q[rows].astype(np.float64)
        W = rhs_q[g].astype(np.float64)
        W = W.T if transpose_rhs else W
        tot = np.zeros((m, N))
        atot = np.zeros((m, N))
        for b in range(kb):
            ks = slice(b * bk, (b + 1) * bk)
            rsb = np.repeat(rs[g, b, 0, :], N // nb)
            tot = tot + rsb[None, :] * (X[:, ks] @ W[ks, :])
            atot = atot + np.abs(rsb)[None, :] * (np.abs(X[:, ks]) @ np.abs(W[ks, :]))
        o[rows] = ls[rows, None] * tot
        a[rows] = np.abs(ls[rows, None]) * atot
    return {"out": o, "abs_sum": a, "f32": o.astype(np.float32), "bf16": bf16_rne_from_f64(o)}
