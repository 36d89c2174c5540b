"""Absmax quantization of activations and weights to e4m3fn, and the SiLU*mul
activation that feeds the second quantization of the gated FFN.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix:

* Activations are quantized per token with a dynamic absmax scale before the
  expert-parallel all-gather and the activation sort ("Quantize activations
  before EP all gather", description and the ``ragged_sort.py`` review
  comments: the scale of a ``QArray`` has the token dimension first when it
  is per-token, otherwise it is a per-tensor / per-channel scale).
* The quantization schemes are ``fp8_dynamic`` (absmax for weights,
  activations and gradients) and ``fp8_static_wa`` (fixed weight scale,
  fixed activation scale, absmax gradients) ("Support quantization for
  tokamax gmm v2", tolerance discussion).
* Weights are pre-quantized outside the kernel to float8_e4m3fn with
  [E, blocks, 1, N] scales, blockwise or channelwise ("Keep qwix out of
  tpu-inference's fused MoE kernel and pre-quantize weights", "Changes in
  this PR", and the review note on inserting the scale's singleton
  dimension).

Readings where the pages are silent (each is listed in the design notes):

* scale ``s = float32(amax / 448)`` with an IEEE float32 divide, and the
  element ``q = e4m3_rne(clip(float32(x / s), -448, 448))``, again an IEEE
  float32 divide (not a multiply by a reciprocal);
* an all-zero row (or block, or tensor) gets ``s = 1.0``;
* values beyond 448 after scaling saturate to +-448 (only possible with a
  static scale).
"""

import numpy as np

from .codec import E4M3_MAX, bf16_decode, bf16_rne_from_f32, e4m3_rne

SCALE_ROW_DYNAMIC = 0
SCALE_TENSOR_DYNAMIC = 1
SCALE_TENSOR_STATIC = 2
SCALE_TENSOR_FROM_ROW_AMAX = 3

_F448 = np.float32(E4M3_MAX)


def _scale_from_amax(amax) -> np.ndarray:
    amax = np.asarray(amax, dtype=np.float32)
    s = amax / _F448                      # float32 / float32: IEEE float32 divide
    return np.where(amax == np.float32(0.0), np.float32(1.0), s).astype(np.float32)


def _quantize_with_scale(xf: np.ndarray, s_bcast: np.ndarray) -> np.ndarray:
    v = (xf / s_bcast).astype(np.float32)      # IEEE float32 divide, elementwise
    v = np.clip(v, -_F448, _F448)
    return e4m3_rne(v)


# ---------------------------------------------------------------------------
# Pinned float32 exponential used by SiLU.  The pages do not discuss the
# activation; both sides of the parity check implement this one written
# recipe so that the requantized bytes can be compared bit for bit:
#   * Cody & Waite's argument reduction with ln 2 split in two parts
#     (W. J. Cody, W. Waite, "Software Manual for the Elementary Functions",
#     1980): n = rint(x * log2(e)), r = (x - n*C1) - n*C2, where C1 is ln 2
#     cut to 16 significant bits (so n*C1 is exact for |n| < 256) and
#     C2 = float32(ln 2 - C1);
#   * exp(r) by the degree-7 Taylor polynomial with float32(1/i!)
#     coefficients evaluated in Horner form, every multiply and add rounded
#     separately (no fused multiply-add);
#   * scaling by 2**n (exact in the clamped range);
#   * x clamped to [-87, 88] first so that the result stays a finite normal
#     float32.
# ---------------------------------------------------------------------------

def _ln2_split():
    ln2 = np.log(2.0)
    m, e = np.frexp(ln2)                       # ln2 = m * 2**e, m in [0.5, 1)
    c1 = np.floor(m * 2.0 ** 16) / 2.0 ** 16 * 2.0 ** e
    c1_32 = np.float32(c1)
    assert float(c1_32) == c1
    c2_32 = np.float32(ln2 - c1)
    return c1_32, c2_32


EXP_C1, EXP_C2 = _ln2_split()
EXP_LOG2E = np.float32(1.0 / np.log(2.0))
EXP_COEFFS = [np.float32(1.0 / np.prod(np.arange(1, i + 1, dtype=np.float64))) for i in range(8)]
EXP_LO = np.float32(-87.0)
EXP_HI = np.float32(88.0)


def pinned_exp_f32(x) -> np.ndarray:
    """The pinned float32 exp (see the recipe above); float32 in, float32 out."""
    x = np.clip(np.asarray(x, dtype=np.float32), EXP_LO, EXP_HI)
    n = np.rint(x * EXP_LOG2E).astype(np.float32)
    r = ((x - n * EXP_C1).astype(np.float32) - (n * EXP_C2).astype(np.float32)).astype(np.float32)
    p = EXP_COEFFS[7]
    for i in range(6, -1, -1):
        p = ((p * r).astype(np.float32) + EXP_COEFFS[i]).astype(np.float32)
    return np.ldexp(p, n.astype(np.int32)).astype(np.float32)


def silu_mul_f32(a, b) -> np.ndarray:
    """h = float32(silu(a) * b), silu(a) = float32(a / float32(1 + e(-a))).

    ``a`` (gate) and ``b`` (up) are float32 arrays (decoded bf16)."""
    a = np.asarray(a, dtype=np.float32)
    b = np.asarray(b, dtype=np.float32)
    den = (np.float32(1.0) + pinned_exp_f32(-a)).astype(np.float32)
    silu = (a / den).astype(np.float32)
    return (silu * b).astype(np.float32)


def silu_mul_backward_f32(a, b, dh):
    """Gradients of h = silu(a) * b for an upstream gradient dh (float32 arrays
    of decoded bf16 values), by a pinned float32 recipe, one rounding per step
    and no fused multiply-add:

      den = 1 + e(-a)     (the pinned exp, as in the forward)
      s   = 1 / den       (the logistic sigmoid of a)
      q   = a / den       (silu(a), the forward's quotient)
      db  = dh * q
      da  = (dh * b) * (s * (1 + a * (1 - s)))

    The pages do not discuss the activation (a gated FFN is the plain reading
    of the gated layer); the derivative is silu'(a) = s * (1 + a * (1 - s)).
    Returns (da, db) float32.
    """
    a = np.asarray(a, dtype=np.float32)
    b = np.asarray(b, dtype=np.float32)
    dh = np.asarray(dh, dtype=np.float32)
    one = np.float32(1.0)
    den = (one + pinned_exp_f32(-a)).astype(np.float32)
    s = (one / den).astype(np.float32)
    q = (a / den).astype(np.float32)
    db = (dh * q).astype(np.float32)
    ds = (s * (one + (a * (one - s).astype(np.float32)).astype(np.float32)).astype(np.float32)).astype(np.float32)
    da = ((dh * b).astype(np.float32) * ds).astype(np.float32)
    return da, db


def silu_mul_backward(a_bits, b_bits, dh_bits):
    """silu_mul_backward_f32 on bf16 bit patterns; (da, db) as bf16 bit
    patterns, each rounded once to nearest even from float32."""
    da, db = silu_mul_backward_f32(bf16_decode(a_bits), bf16_decode(b_bits), bf16_decode(dh_bits))
    return bf16_rne_from_f32(da), bf16_rne_from_f32(db)


def quantize_rows(x_bits, mode, static_scale=None, x_up_bits=None, row_amax_in=None):
    """Quantize a [R, C] bf16 matrix to e4m3fn.

    mode: SCALE_ROW_DYNAMIC (scale per row, shape [R]), SCALE_TENSOR_DYNAMIC
    (one scale from the whole tensor's absmax, shape [1]),
    SCALE_TENSOR_STATIC (the given ``static_scale``, shape [1]) or
    SCALE_TENSOR_FROM_ROW_AMAX (one scale from the maximum of the given row
    maxima ``row_amax_in``, shape [1]; the tensor-dynamic scale when those
    are the rows' own maxima).
    With ``x_up_bits`` the quantized matrix is silu_mul_f32(x, x_up) instead
    of x (the gated FFN's activation).

    Returns (q uint8 [R, C], scale float32, row_amax float32 [R]).
    """
    xf = bf16_decode(x_bits)
    if xf.ndim != 2:
        raise ValueError("quantize_rows: expected a 2-D input")
    if x_up_bits is not None:
        xf = silu_mul_f32(xf, bf16_decode(x_up_bits))
    R = xf.shape[0]
    row_amax = (np.max(np.abs(xf), axis=1) if xf.shape[1] else np.zeros(R)).astype(np.float32)
    if mode == SCALE_ROW_DYNAMIC:
        s = _scale_from_amax(row_amax)
        q = _quantize_with_scale(xf, s[:, None])
    elif mode == SCALE_TENSOR_DYNAMIC:
        amax = np.max(row_amax) if R else np.float32(0.0)
        s = _scale_from_amax(np.array([amax], dtype=np.float32))
        q = _quantize_with_scale(xf, s[0])
    elif mode == SCALE_TENSOR_STATIC:
        s = np.array([static_scale], dtype=np.float32)
        q = _quantize_with_scale(xf, s[0])
    elif mode == SCALE_TENSOR_FROM_ROW_AMAX:
        given = np.asarray(row_amax_in, dtype=np.float32)
        amax = np.max(given) if R else np.float32(0.0)
        s = _scale_from_amax(np.array([amax], dtype=np.float32))
        q = _quantize_with_scale(xf, s[0])
    else:
        raise ValueError("quantize_rows: unknown scale mode")
    return q, s, row_amax


def quantize_weights(w_bits, kb, nb, static_scale=None):
    """Blockwise absmax quantization of expert weights [E, K, N] (bf16 bits).

    The scale tensor has the pages' [E, blocks, 1, N]-style shape
    [E, kb, 1, nb]: block (b, c) covers rows b*K/kb .. (b+1)*K/kb - 1 of the
    contraction dimension and columns c*N/nb .. (c+1)*N/nb - 1.  kb = 1,
    nb = N is the per-output-channel case; kb = K/128, nb = N the 128-row
    K-block case; kb = K/128, nb = N/128 the 128x128 block case.  With
    ``static_scale`` every block gets that fixed scale.

    Returns (q uint8 [E, K, N], s float32 [E, kb, 1, nb]).
    """
    w = bf16_decode(w_bits)
    E, K, N = w.shape
    if K % kb or N % nb:
        raise ValueError("quantize_weights: blocks must tile the matrix")
    bk, bn = K // kb, N // nb
    blocks = np.abs(w).reshape(E, kb, bk, nb, bn)
    if static_scale is None:
        amax = blocks.max(axis=(2, 4)) if bk and bn else np.zeros((E, kb, nb), np.float32)
        s = _scale_from_amax(amax)
    else:
        s = np.full((E, kb, nb), static_scale, dtype=np.float32)
    s_full = np.repeat(np.repeat(s, bk, axis=1), bn, axis=2)     # [E, K, N]
    q = _quantize_with_scale(w, s_full)
    return q, s.reshape(E, kb, 1, nb).astype(np.float32)
