"""Un-sort plus top-k weighted combine of the expert outputs.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix ("Quantize activations before EP all gather", review
comments on ``ragged_gather_reduce_v2.py``): the expert outputs, held in
sorted-row order, are reduced back to one row per token over the rows that
take part (a valid-rows mask), and the output dtype defaults to bfloat16
when it is unspecified or an fp8 type.

Readings: each token's output is the sum over its k routing slots, in slot
order j = 0..k-1, of the router weight times the expert output row of that
slot; a slot whose row is not local (inverse position -1) contributes
nothing; router weights are used as given (no renormalisation).
"""

import numpy as np

from .codec import bf16_decode, bf16_rne_from_f64


def gather_reduce(y, y_is_bf16, inv_pos, topk_weights, sample_tokens=None):
    """out[t, :] = sum_{j < k, inv_pos[t, j] >= 0} w[t, j] * y[inv_pos[t, j], :].

    y: [M_cap, N] bf16 bit patterns (uint16) when ``y_is_bf16`` else float32;
    inv_pos int [T, k]; topk_weights float32 [T, k].  Accumulates in float64
    in slot order.  ``sample_tokens`` restricts the result to those tokens.
    Returns the dict of ``oracle.gmm`` (out, abs_sum, f32, bf16).
    """
    yf = bf16_decode(y) if y_is_bf16 else np.asarray(y, dtype=np.float32)
    yf = yf.astype(np.float64)
    inv = np.asarray(inv_pos, dtype=np.int64)
    w = np.asarray(topk_weights, dtype=np.float32).astype(np.float64)
    T, k = inv.shape
    toks = np.arange(T) if sample_tokens is None else np.asarray(sample_tokens, dtype=np.int64)
    N = yf.shape[1]
    o = np.zeros((len(toks), N))
    a = np.zeros((len(toks), N))
    for j in range(k):
        idx = inv[toks, j]
        ok = idx >= 0
        rows = yf[np.where(ok, idx, 0)]
        contrib = np.where(ok[:, None], w[toks, j][:, None] * rows, 0.0)
        o = o + contrib
        a = a + np.abs(contrib)
    return {"out": o, "abs_sum": a, "f32": o.astype(np.float32), "bf16": bf16_rne_from_f64(o)}
