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


def gather_reduce_backward(dout, y, inv_pos, topk_weights, m_cap, n_local):
    """The backward of ``gather_reduce`` for a bfloat16 upstream gradient.

    "Support quantization for tokamax gmm v2" ("What this does": the layer's
    backward is split into gmm / tgmm calls; the accuracy tables compare
    gradients as well as outputs) needs the gradients that flow from the
    combined token rows back into the sorted expert rows and into the router
    weights.  The pages do not spell the combine's backward out; the reading
    taken is the plain derivative of out[t] = sum_j w[t, j] * y[inv_pos[t, j]]:

      dy[inv_pos[t, j], :] = w[t, j] * dout[t, :]    (each local row is the
                                                        image of one slot)
      dw[t, j]             = sum_c dout[t, c] * y[inv_pos[t, j], c]

    for slots with a local row; a slot whose row is not local (-1) gets
    dw = 0, and sorted rows [n_local, m_cap) of dy are zero.  dy is rounded
    once to bfloat16 (through float32, as the products are exact in float64),
    dw once to float32 from a float64 sum.

    dout: [T, N] bf16 bits; y: [m_cap, N] bf16 bits; inv_pos int [T, k];
    topk_weights float32 [T, k].  Returns dy (bf16 bits [m_cap, N]), dy64
    (float64), dw (float32 [T, k]), dw64 and dw_abs (the sum of |terms|, the
    denominator of the float32 match rule).
    """
    d = bf16_decode(dout).astype(np.float64)
    yf = bf16_decode(y).astype(np.float64)
    inv = np.asarray(inv_pos, dtype=np.int64)
    w = np.asarray(topk_weights, dtype=np.float32).astype(np.float64)
    T, k = inv.shape
    N = d.shape[1]
    dy64 = np.zeros((m_cap, N))
    dw64 = np.zeros((T, k))
    dw_abs = np.zeros((T, k))
    for t in range(T):
        for j in range(k):
            r = inv[t, j]
            if r < 0:
                continue
            dy64[r] = w[t, j] * d[t]
            dw64[t, j] = np.dot(d[t], yf[r])
            dw_abs[t, j] = np.dot(np.abs(d[t]), np.abs(yf[r]))
    dy64[n_local:] = 0.0
    return {"dy": bf16_rne_from_f64(dy64), "dy64": dy64, "dw": dw64.astype(np.float32), "dw64": dw64,
            "dw_abs": dw_abs}
