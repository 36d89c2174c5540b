"""Grouped matmul of fp8 operands (gmm) and its transposed form (tgmm).

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix:

* ``gmm_v2(lhs_q, rhs_q, group_sizes, rhs_scale=..., group_offset=...,
  maybe_quantize_lhs=False)`` multiplies pre-quantized rows of each expert
  group with that expert's pre-quantized weight, applying the rhs scale in
  the kernel; the per-row lhs scale [M, 1] is a factor of the whole
  contraction and can be applied to the output ("Quantize activations
  before EP all gather", review comment on the prequantized ``gmm_v2``
  test).
* The accumulator of an fp8 x fp8 matmul is 32-bit ("Keep qwix out of
  tpu-inference's fused MoE kernel and pre-quantize weights", the Mosaic
  error in the description); weight scales are [E, blocks, 1, N] ("Changes
  in this PR").
* The backward pass splits into a gmm against the transposed weight (input
  gradient) and a tgmm, a per-group lhs^T . rhs over the group's rows
  (weight gradient) ("Support quantization for tokamax gmm v2", "What this
  does": quantization of gmm2 / tgmm2 and the forward/backward split).

Exactness: every e4m3 value is an integer multiple of 2**-9 with magnitude at
most 448, so every product is a multiple of 2**-18 below 2**18 and every
partial sum of up to 2**33 of them is an integer multiple of 2**-18 below
2**51: float64 holds all of them exactly, whatever the summation order.  The
block sums P_b below are therefore exact; only the scale multiplications
round (in float64).

Readings: the lhs scale is applied to the float64 result before the single
rounding to the output type (float32, then bfloat16); rows [n, M) that
belong to no local group are zero; with ``transpose_rhs`` the weight is
stored [E_loc, N, K].
"""

import numpy as np

from .codec import bf16_rne_from_f64, e4m3_decode


def local_group_offsets(group_sizes, group_offset, num_local_experts):
    """Start row of each local group in the compact sorted buffer, and n."""
    gs = np.asarray(group_sizes, dtype=np.int64)[group_offset:group_offset + num_local_experts]
    if np.any(gs < 0):
        raise ValueError("negative group size")
    offs = np.concatenate([[0], np.cumsum(gs)])
    return offs[:-1], gs, int(offs[-1])


def _expand_cols(v, N, nb):
    return np.repeat(np.asarray(v, dtype=np.float64), N // nb)


def _lhs_scale_vec(lhs_scale, M):
    ls = np.asarray(lhs_scale, dtype=np.float64).reshape(-1)
    if ls.size == 1:
        return np.full(M, ls[0])
    if ls.size != M:
        raise ValueError("lhs_scale must have 1 or M entries")
    return ls


def _finish(o, a):
    o32 = o.astype(np.float32)
    return {"out": o, "abs_sum": a, "f32": o32, "bf16": bf16_rne_from_f64(o)}


def gmm(lhs_q, lhs_scale, rhs_q, rhs_scale, group_sizes, group_offset, num_local_experts,
        transpose_rhs=False, sample=None):
    """out[r, c] = ls[r] * sum_b rs[g, b, c] * sum_{k in block b} X[r, k] W_g[k, c].

    lhs_q uint8 [M, K]; lhs_scale float32 [M] or [1]; rhs_q uint8 [E_loc, K, N]
    (or [E_loc, N, K] with transpose_rhs); rhs_scale float32 [E_loc, Kb, 1, Nb].
    ``sample`` = (rows, cols) evaluates only those elements (1-D result).
    Returns a dict with the float64 result ``out``, the abs-sum ``abs_sum``
    (same formula on absolute values), ``f32`` and ``bf16`` (bit patterns).
    """
    lhs_q = np.asarray(lhs_q, dtype=np.uint8)
    M, K = lhs_q.shape
    rhs_q = np.asarray(rhs_q, dtype=np.uint8)
    E_loc = num_local_experts
    N = rhs_q.shape[1] if transpose_rhs else rhs_q.shape[2]
    rs = np.asarray(rhs_scale, dtype=np.float64)
    if rs.ndim != 4 or rs.shape[0] != E_loc or rs.shape[2] != 1:
        raise ValueError("rhs_scale must be [E_loc, Kb, 1, Nb]")
    kb, nb = rs.shape[1], rs.shape[3]
    if K % kb or N % nb:
        raise ValueError("scale blocks must tile K and N")
    bk = K // kb
    offs, sizes, n = local_group_offsets(group_sizes, group_offset, E_loc)
    if n > M:
        raise ValueError("local rows exceed M")
    ls = _lhs_scale_vec(lhs_scale, M)

    def weight(g):
        w = e4m3_decode(rhs_q[g])
        return w.T if transpose_rhs else w          # [K, N]

    if sample is None:
        o = np.zeros((M, N))
        a = np.zeros((M, N))
        for g in range(E_loc):
            m = sizes[g]
            if m == 0:
                continue
            rows = slice(offs[g], offs[g] + m)
            X = e4m3_decode(lhs_q[rows])
            W = weight(g)
            tot = np.zeros((m, N))
            atot = np.zeros((m, N))
            for b in range(kb):
                ks = slice(b * bk, (b + 1) * bk)
                P = X[:, ks] @ W[ks, :]                          # exact
                PA = np.abs(X[:, ks]) @ np.abs(W[ks, :])         # exact
                rsb = _expand_cols(rs[g, b, 0, :], N, nb)
                tot = tot + rsb[None, :] * P
                atot = atot + np.abs(rsb)[None, :] * PA
            o[rows] = ls[rows, None] * tot
            a[rows] = np.abs(ls[rows, None]) * atot
        return _finish(o, a)

    rows_s, cols_s = (np.asarray(v, dtype=np.int64) for v in sample)
    o = np.zeros(rows_s.shape)
    a = np.zeros(rows_s.shape)
    grp = np.searchsorted(offs + sizes, rows_s, side="right")    # group of each row
    inside = rows_s < n
    for g in np.unique(grp[inside]):
        sel = np.nonzero(inside & (grp == g))[0]
        W = weight(g)
        X = e4m3_decode(lhs_q[rows_s[sel]])                     # [P, K]
        Wc = W[:, cols_s[sel]].T                                 # [P, K]
        prod = (X * Wc).reshape(len(sel), kb, bk)
        P = prod.sum(axis=2)                                     # exact
        PA = np.abs(prod).sum(axis=2)
        rsb = rs[g, :, 0, :][:, cols_s[sel] // (N // nb)].T      # [P, kb]
        tot = np.zeros(len(sel))
        atot = np.zeros(len(sel))
        for b in range(kb):
            tot = tot + rsb[:, b] * P[:, b]
            atot = atot + np.abs(rsb[:, b]) * PA[:, b]
        o[sel] = ls[rows_s[sel]] * tot
        a[sel] = np.abs(ls[rows_s[sel]]) * atot
    return _finish(o, a)


def tgmm(lhs_q, lhs_scale, rhs_q, rhs_scale, group_sizes, group_offset, num_local_experts,
         sample=None):
    """dW[g, k, c] = (ls[k] * rs[c]) * sum_{r in group g} X[r, k] * dY[r, c].

    lhs_q uint8 [M, K] with scale [1] or [K]; rhs_q uint8 [M, N] with scale
    [1] or [N] (scales must be constant along the contracted rows).  An empty
    group gives zeros.  ``sample`` = (g, k, c) index arrays evaluates only
    those elements.  Returns the same dict as ``gmm``.
    """
    lhs_q = np.asarray(lhs_q, dtype=np.uint8)
    rhs_q = np.asarray(rhs_q, dtype=np.uint8)
    M, K = lhs_q.shape
    N = rhs_q.shape[1]
    if rhs_q.shape[0] != M:
        raise ValueError("tgmm: lhs and rhs must have the same rows")
    lsv = np.asarray(lhs_scale, dtype=np.float64).reshape(-1)
    rsv = np.asarray(rhs_scale, dtype=np.float64).reshape(-1)
    lsv = np.full(K, lsv[0]) if lsv.size == 1 else lsv
    rsv = np.full(N, rsv[0]) if rsv.size == 1 else rsv
    if lsv.size != K or rsv.size != N:
        raise ValueError("tgmm: scales must have 1, K (lhs) or N (rhs) entries")
    offs, sizes, n = local_group_offsets(group_sizes, group_offset, num_local_experts)
    if n > M:
        raise ValueError("local rows exceed M")
    if sample is None:
        o = np.zeros((num_local_experts, K, N))
        a = np.zeros((num_local_experts, K, N))
        for g in range(num_local_experts):
            if sizes[g] == 0:
                continue
            rows = slice(offs[g], offs[g] + sizes[g])
            X = e4m3_decode(lhs_q[rows])
            D = e4m3_decode(rhs_q[rows])
            sc = lsv[:, None] * rsv[None, :]
            o[g] = sc * (X.T @ D)
            a[g] = np.abs(sc) * (np.abs(X).T @ np.abs(D))
        return _finish(o, a)
    g_s, k_s, c_s = (np.asarray(v, dtype=np.int64) for v in sample)
    o = np.zeros(g_s.shape)
    a = np.zeros(g_s.shape)
    for g in np.unique(g_s):
        sel = np.nonzero(g_s == g)[0]
        if sizes[g] == 0:
            continue
        rows = slice(offs[g], offs[g] + sizes[g])
        X = e4m3_decode(lhs_q[rows][:, k_s[sel]])     # [m, P]
        D = e4m3_decode(rhs_q[rows][:, c_s[sel]])     # [m, P]
        sc = lsv[k_s[sel]] * rsv[c_s[sel]]
        o[sel] = sc * (X * D).sum(axis=0)
        a[sel] = np.abs(sc) * np.abs(X * D).sum(axis=0)
    return _finish(o, a)
