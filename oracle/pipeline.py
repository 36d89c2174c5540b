"""The oracle's steps chained into the three workload pipelines, plus the
unquantized bfloat16 dense reference used only for the accuracy context.

TEST INFRASTRUCTURE ONLY (see the package docstring).

* up-projection: quantize tokens -> sort -> one gmm -> gather-reduce;
* gated FFN forward: quantize -> sort -> gmm(wi_0) = a, gmm(wi_1) = b (bf16)
  -> requantize silu(a)*b per row -> gmm(wo) -> gather-reduce;
* backward: x quantized with the static scale and sorted; dY quantized per
  row (for the input gradient, a gmm against the transposed weight) and per
  tensor (for tgmm, whose contraction runs over rows); dW = tgmm.

The pages report the error of fp8 against a bf16 dense reference as
``relative_norm_diff`` ("Support quantization for tokamax gmm v2", table
"relative_norm_diff Across All Cases"); read here as the Frobenius-norm
ratio ||y - y_ref|| / ||y_ref||.
"""

import numpy as np

from .codec import bf16_decode, bf16_rne_from_f64
from .quantize import (SCALE_ROW_DYNAMIC, SCALE_TENSOR_DYNAMIC, SCALE_TENSOR_STATIC,
                       quantize_rows, quantize_weights)
from .sort import sort_by_expert
from .gmm import gmm, tgmm
from .gather_reduce import gather_reduce


def quantize_config_weights(cfg, weights, static_scale=None):
    """Quantize every weight of a workload with the config's block layout."""
    out = {}
    for name, w in weights.items():
        _, K, N = w.shape
        kb, nb = cfg.scale_blocks(K, N)
        out[name] = quantize_weights(w, kb, nb, static_scale=static_scale)
    return out


def forward_pipeline(cfg, data, qweights, act_mode=SCALE_ROW_DYNAMIC, act_static=None, m_cap=None):
    """Run the up-projection or gated-FFN forward; returns every stage."""
    st = {}
    q, s, _ = quantize_rows(data["x"], act_mode, static_scale=act_static)
    st["xq"], st["xscale"] = q, s
    srt = sort_by_expert(data["ids"], cfg.E, cfg.group_offset, cfg.E_loc, xq=q, xscale=s,
                         xscale_mode=act_mode, m_cap=m_cap)
    st["sort"] = srt
    gs, g0, El = srt["group_sizes"], cfg.group_offset, cfg.E_loc
    if cfg.pipeline == "up":
        wq, ws = qweights["w_up"]
        y = gmm(srt["xs"], srt["ss"], wq, ws, gs, g0, El)
        st["y"] = y
    else:
        w0, s0 = qweights["wi_0"]
        w1, s1 = qweights["wi_1"]
        wo, so = qweights["wo"]
        a = gmm(srt["xs"], srt["ss"], w0, s0, gs, g0, El)
        b = gmm(srt["xs"], srt["ss"], w1, s1, gs, g0, El)
        st["a"], st["b"] = a, b
        hq, hs, _ = quantize_rows(a["bf16"], SCALE_ROW_DYNAMIC, x_up_bits=b["bf16"])
        st["hq"], st["hs"] = hq, hs
        y = gmm(hq, hs, wo, so, gs, g0, El)
        st["y"] = y
    st["out"] = gather_reduce(y["bf16"], True, srt["inv_pos"].reshape(cfg.T, cfg.k), data["topk_w"])
    return st


def backward_pipeline(cfg, data, w_static_scale, act_static_scale, m_cap=None):
    """Config-5 backward: dX = gmm(dYq, W^T), dW = tgmm(Xs, dYq)."""
    st = {}
    (wq, ws), = quantize_config_weights(cfg, {"w_up": data["weights"]["w_up"]},
                                        static_scale=w_static_scale).values()
    st["wq"], st["ws"] = wq, ws
    xq, xsc, _ = quantize_rows(data["x"], SCALE_TENSOR_STATIC, static_scale=act_static_scale)
    srt = sort_by_expert(data["ids"], cfg.E, cfg.group_offset, cfg.E_loc, xq=xq, xscale=xsc,
                         xscale_mode=SCALE_TENSOR_STATIC, m_cap=m_cap)
    st["sort"] = srt
    dyq_r, dys_r, _ = quantize_rows(data["dy"], SCALE_ROW_DYNAMIC)
    dyq_t, dys_t, _ = quantize_rows(data["dy"], SCALE_TENSOR_DYNAMIC)
    st["dyq_row"], st["dys_row"], st["dyq_t"], st["dys_t"] = dyq_r, dys_r, dyq_t, dys_t
    gs, g0, El = srt["group_sizes"], cfg.group_offset, cfg.E_loc
    # dX[r, :] = dY[r, :] @ W_g^T: the weight [E, H, I] is the rhs stored [E, N=H, K=I]
    st["dx"] = gmm(dyq_r, dys_r, wq, ws, gs, g0, El, transpose_rhs=True)
    st["dw"] = lambda sample=None: tgmm(srt["xs"], xsc, dyq_t, dys_t, gs, g0, El, sample=sample)
    return st


def dense_bf16_reference(cfg, data):
    """Unquantized reference: bf16 operands, float64 products, bf16 between stages."""
    x = bf16_decode(data["x"]).astype(np.float64)
    ids = data["ids"]
    T, k = ids.shape
    W = {n: bf16_decode(w).astype(np.float64) for n, w in data["weights"].items()}
    gl = lambda v: bf16_decode(bf16_rne_from_f64(v)).astype(np.float64)
    out = np.zeros((T, cfg.H if cfg.pipeline == "ffn" else cfg.I))
    for j in range(k):
        e = ids[:, j]
        loc = (e >= cfg.group_offset) & (e < cfg.group_offset + cfg.E_loc)
        for g in np.unique(e[loc]):
            rows = np.nonzero(e == g)[0]
            gi = g - cfg.group_offset
            if cfg.pipeline == "up":
                y = gl(x[rows] @ W["w_up"][gi])
            else:
                a = gl(x[rows] @ W["wi_0"][gi])
                b = gl(x[rows] @ W["wi_1"][gi])
                h = gl(a / (1.0 + np.exp(-a)) * b)
                y = gl(h @ W["wo"][gi])
            out[rows] += data["topk_w"][rows, j].astype(np.float64)[:, None] * y
    return bf16_rne_from_f64(out)


def dense_bf16_backward_reference(cfg, data, dout_bits):
    """The gated FFN's backward with unquantized bf16 operands (float64
    products, bf16 between stages), for context next to the pages' gradient
    columns ("Support quantization for tokamax gmm v2", table
    "relative_norm_diff Across All Cases": grad_wi_0, grad_wi_1, grad_wo).
    The forward is dense_bf16_reference's; for out = sum_j w_j y_j the
    backward is dy_j = w_j * dout, dh = dy wo^T, dwo += h^T dy, the SiLU*mul
    derivative (da = dh * b * s (1 + a (1 - s)), db = dh * a s with s the
    logistic of a), dw0 += x^T da, dw1 += x^T db, dx += da w0^T + db w1^T.
    Returns dx (bf16 bits [T, H]) and float64 dw0, dw1 [E_loc, H, I], dwo
    [E_loc, I, H]."""
    x = bf16_decode(data["x"]).astype(np.float64)
    dout = bf16_decode(dout_bits).astype(np.float64)
    ids = data["ids"]
    T, k = ids.shape
    W = {n: bf16_decode(w).astype(np.float64) for n, w in data["weights"].items()}
    gl = lambda v: bf16_decode(bf16_rne_from_f64(v)).astype(np.float64)
    El, H, I = cfg.E_loc, cfg.H, cfg.I
    dw0, dw1, dwo = np.zeros((El, H, I)), np.zeros((El, H, I)), np.zeros((El, I, H))
    dx = np.zeros((T, H))
    for j in range(k):
        e = ids[:, j]
        loc = (e >= cfg.group_offset) & (e < cfg.group_offset + cfg.E_loc)
        for g in np.unique(e[loc]):
            rows = np.nonzero(e == g)[0]
            gi = g - cfg.group_offset
            xr = x[rows]
            a = gl(xr @ W["wi_0"][gi])
            b = gl(xr @ W["wi_1"][gi])
            sg = 1.0 / (1.0 + np.exp(-a))
            h = gl(a * sg * b)
            dy = gl(data["topk_w"][rows, j].astype(np.float64)[:, None] * dout[rows])
            dh = gl(dy @ W["wo"][gi].T)
            dwo[gi] += h.T @ dy
            da = gl(dh * b * sg * (1.0 + a * (1.0 - sg)))
            db = gl(dh * a * sg)
            dw0[gi] += xr.T @ da
            dw1[gi] += xr.T @ db
            dx[rows] += da @ W["wi_0"][gi].T + db @ W["wi_1"][gi].T
    return bf16_rne_from_f64(dx), dw0, dw1, dwo


def rel_norm_diff_f(g, ref):
    """Frobenius-norm ratio of two float arrays (the pages' relative_norm_diff)."""
    g = np.asarray(g, np.float64)
    r = np.asarray(ref, np.float64)
    return float(np.linalg.norm(g - r) / np.linalg.norm(r))


def rel_norm_diff(y_bits, ref_bits):
    y = bf16_decode(y_bits).astype(np.float64)
    r = bf16_decode(ref_bits).astype(np.float64)
    return float(np.linalg.norm(y - r) / np.linalg.norm(r)), float(np.abs(y - r).max())
