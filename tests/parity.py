"""Match rules between the HIP path and the oracle, and numpy <-> device
helpers for the GPU parity tests.

Rules (the floating-point tolerance of the path: 1e-5 relative in float32
before output rounding, 1 bf16 ulp after it):

1. bytes, scales, permutations and group sizes: bit-exact;
2. float32 results: |g - o| <= 1e-5 * A, where A is the oracle's abs-sum
   (the same formula on absolute values, the componentwise measure of a dot
   product's error);
3. bf16 results: where 1e-5 * A is below half a bf16 ulp of o, the bf16
   result is within 1 ulp of bf16(o) (ordered bit patterns); elsewhere
   (cancellation) |g - o| <= 1e-5 * A + half an ulp.

The fp8 matrix cores do not compute exact dot products: they sum products in
aligned chunks of 8 contraction indices, each truncated below 2^-13 of the
chunk's largest exponent sum (tests/mfma_model.py models this; its CPU tests
pin it).  On a few elements of some stages -- operands with a wide spread of
exponents inside a chunk, such as the requantized SiLU output or short
contractions -- that arithmetic itself lands outside 1e-5 * A of the exact
value.  Workload checks therefore take ``model``: a function giving the
modelled matrix-core result at the given flat indices.  Every element is
held to rules 2-3 against the oracle, except those that fail it, which must
then equal the modelled hardware arithmetic within the same 1e-5 * A (rule
3 with the model's value in place of o).  The fraction of such elements is
printed with every check (``model_frac``).

Only tests on synthetic operands with uniformly random e4m3 codes --
exponents spread over the whole format, far from any workload -- may pass
``hw_allowance`` instead: the a-priori bound B_hw below, added to the
tolerance of rules 2 and 3.  Such a test also bounds max |g - o| / A by
HW_MAX_ERR_OVER_A, the most the chunk rule can lose, so a widening of the
allowance shows up.

B_hw: inside a chunk every product is aligned to the chunk's largest
exponent sum e(a) + e(b) -- e(v) is the binary exponent of v, -6 for a
subnormal, and a product with a zero operand takes no part -- and bits below
2^(that sum - 13) are dropped (measured on the device for
v_mfma_f32_16x16x128_f8f6f4 and v_mfma_f32_16x16x32_fp8_fp8).  So product i
loses less than min(|p_i|, 2^-13 * max_j 2^(e(a_j) + e(b_j))) over its
chunk; the allowance uses 2^-12 (a factor-2 margin) and the maximum over the
window of the 15 products around i, which contains every aligned chunk
holding i.
"""

import numpy as np
import torch

from oracle.codec import bf16_decode, bf16_rne_from_f64, e4m3_decode

REL_TOL = 1e-5
HW_FRAC = 2.0 ** -12
# the largest |g - o| / A the chunk rule allows: at most 7 products of a chunk
# lose bits, each less than 2^(e_max - 13), and the chunk's largest product is
# at least 2^(e_max - 3) (a subnormal operand of mantissa 1/8 aligned at -6)
HW_MAX_ERR_OVER_A = 7 * 2.0 ** -13 * 8


# ------------------------------------------------------------ device helpers
def dev_u8(a, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(device)


def dev_i32(a, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)


def dev_f32(a, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def dev_bf16(bits, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).to(device).view(torch.bfloat16)


def host(t):
    """Device tensor -> numpy (bf16 as uint16 bit patterns)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


# ------------------------------------------------------------ allowance
def _window_max(absp):
    """max over [i-7, i+7] along the last axis."""
    K = absp.shape[-1]
    pad = np.zeros(absp.shape[:-1] + (K + 14,), dtype=absp.dtype)
    pad[..., 7:7 + K] = absp
    out = absp.copy()
    for d in range(-7, 8):
        out = np.maximum(out, pad[..., 7 + d:7 + d + K])
    return out


def _exp_field(codes):
    """Alignment exponent of e4m3 codes: binary exponent, -6 for subnormals."""
    e = (np.asarray(codes, np.int64) >> 3) & 0xF
    return np.where(e == 0, -6, e - 7)


def hw_allowance_products(p, ca, cb):
    """B_hw of dot products with products p [..., K] (float64) of the codes
    ca, cb [..., K]."""
    nz = ((ca & 0x7F) != 0) & ((cb & 0x7F) != 0)
    align = np.where(nz, np.ldexp(1.0, _exp_field(ca) + _exp_field(cb)), 0.0)
    return np.minimum(np.abs(p), HW_FRAC * _window_max(align)).sum(axis=-1)


def gmm_allowance(lhs_q, lhs_scale, rhs_q, rhs_scale, group_sizes, g0, El, rows, cols, transpose_rhs=False):
    """B_hw of sampled gmm outputs (rows, cols), with the scales applied."""
    gs = np.asarray(group_sizes, np.int64)[g0:g0 + El]
    offs = np.concatenate([[0], np.cumsum(gs)])
    K = lhs_q.shape[1]
    rs = np.asarray(rhs_scale, np.float64)
    kb, nb = rs.shape[1], rs.shape[3]
    N = rhs_q.shape[1] if transpose_rhs else rhs_q.shape[2]
    ls = np.asarray(lhs_scale, np.float64).reshape(-1)
    out = np.zeros(len(rows))
    grp = np.searchsorted(offs[1:], rows, side="right")
    for g in np.unique(grp):
        if g >= El:
            continue
        sel = np.nonzero(grp == g)[0]
        Xc = lhs_q[rows[sel]]
        Wg = rhs_q[g]
        Wcc = Wg[cols[sel], :] if transpose_rhs else Wg[:, cols[sel]].T
        p = e4m3_decode(Xc) * e4m3_decode(Wcc)                    # [P, K]
        bk = K // kb
        tot = np.zeros(len(sel))
        for b in range(kb):
            ks = slice(b * bk, (b + 1) * bk)
            tot += np.abs(rs[g, b, 0, cols[sel] // (N // nb)]) * hw_allowance_products(p[:, ks], Xc[:, ks], Wcc[:, ks])
        lsr = np.abs(ls[rows[sel]] if ls.size > 1 else np.full(len(sel), ls[0]))
        out[sel] = lsr * tot
    return out


def tgmm_allowance(lhs_q, lhs_scale, rhs_q, rhs_scale, group_sizes, g0, El, gi, ki, ci):
    gs = np.asarray(group_sizes, np.int64)[g0:g0 + El]
    offs = np.concatenate([[0], np.cumsum(gs)])
    ls = np.asarray(lhs_scale, np.float64).reshape(-1)
    rs = np.asarray(rhs_scale, np.float64).reshape(-1)
    out = np.zeros(len(gi))
    for g in np.unique(gi):
        sel = np.nonzero(gi == g)[0]
        if gs[g] == 0:
            continue
        rows = slice(offs[g], offs[g + 1])
        Xc = lhs_q[rows][:, ki[sel]].T                       # [P, m] codes
        Dc = rhs_q[rows][:, ci[sel]].T
        sc = np.abs((ls[ki[sel]] if ls.size > 1 else ls[0]) * (rs[ci[sel]] if rs.size > 1 else rs[0]))
        out[sel] = sc * hw_allowance_products(e4m3_decode(Xc) * e4m3_decode(Dc), Xc, Dc)
    return out


# ------------------------------------------------------------ rules
def _ordered(bits16):
    b = bits16.astype(np.int32)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def _allowance_at(B, idx):
    """B may be a scalar, an array shaped like the results, or a callable
    returning the allowance of the flat indices ``idx``."""
    if callable(B):
        return np.asarray(B(idx), np.float64)
    B = np.asarray(B, np.float64)
    return B if B.ndim == 0 else B.reshape(-1)[idx]


def _report(what, stats):
    print(f"parity {what}: " + " ".join(f"{k}={v:.4g}" if isinstance(v, float) else f"{k}={v}"
                                         for k, v in stats.items()), flush=True)
    return stats


_CHUNK = 1 << 23      # elements compared at a time (bounds the host memory of full-size checks)


def check_f32(g, o, A, what="", hw_allowance=None, model=None):
    """Rule 2 on every element.  ``model``: elements outside 1e-5 * A must be
    within 1e-5 * A of the modelled matrix-core result there.
    ``hw_allowance`` (synthetic random-code operands only): the tolerance is
    1e-5 * A + B_hw and max |g - o| / A is bounded."""
    g, o, A = np.asarray(g).reshape(-1), np.asarray(o).reshape(-1), np.asarray(A).reshape(-1)
    assert g.size == o.size == A.size, f"{what}: sizes {g.size} {o.size} {A.size}"
    n_strict, ratio, n_bad, excess, model_ratio = 0, 0.0, 0, 0.0, 0.0
    for s0 in range(0, g.size, _CHUNK):
        sl = slice(s0, min(s0 + _CHUNK, g.size))
        gc, oc, Ac = (np.asarray(v[sl], np.float64) for v in (g, o, A))
        err = np.abs(gc - oc)
        strict = err <= REL_TOL * Ac
        n_strict += int(strict.sum())
        pos = Ac > 0
        if pos.any():
            ratio = max(ratio, float(np.max(err[pos] / Ac[pos])))
        if (err[~pos] > 0).any():
            ratio = np.inf
        idx = np.nonzero(~strict)[0]
        if not idx.size:
            continue
        if hw_allowance is not None:
            tol = REL_TOL * Ac[idx] + _allowance_at(hw_allowance, idx + s0)
            bad = err[idx] > tol
            n_bad += int(bad.sum())
            if bad.any():
                excess = max(excess, float(np.max(err[idx] - tol)))
        elif model is not None:
            mv = np.asarray(model(idx + s0), np.float32).astype(np.float64)
            merr = np.abs(gc[idx] - mv)
            n_bad += int((merr > REL_TOL * Ac[idx]).sum())
            model_ratio = max(model_ratio, float(np.max(merr / np.where(Ac[idx] > 0, Ac[idx], 1))))
        else:
            n_bad += idx.size
    n = g.size
    stats = {"strict_frac": n_strict / n if n else 1.0, "max_err_over_A": ratio, "n": int(n)}
    if model is not None:
        stats["model_frac"] = 1.0 - stats["strict_frac"]
        stats["max_err_vs_model_over_A"] = model_ratio
    _report(what, stats)
    if hw_allowance is not None:
        assert n_bad == 0, (f"{what}: {n_bad} of {n} float32 results outside 1e-5*A + B_hw; "
                            f"worst excess {excess:.3g}")
        assert ratio <= HW_MAX_ERR_OVER_A, f"{what}: max |g-o|/A = {ratio:.3g} > {HW_MAX_ERR_OVER_A}"
    elif model is not None:
        assert n_bad == 0, (f"{what}: {n_bad} of {n} float32 results outside 1e-5*A of both the exact value and "
                            f"the modelled matrix-core value; max |g-o|/A = {ratio:.3g}")
    else:
        assert n_bad == 0, f"{what}: {n_bad} of {n} float32 results outside 1e-5*A; max |g-o|/A = {ratio:.3g}"
    return stats


def _bf16_failing(tol, o, d, gv, hu):
    tight = tol < (2.0 ** -9) * np.abs(o) * (1 - 2.0 ** -8)
    return (tight & (d > 1)) | ((~tight) & (np.abs(gv - o) > tol + hu))


def _bf16_parts(gb, oc):
    d = np.abs(_ordered(gb) - _ordered(bf16_rne_from_f64(oc)))
    gv = bf16_decode(gb).astype(np.float64)
    hu = np.ldexp(1.0, np.frexp(np.maximum(np.abs(oc), 1e-38))[1] - 9)
    return d, gv, hu


def check_bf16(g_bits, o, A, what="", hw_allowance=None, model=None):
    """Rule 3 on every element (tolerance 1e-5 * A).  ``model``: elements
    that fail it must meet rule 3 with the modelled matrix-core float32
    result in place of o.  ``hw_allowance``: B_hw is added to the tolerance
    (synthetic random-code operands only)."""
    g_bits, o, A = np.asarray(g_bits).reshape(-1), np.asarray(o).reshape(-1), np.asarray(A).reshape(-1)
    assert g_bits.size == o.size == A.size, f"{what}: sizes {g_bits.size} {o.size} {A.size}"
    n_exact, n_strict_bad, n_bad, dmax = 0, 0, 0, 0
    for s0 in range(0, g_bits.size, _CHUNK):
        sl = slice(s0, min(s0 + _CHUNK, g_bits.size))
        gb = np.asarray(g_bits[sl], np.uint16)
        oc = np.asarray(o[sl], np.float64)
        Ac = np.asarray(A[sl], np.float64)
        d, gv, hu = _bf16_parts(gb, oc)
        n_exact += int((d == 0).sum())
        dmax = max(dmax, int(d.max()) if d.size else 0)
        idx = np.nonzero(_bf16_failing(REL_TOL * Ac, oc, d, gv, hu))[0]
        n_strict_bad += idx.size
        if not idx.size:
            continue
        if hw_allowance is not None:
            tol = REL_TOL * Ac[idx] + _allowance_at(hw_allowance, idx + s0)
            n_bad += int(_bf16_failing(tol, oc[idx], d[idx], gv[idx], hu[idx]).sum())
        elif model is not None:
            mv = np.asarray(model(idx + s0), np.float32).astype(np.float64)
            dm, gvm, hum = _bf16_parts(gb[idx], mv)
            n_bad += int(_bf16_failing(REL_TOL * Ac[idx], mv, dm, gvm, hum).sum())
        else:
            n_bad += idx.size
    n = g_bits.size
    stats = {"exact_frac": n_exact / n if n else 1.0, "max_ulp_diff": dmax,
             "strict_frac": 1.0 - n_strict_bad / n if n else 1.0, "n": int(n)}
    if model is not None:
        stats["model_frac"] = n_strict_bad / n if n else 0.0
    _report(what, stats)
    if hw_allowance is not None:
        assert n_bad == 0, f"{what}: {n_bad} bf16 results outside 1 ulp of bf16(o) (or the cancellation " \
                           f"tolerance with B_hw)"
    elif model is not None:
        assert n_bad == 0, (f"{what}: {n_bad} of {n} bf16 results outside rule 3 against both the exact value and "
                            f"the modelled matrix-core value")
    else:
        assert n_bad == 0, (f"{what}: {n_bad} of {n} bf16 results outside 1 ulp of bf16(o) "
                            f"(or 1e-5*A + half an ulp where the sum cancels)")
    return stats


def assert_bits_equal(g, o, what=""):
    g = np.ascontiguousarray(g)
    o = np.ascontiguousarray(o)
    assert g.shape == o.shape, f"{what}: shape {g.shape} != {o.shape}"
    if g.dtype == np.float32:
        g = g.view(np.uint32)
        o = o.astype(np.float32).view(np.uint32)
    neq = g != o
    assert not neq.any(), f"{what}: {neq.sum()} of {neq.size} differ; first at {np.argwhere(neq)[0].tolist()}"
