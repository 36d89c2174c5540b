"""Pins of the oracle's int8 variant: the codec against torch's rounding,
the quantizers against exact rational arithmetic and the invariants of
absmax scaling, and the int32-accumulated grouped matmul against Python
integer brute force and numpy's integer matmul."""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle.codec import bf16_decode
from oracle.int8 import (I8_MAX, SCALE_ROW_DYNAMIC, SCALE_TENSOR_DYNAMIC, SCALE_TENSOR_FROM_ROW_AMAX,
                         SCALE_TENSOR_STATIC, gmm_int8, int8_rne, quantize_rows_int8, quantize_weights_int8)
from oracle.sort import sort_by_expert
from tests.test_oracle_quantize import rn32_div
from workloads import to_bf16_bits


def _bf16(a):
    return to_bf16_bits(np.asarray(a, dtype=np.float32))


def _round_half_even(f: Fraction) -> int:
    fl = f.numerator // f.denominator
    rem = f - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        return fl + 1
    return fl


def test_codec_matches_torch_round_and_saturates():
    halves = np.arange(-300, 301, dtype=np.float32) / np.float32(2)        # every tie of the range and past it
    rng = np.random.default_rng(0)
    rand = rng.uniform(-200, 200, 20000).astype(np.float32)
    for v in (halves, rand):
        ref = torch.clamp(torch.round(torch.from_numpy(v)), -I8_MAX, I8_MAX).to(torch.int8).numpy()
        assert (int8_rne(v) == ref).all()
    assert int8_rne(np.float32(127.5)) == 127 and int8_rne(np.float32(-1000)) == -127    # never -128
    assert int8_rne(np.float32(2.5)) == 2 and int8_rne(np.float32(3.5)) == 4 and int8_rne(np.float32(-0.5)) == 0


def test_row_quantize_matches_exact_rational_bruteforce():
    rng = np.random.default_rng(1)
    x = _bf16(rng.standard_normal((6, 48)) * rng.uniform(0.01, 100, (6, 1)))
    q, s, amax = quantize_rows_int8(x, SCALE_ROW_DYNAMIC)
    xf = bf16_decode(x)
    for r in range(x.shape[0]):
        a = max(abs(Fraction(float(v))) for v in xf[r])
        assert Fraction(float(amax[r])) == a
        assert s[r] == rn32_div(np.float32(a), np.float32(127))       # s = RN(amax / 127)
        for c in range(x.shape[1]):
            v = rn32_div(xf[r, c], s[r])                              # RN(x / s), then ties-to-even integer
            want = max(-I8_MAX, min(I8_MAX, _round_half_even(Fraction(float(v)))))
            assert int(q[r, c]) == want


def test_static_scale_saturates_and_matches_bruteforce():
    x = _bf16([[0.0, -0.0, 1.0, -1.0, 3.99, 4.0, 1000.0, -1000.0, 0.031, 0.0156, 0.0157, 2.0 ** -20, 5.5, -6.5,
                7.5, 8.5]])
    s = np.float32(4.0 / 127)
    q, sc, _ = quantize_rows_int8(x, SCALE_TENSOR_STATIC, static_scale=s)
    assert sc[0] == s
    for c, v in enumerate(bf16_decode(x)[0]):
        want = max(-I8_MAX, min(I8_MAX, _round_half_even(Fraction(float(rn32_div(v, s))))))
        assert int(q[0, c]) == want
    assert q[0, 6] == 127 and q[0, 7] == -127


def test_every_nonzero_row_reaches_127_and_error_bound():
    rng = np.random.default_rng(2)
    x = _bf16(rng.standard_normal((200, 64)) * rng.uniform(1e-3, 1e3, (200, 1)))
    x[5] = 0
    q, s, amax = quantize_rows_int8(x, SCALE_ROW_DYNAMIC)
    nz = amax > 0
    assert (np.abs(q[nz]).max(axis=1) == 127).all()
    assert (q[5] == 0).all() and s[5] == 1.0
    assert (q != -128).all()
    xf = bf16_decode(x).astype(np.float64)
    err = np.abs(xf - q.astype(np.float64) * s[:, None].astype(np.float64))
    # half a quantum, plus the float32 quotient's rounding (|x / s| <= 127: at most 127 * 2^-24 of a quantum)
    assert (err <= s[:, None] * (0.5 + 127 * 2.0 ** -24)).all()


def test_tensor_modes():
    rng = np.random.default_rng(3)
    x = _bf16(rng.standard_normal((40, 32)))
    q1, s1, am = quantize_rows_int8(x, SCALE_TENSOR_DYNAMIC)
    assert s1[0] == rn32_div(np.float32(np.abs(bf16_decode(x)).max()), np.float32(127))
    q2, s2, _ = quantize_rows_int8(x, SCALE_TENSOR_FROM_ROW_AMAX, row_amax_in=am)
    assert s2[0] == s1[0] and (q2 == q1).all()
    q3, s3, _ = quantize_rows_int8(x, SCALE_TENSOR_STATIC, static_scale=s1[0])
    assert (q3 == q1).all()


def test_quantize_then_gather_equals_gather_then_quantize():
    rng = np.random.default_rng(4)
    T, H, E, k = 50, 32, 6, 3
    x = _bf16(rng.standard_normal((T, H)) * rng.uniform(0.1, 10, (T, 1)))
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    q, s, _ = quantize_rows_int8(x, SCALE_ROW_DYNAMIC)
    srt = sort_by_expert(ids, E, 0, E, xq=q.view(np.uint8), xscale=s, xscale_mode=SCALE_ROW_DYNAMIC)
    q2, s2, _ = quantize_rows_int8(x[srt["perm"] // k], SCALE_ROW_DYNAMIC)
    assert (srt["xs"].view(np.int8) == q2).all() and (srt["ss"] == s2).all()


@pytest.mark.parametrize("kb,nb", [(1, 32), (2, 32), (2, 2), (1, 1)])
def test_weight_quantizer_blocks_bruteforce(kb, nb):
    rng = np.random.default_rng(kb * 10 + nb)
    E, K, N = 2, 256, 32
    w = _bf16(rng.standard_normal((E, K, N)) * 0.02)
    w[1, :K // kb, :N // nb] = 0                                   # an all-zero block
    q, s = quantize_weights_int8(w, kb, nb)
    wf = bf16_decode(w)
    bk, bn = K // kb, N // nb
    for e in range(E):
        for b in range(kb):
            for c in range(nb):
                blk = wf[e, b * bk:(b + 1) * bk, c * bn:(c + 1) * bn]
                a = np.float32(np.abs(blk).max())
                want = np.float32(1.0) if a == 0 else rn32_div(a, np.float32(127))
                assert s[e, b, 0, c] == want
                qq = int8_rne((blk / s[e, b, 0, c]).astype(np.float32))
                assert (q[e, b * bk:(b + 1) * bk, c * bn:(c + 1) * bn] == qq).all()
    assert (q[1, :bk, :bn] == 0).all()


def test_gmm_int8_is_the_exact_integer_dot_product():
    """Against Python integers on unsorted (token, slot) pairs and numpy's
    int64 matmul on each group; blockwise scales equal per-channel ones when
    every block scale of a column is the same."""
    rng = np.random.default_rng(5)
    E, K, N = 4, 256, 48
    gs = np.array([3, 0, 5, 2], np.int32)
    M = int(gs.sum()) + 2
    X = rng.integers(-127, 128, (M, K)).astype(np.int8)
    W = rng.integers(-127, 128, (E, K, N)).astype(np.int8)
    ls = rng.uniform(0.01, 1, M).astype(np.float32)
    rs = rng.uniform(0.01, 1, (E, 2, 1, N)).astype(np.float32)
    o = gmm_int8(X, ls, W, rs, gs, 0, E)
    offs = np.concatenate([[0], np.cumsum(gs)])
    for g in range(E):
        for r in range(offs[g], offs[g + 1]):
            for c in range(0, N, 7):
                p0 = sum(int(X[r, k]) * int(W[g, k, c]) for k in range(128))
                p1 = sum(int(X[r, k]) * int(W[g, k, c]) for k in range(128, 256))
                want = float(ls[r]) * (float(rs[g, 0, 0, c]) * p0 + float(rs[g, 1, 0, c]) * p1)
                assert o["out"][r, c] == want
        if gs[g]:
            P = X[offs[g]:offs[g + 1]].astype(np.int64) @ W[g].astype(np.int64)
            same = np.repeat(rs[g, :1], 2, axis=0)[None]
            o1 = gmm_int8(X[offs[g]:offs[g + 1]], ls[offs[g]:offs[g + 1]], W[g:g + 1], same, [gs[g]], 0, 1)
            want = ls[offs[g]:offs[g + 1], None].astype(np.float64) * (rs[g, 0, 0][None].astype(np.float64) * P)
            assert np.allclose(o1["out"], want, rtol=1e-15, atol=0)
    assert not o["out"][offs[-1]:].any()
    ot = gmm_int8(X, ls, np.ascontiguousarray(W.transpose(0, 2, 1)), rs, gs, 0, E, transpose_rhs=True)
    assert (ot["out"] == o["out"]).all()
