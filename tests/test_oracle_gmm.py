"""Pins of the oracle's grouped matmul (gmm) and transposed grouped matmul
(tgmm): brute force per routed row without sorting, exact rational dot
products, library matmul on a single group, and structural invariants."""

from fractions import Fraction

import numpy as np
import pytest

from oracle.codec import e4m3_decode
from oracle.gmm import gmm, tgmm
from oracle.sort import sort_by_expert


def _rand_e4m3(rng, shape):
    """Random finite e4m3 codes with a realistic magnitude spread."""
    c = rng.integers(0, 256, shape).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x38
    return c


def _dot_blocks(x, w, rs_row, kb):
    """sum_b rs_b * (x_b . w_b), blocks in ascending order, float64."""
    K = len(x)
    bk = K // kb
    tot = 0.0
    for b in range(kb):
        tot = tot + rs_row[b] * float(np.dot(x[b * bk:(b + 1) * bk], w[b * bk:(b + 1) * bk]))
    return tot


@pytest.mark.parametrize("kb,nb", [(1, 24), (2, 24), (4, 3), (1, 1)])
def test_gmm_equals_unsorted_per_row_bruteforce(kb, nb):
    rng = np.random.default_rng(20 + kb)
    T, k, E, K, N = 11, 2, 6, 32, 24
    g0, El = 1, 4
    ids = rng.integers(0, E, (T, k)).astype(np.int32)
    xq = _rand_e4m3(rng, (T, K))
    xsc = rng.uniform(0.01, 1, T).astype(np.float32)
    srt = sort_by_expert(ids, E, g0, El, xq=xq, xscale=xsc, m_cap=T * k)
    wq = _rand_e4m3(rng, (El, K, N))
    ws = rng.uniform(0.001, 0.1, (El, kb, 1, nb)).astype(np.float32)
    res = gmm(srt["xs"], srt["ss"], wq, ws, srt["group_sizes"], g0, El)
    inv = srt["inv_pos"]
    for f in range(T * k):
        r = inv[f]
        e = ids.reshape(-1)[f]
        if r < 0:
            assert not (g0 <= e < g0 + El)
            continue
        t = f // k
        x = e4m3_decode(xq[t])
        W = e4m3_decode(wq[e - g0])
        for c in range(N):
            rs_row = ws[e - g0, :, 0, c // (N // nb)].astype(np.float64)
            expect = float(xsc[t]) * _dot_blocks(x, W[:, c], rs_row, kb)
            assert res["out"][r, c] == expect
    n = srt["n"]
    assert not res["out"][n:].any() and not res["f32"][n:].any() and not res["bf16"][n:].any()


def test_gmm_exact_rational_on_tiny_input():
    rng = np.random.default_rng(21)
    M, K, N, E = 5, 16, 3, 2
    gs = np.array([2, 3], np.int32)
    xq = _rand_e4m3(rng, (M, K))
    wq = _rand_e4m3(rng, (E, K, N))
    ls = rng.uniform(0.01, 1, M).astype(np.float32)
    ws = rng.uniform(0.001, 0.1, (E, 2, 1, N)).astype(np.float32)
    res = gmm(xq, ls, wq, ws, gs, 0, E)
    for r in range(M):
        g = 0 if r < 2 else 1
        for c in range(N):
            ex = Fraction(0)
            for b in range(2):
                s = sum(Fraction(float(e4m3_decode(xq[r, kk]))) * Fraction(float(e4m3_decode(wq[g, kk, c])))
                        for kk in range(b * 8, b * 8 + 8))
                ex += Fraction(float(ws[g, b, 0, c])) * s
            ex *= Fraction(float(ls[r]))
            got = res["out"][r, c]
            assert abs(Fraction(got) - ex) <= abs(ex) * Fraction(1, 2 ** 50)
            aex = 0
            for b in range(2):
                s = sum(abs(Fraction(float(e4m3_decode(xq[r, kk]))) * Fraction(float(e4m3_decode(wq[g, kk, c]))))
                        for kk in range(b * 8, b * 8 + 8))
                aex += Fraction(float(ws[g, b, 0, c])) * s
            aex *= Fraction(float(ls[r]))
            assert abs(Fraction(res["abs_sum"][r, c]) - aex) <= aex * Fraction(1, 2 ** 50)
            assert res["abs_sum"][r, c] >= abs(got)


def test_gmm_single_group_is_library_matmul_and_scales_factor_out():
    rng = np.random.default_rng(22)
    M, K, N = 9, 64, 10
    xq = _rand_e4m3(rng, (M, K))
    wq = _rand_e4m3(rng, (1, K, N))
    one = np.ones((1, 1, 1, N), np.float32)
    res = gmm(xq, np.ones(1, np.float32), wq, one, np.array([M], np.int32), 0, 1)
    assert np.array_equal(res["out"], np.matmul(e4m3_decode(xq), e4m3_decode(wq[0])))
    res2 = gmm(xq, np.full(1, 0.5, np.float32), wq, 4 * one, np.array([M], np.int32), 0, 1)
    assert np.array_equal(res2["out"], 2 * res["out"])


def test_gmm_blockwise_with_equal_scales_equals_per_channel():
    rng = np.random.default_rng(23)
    M, K, N = 7, 256, 8
    xq = _rand_e4m3(rng, (M, K))
    wq = _rand_e4m3(rng, (1, K, N))
    ls = rng.uniform(0.01, 1, M).astype(np.float32)
    pc = rng.uniform(0.001, 0.1, (1, 1, 1, N)).astype(np.float32)
    blk = np.repeat(pc, 2, axis=1)
    gs = np.array([M], np.int32)
    a = gmm(xq, ls, wq, pc, gs, 0, 1)
    b = gmm(xq, ls, wq, blk, gs, 0, 1)
    # per-channel: rs * (P0 + P1); blockwise: rs*P0 + rs*P1 -- equal up to a few
    # roundings of the partial products, each bounded by the abs-sum
    assert np.all(np.abs(a["out"] - b["out"]) <= 2.0 ** -50 * a["abs_sum"])
    assert np.array_equal(a["abs_sum"] > 0, b["abs_sum"] > 0)


def test_gmm_transpose_rhs_sampling_and_empty_groups():
    rng = np.random.default_rng(24)
    E, K, N = 5, 32, 16
    gs = np.array([0, 3, 0, 4, 0], np.int32)        # empty first, middle, last
    M = 10
    xq = _rand_e4m3(rng, (M, K))
    wq = _rand_e4m3(rng, (E, K, N))
    ws = rng.uniform(0.001, 0.1, (E, 1, 1, N)).astype(np.float32)
    ls = rng.uniform(0.01, 1, M).astype(np.float32)
    a = gmm(xq, ls, wq, ws, gs, 0, E)
    b = gmm(xq, ls, np.ascontiguousarray(wq.transpose(0, 2, 1)), ws, gs, 0, E, transpose_rhs=True)
    assert np.array_equal(a["out"], b["out"])
    assert not a["out"][7:].any()
    rows = rng.integers(0, M, 40)
    cols = rng.integers(0, N, 40)
    s = gmm(xq, ls, wq, ws, gs, 0, E, sample=(rows, cols))
    assert np.array_equal(s["out"], a["out"][rows, cols])
    assert np.array_equal(s["abs_sum"], a["abs_sum"][rows, cols])
    # local slice: experts 1..3 only
    c = gmm(xq[:7], ls[:7], wq[1:4], ws[1:4], gs, 1, 3)
    assert np.array_equal(c["out"], a["out"][:7])


def test_gmm_rejects_rows_beyond_buffer():
    with pytest.raises(ValueError):
        gmm(np.zeros((3, 16), np.uint8), np.ones(3, np.float32), np.zeros((1, 16, 4), np.uint8),
            np.ones((1, 1, 1, 4), np.float32), np.array([4], np.int32), 0, 1)


def test_tgmm_bruteforce_dense_sum_and_empty_group():
    rng = np.random.default_rng(25)
    E, M, K, N = 4, 12, 8, 6
    gs = np.array([5, 0, 4, 3], np.int32)
    X = _rand_e4m3(rng, (M, K))
    D = _rand_e4m3(rng, (M, N))
    lsk = rng.uniform(0.01, 1, K).astype(np.float32)
    rsn = rng.uniform(0.01, 1, N).astype(np.float32)
    res = tgmm(X, lsk, D, rsn, gs, 0, E)
    offs = [0, 5, 5, 9]
    for g in range(E):
        for kk in range(K):
            for c in range(N):
                acc = 0.0
                for r in range(offs[g], offs[g] + gs[g]):
                    acc += float(e4m3_decode(X[r, kk])) * float(e4m3_decode(D[r, c]))
                assert res["out"][g, kk, c] == float(lsk[kk]) * float(rsn[c]) * acc
    assert not res["out"][1].any()
    unit = tgmm(X, np.ones(1, np.float32), D, np.ones(1, np.float32), gs, 0, E)
    assert np.array_equal(unit["out"].sum(axis=0), e4m3_decode(X).T @ e4m3_decode(D))
    gi = rng.integers(0, E, 30)
    ki = rng.integers(0, K, 30)
    ci = rng.integers(0, N, 30)
    s = tgmm(X, lsk, D, rsn, gs, 0, E, sample=(gi, ki, ci))
    assert np.array_equal(s["out"], res["out"][gi, ki, ci])
    assert np.array_equal(s["abs_sum"], res["abs_sum"][gi, ki, ci])
    # local slice of experts 2..3: their rows (5..11) start at row 0 of the compact buffer
    loc = tgmm(X[5:], lsk, D[5:], rsn, gs, 2, 2)
    assert np.array_equal(loc["out"], res["out"][2:4])
