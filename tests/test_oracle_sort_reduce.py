"""Pins of the oracle's stable ragged sort and its gather-reduce."""

import numpy as np
import pytest

from oracle.codec import bf16_decode
from oracle.gather_reduce import gather_reduce
from oracle.quantize import SCALE_ROW_DYNAMIC, SCALE_TENSOR_STATIC, quantize_rows
from oracle.sort import sort_by_expert
from workloads import to_bf16_bits


def _routing(rng, T, k, E, skew=False):
    if skew:                 # several empty experts, including the first local one
        p = np.array([0.5, 0.0, 0.0, 0.3, 0.15, 0.05, 0.0, 0.0])[:E]
        return rng.choice(E, (T, k), p=p / p.sum()).astype(np.int32)
    return rng.integers(0, E, (T, k)).astype(np.int32)


@pytest.mark.parametrize("T,k,E,g0,El,skew", [(13, 2, 8, 0, 8, False), (29, 3, 8, 2, 4, True),
                                              (7, 4, 6, 5, 1, False), (0, 2, 4, 0, 4, False)])
def test_sort_matches_python_bruteforce(T, k, E, g0, El, skew):
    rng = np.random.default_rng(T * 31 + k)
    ids = _routing(rng, T, k, E, skew)
    H = 16
    xq = rng.integers(0, 256, (T, H)).astype(np.uint8)
    xs_scale = rng.uniform(0.1, 2, T).astype(np.float32)
    out = sort_by_expert(ids, E, g0, El, xq=xq, xscale=xs_scale, m_cap=T * k + 5)
    M = T * k
    flat = [int(v) for v in ids.reshape(-1)]
    order = sorted(range(M), key=lambda f: (flat[f], f))          # stable by construction
    assert out["perm"].tolist() == order
    counts = [0] * E
    for v in flat:
        counts[v] += 1
    assert out["group_sizes"].tolist() == counts
    assert sum(counts) == M
    start = sum(counts[:g0])
    n = sum(counts[g0:g0 + El])
    assert (out["start"], out["n"]) == (start, n)
    for f in range(M):
        r = order.index(f)
        expect = r - start if start <= r < start + n else -1
        assert out["inv_pos"][f] == expect
    for r in range(n):
        t = order[start + r] // k
        assert np.array_equal(out["xs"][r], xq[t])
        assert out["ss"][r] == xs_scale[t]
    assert not out["xs"][n:].any() and not out["ss"][n:].any()
    # token ids ascend inside each group (stability)
    toks = np.asarray(order) // max(k, 1)
    for e in range(E):
        lo = sum(counts[:e])
        assert np.all(np.diff(toks[lo:lo + counts[e]]) >= 0)


def test_sort_passes_tensor_scale_through():
    ids = np.array([[1, 0], [0, 2]], np.int32)
    out = sort_by_expert(ids, 3, 0, 3, xq=np.zeros((2, 16), np.uint8),
                         xscale=np.array([0.5], np.float32), xscale_mode=SCALE_TENSOR_STATIC)
    assert out["ss"].tolist() == [0.5]


def test_sort_rejects_bad_ids_and_small_capacity():
    with pytest.raises(ValueError):
        sort_by_expert(np.array([[0, 4]], np.int32), 4, 0, 4)
    with pytest.raises(ValueError):
        sort_by_expert(np.array([[0, 1]], np.int32), 4, 0, 4, xq=np.zeros((1, 16), np.uint8), m_cap=1)


def test_quantize_before_sort_equals_sort_before_quantize():
    # "Quantize activations before EP all gather", Testing strategy.
    rng = np.random.default_rng(11)
    T, k, E, H = 50, 3, 6, 32
    ids = rng.integers(0, E, (T, k)).astype(np.int32)
    xb = to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    q, s, _ = quantize_rows(xb, SCALE_ROW_DYNAMIC)
    a = sort_by_expert(ids, E, 2, 3, xq=q, xscale=s)
    perm = a["perm"][a["start"]:a["start"] + a["n"]]
    xb_sorted = xb[perm // k]
    q2, s2, _ = quantize_rows(xb_sorted, SCALE_ROW_DYNAMIC)
    assert np.array_equal(a["xs"], q2)
    assert np.array_equal(a["ss"].view(np.uint32), s2.view(np.uint32))


def _y_bits(rng, rows, N):
    return to_bf16_bits(rng.standard_normal((rows, N)).astype(np.float32))


def test_gather_reduce_k1_unit_weight_is_inverse_permutation():
    rng = np.random.default_rng(12)
    T, N = 20, 16
    ids = rng.integers(0, 5, (T, 1)).astype(np.int32)
    srt = sort_by_expert(ids, 5, 0, 5)
    y = _y_bits(rng, T, N)
    out = gather_reduce(y, True, srt["inv_pos"].reshape(T, 1), np.ones((T, 1), np.float32))
    assert np.array_equal(out["bf16"], y[srt["inv_pos"]])


def test_gather_reduce_bruteforce_linearity_and_nonlocal_tokens():
    rng = np.random.default_rng(13)
    T, k, E, N = 17, 3, 8, 8
    ids = rng.integers(0, E, (T, k)).astype(np.int32)
    ids[4] = [0, 1, 7]                   # token with no local expert below
    srt = sort_by_expert(ids, E, 2, 4)
    inv = srt["inv_pos"].reshape(T, k)
    assert np.all(inv[4] == -1)
    y = _y_bits(rng, max(srt["n"], 1), N)
    w = rng.uniform(0, 1, (T, k)).astype(np.float32)
    out = gather_reduce(y, True, inv, w)
    yf = bf16_decode(y).astype(np.float64)
    for t in range(T):
        for c in range(N):
            acc = 0.0
            for j in range(k):
                if inv[t, j] >= 0:
                    acc += float(w[t, j]) * float(yf[inv[t, j], c])
            assert out["out"][t, c] == acc
    assert not out["out"][4].any()
    out2 = gather_reduce(y, True, inv, 2 * w)
    assert np.array_equal(out2["out"], 2 * out["out"])
    # float32 input path and sampling
    y32 = bf16_decode(y)
    out3 = gather_reduce(y32, False, inv, w, sample_tokens=[3, 9])
    assert np.array_equal(out3["out"], out["out"][[3, 9]])
