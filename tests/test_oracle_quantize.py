"""Pins of the oracle's quantizers and of the pinned SiLU recipe."""

from fractions import Fraction

import numpy as np
import pytest

from oracle.codec import bf16_decode, e4m3_decode, e4m3_rne
from oracle.quantize import (EXP_C1, EXP_C2, SCALE_ROW_DYNAMIC, SCALE_TENSOR_DYNAMIC,
                             SCALE_TENSOR_STATIC, pinned_exp_f32, quantize_rows,
                             quantize_weights, silu_mul_f32)
from workloads import to_bf16_bits

F32_INF = np.float32(np.inf)


def rn32_div(x, s):
    """Correctly rounded float32 quotient from exact rational arithmetic."""
    q = Fraction(float(x)) / Fraction(float(s))
    if q == 0:          # IEEE: the sign of a zero quotient is the xor of the signs
        neg = bool(np.signbit(np.float32(x))) != bool(np.signbit(np.float32(s)))
        return np.float32(-0.0) if neg else np.float32(0.0)
    a = np.float32(float(q))
    cands = [np.nextafter(a, -F32_INF), a, np.nextafter(a, F32_INF)]
    best = None
    for c in cands:
        d = abs(Fraction(float(c)) - q)
        even = (np.array(c, np.float32).view(np.uint32) & 1) == 0
        if best is None or d < best[0] or (d == best[0] and even):
            best = (d, c)
    return np.float32(best[1])


def nearest_e4m3_code(v):
    x = Fraction(float(v))
    best = None
    for c in range(127):
        val = Fraction(float(e4m3_decode(np.uint8(c))))
        d = abs(abs(x) - val)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return best[1] | (0x80 if np.signbit(np.float32(v)) else 0)


def _bf16(a):
    return to_bf16_bits(np.asarray(a, dtype=np.float32))


def test_row_quantize_matches_exact_rational_bruteforce():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 24)).astype(np.float32)
    x[1] *= 1e-3
    x[2, :] = 0.0
    x[3, 5] = -0.0
    xb = _bf16(x)
    q, s, amax = quantize_rows(xb, SCALE_ROW_DYNAMIC)
    xf = bf16_decode(xb)
    for r in range(xf.shape[0]):
        am = max(abs(float(v)) for v in xf[r])
        sr = np.float32(1.0) if am == 0 else rn32_div(am, 448.0)
        assert s[r].view(np.uint32) == sr.view(np.uint32)
        assert amax[r] == am
        for c in range(xf.shape[1]):
            v = rn32_div(xf[r, c], sr)
            v = min(max(v, np.float32(-448)), np.float32(448))
            assert q[r, c] == nearest_e4m3_code(v), (r, c)


def test_static_quantize_saturates_and_matches_bruteforce():
    s_static = float(np.float32(4.0) / np.float32(448.0))
    x = np.array([[0.0, 1.0, -3.9, 3.95, 4.0, 5.0, -100.0, 3.857]], np.float32)
    xb = _bf16(x)
    q, s, _ = quantize_rows(xb, SCALE_TENSOR_STATIC, static_scale=s_static)
    assert s.shape == (1,) and s[0] == np.float32(s_static)
    xf = bf16_decode(xb)[0]
    for c in range(x.shape[1]):
        v = rn32_div(xf[c], np.float32(s_static))
        v = min(max(v, np.float32(-448)), np.float32(448))
        assert q[0, c] == nearest_e4m3_code(v)
    # |x/s| >= 432 (the midpoint 432 rounds to the even code 448) <=> code +-448
    big = np.abs((bf16_decode(xb) / np.float32(s_static)).astype(np.float32)) >= 432
    assert np.array_equal(np.isin(q, [0x7E, 0xFE]), big)


def test_every_nonzero_row_reaches_448_and_error_bound():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((64, 256)).astype(np.float32) * rng.uniform(1e-3, 1e3, (64, 1)).astype(np.float32)
    xb = _bf16(x)
    q, s, _ = quantize_rows(xb, SCALE_ROW_DYNAMIC)
    assert np.all(np.any(np.isin(q, [0x7E, 0xFE]), axis=1))
    xf = bf16_decode(xb).astype(np.float64)
    v = xf / s[:, None].astype(np.float64)
    d = e4m3_decode(q)
    # half the e4m3 spacing at |v| (2^-10 below 2^-6), plus the float32 divide's half-ulp
    ex = np.floor(np.log2(np.maximum(np.abs(v), 2.0 ** -6)))
    half_spacing = np.where(np.abs(v) >= 2.0 ** -6, 2.0 ** (ex - 4), 2.0 ** -10)
    assert np.all(np.abs(v - d) <= half_spacing * (1 + 2.0 ** -20) + np.abs(v) * 2.0 ** -24)


def test_tensor_dynamic_scale_is_global_absmax():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((16, 32)).astype(np.float32)
    x[7, 3] = 9.0
    xb = _bf16(x)
    q, s, amax = quantize_rows(xb, SCALE_TENSOR_DYNAMIC)
    qr, sr, _ = quantize_rows(xb[7:8], SCALE_ROW_DYNAMIC)
    assert s.shape == (1,) and s[0] == sr[0] == rn32_div(9.0, 448.0)
    assert np.array_equal(q[7], qr[0])
    assert np.array_equal(amax, np.abs(bf16_decode(xb)).max(axis=1))


def test_quantize_then_gather_equals_gather_then_quantize():
    # "Quantize activations before EP all gather", Testing strategy: moving the
    # quantization before the gather must not change the math.
    rng = np.random.default_rng(6)
    xb = _bf16(rng.standard_normal((40, 64)).astype(np.float32))
    idx = rng.integers(0, 40, 100)
    q, s, _ = quantize_rows(xb, SCALE_ROW_DYNAMIC)
    q2, s2, _ = quantize_rows(xb[idx], SCALE_ROW_DYNAMIC)
    assert np.array_equal(q[idx], q2)
    assert np.array_equal(s[idx].view(np.uint32), s2.view(np.uint32))


def test_zero_rows_and_empty_inputs():
    xb = _bf16(np.zeros((3, 16), np.float32))
    xb[1, 2] = 0x8000              # -0.0
    q, s, _ = quantize_rows(xb, SCALE_ROW_DYNAMIC)
    assert np.all(s == 1.0)
    assert q[1, 2] == 0x80 and np.count_nonzero(q) == 1
    q, s, _ = quantize_rows(np.zeros((0, 16), np.uint16), SCALE_TENSOR_DYNAMIC)
    assert q.shape == (0, 16) and s[0] == 1.0


def test_pinned_exp_constants_and_accuracy():
    # Cody-Waite split: C1 has at most 16 significant bits, C1 + C2 = ln 2 closely
    m, _ = np.frexp(float(EXP_C1))
    assert (m * 2 ** 16) == int(m * 2 ** 16)
    assert abs(float(EXP_C1) + float(EXP_C2) - np.log(2.0)) < 2.0 ** -40
    assert pinned_exp_f32(np.float32(0.0)) == np.float32(1.0)
    x = np.linspace(-87.0, 88.0, 200001, dtype=np.float32)
    e = pinned_exp_f32(x).astype(np.float64)
    ref = np.exp(x.astype(np.float64))
    ulp = np.spacing(ref.astype(np.float32)).astype(np.float64)
    assert np.max(np.abs(e - ref) / ulp) <= 2.0
    # clamped outside [-87, 88]
    assert pinned_exp_f32(np.float32(-200.0)) == pinned_exp_f32(np.float32(-87.0))
    assert np.isfinite(pinned_exp_f32(np.float32(1000.0)))


def test_silu_mul_close_to_float64():
    rng = np.random.default_rng(7)
    a = (rng.standard_normal(100000) * 4).astype(np.float32)
    b = rng.standard_normal(100000).astype(np.float32)
    h = silu_mul_f32(a, b).astype(np.float64)
    a64, b64 = a.astype(np.float64), b.astype(np.float64)
    ref = a64 / (1.0 + np.exp(-a64)) * b64
    ulp = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
    assert np.max(np.abs(h - ref) / ulp) <= 4.0
    assert silu_mul_f32(np.float32(0.0), np.float32(3.0)) == 0.0


def test_silu_mul_quantize_is_row_quantize_of_h():
    rng = np.random.default_rng(8)
    a = _bf16(rng.standard_normal((6, 32)).astype(np.float32))
    b = _bf16(rng.standard_normal((6, 32)).astype(np.float32))
    q, s, _ = quantize_rows(a, SCALE_ROW_DYNAMIC, x_up_bits=b)
    h = silu_mul_f32(bf16_decode(a), bf16_decode(b))
    for r in range(6):
        am = float(np.max(np.abs(h[r])))
        sr = rn32_div(am, 448.0)
        assert s[r] == sr
        for c in range(32):
            v = min(max(rn32_div(h[r, c], sr), np.float32(-448)), np.float32(448))
            assert q[r, c] == nearest_e4m3_code(v)


@pytest.mark.parametrize("kb,nb", [(1, 6), (2, 6), (2, 3), (1, 1)])
def test_weight_quantizer_blocks_bruteforce(kb, nb):
    rng = np.random.default_rng(9 + kb + nb)
    E, K, N = 2, 8, 6
    w = _bf16(rng.standard_normal((E, K, N)).astype(np.float32) * 0.02)
    w[1, 0:K // kb, 0:N // nb] = 0           # an all-zero block (or more)
    q, s = quantize_weights(w, kb, nb)
    assert s.shape == (E, kb, 1, nb)
    wf = bf16_decode(w)
    bk, bn = K // kb, N // nb
    for e in range(E):
        for b in range(kb):
            for c in range(nb):
                blk = wf[e, b * bk:(b + 1) * bk, c * bn:(c + 1) * bn]
                am = max(abs(float(v)) for v in blk.ravel())
                sr = np.float32(1.0) if am == 0 else rn32_div(am, 448.0)
                assert s[e, b, 0, c] == sr
                for i in range(bk):
                    for j in range(bn):
                        v = rn32_div(blk[i, j], sr)
                        assert q[e, b * bk + i, c * bn + j] == nearest_e4m3_code(v)


def test_weight_quantizer_static_scale():
    rng = np.random.default_rng(10)
    w = _bf16(rng.standard_normal((2, 4, 4)).astype(np.float32) * 0.02)
    st = float(np.float32(0.08) / np.float32(448))
    q, s = quantize_weights(w, 1, 1, static_scale=st)
    assert np.all(s == np.float32(st))
    v = np.clip((bf16_decode(w) / np.float32(st)).astype(np.float32), -448, 448)
    assert np.array_equal(q, e4m3_rne(v))


def test_tensor_scale_from_row_maxima_is_the_tensor_dynamic_result():
    """The tensor scale from a row-mode call's row maxima gives the tensor-dynamic
    codes and scale bit for bit (max is exact in any grouping), also for the
    SiLU*mul activation; rows of zeros and an all-zero matrix keep scale 1."""
    from oracle.quantize import SCALE_TENSOR_FROM_ROW_AMAX
    rng = np.random.default_rng(12)
    x = to_bf16_bits((rng.standard_normal((40, 96)) * 2.0).astype(np.float32))
    x[3] = 0
    up = to_bf16_bits(rng.standard_normal((40, 96)).astype(np.float32))
    for xu in (None, up):
        _, _, ra = quantize_rows(x, SCALE_ROW_DYNAMIC, x_up_bits=xu)
        q1, s1, _ = quantize_rows(x, SCALE_TENSOR_DYNAMIC, x_up_bits=xu)
        q2, s2, _ = quantize_rows(x, SCALE_TENSOR_FROM_ROW_AMAX, x_up_bits=xu, row_amax_in=ra)
        assert np.array_equal(q1, q2) and np.array_equal(s1.view(np.uint32), s2.view(np.uint32))
    z = np.zeros((5, 32), np.uint16)
    q, s, _ = quantize_rows(z, SCALE_TENSOR_FROM_ROW_AMAX, row_amax_in=np.zeros(5, np.float32))
    assert s[0] == 1.0 and not q.any()
