"""Pins of the oracle's number formats (e4m3fn, bfloat16) against the OCP
format definition, torch's CPU casts and brute-force nearest search."""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle.codec import (E4M3_MAX, bf16_decode, bf16_rne_from_f32, e4m3_decode, e4m3_rne)


def _finite_codes():
    return np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)


def test_e4m3_value_set_matches_format_definition():
    vals = e4m3_decode(np.arange(256, dtype=np.uint8))
    # OCP e4m3fn: NaN only at S.1111.111, max 448, min normal 2^-6, min subnormal 2^-9.
    assert np.isnan(vals[0x7F]) and np.isnan(vals[0xFF])
    assert np.count_nonzero(np.isnan(vals)) == 2
    assert vals[0x7E] == 448.0 and vals[0xFE] == -448.0
    assert vals[0x08] == 2.0 ** -6 and vals[0x01] == 2.0 ** -9
    assert vals[0x38] == 1.0 and vals[0x00] == 0.0 and np.signbit(vals[0x80])
    fin = vals[~np.isnan(vals)]
    assert np.max(np.abs(fin)) == E4M3_MAX
    # 126 distinct positive values, symmetric set
    pos = np.unique(fin[fin > 0])
    assert len(pos) == 126
    assert np.array_equal(np.unique(-fin[fin < 0]), pos)
    # spacing: 2^-9 below 2^-6, then 8 values per binade with spacing 2^(e-3)
    for e in range(-6, 9):
        binade = pos[(pos >= 2.0 ** e) & (pos < 2.0 ** (e + 1))]
        expect = 8 if e < 8 else 7          # 2^8 binade stops at 448 (1.75 * 2^8)
        assert len(binade) == expect
        assert np.allclose(np.diff(binade), 2.0 ** (e - 3))


def test_e4m3_decode_matches_torch():
    codes = _finite_codes()
    t = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(e4m3_decode(codes), t)


def test_e4m3_round_trip_every_finite_value():
    codes = _finite_codes()
    vals = e4m3_decode(codes).astype(np.float32)
    assert np.array_equal(e4m3_rne(vals), codes)


def test_e4m3_named_probes():
    cases = [(1.0625, 0x38), (1.1875, 0x3A), (2.0 ** -10, 0x00), (3 * 2.0 ** -11, 0x01),
             (448.0, 0x7E), (-448.0, 0xFE), (432.0, 0x7E), (431.0, 0x7D), (-1e-9, 0x80),
             (-0.0, 0x80), (0.0, 0x00), (2.0 ** -6 - 2.0 ** -10, 0x08),
             (7 * 2.0 ** -9 + 2.0 ** -10, 0x08)]
    for v, c in cases:
        assert int(e4m3_rne(np.float32(v))) == c, (v, hex(c))


def _nearest_even_bruteforce(v):
    """Nearest e4m3 value by exhaustive search over the value set; ties to
    the code with an even mantissa field; zero keeps the input's sign."""
    x = Fraction(float(v))
    best = None
    for c in range(128):
        if c == 0x7F:
            continue
        val = Fraction(float(e4m3_decode(np.uint8(c))))
        d = abs(abs(x) - val)
        if best is None or d < best[0] or (d == best[0] and (c & 1) == 0):
            best = (d, c)
    code = best[1]
    if np.signbit(np.float32(v)):
        code |= 0x80
    return code


def test_e4m3_rne_matches_bruteforce_nearest_search():
    rng = np.random.default_rng(1)
    v = np.concatenate([
        rng.uniform(-448, 448, 300),
        rng.standard_normal(300) * 4.0,
        rng.uniform(-2.0 ** -5, 2.0 ** -5, 300),
    ]).astype(np.float32)
    got = e4m3_rne(v)
    for x, g in zip(v, got):
        assert int(g) == _nearest_even_bruteforce(x), x


def test_e4m3_tie_midpoints_and_neighbours():
    vals = np.unique(np.abs(e4m3_decode(_finite_codes())))     # +0.0 first
    for lo, hi in zip(vals[:-1], vals[1:]):
        mid = np.float32((lo + hi) / 2)            # exact in float32
        assert float(mid) == (lo + hi) / 2
        lo_c, hi_c = int(e4m3_rne(np.float32(lo))), int(e4m3_rne(np.float32(hi)))
        even = lo_c if lo_c % 2 == 0 else hi_c
        assert int(e4m3_rne(mid)) == even
        assert int(e4m3_rne(np.nextafter(mid, np.float32(0)))) == lo_c
        assert int(e4m3_rne(np.nextafter(mid, np.float32(1e9)))) == hi_c
        assert int(e4m3_rne(-mid)) == even | 0x80


def test_e4m3_rne_matches_torch_cast_on_every_bf16_value():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = bf16_decode(bits)
    f = f[np.isfinite(f)]
    f = np.clip(f, -E4M3_MAX, E4M3_MAX).astype(np.float32)
    ours = e4m3_rne(f)
    theirs = torch.from_numpy(f.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, theirs)


def test_e4m3_rejects_unclipped_and_nonfinite():
    with pytest.raises(ValueError):
        e4m3_rne(np.float32(449.0))
    with pytest.raises(ValueError):
        e4m3_rne(np.float32(np.nan))


def test_bf16_round_trip_and_torch_cast():
    rng = np.random.default_rng(2)
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32) * 10,
                        rng.uniform(-1e-38, 1e-38, 2000).astype(np.float32),
                        np.array([3.3895314e38, -3.3895314e38, 0.0, -0.0], np.float32)])
    # exact ties: bf16 value + half an ulp
    b = rng.integers(0, 0x7F00, 2000).astype(np.uint32)
    ties = ((b << 16) | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, -ties])
    ours = bf16_rne_from_f32(x)
    theirs = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)
    bits = np.arange(0, 65536, 7, dtype=np.uint32).astype(np.uint16)
    f = bf16_decode(bits)
    keep = np.isfinite(f)
    assert np.array_equal(bf16_rne_from_f32(f[keep]), bits[keep])
