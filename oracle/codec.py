"""Number formats of the path: OCP float8 e4m3fn and bfloat16.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages quantize to ``float8_e4m3fn`` ("Keep qwix out of tpu-inference's
fused MoE kernel and pre-quantize weights", "Changes in this PR"; the Mosaic
error message in its description names the type ``f8E4M3FN``).  That is the
OCP 8-bit format with 4 exponent bits (bias 7), 3 mantissa bits, no
infinities, a single NaN pattern per sign (S.1111.111), largest finite value
448 and subnormals down to 2**-9.  It is not the "fnuz" variant.

The pages do not state the rounding mode of the cast; this oracle rounds to
nearest, ties to even, keeps the sign of a result that rounds to zero and
keeps subnormals (no flush).  Values must be finite and already clipped to
[-448, 448] (the saturating clip lives in the quantizers).
"""

import numpy as np

E4M3_MAX = 448.0
E4M3_MIN_NORMAL_EXP = -6          # smallest normal: 2**-6
E4M3_SUBNORMAL_QUANTUM = 2.0 ** -9


def _e4m3_value_table() -> np.ndarray:
    """Decoded value of every one of the 256 codes (float64, NaN for S.1111.111)."""
    vals = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            vals[code] = np.nan
        elif e == 0:
            vals[code] = sign * (m / 8.0) * 2.0 ** -6
        else:
            vals[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


_E4M3_TABLE = _e4m3_value_table()


def e4m3_decode(codes) -> np.ndarray:
    """Exact float64 value of each e4m3fn byte."""
    return _E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_rne(v) -> np.ndarray:
    """Round finite float32 values in [-448, 448] to e4m3fn codes (uint8).

    Steps: take the magnitude a; its binary exponent ex = floor(log2 a); the
    spacing of e4m3 values around a is 2**(ex-3) for normal numbers and
    2**-9 below 2**-6; divide by that spacing (exact: a power of two), round
    half to even, and encode the resulting multiple of the spacing.
    """
    v = np.asarray(v, dtype=np.float32)
    if not np.all(np.isfinite(v)):
        raise ValueError("e4m3_rne: non-finite input")
    if np.any(np.abs(v) > E4M3_MAX):
        raise ValueError("e4m3_rne: input outside [-448, 448]; clip first")
    sign = np.signbit(v).astype(np.uint8) << 7
    a = np.abs(v.astype(np.float64))
    _, fe = np.frexp(a)                 # a = f * 2**fe, f in [0.5, 1)
    ex = fe.astype(np.int64) - 1        # floor(log2 a) for a > 0
    quantum = np.where(ex >= E4M3_MIN_NORMAL_EXP, np.ldexp(1.0, ex - 3), E4M3_SUBNORMAL_QUANTUM)
    n = np.rint(a / quantum)            # round half to even
    w = n * quantum                     # rounded magnitude, exact in float64
    code = np.zeros(v.shape, dtype=np.int64)
    sub = (w > 0) & (w < 2.0 ** E4M3_MIN_NORMAL_EXP)
    code[sub] = (w[sub] / E4M3_SUBNORMAL_QUANTUM).astype(np.int64)
    nrm = w >= 2.0 ** E4M3_MIN_NORMAL_EXP
    _, we = np.frexp(w[nrm])
    e_unb = we.astype(np.int64) - 1
    mant = (np.ldexp(w[nrm], -e_unb) - 1.0) * 8.0
    code[nrm] = ((e_unb + 7) << 3) | mant.astype(np.int64)
    return (code.astype(np.uint8) | sign).astype(np.uint8)


def bf16_decode(bits) -> np.ndarray:
    """bfloat16 bit patterns (uint16) to float32, exactly."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def bf16_rne_from_f32(x) -> np.ndarray:
    """float32 to bfloat16 bit patterns, round to nearest, ties to even.

    bfloat16 is the upper half of the float32 encoding; rounding adds half of
    the dropped field's range minus one, plus the kept field's lowest bit (so
    that exact halves go to the even neighbour), then truncates.  NaN maps to
    the quiet NaN of the same sign.
    """
    x = np.asarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    lsb = (bits >> np.uint64(16)) & np.uint64(1)
    rounded = ((bits + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(x)
    if np.any(nan):
        rounded = rounded.copy()
        rounded[nan] = ((bits[nan] >> np.uint64(16)).astype(np.uint16) & np.uint16(0x8000)) | np.uint16(0x7FC0)
    return rounded


def bf16_rne_from_f64(x) -> np.ndarray:
    """float64 to bfloat16 through float32 (two round-to-nearest-even steps)."""
    return bf16_rne_from_f32(np.asarray(x, dtype=np.float64).astype(np.float32))
