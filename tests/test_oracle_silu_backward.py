"""Pins of the oracle's SiLU*mul backward (oracle/quantize.py): torch
autograd of h = a * sigmoid(a) * b in float64, the closed forms at a = 0 and
for large |a|, and the bf16 rounding by torch's own cast."""

import numpy as np
import torch

from oracle.codec import bf16_decode
from oracle.quantize import silu_mul_backward, silu_mul_backward_f32
from workloads import to_bf16_bits


def _bits(rng, n, scale):
    return to_bf16_bits((rng.standard_normal(n) * scale).astype(np.float32))


def test_matches_float64_autograd_within_float32_rounding():
    rng = np.random.default_rng(1)
    n = 20000
    a = bf16_decode(_bits(rng, n, 4.0))
    b = bf16_decode(_bits(rng, n, 1.0))
    dh = bf16_decode(_bits(rng, n, 1e-2))
    da, db = silu_mul_backward_f32(a, b, dh)
    at = torch.tensor(a.astype(np.float64), requires_grad=True)
    bt = torch.tensor(b.astype(np.float64), requires_grad=True)
    h = at * torch.sigmoid(at) * bt
    h.backward(torch.tensor(dh.astype(np.float64)))
    ga, gb = at.grad.numpy(), bt.grad.numpy()
    # a handful of float32 roundings (the pinned exp is within ~2 ulp): relative 1e-6 of the
    # magnitudes of the factors involved
    sa = np.abs(dh.astype(np.float64) * b) * (1.0 + np.abs(a)) + 1e-30
    sb = np.abs(dh.astype(np.float64) * a) + 1e-30
    assert np.all(np.abs(da - ga) <= 2e-6 * sa), np.max(np.abs(da - ga) / sa)
    assert np.all(np.abs(db - gb) <= 2e-6 * sb), np.max(np.abs(db - gb) / sb)


def test_closed_forms():
    # a = 0: sigmoid = 1/2, silu = 0, silu' = 1/2 exactly
    da, db = silu_mul_backward_f32(np.float32(0.0), np.float32(3.0), np.float32(0.25))
    assert da == np.float32(0.375) and db == 0.0
    # large positive a: sigmoid rounds to 1, silu' = 1, silu = a
    da, db = silu_mul_backward_f32(np.float32(40.0), np.float32(2.0), np.float32(0.5))
    assert da == np.float32(1.0) and db == np.float32(20.0)
    # very negative a: both gradients vanish but stay finite
    da, db = silu_mul_backward_f32(np.float32(-100.0), np.float32(2.0), np.float32(0.5))
    assert np.isfinite(da) and np.isfinite(db) and abs(da) < 1e-30 and abs(db) < 1e-30


def test_bf16_outputs_are_torch_casts_of_the_float32_results():
    rng = np.random.default_rng(2)
    a, b, dh = _bits(rng, 5000, 4.0), _bits(rng, 5000, 1.0), _bits(rng, 5000, 1e-2)
    da_bits, db_bits = silu_mul_backward(a, b, dh)
    da, db = silu_mul_backward_f32(bf16_decode(a), bf16_decode(b), bf16_decode(dh))
    for got, f in ((da_bits, da), (db_bits, db)):
        ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(got, ref)
