"""Pins of the oracle's gather-reduce backward (oracle/gather_reduce.py):
torch's automatic differentiation of the forward combine in float64, torch's
own float32 product and bfloat16 cast for the rounding, the adjoint identity
with the forward oracle, and the k = 1 un-sort special case."""

import numpy as np
import pytest
import torch

from oracle.codec import bf16_decode
from oracle.gather_reduce import gather_reduce, gather_reduce_backward
from oracle.sort import sort_by_expert
from workloads import to_bf16_bits


def _case(T, k, E, g0, El, N, seed, extra=8):
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    srt = sort_by_expert(ids, E, g0, El)
    n = int(srt["n"])
    m_cap = n + extra
    inv = srt["inv_pos"].reshape(T, k)
    y = to_bf16_bits(rng.standard_normal((m_cap, N)).astype(np.float32))
    dout = to_bf16_bits((rng.standard_normal((T, N)) * 1e-2).astype(np.float32))
    w = rng.uniform(0.0, 1.0, (T, k)).astype(np.float32)
    return inv, y, dout, w, n, m_cap


@pytest.mark.parametrize("T,k,E,g0,El,N", [(40, 2, 8, 0, 8, 64), (33, 4, 16, 4, 8, 128), (17, 8, 64, 0, 64, 32)])
def test_backward_matches_autograd_of_the_forward(T, k, E, g0, El, N):
    inv, y, dout, w, n, m_cap = _case(T, k, E, g0, El, N, T + N)
    o = gather_reduce_backward(dout, y, inv, w, m_cap, n)
    yt = torch.tensor(bf16_decode(y).astype(np.float64), requires_grad=True)
    wt = torch.tensor(w.astype(np.float64), requires_grad=True)
    invt = torch.tensor(inv.astype(np.int64))
    mask = (invt >= 0).to(torch.float64)
    rows = yt.index_select(0, invt.clamp(min=0).reshape(-1)).reshape(T, k, N)
    out = (wt.unsqueeze(-1) * mask.unsqueeze(-1) * rows).sum(dim=1)
    dt = torch.tensor(bf16_decode(dout).astype(np.float64))
    (out * dt).sum().backward()
    assert np.array_equal(o["dy64"], yt.grad.numpy())           # single exact products: equal bits
    np.testing.assert_allclose(o["dw64"], wt.grad.numpy() * mask.numpy(), rtol=1e-12, atol=1e-300)
    assert (o["dw"][inv < 0] == 0).all()
    assert not o["dy64"][n:].any()


def test_dy_rounding_is_torch_float32_product_then_bfloat16():
    inv, y, dout, w, n, m_cap = _case(64, 4, 8, 2, 5, 96, 3)
    o = gather_reduce_backward(dout, y, inv, w, m_cap, n)
    d32 = torch.from_numpy(bf16_decode(dout).astype(np.float32))
    for t in range(inv.shape[0]):
        for j in range(inv.shape[1]):
            r = inv[t, j]
            if r < 0:
                continue
            ref = (torch.tensor(w[t, j], dtype=torch.float32) * d32[t]).to(torch.bfloat16)
            assert np.array_equal(o["dy"][r], ref.view(torch.int16).numpy().view(np.uint16))


def test_adjoint_identity_with_the_forward_oracle():
    """<gather_reduce(y, w), dout> = <y, dy> = <w, dw>, all in float64."""
    inv, y, dout, w, n, m_cap = _case(50, 3, 12, 3, 6, 80, 11)
    o = gather_reduce_backward(dout, y, inv, w, m_cap, n)
    fwd = gather_reduce(y, True, inv, w)["out"]
    lhs = float(np.sum(fwd * bf16_decode(dout).astype(np.float64)))
    via_y = float(np.sum(bf16_decode(y).astype(np.float64) * o["dy64"]))
    via_w = float(np.sum(w.astype(np.float64) * o["dw64"]))
    assert lhs == pytest.approx(via_y, rel=1e-12)
    assert lhs == pytest.approx(via_w, rel=1e-12)


def test_top1_unit_weights_is_the_exact_unsort():
    T, N = 30, 48
    inv, y, dout, _, n, m_cap = _case(T, 1, 4, 0, 4, N, 5)
    w = np.ones((T, 1), np.float32)
    o = gather_reduce_backward(dout, y, inv, w, m_cap, n)
    assert np.array_equal(o["dy"][inv[:, 0]], dout)                 # bitwise: w = 1 leaves bf16 values exact
    # dw[t] is the row dot product: torch's float64 matmul of the gathered rows
    yt = torch.from_numpy(bf16_decode(y).astype(np.float64))[torch.from_numpy(inv[:, 0].astype(np.int64))]
    dt = torch.from_numpy(bf16_decode(dout).astype(np.float64))
    np.testing.assert_allclose(o["dw64"][:, 0], (dt.unsqueeze(1) @ yt.unsqueeze(2)).reshape(-1).numpy(), rtol=1e-12)
    assert not o["dy"][n:].any()
