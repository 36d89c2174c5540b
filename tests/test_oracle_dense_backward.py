"""Pin of the oracle's unquantized bf16 backward of the gated FFN (the
context reference for the gradient columns of "Support quantization for
tokamax gmm v2", table "relative_norm_diff Across All Cases"): against torch
autograd in float64 of the same layer without the bf16 roundings between
stages.  A dropped term, a wrong sign or a transposed operand shows up as an
O(1) difference; the roundings alone stay near 1e-2."""

import numpy as np
import torch

from oracle.codec import bf16_decode
from oracle.pipeline import dense_bf16_backward_reference, rel_norm_diff_f
from workloads import generate, scaled_config, to_bf16_bits


def _autograd(cfg, data, dout_bits):
    x = torch.tensor(bf16_decode(data["x"]).astype(np.float64), requires_grad=True)
    W = {n: torch.tensor(bf16_decode(w).astype(np.float64), requires_grad=True) for n, w in data["weights"].items()}
    dout = torch.tensor(bf16_decode(dout_bits).astype(np.float64))
    ids = torch.tensor(data["ids"].astype(np.int64))
    wts = torch.tensor(data["topk_w"].astype(np.float64))
    out = torch.zeros(cfg.T, cfg.H, dtype=torch.float64)
    for j in range(cfg.k):
        for t in range(cfg.T):
            g = int(ids[t, j]) - cfg.group_offset
            if not 0 <= g < cfg.E_loc:
                continue
            a = x[t] @ W["wi_0"][g]
            b = x[t] @ W["wi_1"][g]
            y = (torch.nn.functional.silu(a) * b) @ W["wo"][g]
            out[t] = out[t] + wts[t, j] * y
    (out * dout).sum().backward()
    return x.grad.numpy(), W["wi_0"].grad.numpy(), W["wi_1"].grad.numpy(), W["wo"].grad.numpy()


def test_dense_backward_matches_autograd_up_to_bf16_roundings():
    cfg = scaled_config(2, T=24, H=64, E=6, k=2, I=48, group_offset=1, num_local_experts=4)
    data = generate(cfg)
    rng = np.random.default_rng(3)
    dout = to_bf16_bits(rng.standard_normal((cfg.T, cfg.H)).astype(np.float32))
    dx, dw0, dw1, dwo = dense_bf16_backward_reference(cfg, data, dout)
    gx, g0, g1, go = _autograd(cfg, data, dout)
    for name, got, ref in (("dx", bf16_decode(dx), gx), ("dw0", dw0, g0), ("dw1", dw1, g1), ("dwo", dwo, go)):
        r = rel_norm_diff_f(got, ref)
        assert r < 2e-2, (name, r)
    # a token routed to no local expert gets no gradient
    none = ~np.isin(data["ids"], np.arange(1, 5)).any(axis=1)
    if none.any():
        assert not bf16_decode(dx)[none].any()
