"""Seeded synthetic workloads for the fp8 MoE grouped-matmul path.

This module only draws inputs: routing, activations, weights and gradients in
bfloat16.  It holds none of the path's arithmetic (no quantization, no sort,
no matmul): both the HIP library's tests/benchmark and the CPU oracle take
their inputs from here.

The pages run their accuracy comparison on unit-test shapes they do not print
("Support quantization for tokamax gmm v2", tables "relative_norm_diff
Across All Cases" and "max_abs_diff Across All Cases"); these five
configurations stand in for them:

1. tiny MoE up-projection: T=256, H=512, E=8, top-2, N=1024, per-channel
   weight scales, per-token dynamic activation scales;
2. full gated MoE FFN forward: T=4096, H=2048, E=64, top-8, I=768;
3. config 1 shapes with Zipf-skewed routing (several empty experts),
   blockwise [E, K/128, 1, N] weight scales, plus a static-scale variant;
4. one GPU's expert slice of a large layer: T=8192, H=7168, E=256, top-8,
   I=2048, 32 local experts from group_offset 64, 128x128 weight blocks,
   1% outlier token rows scaled by 50;
5. MoE backward: T=8192, H=4096, E=64, top-4, I=1536, uniform routing,
   dY ~ N(0, 1e-3) in sorted-row space, static activation/weight scales.

A sixth, derived workload carries config 3's structure to the large-matmul
shapes of config 4, so the ragged tile scheduler is measured where matrix-core
rate means something: T=1024 tokens, H=7168, E=32 experts (all local), top-8
(8192 routed rows, as config 4's local slice), N=2048, the same Zipf-skewed
routing (15 experts receive 2..1024 rows, 17 receive none), [E, K/128, 1, N]
weight scales, and the static-scale variant.

Generator: every tensor has its own stream, ``numpy.random.default_rng([1000
+ c, s])`` with s = 0 routing (logits, then the Zipf rank permutation), 1
activations x, 2 outlier rows, 3 dY, 10 + i the i-th weight (wi_0, wi_1, wo,
or the single up weight), so that any subset can be drawn on its own; every
float32 draw is rounded to bfloat16 by torch's CPU cast (round to nearest
even).
"""

from dataclasses import dataclass, field
import math

import numpy as np
import torch

# Static scales of the fp8_static_wa scheme ("Support quantization for tokamax
# gmm v2": fixed weight scale + fixed activation scale).  The activation value
# maps 4 standard deviations of N(0,1) to the largest e4m3 value; the weight
# value does the same for N(0, 0.02).
STATIC_ACT_SCALE = float(np.float32(4.0) / np.float32(448.0))
STATIC_WEIGHT_SCALE = float(np.float32(0.08) / np.float32(448.0))

ZIPF_S = 1.2
ZIPF_STRENGTH = 4.0


@dataclass
class MoEConfig:
    cid: int
    name: str
    T: int
    H: int
    E: int
    k: int
    I: int                        # expert intermediate size (config 1: N of the up-projection)
    pipeline: str                 # "up", "ffn" or "bwd"
    routing: str = "softmax"      # "softmax", "zipf", "uniform"
    group_offset: int = 0
    num_local_experts: int = -1
    weight_block_k: int = 0       # 0: per-channel (one K block); else K rows per block
    weight_block_n: int = 1       # columns per scale block (1 = per channel)
    outlier_frac: float = 0.0
    outlier_mult: float = 1.0
    static: bool = False
    extra: dict = field(default_factory=dict)

    @property
    def E_loc(self):
        return self.E if self.num_local_experts < 0 else self.num_local_experts

    @property
    def M(self):
        return self.T * self.k

    def weight_shapes(self):
        """(name, [E_loc, K, N]) of each weight, in draw order."""
        if self.pipeline == "up":
            return [("w_up", (self.E_loc, self.H, self.I))]
        if self.pipeline == "ffn":
            return [("wi_0", (self.E_loc, self.H, self.I)), ("wi_1", (self.E_loc, self.H, self.I)),
                    ("wo", (self.E_loc, self.I, self.H))]
        return [("w_up", (self.E_loc, self.H, self.I))]

    def scale_blocks(self, K, N):
        """(kb, nb) of the [E, kb, 1, nb] weight-scale tensor of a [K, N] weight."""
        kb = 1 if self.weight_block_k == 0 else K // self.weight_block_k
        nb = N if self.weight_block_n == 1 else N // self.weight_block_n
        return kb, nb


CONFIGS = {
    1: MoEConfig(1, "tiny-up-proj", T=256, H=512, E=8, k=2, I=1024, pipeline="up"),
    2: MoEConfig(2, "gated-ffn-fwd", T=4096, H=2048, E=64, k=8, I=768, pipeline="ffn"),
    3: MoEConfig(3, "tiny-up-proj-zipf-blockwise", T=256, H=512, E=8, k=2, I=1024, pipeline="up",
                 routing="zipf", weight_block_k=128),
    4: MoEConfig(4, "ep-slice-ffn-fwd", T=8192, H=7168, E=256, k=8, I=2048, pipeline="ffn",
                 group_offset=64, num_local_experts=32, weight_block_k=128, weight_block_n=128,
                 outlier_frac=0.01, outlier_mult=50.0),
    5: MoEConfig(5, "moe-bwd", T=8192, H=4096, E=64, k=4, I=1536, pipeline="bwd",
                 routing="uniform", static=True),
    6: MoEConfig(6, "skewed-up-proj-large", T=1024, H=7168, E=32, k=8, I=2048, pipeline="up",
                 routing="zipf", weight_block_k=128),
}


def scaled_config(cid, **over):
    """A copy of config ``cid`` with fields replaced (small parity cases)."""
    base = CONFIGS[cid]
    d = dict(base.__dict__)
    d.update(over)
    d["extra"] = dict(base.extra)
    return MoEConfig(**d)


def to_bf16_bits(a_f32: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16) by torch's CPU cast."""
    t = torch.from_numpy(np.ascontiguousarray(a_f32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def _route_softmax(logits, k):
    z = logits.astype(np.float64)
    z = z - z.max(axis=1, keepdims=True)
    p = np.exp(z)
    p /= p.sum(axis=1, keepdims=True)
    order = np.argsort(-p, axis=1, kind="stable")[:, :k]       # ties -> lower expert id
    w = np.take_along_axis(p, order, axis=1).astype(np.float32)
    return order.astype(np.int32), w


def _rng(cfg, seed, stream):
    return np.random.default_rng([1000 + cfg.cid if seed is None else seed, stream])


def generate(cfg: MoEConfig, seed=None, with_weights=True):
    """Draw one workload.  Returns a dict of numpy arrays:

    ids int32 [T, k], topk_w float32 [T, k], x uint16 [T, H] (bf16 bits),
    weights {name: uint16 [E_loc, K, N]}, and for the backward config
    dy uint16 [T*k, I].  ``with_weights`` is True (all weights), False (none)
    or a collection of weight names.
    """
    T, H, E, k = cfg.T, cfg.H, cfg.E, cfg.k
    out = {"cfg": cfg}
    rng = _rng(cfg, seed, 0)
    if cfg.routing == "uniform":
        ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32) if T else \
            np.zeros((0, k), np.int32)
        out["ids"], out["topk_w"] = ids, np.ones((T, k), np.float32)
    else:
        logits = rng.standard_normal((T, E))
        if cfg.routing == "zipf":
            rank = 1 + rng.permutation(E)
            logits = logits - ZIPF_STRENGTH * ZIPF_S * np.log(rank)[None, :]
        out["ids"], out["topk_w"] = _route_softmax(logits, k) if T else \
            (np.zeros((0, k), np.int32), np.zeros((0, k), np.float32))
        if cfg.routing == "zipf" and T >= 64:
            empty = int((np.bincount(out["ids"].ravel(), minlength=E) == 0).sum())
            assert empty >= 2, "Zipf-skewed routing is expected to leave experts empty"
    x = _rng(cfg, seed, 1).standard_normal((T, H), dtype=np.float32)
    if cfg.outlier_frac > 0 and T:
        n_out = int(round(cfg.outlier_frac * T))
        rows = _rng(cfg, seed, 2).choice(T, n_out, replace=False)
        x[rows] *= np.float32(cfg.outlier_mult)
        out["outlier_rows"] = np.sort(rows)
    out["x"] = to_bf16_bits(x)
    del x
    weights = {}
    for i, (name, shp) in enumerate(cfg.weight_shapes()):
        if with_weights is True or (with_weights and name in with_weights):
            w = _rng(cfg, seed, 10 + i).standard_normal(shp, dtype=np.float32)
            w *= np.float32(0.02)
            weights[name] = to_bf16_bits(w)
            del w
    out["weights"] = weights
    if cfg.pipeline == "bwd":
        dy = _rng(cfg, seed, 3).standard_normal((T * k, cfg.I), dtype=np.float32)
        dy *= np.float32(1e-3)
        out["dy"] = to_bf16_bits(dy)
    return out


def m_cap_for(cfg: MoEConfig, n_local: int, align: int = 256) -> int:
    """Row capacity of the sorted buffers: all routed rows when every expert
    is local, else the realised local count rounded up to ``align``."""
    if cfg.E_loc == cfg.E:
        return cfg.M
    return int(math.ceil(max(n_local, 1) / align) * align)
