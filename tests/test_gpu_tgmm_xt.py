"""The sort's row gather written in the weight-gradient product's transposed
layout (moe_sort_gather_transposed) and the product on it (moe_tgmm_fp8_xt):
the layout bit for bit against the oracle's sorted rows laid out by hand,
and the product bit for bit against moe_tgmm_fp8 on the sorted rows."""

import numpy as np
import pytest
import torch

import moe_fp8_grouped_amd as m
from oracle.gmm import tgmm
from oracle.quantize import SCALE_TENSOR_DYNAMIC, SCALE_TENSOR_STATIC, quantize_rows
from oracle.sort import sort_by_expert
from tests.parity import assert_bits_equal, check_f32, dev_f32, dev_i32, dev_u8, host
from tests.mfma_model import tgmm_samples
from workloads import CONFIGS, STATIC_ACT_SCALE, generate, to_bf16_bits

pytestmark = pytest.mark.gpu
CANARY = 0x5A


def expected_xt(xs, group_sizes, g0, El, M, E):
    """The transposed layout from the sorted local rows xs [>= n, H]: group g's
    rows as columns from 128 * (sum of the earlier groups' 128-row blocks),
    zeros up to its own next multiple of 128, the canary past the last one."""
    H = xs.shape[1]
    cols = m.tgmm_xt_cols(M, E)
    xt = np.full((H, cols), CANARY, np.uint8)
    r0 = p0 = 0
    for g in range(El):
        mg = int(group_sizes[g0 + g])
        blocks = (mg + 127) // 128
        xt[:, p0:p0 + 128 * blocks] = 0
        xt[:, p0:p0 + mg] = xs[r0:r0 + mg].T
        r0 += mg
        p0 += 128 * blocks
    return xt


def gpu_gather_t(x_dev, x_dtype, scale, T, k, H, perm, gs, E, g0, El, M):
    cols = m.tgmm_xt_cols(M, E)
    xt = torch.full((H, cols), CANARY, dtype=torch.uint8, device="cuda")
    sc = torch.zeros(1, dtype=torch.float32, device="cuda")
    ws = torch.zeros(256, dtype=torch.uint8, device="cuda")
    print(f"sort_gather_transposed T={T} k={k} H={H} E={E} g0={g0} El={El} M={M} dtype={x_dtype}", flush=True)
    m.moe_sort_gather_transposed(x_dev, x_dtype, scale, T, k, H, dev_i32(perm), dev_i32(gs), E, g0, El, M, xt, sc, ws)
    assert m.moe_debug_check(ws) == 0
    return xt, sc


def routing(rng, T, k, E, skew=0.0):
    w = np.exp(-skew * np.log1p(np.arange(E))) if skew else np.ones(E)
    return np.stack([rng.choice(E, k, replace=False, p=w / w.sum()) for _ in range(T)]).astype(np.int32)


@pytest.mark.parametrize("T,k,E,g0,El,H,skew", [
    (300, 4, 16, 0, 16, 256, 0.0),
    (500, 2, 24, 5, 9, 512, 1.5),        # a local slice; skewed routing leaves empty groups
    (64, 8, 8, 2, 4, 768, 0.0),
])
def test_gather_transposed_e4m3_codes_bit_exact(T, k, E, g0, El, H, skew):
    rng = np.random.default_rng(T + E + H)
    ids = routing(rng, T, k, E, skew)
    xq = rng.integers(0, 256, (T, H)).astype(np.uint8)
    srt = sort_by_expert(ids, E, g0, El, xq=xq, xscale=np.ones(1, np.float32), xscale_mode=SCALE_TENSOR_STATIC)
    n = srt["n"]
    M = n + 19
    want = expected_xt(srt["xs"], srt["group_sizes"], g0, El, M, E)
    xt, _ = gpu_gather_t(dev_u8(xq), m.MOE_E4M3FN, 1.0, T, k, H, srt["perm"], srt["group_sizes"], E, g0, El, M)
    assert_bits_equal(host(xt), want, "transposed gather, e4m3 codes")


def test_gather_transposed_bf16_static_quantizes_like_the_row_quantizer():
    """bf16 rows quantized on the way with the static scale: the codes of
    moe_quantize_rows' static mode (saturation, signed zeros, subnormals)."""
    rng = np.random.default_rng(11)
    T, k, E, H = 400, 3, 12, 512
    ids = routing(rng, T, k, E, 1.0)
    x = to_bf16_bits((rng.standard_normal((T, H)) * rng.uniform(0.01, 8, (T, 1))).astype(np.float32))
    x[3, :7] = to_bf16_bits(np.array([0.0, -0.0, 1e30, -1e30, 1e-30, -1e-30, 448.0], np.float32))
    s = np.float32(0.0157)
    xq, xsc, _ = quantize_rows(x, SCALE_TENSOR_STATIC, static_scale=s)
    srt = sort_by_expert(ids, E, 0, E, xq=xq, xscale=xsc, xscale_mode=SCALE_TENSOR_STATIC)
    M = srt["n"]
    want = expected_xt(srt["xs"], srt["group_sizes"], 0, E, M, E)
    xd = torch.from_numpy(x.view(np.int16)).to("cuda")
    xt, sc = gpu_gather_t(xd, m.MOE_BF16, float(s), T, k, H, srt["perm"], srt["group_sizes"], E, 0, E, M)
    assert_bits_equal(host(xt), want, "transposed gather, bf16 quantized")
    assert host(sc)[0] == s


@pytest.mark.parametrize("out_dtype", [m.MOE_F32, m.MOE_BF16])
def test_tgmm_on_the_transposed_layout_equals_tgmm(out_dtype):
    rng = np.random.default_rng(5 + out_dtype)
    T, k, E, g0, El, H, N = 700, 4, 20, 3, 12, 512, 384
    ids = routing(rng, T, k, E, 1.2)
    xq = rng.integers(0, 0x7E, (T, H)).astype(np.uint8) | (rng.integers(0, 2, (T, H)).astype(np.uint8) << 7)
    srt = sort_by_expert(ids, E, g0, El, xq=xq, xscale=np.ones(1, np.float32), xscale_mode=SCALE_TENSOR_STATIC)
    n = srt["n"]
    M = n + 5
    X = np.zeros((M, H), np.uint8)
    X[:n] = srt["xs"][:n]
    D = rng.integers(0, 0x7E, (M, N)).astype(np.uint8) | (rng.integers(0, 2, (M, N)).astype(np.uint8) << 7)
    xs = rng.uniform(0.01, 1, H).astype(np.float32)
    ds = np.array([0.003], np.float32)
    gs = srt["group_sizes"]
    xt, _ = gpu_gather_t(dev_u8(xq), m.MOE_E4M3FN, 1.0, T, k, H, srt["perm"], gs, E, g0, El, M)
    dt = torch.float32 if out_dtype == m.MOE_F32 else torch.bfloat16
    a = torch.full((El, H, N), 7.0, dtype=dt, device="cuda")
    b = torch.full((El, H, N), 9.0, dtype=dt, device="cuda")
    ws = m.workspace(m.MOE_OP_TGMM, M, H, N, E)
    print(f"tgmm and tgmm_xt M={M} K={H} N={N} E={E} g0={g0} El={El}", flush=True)
    m.moe_tgmm_fp8(dev_u8(X), dev_f32(xs), H, dev_u8(D), dev_f32(ds), 1, dev_i32(gs), E, g0, El, M, H, N, out_dtype,
                   a, ws)
    m.moe_tgmm_fp8_xt(xt, dev_f32(xs), H, dev_u8(D), dev_f32(ds), 1, dev_i32(gs), E, g0, El, M, H, N, out_dtype,
                      b, ws)
    assert m.moe_debug_check(ws) == 0
    assert torch.equal(a, b), "tgmm on the transposed layout differs from tgmm on the sorted rows"
    if out_dtype == m.MOE_F32:
        o = tgmm(X, xs, D, ds, gs, g0, El)
        check_f32(host(b), o["out"], o["abs_sum"], "tgmm_xt against the oracle",
                  model=lambda idx: tgmm_samples(X, xs, D, ds, gs, g0, El, idx // (H * N), (idx // N) % H, idx % N))


def test_config5_weight_gradient_through_the_transposed_gather():
    """Config 5 at full size: X quantized with its static scale on the way
    into the transposed layout, the layout bit-exact against the oracle's
    quantized and sorted rows, and dW equal to moe_tgmm_fp8's on those rows."""
    cfg = CONFIGS[5]
    d = generate(cfg, with_weights=False)
    T, k, E, H, N = cfg.T, cfg.k, cfg.E, cfg.H, cfg.I
    xq, xsc, _ = quantize_rows(d["x"], SCALE_TENSOR_STATIC, static_scale=STATIC_ACT_SCALE)
    srt = sort_by_expert(d["ids"], E, 0, E, xq=xq, xscale=xsc, xscale_mode=SCALE_TENSOR_STATIC)
    M = srt["n"]
    gs = srt["group_sizes"]
    xd = torch.from_numpy(d["x"].view(np.int16)).to("cuda")
    xt, sc = gpu_gather_t(xd, m.MOE_BF16, float(STATIC_ACT_SCALE), T, k, H, srt["perm"], gs, E, 0, E, M)
    assert_bits_equal(host(xt), expected_xt(srt["xs"], gs, 0, E, M, E), "config 5 transposed X")
    dyq, dys, _ = quantize_rows(d["dy"], SCALE_TENSOR_DYNAMIC)
    a = torch.empty((E, H, N), dtype=torch.float32, device="cuda")
    b = torch.empty((E, H, N), dtype=torch.float32, device="cuda")
    ws = m.workspace(m.MOE_OP_TGMM, M, H, N, E)
    print(f"config 5 tgmm and tgmm_xt M={M}", flush=True)
    m.moe_tgmm_fp8(dev_u8(srt["xs"][:M]), sc, 1, dev_u8(dyq), dev_f32(dys), 1, dev_i32(gs), E, 0, E, M, H, N,
                   m.MOE_F32, a, ws)
    m.moe_tgmm_fp8_xt(xt, sc, 1, dev_u8(dyq), dev_f32(dys), 1, dev_i32(gs), E, 0, E, M, H, N, m.MOE_F32, b, ws)
    assert m.moe_debug_check(ws) == 0
    assert torch.equal(a, b)
