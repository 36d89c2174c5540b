"""GPU parity of the grouped matmuls (gmm, tgmm) against the oracle, under
the float32 / bf16 match rules of tests/parity.py.  Every workload case
compares every output element under the strict rules (1e-5 * A in float32,
1 bf16 ulp); only the synthetic random-code cases carry the matrix-core
allowance."""

import numpy as np
import pytest
import torch

import moe_fp8_grouped_amd as m
from oracle.gmm import gmm, tgmm
from oracle.quantize import SCALE_ROW_DYNAMIC, SCALE_TENSOR_DYNAMIC, SCALE_TENSOR_STATIC, quantize_rows, quantize_weights
from oracle.sort import sort_by_expert
from tests.parity import (assert_bits_equal, check_bf16, check_f32, dev_f32, dev_i32, dev_u8, gmm_allowance, host,
                          tgmm_allowance)
from tests.mfma_model import gmm_samples, tgmm_samples
from workloads import CONFIGS, STATIC_ACT_SCALE, STATIC_WEIGHT_SCALE, generate, to_bf16_bits

pytestmark = pytest.mark.gpu


def gpu_gmm(lhs, ls, ls_mode, rhs, rs, group_sizes, E, g0, El, transpose_rhs, out_dtype, M=None):
    M = lhs.shape[0] if M is None else M
    K = lhs.shape[1]
    N = rhs.shape[1] if transpose_rhs else rhs.shape[2]
    assert rhs.shape[0] == El and rs.shape[0] == El and rs.ndim == 4
    assert (ls.size == M) if ls_mode == m.MOE_SCALE_ROW_DYNAMIC else ls.size == 1
    out = torch.full((M, N), 3.0, dtype=torch.float32 if out_dtype == m.MOE_F32 else torch.bfloat16, device="cuda")
    ws = m.workspace(m.MOE_OP_GMM, M, K, N, E)
    print(f"gmm M={M} K={K} N={N} E={E} g0={g0} El={El} Kb={rs.shape[1]} Nb={rs.shape[3]} "
          f"tr={transpose_rhs} out={out_dtype}", flush=True)
    m.moe_gmm_fp8(dev_u8(lhs), dev_f32(ls), ls_mode, dev_u8(rhs), dev_f32(rs), rs.shape[1], rs.shape[3],
                  transpose_rhs, dev_i32(group_sizes), E, g0, El, M, K, N, out_dtype, out, ws)
    err = m.moe_debug_check(ws)
    return host(out), err


def _check_gmm_full(lhs, ls, ls_mode, wq, ws_, gs, E, g0, El, tr, what, hw=False, M=None):
    """Every element of the f32 and the bf16 output against the oracle: the
    strict rules, or (hw: synthetic random-code operands) the rules with the
    matrix-core allowance."""
    rhs = np.ascontiguousarray(wq.transpose(0, 2, 1)) if tr else wq
    lhs_o, ls_o = lhs, ls
    if M is not None and M > lhs.shape[0]:           # rows past the local ones: zero codes, zero scales
        lhs_o = np.zeros((M, lhs.shape[1]), np.uint8)
        lhs_o[:lhs.shape[0]] = lhs
        if ls.size > 1:
            ls_o = np.zeros(M, np.float32)
            ls_o[:ls.size] = ls
    o = gmm(lhs_o, ls_o, wq, ws_, gs, g0, El)
    Mo, N = o["out"].shape
    B = (lambda idx: gmm_allowance(lhs_o, ls_o, wq, ws_, gs, g0, El, idx // N, idx % N)) if hw else None
    mdl = None if hw else (lambda idx: gmm_samples(lhs_o, ls_o, wq, ws_, gs, g0, El, idx // N, idx % N))
    g32, err = gpu_gmm(lhs_o, ls_o, ls_mode, rhs, ws_, gs, E, g0, El, tr, m.MOE_F32)
    assert err == 0
    st = check_f32(g32, o["out"], o["abs_sum"], what + " f32", hw_allowance=B, model=mdl)
    del g32
    g16, _ = gpu_gmm(lhs_o, ls_o, ls_mode, rhs, ws_, gs, E, g0, El, tr, m.MOE_BF16)
    check_bf16(g16, o["out"], o["abs_sum"], what + " bf16", hw_allowance=B, model=mdl)
    n = int(np.asarray(gs)[g0:g0 + El].sum())
    assert not g16[n:].any()
    return st


def _config_stage(cid, static=False, weight="w_up", gpu_weights=False):
    cfg = CONFIGS[cid]
    d = generate(cfg, with_weights=[weight])
    mode = SCALE_TENSOR_STATIC if static else SCALE_ROW_DYNAMIC
    xq, xsc, _ = quantize_rows(d["x"], mode, static_scale=STATIC_ACT_SCALE if static else None)
    srt = sort_by_expert(d["ids"], cfg.E, cfg.group_offset, cfg.E_loc, xq=xq, xscale=xsc, xscale_mode=mode)
    w = d["weights"][weight]
    kb, nb = cfg.scale_blocks(w.shape[1], w.shape[2])
    static_w = STATIC_WEIGHT_SCALE if static else None
    wq, ws_ = _gpu_weights(w, kb, nb, static_w) if gpu_weights else quantize_weights(w, kb, nb, static_scale=static_w)
    return cfg, srt, wq, ws_, mode


@pytest.mark.parametrize("tr", [1, 0])
def test_gmm_config1_full(tr):
    cfg, srt, wq, ws_, mode = _config_stage(1)
    _check_gmm_full(srt["xs"], srt["ss"], mode, wq, ws_, srt["group_sizes"], cfg.E, 0, cfg.E, tr, f"config 1 tr={tr}")


@pytest.mark.parametrize("static", [False, True])
def test_gmm_config3_blockwise_skewed_full(static):
    cfg, srt, wq, ws_, mode = _config_stage(3, static=static)
    assert ws_.shape == (8, 4, 1, 1024)
    assert (srt["group_sizes"] == 0).sum() >= 2
    ls = srt["ss"] if mode == SCALE_ROW_DYNAMIC else np.array([STATIC_ACT_SCALE], np.float32)
    what = "config 3" + (" static" if static else "")
    _check_gmm_full(srt["xs"], ls, mode, wq, ws_, srt["group_sizes"], cfg.E, 0, cfg.E, 1, what)
    _check_gmm_full(srt["xs"], ls, mode, wq, ws_, srt["group_sizes"], cfg.E, 0, cfg.E, 0, what + " kn")


def test_gmm_config2_wi0_full():
    cfg, srt, wq, ws_, mode = _config_stage(2, weight="wi_0", gpu_weights=True)
    _check_gmm_full(srt["xs"], srt["ss"], mode, wq, ws_, srt["group_sizes"], cfg.E, 0, cfg.E, 1, "config 2 wi_0")


def test_gmm_config2_wo_full():
    cfg = CONFIGS[2]
    d = generate(cfg, with_weights=["wo"])
    rng = np.random.default_rng(7)
    gs = np.bincount(d["ids"].ravel(), minlength=cfg.E).astype(np.int32)
    hq, hs, _ = quantize_rows(generate_h(rng, cfg.M, cfg.I), SCALE_ROW_DYNAMIC)
    wq, ws_ = _gpu_weights(d["weights"]["wo"], 1, cfg.H)
    _check_gmm_full(hq, hs, SCALE_ROW_DYNAMIC, wq, ws_, gs, cfg.E, 0, cfg.E, 1, "config 2 wo")


def generate_h(rng, M, I):
    from workloads import to_bf16_bits
    return to_bf16_bits((rng.standard_normal((M, I)) * 0.05).astype(np.float32))


def _gpu_weights(w_bits, kb, nb, static=None):
    """The weight pre-quantization on the GPU ([E, K, N] layout), its first
    two experts bit-checked against the oracle's; the oracle's later stages
    take these (the oracle's own quantizer is slow on weights this large)."""
    E, K, N = w_bits.shape
    q = torch.empty((E, K, N), dtype=torch.uint8, device="cuda")
    s = torch.empty((E, kb, 1, nb), dtype=torch.float32, device="cuda")
    wd = torch.from_numpy(np.ascontiguousarray(w_bits).view(np.int16)).to("cuda")
    m.moe_quantize_weights(wd, E, K, N, kb, nb, m.MOE_SCALE_TENSOR_STATIC if static else m.MOE_SCALE_ROW_DYNAMIC,
                           static or 0.0, 0, q, s)
    torch.cuda.synchronize()
    q, s = host(q), host(s)
    qo, so = quantize_weights(w_bits[:2], kb, nb, static_scale=static)
    assert_bits_equal(q[:2], qo, "weights q (first experts)")
    assert_bits_equal(s[:2], so, "weights scale (first experts)")
    return q, s


def test_gmm_config4_expert_slice_full():
    cfg = CONFIGS[4]
    d = generate(cfg, with_weights=["wi_0"])
    xq, xsc, _ = quantize_rows(d["x"], SCALE_ROW_DYNAMIC)
    srt = sort_by_expert(d["ids"], cfg.E, cfg.group_offset, cfg.E_loc, xq=xq, xscale=xsc,
                         xscale_mode=SCALE_ROW_DYNAMIC)
    kb, nb = cfg.scale_blocks(cfg.H, cfg.I)
    wq, ws_ = _gpu_weights(d["weights"]["wi_0"], kb, nb)
    assert ws_.shape == (32, 56, 1, 16)
    n = srt["n"]
    m_cap = ((n + 255) // 256) * 256
    _check_gmm_full(srt["xs"][:n], srt["ss"][:n], SCALE_ROW_DYNAMIC, wq, ws_, srt["group_sizes"], cfg.E,
                    cfg.group_offset, cfg.E_loc, 1, "config 4 wi_0", M=m_cap)


@pytest.mark.parametrize("static", [False, True])
def test_gmm_skewed_large_blockwise_full(static):
    """Config 3's skewed routing and [E, K/128, 1, N] scales at the large
    matmul shape (8192 rows, K=7168, N=2048, 32 experts, 17 of them empty)."""
    cfg = CONFIGS[6]
    d = generate(cfg, with_weights=["w_up"])
    mode = SCALE_TENSOR_STATIC if static else SCALE_ROW_DYNAMIC
    xq, xsc, _ = quantize_rows(d["x"], mode, static_scale=STATIC_ACT_SCALE if static else None)
    srt = sort_by_expert(d["ids"], cfg.E, 0, cfg.E, xq=xq, xscale=xsc, xscale_mode=mode)
    kb, nb = cfg.scale_blocks(cfg.H, cfg.I)
    wq, ws_ = _gpu_weights(d["weights"]["w_up"], kb, nb, STATIC_WEIGHT_SCALE if static else None)
    assert ws_.shape == (32, 56, 1, 2048)
    gs = srt["group_sizes"]
    assert (gs == 0).sum() >= 2 and gs.max() >= 512 and (gs[gs > 0] < 128).any()
    ls = srt["ss"] if not static else xsc
    _check_gmm_full(srt["xs"], ls, mode, wq, ws_, gs, cfg.E, 0, cfg.E, 1, "skewed large" + (" static" if static else ""))


def test_gmm_config5_input_gradient_full():
    cfg = CONFIGS[5]
    d = generate(cfg, with_weights=["w_up"])
    gs = np.bincount(d["ids"].ravel(), minlength=cfg.E).astype(np.int32)
    dyq, dys, _ = quantize_rows(d["dy"], SCALE_ROW_DYNAMIC)
    wq, ws_ = _gpu_weights(d["weights"]["w_up"], 1, 1, STATIC_WEIGHT_SCALE)      # [E, H, I]
    # dX = dY @ W^T: the rhs is W stored [E, N=H, K=I]; the oracle takes it as [E, K, N] = W^T
    wT = np.ascontiguousarray(wq.transpose(0, 2, 1))
    o = gmm(dyq, dys, wT, ws_, gs, 0, cfg.E)
    g32, err = gpu_gmm(dyq, dys, m.MOE_SCALE_ROW_DYNAMIC, wq, ws_, gs, cfg.E, 0, cfg.E, 1, m.MOE_F32)
    assert err == 0
    N = cfg.H
    check_f32(g32, o["out"], o["abs_sum"], "config 5 dX f32",
              model=lambda idx: gmm_samples(dyq, dys, wT, ws_, gs, 0, cfg.E, idx // N, idx % N))


@pytest.mark.parametrize("sizes", [[0, 5, 0, 130, 1, 0, 257, 0], [0, 0, 0, 0], [300], [1, 1, 1, 1, 1, 1, 1, 1]])
def test_gmm_ragged_groups_and_zero_tail(sizes):
    rng = np.random.default_rng(len(sizes) + sum(sizes))
    E = len(sizes)
    gs = np.array(sizes, np.int32)
    n = int(gs.sum())
    M = n + 37
    K, N = 256, 256
    lhs = rng.integers(0, 256, (M, K)).astype(np.uint8)
    lhs[(lhs & 0x7F) == 0x7F] = 0x30
    ls = rng.uniform(0.01, 1, M).astype(np.float32)
    w = rng.integers(0, 256, (E, K, N)).astype(np.uint8)
    w[(w & 0x7F) == 0x7F] = 0x30
    rs = rng.uniform(0.001, 0.1, (E, 2, 1, 2)).astype(np.float32)
    _check_gmm_full(lhs, ls, m.MOE_SCALE_ROW_DYNAMIC, w, rs, gs, E, 0, E, 1, f"ragged {sizes}", hw=True)
    _check_gmm_full(lhs, ls, m.MOE_SCALE_ROW_DYNAMIC, w, rs, gs, E, 0, E, 0, f"ragged kn {sizes}", hw=True)


@pytest.mark.parametrize("sizes,N,nb,static", [
    ([0, 5, 0, 130, 1, 0, 257, 300, 128, 129, 256, 384, 513], 1536, "channel", False),
    ([2, 0, 700, 64, 255], 2048, "coarse", False),
    ([1, 1, 1, 1], 1536, "tensor", True),
])
def test_gmm_wide_outputs_ragged(sizes, N, nb, static):
    """Weights [E, N, K] with 1536 or more output columns, bf16 out and
    per-channel, coarse or tensor weight scales: empty groups, one-row
    groups, groups of 129..144 rows (one absorbing row block) and of more,
    tiles reaching past the buffer, and the zero rows after the last group --
    against the oracle over the whole output."""
    rng = np.random.default_rng(sum(sizes) + N)
    E = len(sizes)
    gs = np.array(sizes, np.int32)
    n = int(gs.sum())
    M = n + 37
    K = 384
    lhs = rng.integers(0, 0x70, (M, K)).astype(np.uint8)
    w = rng.integers(0, 0x70, (E, K, N)).astype(np.uint8)
    nbv = {"channel": N, "coarse": N // 128, "tensor": 1}[nb]
    rs = rng.uniform(0.001, 0.1, (E, 1, 1, nbv)).astype(np.float32)
    if static:
        ls, mode = np.array([0.25], np.float32), m.MOE_SCALE_TENSOR_STATIC
    else:
        ls, mode = rng.uniform(0.01, 1, M).astype(np.float32), m.MOE_SCALE_ROW_DYNAMIC
    _check_gmm_full(lhs, ls, mode, w, rs, gs, E, 0, E, 1, f"wide outputs {sizes} N={N} {nb}", hw=True)


@pytest.mark.parametrize("N,nb,Kb", [(512, "block", 2), (384, "channel", 1), (256, "block", 3), (512, "block64", 4),
                                     (384, "block64", 2)])
def test_gmm_absorbing_row_blocks(N, nb, Kb):
    """Group sizes at the boundaries of the absorbing row blocks (a group of
    m rows takes ceil(m / 144) blocks of 128 rows plus up to 16 each, so
    wide tiles of 129..144 rows): every element of the float32 and bf16
    outputs against the oracle, with an even and an odd count of 128-column
    blocks (the odd one's last column takes plain tiles), blockwise and
    per-channel scales, and rows past the groups."""
    sizes = [0, 1, 16, 17, 128, 129, 140, 144, 145, 256, 257, 272, 285, 288, 289, 300, 431, 432, 433]
    rng = np.random.default_rng(N + Kb)
    E = len(sizes)
    gs = np.array(sizes, np.int32)
    n = int(gs.sum())
    M = n + 37
    K = 128 * Kb if Kb > 1 else 512
    lhs = rng.integers(0, 0x70, (M, K)).astype(np.uint8)
    w = rng.integers(0, 0x70, (E, K, N)).astype(np.uint8)
    nbv = {"block": N // 128, "block64": N // 64, "channel": N}[nb]     # 128- or 64-column scale blocks
    rs = rng.uniform(0.001, 0.1, (E, Kb, 1, nbv)).astype(np.float32)
    ls = rng.uniform(0.01, 1, M).astype(np.float32)
    _check_gmm_full(lhs, ls, m.MOE_SCALE_ROW_DYNAMIC, w, rs, gs, E, 0, E, 1, f"absorbing N={N} {nb} Kb={Kb}", hw=True)


@pytest.mark.parametrize("sizes,N,blockwise", [([300, 200, 50], 1024, True), ([40, 0, 513, 7], 2048, False),
                                                ([100], 2048, True)])
def test_gmm_split_last_round(sizes, N, blockwise):
    """Few tiles over many workgroups: each XCD's last (here only) round of
    tiles is split along K (K = 2048: parts of at least four 128-deep steps),
    whose float32 sums meet in the workspace.  Quantized gaussian operands, as
    in the workloads: every element of both outputs under the strict rule
    (the matrix-core model for the rare misses), the same bits on a second
    call, and the same rule with a header-only workspace (no split)."""
    rng = np.random.default_rng(sum(sizes) + N)
    E = len(sizes)
    gs = np.array(sizes, np.int32)
    n = int(gs.sum())
    M, K = n + 37, 2048
    x = to_bf16_bits(rng.standard_normal((n, K)).astype(np.float32))
    xq, xsc, _ = quantize_rows(x, SCALE_ROW_DYNAMIC)
    w = to_bf16_bits((rng.standard_normal((E, K, N)) * 0.02).astype(np.float32))
    kb, nb = (K // 128, N // 128) if blockwise else (1, N)
    wq, ws_ = quantize_weights(w, kb, nb)
    what = f"split {sizes} N={N} {'blockwise' if blockwise else 'per-channel'}"
    _check_gmm_full(xq, xsc, SCALE_ROW_DYNAMIC, wq, ws_, gs, E, 0, E, 1, what, M=M)
    lhs = np.zeros((M, K), np.uint8)
    lhs[:n] = xq
    ls = np.zeros(M, np.float32)
    ls[:n] = xsc
    rhs = np.ascontiguousarray(wq.transpose(0, 2, 1))
    a, err_a = gpu_gmm(lhs, ls, SCALE_ROW_DYNAMIC, rhs, ws_, gs, E, 0, E, 1, m.MOE_BF16)
    b, err_b = gpu_gmm(lhs, ls, SCALE_ROW_DYNAMIC, rhs, ws_, gs, E, 0, E, 1, m.MOE_BF16)
    assert err_a == 0 and err_b == 0
    assert_bits_equal(a, b, "split: second call")
    # a header-only workspace: the same product without the split
    out = torch.full((M, N), 3.0, dtype=torch.float32, device="cuda")
    small = torch.zeros(256, dtype=torch.uint8, device="cuda")
    print(f"gmm header-only workspace M={M} K={K} N={N}", flush=True)
    m.moe_gmm_fp8(dev_u8(lhs), dev_f32(ls), SCALE_ROW_DYNAMIC, dev_u8(rhs), dev_f32(ws_), kb, nb, 1, dev_i32(gs), E, 0,
                  E, M, K, N, m.MOE_F32, out, small)
    assert m.moe_debug_check(small) == 0
    o = gmm(lhs, ls, wq, ws_, gs, 0, E)
    check_f32(host(out), o["out"], o["abs_sum"], what + " header-only workspace",
              model=lambda idx: gmm_samples(lhs, ls, wq, ws_, gs, 0, E, idx // N, idx % N))


def test_gmm_wide_outputs_local_slice():
    rng = np.random.default_rng(21)
    E, g0, El = 10, 3, 4
    gs = rng.integers(0, 300, E).astype(np.int32)
    n = int(gs[g0:g0 + El].sum())
    K, N = 256, 1536
    lhs = rng.integers(0, 0x70, (n + 10, K)).astype(np.uint8)
    w = rng.integers(0, 0x70, (El, K, N)).astype(np.uint8)
    rs = rng.uniform(0.01, 0.1, (El, 1, 1, N)).astype(np.float32)
    ls = rng.uniform(0.01, 1, n + 10).astype(np.float32)
    _check_gmm_full(lhs, ls, m.MOE_SCALE_ROW_DYNAMIC, w, rs, gs, E, g0, El, 1, "wide outputs local slice", hw=True)


def test_gmm_local_slice_and_no_local_experts():
    rng = np.random.default_rng(11)
    E, g0, El = 10, 3, 4
    gs = rng.integers(0, 200, E).astype(np.int32)
    n = int(gs[g0:g0 + El].sum())
    K, N = 384, 128
    lhs = rng.integers(0, 0x70, (n + 10, K)).astype(np.uint8)
    w = rng.integers(0, 0x70, (El, K, N)).astype(np.uint8)
    rs = rng.uniform(0.01, 0.1, (El, 3, 1, N)).astype(np.float32)
    ls = np.array([0.5], np.float32)
    _check_gmm_full(lhs, ls, m.MOE_SCALE_TENSOR_STATIC, w, rs, gs, E, g0, El, 1, "local slice", hw=True)
    # no local experts: every row is zero
    g32, err = gpu_gmm(lhs, ls, m.MOE_SCALE_TENSOR_STATIC, w[:0], rs[:0], gs, E, g0, 0, 1, m.MOE_F32)
    assert err == 0 and not g32.any()


def test_gmm_flags_rows_beyond_buffer():
    gs = np.array([100, 100], np.int32)
    lhs = np.ones((150, 128), np.uint8)
    w = np.ones((2, 128, 128), np.uint8)
    rs = np.ones((2, 1, 1, 128), np.float32)
    g32, err = gpu_gmm(lhs, np.ones(1, np.float32), m.MOE_SCALE_TENSOR_STATIC, w, rs, gs, 2, 0, 2, 1, m.MOE_F32)
    assert err & m.MOE_DEVERR_ROWS


# ------------------------------------------------------------------ tgmm
def gpu_tgmm(X, xs, D, ds, gs, E, g0, El, out_dtype=m.MOE_F32):
    M, K = X.shape
    N = D.shape[1]
    out = torch.full((El, K, N), 5.0, dtype=torch.float32 if out_dtype == m.MOE_F32 else torch.bfloat16,
                     device="cuda")
    ws = m.workspace(m.MOE_OP_TGMM, M, K, N, E)
    print(f"tgmm M={M} K={K} N={N} E={E} El={El}", flush=True)
    m.moe_tgmm_fp8(dev_u8(X), dev_f32(xs), xs.size, dev_u8(D), dev_f32(ds), ds.size, dev_i32(gs), E, g0, El, M, K,
                   N, out_dtype, out, ws)
    err = m.moe_debug_check(ws)
    return host(out), err


@pytest.mark.parametrize("sizes", [[0, 3, 200, 0, 1, 129, 0], [64, 64], [0]])
def test_tgmm_small_full(sizes):
    rng = np.random.default_rng(sum(sizes) + 1)
    E = len(sizes)
    gs = np.array(sizes, np.int32)
    M = int(gs.sum()) + 5
    K, N = 256, 384
    X = rng.integers(0, 0x7E, (M, K)).astype(np.uint8) | (rng.integers(0, 2, (M, K)).astype(np.uint8) << 7)
    D = rng.integers(0, 0x7E, (M, N)).astype(np.uint8) | (rng.integers(0, 2, (M, N)).astype(np.uint8) << 7)
    xs = rng.uniform(0.01, 1, K).astype(np.float32)
    ds = np.array([0.003], np.float32)
    o = tgmm(X, xs, D, ds, gs, 0, E)
    g, err = gpu_tgmm(X, xs, D, ds, gs, E, 0, E)
    assert err == 0
    B = lambda idx: tgmm_allowance(X, xs, D, ds, gs, 0, E, idx // (K * N), (idx // N) % K, idx % N)
    check_f32(g, o["out"], o["abs_sum"], f"tgmm {sizes}", hw_allowance=B)
    for e in np.nonzero(gs == 0)[0]:
        assert not g[e].any()
    g16, _ = gpu_tgmm(X, xs, D, ds, gs, E, 0, E, m.MOE_BF16)
    check_bf16(g16, o["out"], o["abs_sum"], f"tgmm bf16 {sizes}", hw_allowance=B)


def test_tgmm_config5_full():
    cfg = CONFIGS[5]
    d = generate(cfg, with_weights=False)
    xq, xsc, _ = quantize_rows(d["x"], SCALE_TENSOR_STATIC, static_scale=STATIC_ACT_SCALE)
    srt = sort_by_expert(d["ids"], cfg.E, 0, cfg.E, xq=xq, xscale=xsc, xscale_mode=SCALE_TENSOR_STATIC)
    dyq, dys, _ = quantize_rows(d["dy"], SCALE_TENSOR_DYNAMIC)
    gs = srt["group_sizes"]
    g, err = gpu_tgmm(srt["xs"], xsc, dyq, dys, gs, cfg.E, 0, cfg.E)
    assert err == 0
    o = tgmm(srt["xs"], xsc, dyq, dys, gs, 0, cfg.E)
    K, N = cfg.H, cfg.I
    check_f32(g, o["out"], o["abs_sum"], "config 5 dW",
              model=lambda idx: tgmm_samples(srt["xs"], xsc, dyq, dys, gs, 0, cfg.E, idx // (K * N), (idx // N) % K,
                                             idx % N))


def test_tgmm_dy_by_rows_ends_at_the_buffer():
    """The product reads dY by rows, a group's last K step reaching up to 127
    rows past its end: here the buffer ends at the last group's last row, so
    those reads are kept inside it, and the next group's rows (large codes
    of both signs) must add nothing to a group's gradient."""
    rng = np.random.default_rng(123)
    gs = np.array([37, 300, 0, 91], np.int32)
    E = len(gs)
    M = int(gs.sum())
    K, N = 512, 256
    X = rng.integers(0, 0x7E, (M, K)).astype(np.uint8) | (rng.integers(0, 2, (M, K)).astype(np.uint8) << 7)
    D = rng.integers(0x60, 0x7E, (M, N)).astype(np.uint8) | (rng.integers(0, 2, (M, N)).astype(np.uint8) << 7)
    xs = rng.uniform(0.01, 1, K).astype(np.float32)
    ds = rng.uniform(0.001, 0.01, N).astype(np.float32)
    o = tgmm(X, xs, D, ds, gs, 0, E)
    g, err = gpu_tgmm(X, xs, D, ds, gs, E, 0, E)
    assert err == 0
    B = lambda idx: tgmm_allowance(X, xs, D, ds, gs, 0, E, idx // (K * N), (idx // N) % K, idx % N)
    check_f32(g, o["out"], o["abs_sum"], "tgmm dY by rows, buffer end", hw_allowance=B)
    assert not g[2].any()


@pytest.mark.parametrize("K,small_ws", [(384, False), (256, True)])
def test_tgmm_one_kernel_path(K, small_ws):
    """The one-kernel tgmm (operands transposed in LDS while multiplying) serves
    K not a multiple of 256 and workspaces too small for the transposed copies."""
    rng = np.random.default_rng(K + small_ws)
    gs = np.array([5, 0, 140, 67], np.int32)
    E = len(gs)
    M = int(gs.sum()) + 3
    N = 256
    X = rng.integers(0, 0x7E, (M, K)).astype(np.uint8) | (rng.integers(0, 2, (M, K)).astype(np.uint8) << 7)
    D = rng.integers(0, 0x7E, (M, N)).astype(np.uint8) | (rng.integers(0, 2, (M, N)).astype(np.uint8) << 7)
    xs = np.array([0.02], np.float32)
    ds = rng.uniform(0.01, 1, N).astype(np.float32)
    o = tgmm(X, xs, D, ds, gs, 0, E)
    out = torch.full((E, K, N), 5.0, dtype=torch.float32, device="cuda")
    ws = m.workspace(m.MOE_OP_GMM if small_ws else m.MOE_OP_TGMM, M, K, N, E)
    print(f"tgmm one-kernel K={K} ws={ws.numel()}", flush=True)
    m.moe_tgmm_fp8(dev_u8(X), dev_f32(xs), 1, dev_u8(D), dev_f32(ds), N, dev_i32(gs), E, 0, E, M, K, N, m.MOE_F32,
                   out, ws)
    assert m.moe_debug_check(ws) == 0
    g = host(out)
    B = lambda idx: tgmm_allowance(X, xs, D, ds, gs, 0, E, idx // (K * N), (idx // N) % K, idx % N)
    check_f32(g, o["out"], o["abs_sum"], f"tgmm one-kernel K={K}", hw_allowance=B)
    assert not g[1].any()


# ------------------------------------------------- group sizes past 2^31
BIG_SIZES = np.array([1 << 30] * 3, np.int32)        # they sum to 3 * 2^30, past the int32 range


@pytest.mark.parametrize("N,out_dtype", [(256, m.MOE_F32), (1536, m.MOE_BF16)])
def test_gmm_group_sizes_summing_past_2_31_stay_in_bounds(N, out_dtype):
    """Three groups of 2^30 rows against a 1000-row buffer: the row table
    saturates at the buffer (group 0 gets every row, the others none), the
    rows flag is raised, and nothing past the output's last row is written
    (float32 and bf16 out)."""
    rng = np.random.default_rng(N)
    M, K, E = 1000, 256, 3
    lhs = rng.integers(0, 0x70, (M, K)).astype(np.uint8)
    w = rng.integers(0, 0x70, (E, K, N)).astype(np.uint8)
    rs = rng.uniform(0.01, 0.1, (E, 1, 1, N)).astype(np.float32)
    ls = rng.uniform(0.01, 1, M).astype(np.float32)
    dt = torch.float32 if out_dtype == m.MOE_F32 else torch.bfloat16
    buf = torch.full((M + 300, N), 3.0, dtype=dt, device="cuda")      # 300 canary rows after the output
    ws = m.workspace(m.MOE_OP_GMM, M, K, N, E)
    print(f"gmm group sizes past 2^31 M={M} N={N} out={out_dtype}", flush=True)
    m.moe_gmm_fp8(dev_u8(lhs), dev_f32(ls), m.MOE_SCALE_ROW_DYNAMIC, dev_u8(np.ascontiguousarray(w.transpose(0, 2, 1))),
                  dev_f32(rs), 1, N, 1, dev_i32(BIG_SIZES), E, 0, E, M, K, N, out_dtype, buf, ws)
    err = m.moe_debug_check(ws)
    assert err & m.MOE_DEVERR_ROWS
    g = host(buf)
    canary = g[M:]
    assert (canary == (3.0 if out_dtype == m.MOE_F32 else 0x4040)).all(), "rows past the buffer were written"
    o = gmm(lhs, ls, w, rs, np.array([M, 0, 0], np.int32), 0, E)
    Nn = N
    B = lambda idx: gmm_allowance(lhs, ls, w, rs, np.array([M, 0, 0], np.int32), 0, E, idx // Nn, idx % Nn)
    if out_dtype == m.MOE_F32:
        check_f32(g[:M], o["out"], o["abs_sum"], "sizes past 2^31", hw_allowance=B)
    else:
        check_bf16(g[:M], o["out"], o["abs_sum"], "sizes past 2^31 bf16", hw_allowance=B)


def test_tgmm_group_sizes_summing_past_2_31_stay_in_bounds():
    """The weight-gradient product with the same sizes: group 0 takes the
    buffer's 1000 rows, the other groups are zero, the flag is raised, and the
    canary after the output is untouched."""
    rng = np.random.default_rng(5)
    M, K, N, E = 1000, 256, 256, 3
    X = rng.integers(0, 0x70, (M, K)).astype(np.uint8)
    D = rng.integers(0, 0x70, (M, N)).astype(np.uint8)
    xs, ds = np.array([0.02], np.float32), np.array([0.003], np.float32)
    buf = torch.full((E + 1, K, N), 5.0, dtype=torch.float32, device="cuda")   # one canary group after the output
    ws = m.workspace(m.MOE_OP_TGMM, M, K, N, E)
    print(f"tgmm group sizes past 2^31 M={M}", flush=True)
    m.moe_tgmm_fp8(dev_u8(X), dev_f32(xs), 1, dev_u8(D), dev_f32(ds), 1, dev_i32(BIG_SIZES), E, 0, E, M, K, N,
                   m.MOE_F32, buf, ws)
    assert m.moe_debug_check(ws) & m.MOE_DEVERR_ROWS
    g = host(buf)
    assert (g[E] == 5.0).all(), "the canary after the output was written"
    assert not g[1:E].any()
    gs1 = np.array([M, 0, 0], np.int32)
    o = tgmm(X, xs, D, ds, gs1, 0, E)
    B = lambda idx: tgmm_allowance(X, xs, D, ds, gs1, 0, E, idx // (K * N), (idx // N) % K, idx % N)
    check_f32(g[:E], o["out"], o["abs_sum"], "tgmm sizes past 2^31", hw_allowance=B)


# ------------------------------------------------- the matrix-core model
@pytest.mark.parametrize("K", [128, 512, 2048])
def test_matrix_core_model_matches_the_device(K):
    """The model of the fp8 matrix core used by the workload checks
    (tests/mfma_model.py) against the device itself: one group, unit scales,
    float32 output, operands of random codes with exponents spread over the
    whole format.  The device's dot products equal the model's up to the
    order of the float32 additions of the chunk sums, and depart from the
    exact sums by far more than that (so the agreement is not trivial)."""
    from tests.mfma_model import dot_f32
    from oracle.codec import e4m3_decode
    rng = np.random.default_rng(K + 1)
    M, N = 256, 256
    lhs = rng.integers(0, 256, (M, K)).astype(np.uint8)
    lhs[(lhs & 0x7F) == 0x7F] = 0x30
    w = rng.integers(0, 256, (1, K, N)).astype(np.uint8)
    w[(w & 0x7F) == 0x7F] = 0x30
    g32, err = gpu_gmm(lhs, np.ones(1, np.float32), m.MOE_SCALE_TENSOR_STATIC,
                       np.ascontiguousarray(w.transpose(0, 2, 1)), np.ones((1, 1, 1, N), np.float32), np.array([M], np.int32), 1, 0, 1, 1, m.MOE_F32)
    assert err == 0
    rows = np.repeat(np.arange(M), N)
    cols = np.tile(np.arange(N), M)
    model = dot_f32(lhs[rows], w[0][:, cols].T).astype(np.float64)
    p = e4m3_decode(lhs[rows]) * e4m3_decode(w[0][:, cols].T)
    exact, A = p.sum(axis=1), np.abs(p).sum(axis=1)
    g = g32.reshape(-1).astype(np.float64)
    dev_vs_model = np.abs(g - model) / A
    dev_vs_exact = np.abs(g - exact) / A
    print(f"K={K}: device == model on {np.mean(g == model):.4f} of outputs; max |dev-model|/A "
          f"{dev_vs_model.max():.3g}; max |dev-exact|/A {dev_vs_exact.max():.3g}", flush=True)
    assert dev_vs_model.max() <= 2e-6
    assert dev_vs_exact.max() > 20 * dev_vs_model.max()


# ------------------------------------------------- K, N multiples of 16 only
@pytest.mark.parametrize("K,N,tr,nb", [(144, 80, 1, "channel"), (144, 80, 0, "channel"), (16, 16, 1, "tensor"),
                                       (272, 1552, 0, "coarse16"), (400, 208, 1, "channel")])
def test_gmm_sizes_multiple_of_16(K, N, tr, nb):
    """K and N that are multiples of 16 but not of 128 (the edge path):
    ragged groups with empty ones, both weight layouts, per-channel, per-
    tensor and 16-column-block scales, the rows after the last group zero."""
    rng = np.random.default_rng(K * 7 + N + tr)
    sizes = [0, 5, 0, 130, 1, 67, 0, 257]
    E = len(sizes)
    gs = np.array(sizes, np.int32)
    M = int(gs.sum()) + 21
    lhs = rng.integers(0, 0x70, (M, K)).astype(np.uint8)
    w = rng.integers(0, 0x70, (E, K, N)).astype(np.uint8)
    nbv = {"channel": N, "tensor": 1, "coarse16": N // 16}[nb]
    rs = rng.uniform(0.001, 0.1, (E, 1, 1, nbv)).astype(np.float32)
    ls = rng.uniform(0.01, 1, M).astype(np.float32)
    _check_gmm_full(lhs, ls, m.MOE_SCALE_ROW_DYNAMIC, w, rs, gs, E, 0, E, tr, f"K={K} N={N} tr={tr} {nb}", hw=True)


def test_gmm_sizes_multiple_of_16_quantized_operands_local_slice():
    """Quantized gaussian operands at K=144, N=80 on a local slice of the
    experts: the workload rule (1e-5 * A, else the modelled matrix core)."""
    from workloads import to_bf16_bits
    rng = np.random.default_rng(144)
    E, g0, El, K, N = 12, 4, 5, 144, 80
    gs = rng.integers(0, 90, E).astype(np.int32)
    gs[g0 + 1] = 0
    n = int(gs[g0:g0 + El].sum())
    x = to_bf16_bits(rng.standard_normal((n + 7, K)).astype(np.float32))
    w = to_bf16_bits((rng.standard_normal((El, K, N)) * 0.02).astype(np.float32))
    xq, xs, _ = quantize_rows(x, SCALE_ROW_DYNAMIC)
    wq, ws_ = quantize_weights(w, 1, N)
    _check_gmm_full(xq, xs, SCALE_ROW_DYNAMIC, wq, ws_, gs, E, g0, El, 1, "K=144 N=80 quantized slice")
    _check_gmm_full(xq, xs, SCALE_ROW_DYNAMIC, wq, ws_, gs, E, g0, El, 0, "K=144 N=80 quantized slice kn")


@pytest.mark.parametrize("K,N,scales", [(144, 80, "k_and_n"), (16, 48, "tensor"), (144, 1040, "n")])
def test_tgmm_sizes_multiple_of_16(K, N, scales):
    rng = np.random.default_rng(K + N)
    sizes = [0, 3, 200, 0, 1, 129]
    E = len(sizes)
    gs = np.array(sizes, np.int32)
    M = int(gs.sum()) + 4
    X = rng.integers(0, 0x7E, (M, K)).astype(np.uint8) | (rng.integers(0, 2, (M, K)).astype(np.uint8) << 7)
    D = rng.integers(0, 0x7E, (M, N)).astype(np.uint8) | (rng.integers(0, 2, (M, N)).astype(np.uint8) << 7)
    xs = rng.uniform(0.01, 1, K).astype(np.float32) if scales == "k_and_n" else np.array([0.02], np.float32)
    ds = rng.uniform(0.01, 1, N).astype(np.float32) if scales in ("k_and_n", "n") else np.array([0.003], np.float32)
    o = tgmm(X, xs, D, ds, gs, 0, E)
    g, err = gpu_tgmm(X, xs, D, ds, gs, E, 0, E)
    assert err == 0
    B = lambda idx: tgmm_allowance(X, xs, D, ds, gs, 0, E, idx // (K * N), (idx // N) % K, idx % N)
    check_f32(g, o["out"], o["abs_sum"], f"tgmm K={K} N={N}", hw_allowance=B)
    for e in np.nonzero(gs == 0)[0]:
        assert not g[e].any()
    g16, _ = gpu_tgmm(X, xs, D, ds, gs, E, 0, E, m.MOE_BF16)
    check_bf16(g16, o["out"], o["abs_sum"], f"tgmm bf16 K={K} N={N}", hw_allowance=B)
