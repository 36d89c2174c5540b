"""GPU parity of the grouped matmuls (gmm, tgmm) against the oracle, under
the float32 / bf16 match rules of tests/parity.py."""

import numpy as np
import pytest
import torch

import moe_fp8_grouped_amd as m
from oracle.gmm import gmm, tgmm
from oracle.quantize import SCALE_ROW_DYNAMIC, SCALE_TENSOR_DYNAMIC, SCALE_TENSOR_STATIC, quantize_rows, quantize_weights
from oracle.sort import sort_by_expert
from tests.parity import (check_bf16, check_f32, dev_f32, dev_i32, dev_u8, gmm_allowance, host, tgmm_allowance)
from workloads import CONFIGS, STATIC_ACT_SCALE, STATIC_WEIGHT_SCALE, generate

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


def _check_gmm_full(lhs, ls, ls_mode, wq, ws_, gs, E, g0, El, tr, what):
    rhs = np.ascontiguousarray(wq.transpose(0, 2, 1)) if tr else wq
    o = gmm(lhs, ls, wq, ws_, gs, g0, El)
    M, N = o["out"].shape
    B = lambda idx: gmm_allowance(lhs, ls, wq, ws_, gs, g0, El, idx // N, idx % N)
    g32, err = gpu_gmm(lhs, ls, ls_mode, rhs, ws_, gs, E, g0, El, tr, m.MOE_F32)
    assert err == 0
    st = check_f32(g32, o["out"], o["abs_sum"], B, what + " f32")
    g16, _ = gpu_gmm(lhs, ls, ls_mode, rhs, ws_, gs, E, g0, El, tr, m.MOE_BF16)
    check_bf16(g16, o["out"], o["abs_sum"], B, what + " bf16")
    n = int(np.asarray(gs)[g0:g0 + El].sum())
    assert not g32[n:].any() and not g16[n:].any()
    return st


def _config_stage(cid, static=False, weight="w_up"):
    cfg = CONFIGS[cid]
    d = generate(cfg, with_weights=[weight])
    mode = SCALE_TENSOR_STATIC if static else SCALE_ROW_DYNAMIC
    xq, xsc, _ = quantize_rows(d["x"], mode, static_scale=STATIC_ACT_SCALE if static else None)
    srt = sort_by_expert(d["ids"], cfg.E, cfg.group_offset, cfg.E_loc, xq=xq, xscale=xsc, xscale_mode=mode)
    w = d["weights"][weight]
    kb, nb = cfg.scale_blocks(w.shape[1], w.shape[2])
    wq, ws_ = quantize_weights(w, kb, nb, static_scale=STATIC_WEIGHT_SCALE if static else None)
    return cfg, srt, wq, ws_, mode


@pytest.mark.parametrize("tr", [1, 0])
def test_gmm_config1_full(tr):
    cfg, srt, wq, ws_, mode = _config_stage(1)
    st = _check_gmm_full(srt["xs"], srt["ss"], mode, wq, ws_, srt["group_sizes"], cfg.E, 0, cfg.E, tr, "config 1")
    print("config 1 strict 1e-5*A fraction", st)


@pytest.mark.parametrize("static", [False, True])
def test_gmm_config3_blockwise_skewed_full(static):
    cfg, srt, wq, ws_, mode = _config_stage(3, static=static)
    assert ws_.shape == (8, 4, 1, 1024)
    assert (srt["group_sizes"] == 0).sum() >= 2
    _check_gmm_full(srt["xs"], srt["ss"], mode, wq, ws_, srt["group_sizes"], cfg.E, 0, cfg.E, 1, "config 3")
    _check_gmm_full(srt["xs"], srt["ss"], mode, wq, ws_, srt["group_sizes"], cfg.E, 0, cfg.E, 0, "config 3 kn")


def _sampled(lhs, ls, ls_mode, wq, ws_, gs, E, g0, El, tr, n_samples, seed, what, M=None):
    rhs = np.ascontiguousarray(wq.transpose(0, 2, 1)) if tr == 1 else wq
    Mr = lhs.shape[0] if M is None else M
    N = wq.shape[2]
    n = int(np.asarray(gs)[g0:g0 + El].sum())
    rng = np.random.default_rng(seed)
    rows = rng.integers(0, max(n, 1), n_samples)
    cols = rng.integers(0, N, n_samples)
    o = gmm(lhs, ls, wq, ws_, gs, g0, El, sample=(rows, cols))
    B = lambda idx: gmm_allowance(lhs, ls, wq, ws_, gs, g0, El, rows[idx], cols[idx])
    g32, err = gpu_gmm(lhs, ls, ls_mode, rhs, ws_, gs, E, g0, El, tr, m.MOE_F32, M=Mr)
    assert err == 0
    st = check_f32(g32[rows, cols], o["out"], o["abs_sum"], B, what)
    g16, _ = gpu_gmm(lhs, ls, ls_mode, rhs, ws_, gs, E, g0, El, tr, m.MOE_BF16, M=Mr)
    check_bf16(g16[rows, cols], o["out"], o["abs_sum"], B, what + " bf16")
    assert not g32[n:].any() and not g16[n:].any()
    # every row of every group was written (the fill value 3.0 is gone)
    assert not (g32[:n] == 3.0).all(axis=1).any()
    return st


def test_gmm_config2_wi0_sampled():
    cfg, srt, wq, ws_, mode = _config_stage(2, weight="wi_0")
    st = _sampled(srt["xs"], srt["ss"], mode, wq, ws_, srt["group_sizes"], cfg.E, 0, cfg.E, 1, 20000, 1,
                  "config 2 wi_0")
    print("config 2 wi_0", st)


def test_gmm_config2_wo_sampled():
    cfg = CONFIGS[2]
    d = generate(cfg, with_weights=["wo"])
    rng = np.random.default_rng(7)
    gs = np.bincount(d["ids"].ravel(), minlength=cfg.E).astype(np.int32)
    hq, hs, _ = quantize_rows(generate_h(rng, cfg.M, cfg.I), SCALE_ROW_DYNAMIC)
    wq, ws_ = quantize_weights(d["weights"]["wo"], 1, cfg.H)
    _sampled(hq, hs, SCALE_ROW_DYNAMIC, wq, ws_, gs, cfg.E, 0, cfg.E, 1, 20000, 2, "config 2 wo")


def generate_h(rng, M, I):
    from workloads import to_bf16_bits
    return to_bf16_bits((rng.standard_normal((M, I)) * 0.05).astype(np.float32))


def test_gmm_config4_expert_slice_sampled():
    cfg, srt, wq, ws_, mode = _config_stage(4, weight="wi_0")
    assert ws_.shape == (32, 56, 1, 16)
    n = srt["n"]
    m_cap = ((n + 255) // 256) * 256
    lhs = np.zeros((m_cap, cfg.H), np.uint8)
    lhs[:n] = srt["xs"][:n]
    ls = np.zeros(m_cap, np.float32)
    ls[:n] = srt["ss"][:n]
    _sampled(lhs, ls, mode, wq, ws_, srt["group_sizes"], cfg.E, cfg.group_offset, cfg.E_loc, 1, 6000, 3,
             "config 4 wi_0")


@pytest.mark.parametrize("static", [False, True])
def test_gmm_skewed_large_blockwise_sampled(static):
    """Config 3's skewed routing and [E, K/128, 1, N] scales at the large
    matmul shape (8192 rows, K=7168, N=2048, 32 experts, 17 of them empty)."""
    cfg, srt, wq, ws_, mode = _config_stage(6, static=static)
    assert ws_.shape == (32, 56, 1, 2048)
    gs = srt["group_sizes"]
    assert (gs == 0).sum() >= 2 and gs.max() >= 512 and (gs[gs > 0] < 128).any()
    _sampled(srt["xs"], srt["ss"], mode, wq, ws_, gs, cfg.E, 0, cfg.E, 1, 6000, 6 + static,
             "skewed large" + (" static" if static else ""))


def test_gmm_config5_input_gradient_sampled():
    cfg = CONFIGS[5]
    d = generate(cfg, with_weights=["w_up"])
    gs = np.bincount(d["ids"].ravel(), minlength=cfg.E).astype(np.int32)
    dyq, dys, _ = quantize_rows(d["dy"], SCALE_ROW_DYNAMIC)
    wq, ws_ = quantize_weights(d["weights"]["w_up"], 1, 1, static_scale=STATIC_WEIGHT_SCALE)   # [E, H, I]
    # dX = dY @ W^T: the rhs is W stored [E, N=H, K=I]; the oracle takes it as [E, K, N] = W^T
    wT = np.ascontiguousarray(wq.transpose(0, 2, 1))
    rng = np.random.default_rng(4)
    n = cfg.M
    rows = rng.integers(0, n, 8000)
    cols = rng.integers(0, cfg.H, 8000)
    o = gmm(dyq, dys, wT, ws_, gs, 0, cfg.E, sample=(rows, cols))
    B = lambda idx: gmm_allowance(dyq, dys, wT, ws_, gs, 0, cfg.E, rows[idx], cols[idx])
    g32, err = gpu_gmm(dyq, dys, m.MOE_SCALE_ROW_DYNAMIC, wq, ws_, gs, cfg.E, 0, cfg.E, 1, m.MOE_F32)
    assert err == 0
    check_f32(g32[rows, cols], o["out"], o["abs_sum"], B, "config 5 dX")


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
    _check_gmm_full(lhs, ls, m.MOE_SCALE_ROW_DYNAMIC, w, rs, gs, E, 0, E, 1, f"ragged {sizes}")
    _check_gmm_full(lhs, ls, m.MOE_SCALE_ROW_DYNAMIC, w, rs, gs, E, 0, E, 0, f"ragged kn {sizes}")


@pytest.mark.parametrize("sizes,N,nb,static", [
    ([0, 5, 0, 130, 1, 0, 257, 300, 128, 129, 256, 384, 513], 1536, "channel", False),
    ([2, 0, 700, 64, 255], 2048, "coarse", False),
    ([1, 1, 1, 1], 1536, "tensor", True),
])
def test_gmm_256_tiles_ragged(sizes, N, nb, static):
    """The 256 x 256-tile kernel (weights [E, N, K], N >= 1536, bf16 out):
    empty groups, one-row groups, remainders of at most 128 rows (half
    tiles) and of more (a full tile with rows not stored), tiles reaching
    past the buffer, and the zero rows after the last group -- against the
    oracle over the whole output (its float32 twin runs the 256 x 128 kernel)."""
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
    _check_gmm_full(lhs, ls, mode, w, rs, gs, E, 0, E, 1, f"256 tiles {sizes} N={N} {nb}")


def test_gmm_256_tiles_local_slice():
    rng = np.random.default_rng(21)
    E, g0, El = 10, 3, 4
    gs = rng.integers(0, 300, E).astype(np.int32)
    n = int(gs[g0:g0 + El].sum())
    K, N = 256, 1536
    lhs = rng.integers(0, 0x70, (n + 10, K)).astype(np.uint8)
    w = rng.integers(0, 0x70, (El, K, N)).astype(np.uint8)
    rs = rng.uniform(0.01, 0.1, (El, 1, 1, N)).astype(np.float32)
    ls = rng.uniform(0.01, 1, n + 10).astype(np.float32)
    _check_gmm_full(lhs, ls, m.MOE_SCALE_ROW_DYNAMIC, w, rs, gs, E, g0, El, 1, "256 tiles local slice")


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
    _check_gmm_full(lhs, ls, m.MOE_SCALE_TENSOR_STATIC, w, rs, gs, E, g0, El, 1, "local slice")
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
    check_f32(g, o["out"], o["abs_sum"], B, f"tgmm {sizes}")
    for e in np.nonzero(gs == 0)[0]:
        assert not g[e].any()
    g16, _ = gpu_tgmm(X, xs, D, ds, gs, E, 0, E, m.MOE_BF16)
    check_bf16(g16, o["out"], o["abs_sum"], B, f"tgmm bf16 {sizes}")


def test_tgmm_config5_sampled():
    cfg = CONFIGS[5]
    d = generate(cfg, with_weights=False)
    xq, xsc, _ = quantize_rows(d["x"], SCALE_TENSOR_STATIC, static_scale=STATIC_ACT_SCALE)
    srt = sort_by_expert(d["ids"], cfg.E, 0, cfg.E, xq=xq, xscale=xsc, xscale_mode=SCALE_TENSOR_STATIC)
    dyq, dys, _ = quantize_rows(d["dy"], SCALE_TENSOR_DYNAMIC)
    gs = srt["group_sizes"]
    g, err = gpu_tgmm(srt["xs"], xsc, dyq, dys, gs, cfg.E, 0, cfg.E)
    assert err == 0
    rng = np.random.default_rng(8)
    P = 6000
    gi, ki, ci = rng.integers(0, cfg.E, P), rng.integers(0, cfg.H, P), rng.integers(0, cfg.I, P)
    o = tgmm(srt["xs"], xsc, dyq, dys, gs, 0, cfg.E, sample=(gi, ki, ci))
    B = lambda idx: tgmm_allowance(srt["xs"], xsc, dyq, dys, gs, 0, cfg.E, gi[idx], ki[idx], ci[idx])
    st = check_f32(g[gi, ki, ci], o["out"], o["abs_sum"], B, "config 5 dW")
    print("config 5 dW", st)
    # property at full size: every group's gradient was written (no fill value left)
    assert not (g == 5.0).any()


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
    check_f32(g, o["out"], o["abs_sum"], B, f"tgmm one-kernel K={K}")
    assert not g[1].any()
