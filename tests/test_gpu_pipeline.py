"""GPU parity of the gather-reduce and of whole pipelines, checked stage by
stage: the oracle of each stage is fed the GPU's actual inputs for that
stage, so the bit-exact rules apply to every quantization on the path."""

import numpy as np
import pytest
import torch

import moe_fp8_grouped_amd as m
from moe_fp8_grouped_amd.pipeline import BackwardPath, FFNBackwardPath, ForwardPath
from oracle.gather_reduce import gather_reduce, gather_reduce_backward
from oracle.gmm import gmm, tgmm
from oracle.pipeline import dense_bf16_backward_reference, dense_bf16_reference, rel_norm_diff, rel_norm_diff_f
from oracle.quantize import (SCALE_ROW_DYNAMIC, SCALE_TENSOR_DYNAMIC, SCALE_TENSOR_STATIC, quantize_rows,
                             quantize_weights, silu_mul_backward)
from oracle.sort import sort_by_expert
from tests.golden import accuracy_tables
from tests.test_gpu_tgmm_xt import expected_xt
from tests.mfma_model import gmm_samples, tgmm_samples
from tests.parity import assert_bits_equal, check_bf16, check_f32, dev_bf16, dev_f32, dev_i32, host
from workloads import CONFIGS, STATIC_ACT_SCALE, STATIC_WEIGHT_SCALE, generate, scaled_config, to_bf16_bits

pytestmark = pytest.mark.gpu


def gpu_gather_reduce(y, y_bf16, inv, w, out_dtype=m.MOE_BF16):
    T, k = inv.shape
    N = y.shape[1]
    yd = dev_bf16(y) if y_bf16 else dev_f32(y)
    out = torch.full((T, N), 9.0, dtype=torch.bfloat16 if out_dtype == m.MOE_BF16 else torch.float32, device="cuda")
    print(f"gather_reduce T={T} k={k} N={N} y_bf16={y_bf16}", flush=True)
    m.moe_gather_reduce(yd, m.MOE_BF16 if y_bf16 else m.MOE_F32, dev_i32(inv), dev_f32(w), T, k, N, out_dtype, out)
    torch.cuda.synchronize()
    return host(out)


@pytest.mark.parametrize("T,k,E,g0,El,N", [(256, 2, 8, 0, 8, 1024), (4096, 8, 64, 0, 64, 2048),
                                           (2000, 8, 256, 64, 32, 7168), (33, 3, 5, 1, 2, 8)])
def test_gather_reduce(T, k, E, g0, El, N):
    rng = np.random.default_rng(T + N)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    srt = sort_by_expert(ids, E, g0, El)
    inv = srt["inv_pos"].reshape(T, k)
    rows = max(srt["n"], 1)
    y = to_bf16_bits(rng.standard_normal((rows, N)).astype(np.float32))
    w = rng.uniform(0, 1, (T, k)).astype(np.float32)
    o = gather_reduce(y, True, inv, w)
    g = gpu_gather_reduce(y, True, inv, w)
    check_bf16(g, o["out"], o["abs_sum"], "gather_reduce bf16")
    none = np.all(inv < 0, axis=1)
    assert not g[none].any()
    g32 = gpu_gather_reduce(y, True, inv, w, m.MOE_F32)
    check_f32(g32, o["out"], o["abs_sum"], "gather_reduce f32")
    yf = (rng.standard_normal((rows, N))).astype(np.float32)
    o2 = gather_reduce(yf, False, inv, w)
    g2 = gpu_gather_reduce(yf, False, inv, w, m.MOE_F32)
    check_f32(g2, o2["out"], o2["abs_sum"], "gather_reduce f32 in")


def test_gather_reduce_k1_is_exact_unsort():
    rng = np.random.default_rng(3)
    T, E, N = 500, 7, 64
    ids = rng.integers(0, E, (T, 1)).astype(np.int32)
    srt = sort_by_expert(ids, E, 0, E)
    y = to_bf16_bits(rng.standard_normal((T, N)).astype(np.float32))
    g = gpu_gather_reduce(y, True, srt["inv_pos"].reshape(T, 1), np.ones((T, 1), np.float32))
    assert_bits_equal(g, y[srt["inv_pos"]], "k=1 unsort")


def gpu_gather_reduce_backward(dout, y, inv, w, gs, E, g0, El, m_cap):
    T, k = inv.shape
    N = dout.shape[1]
    dy = torch.full((m_cap, N), 9.0, dtype=torch.bfloat16, device="cuda")
    dw = torch.full((T, k), 7.0, dtype=torch.float32, device="cuda")
    quant = N <= 8192
    q = torch.full((m_cap, N), 0x55, dtype=torch.uint8, device="cuda") if quant else None
    qs = torch.full((m_cap,), 5.0, dtype=torch.float32, device="cuda") if quant else None
    qa = torch.full((m_cap,), 5.0, dtype=torch.float32, device="cuda") if quant else None
    print(f"gather_reduce_backward T={T} k={k} N={N} E={E} g0={g0} El={El} m_cap={m_cap} quant={quant}", flush=True)
    m.moe_gather_reduce_backward(dev_bf16(dout), dev_bf16(y), dev_i32(inv), dev_f32(w), T, k, N, dev_i32(gs), E, g0,
                                 El, m_cap, dy, dw, q, qs, qa)
    torch.cuda.synchronize()
    return host(dy), host(dw), ((host(q), host(qs), host(qa)) if quant else None)


@pytest.mark.parametrize("T,k,E,g0,El,N,extra", [(256, 2, 8, 0, 8, 1024, 0), (4096, 8, 64, 0, 64, 2048, 0),
                                                 (600, 8, 256, 64, 32, 7168, 40), (33, 3, 5, 1, 2, 8, 5),
                                                 (90, 4, 16, 0, 16, 520, 0), (40, 2, 4, 0, 4, 16384, 3)])
def test_gather_reduce_backward(T, k, E, g0, El, N, extra):
    """dy bit-exact (one float32 product, one bf16 rounding), dw under the
    float32 rule; rows past the local ones zero; non-local slots dw = 0."""
    rng = np.random.default_rng(T + N + k)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    srt = sort_by_expert(ids, E, g0, El)
    inv = srt["inv_pos"].reshape(T, k)
    n = int(srt["n"])
    m_cap = n + extra
    y = to_bf16_bits(rng.standard_normal((max(m_cap, 1), N)).astype(np.float32))[:m_cap]
    dout = to_bf16_bits((rng.standard_normal((T, N)) * 1e-2).astype(np.float32))
    w = rng.uniform(0, 1, (T, k)).astype(np.float32)
    o = gather_reduce_backward(dout, y, inv, w, m_cap, n)
    gdy, gdw, gq = gpu_gather_reduce_backward(dout, y, inv, w, srt["group_sizes"], E, g0, El, m_cap)
    assert_bits_equal(gdy, o["dy"], "dy")
    if gq is not None:      # dy's row quantization formed in the same pass: moe_quantize_rows' bytes
        q, s_, a = quantize_rows(o["dy"], SCALE_ROW_DYNAMIC)
        assert_bits_equal(gq[0], q, "dy row q")
        assert_bits_equal(gq[1], s_, "dy row scale")
        assert_bits_equal(gq[2], a, "dy row amax")
    check_f32(gdw, o["dw64"], o["dw_abs"], "dw")
    assert (gdw[inv < 0] == 0).all()


def test_gather_reduce_backward_group_sizes_summing_past_2_31():
    """Local group sizes that sum past 2^31: the local row count saturates at
    M_cap, so no zero row is written past dy's buffer (the canary rows after
    it keep their fill) and dy and dw are the oracle's with n = M_cap."""
    rng = np.random.default_rng(9)
    T, k, E, N = 64, 2, 3, 64
    ids = rng.integers(0, E, (T, k)).astype(np.int32)
    srt = sort_by_expert(ids, E, 0, E)
    inv = srt["inv_pos"].reshape(T, k)
    m_cap = int(srt["n"])
    y = to_bf16_bits(rng.standard_normal((m_cap, N)).astype(np.float32))
    dout = to_bf16_bits((rng.standard_normal((T, N)) * 1e-2).astype(np.float32))
    w = rng.uniform(0, 1, (T, k)).astype(np.float32)
    big = np.array([1 << 30] * 3, np.int32)
    buf = torch.full((m_cap + 40, N), 9.0, dtype=torch.bfloat16, device="cuda")
    dw = torch.full((T, k), 7.0, dtype=torch.float32, device="cuda")
    print(f"gather_reduce_backward group sizes past 2^31 T={T} k={k} m_cap={m_cap}", flush=True)
    m.moe_gather_reduce_backward(dev_bf16(dout), dev_bf16(y), dev_i32(inv), dev_f32(w), T, k, N, dev_i32(big), E, 0,
                                 E, m_cap, buf, dw, None, None, None)
    torch.cuda.synchronize()
    g = host(buf)
    assert (g[m_cap:] == 0x4110).all(), "rows past dy's buffer were written"
    o = gather_reduce_backward(dout, y, inv, w, m_cap, m_cap)
    assert_bits_equal(g[:m_cap], o["dy"], "dy")
    check_f32(host(dw), o["dw64"], o["dw_abs"], "dw sizes past 2^31")


# ------------------------------------------------------------------ pipelines
def _full_gmm_stage(lhs, ls, wq_kn, ws_, gs, g0, El, got, what):
    """Every element of a bf16 gmm stage output against the oracle (the
    modelled matrix core where the exact value is out of its reach)."""
    o = gmm(lhs, ls, wq_kn, ws_, gs, g0, El)
    N = wq_kn.shape[2]
    return check_bf16(got, o["out"], o["abs_sum"], what,
                      model=lambda idx: gmm_samples(lhs, ls, wq_kn, ws_, gs, g0, El, idx // N, idx % N))


def _weights_kn(path, name):
    w = path.w[name]
    q = host(w.q)
    return (np.ascontiguousarray(q.transpose(0, 2, 1)) if w.nk else q), host(w.scale)


def _forward_stagewise(cfg, data, static=False, fused=None):
    mc = None
    if cfg.E_loc != cfg.E:
        n_loc = int(np.isin(data["ids"], np.arange(cfg.group_offset, cfg.group_offset + cfg.E_loc)).sum())
        mc = ((n_loc + 255) // 256) * 256
    path = ForwardPath(cfg, data, static_act=STATIC_ACT_SCALE if static else None,
                       static_weight=STATIC_WEIGHT_SCALE if static else None, m_cap=mc, fused_quantize=fused)
    print(f"pipeline {cfg.name} static={static} m_cap={path.m_cap} fused={path.fused_quantize}", flush=True)
    path.step()
    torch.cuda.synchronize()
    assert m.moe_debug_check(path.ws_sort) == 0 and m.moe_debug_check(path.ws_gmm) == 0
    mode = SCALE_TENSOR_STATIC if static else SCALE_ROW_DYNAMIC
    # weights: the GPU quantizer against the oracle's (first experts of large weights)
    for name, wb in data["weights"].items():
        kb, nb = cfg.scale_blocks(wb.shape[1], wb.shape[2])
        ne = wb.shape[0] if wb.size <= (1 << 26) else 2
        wq_o, ws_o = quantize_weights(wb[:ne], kb, nb, static_scale=STATIC_WEIGHT_SCALE if static else None)
        wq_g, ws_g = _weights_kn(path, name)
        assert_bits_equal(wq_g[:ne], wq_o, name + " q")
        assert_bits_equal(ws_g[:ne], ws_o, name + " scale")
    # S1 quantize
    xq, xsc, _ = quantize_rows(data["x"], mode, static_scale=STATIC_ACT_SCALE if static else None)
    if not path.fused_quantize:            # the fused pass writes no [T, H] codes
        assert_bits_equal(host(path.xq), xq, "xq")
        assert_bits_equal(host(path.xscale), xsc, "xscale")
    elif static:
        assert_bits_equal(host(path.xscale), xsc, "xscale")
    # S2/S3 sort
    srt = sort_by_expert(data["ids"], cfg.E, cfg.group_offset, cfg.E_loc, xq=xq, xscale=xsc, xscale_mode=mode,
                         m_cap=path.m_cap)
    assert_bits_equal(host(path.perm), srt["perm"], "perm")
    assert_bits_equal(host(path.inv_pos), srt["inv_pos"], "inv_pos")
    assert_bits_equal(host(path.group_sizes), srt["group_sizes"], "group_sizes")
    assert_bits_equal(host(path.xs), srt["xs"], "xs")
    if mode == SCALE_ROW_DYNAMIC:
        assert_bits_equal(host(path.ss), srt["ss"], "ss")
    gs, g0, El, n = srt["group_sizes"], cfg.group_offset, cfg.E_loc, srt["n"]
    ls = srt["ss"] if mode == SCALE_ROW_DYNAMIC else xsc
    if cfg.pipeline == "up":
        wq, ws_ = _weights_kn(path, "w_up")
        _full_gmm_stage(srt["xs"], ls, wq, ws_, gs, g0, El, host(path.y), f"config {cfg.cid} up gmm")
    else:
        for name, buf in (("wi_0", path.a), ("wi_1", path.b)):       # the halves of the fused launch
            wq, ws_ = _weights_kn(path, name)
            _full_gmm_stage(srt["xs"], ls, wq, ws_, gs, g0, El, host(buf), f"config {cfg.cid} {name}")
        a, b = host(path.a), host(path.b)
        assert not a[n:].any() and not b[n:].any()
        # S5: requantization of silu(a)*b from the GPU's own a and b -- bit-exact
        hq, hs, _ = quantize_rows(a, SCALE_ROW_DYNAMIC, x_up_bits=b)
        assert_bits_equal(host(path.hq), hq, "hq")
        assert_bits_equal(host(path.hs), hs, "hs")
        wq, ws_ = _weights_kn(path, "wo")
        _full_gmm_stage(hq, hs, wq, ws_, gs, g0, El, host(path.y), f"config {cfg.cid} wo")
    # S7 from the GPU's y
    y = host(path.y)
    o = gather_reduce(y, True, host(path.inv_pos).reshape(cfg.T, cfg.k), data["topk_w"])
    out = host(path.out)
    check_bf16(out, o["out"], o["abs_sum"], "gather_reduce")
    return out


@pytest.mark.parametrize("cid,static,fused", [(1, False, False), (3, False, False), (3, True, False), (3, True, True)])
def test_up_projection_pipeline_stagewise_and_context(cid, static, fused):
    cfg = CONFIGS[cid]
    data = generate(cfg)
    out = _forward_stagewise(cfg, data, static=static, fused=fused)
    # fp8 vs unquantized bf16, next to the pages' TPU figures (context only)
    rel, mx = rel_norm_diff(out, dense_bf16_reference(cfg, data))
    tab = accuracy_tables()
    page = tab[("rel", "megablox_fp8_static_ep1" if static else "megablox_fp8_dynamic_ep1")][0]
    print(f"config {cid} {'static' if static else 'dynamic'}: rel_norm_diff {rel:.4f} max_abs {mx:.3g} "
          f"(pages, TPU v5p-8 whole layer: {page})")
    assert rel < 0.2


@pytest.mark.timeout(600)
def test_gated_ffn_pipeline_config2_stagewise():
    cfg = CONFIGS[2]
    data = generate(cfg)
    out = _forward_stagewise(cfg, data)
    # fp8 vs unquantized bf16, next to the pages' TPU figures (context only)
    rel, mx = rel_norm_diff(out, dense_bf16_reference(cfg, data))
    page = accuracy_tables()[("rel", "megablox_fp8_dynamic_ep1")][0]
    print(f"config 2 dynamic: rel_norm_diff {rel:.4f} max_abs {mx:.3g} (pages, TPU v5p-8 whole layer: {page})")
    assert rel < 0.2


def test_gated_ffn_small_full_context():
    cfg = scaled_config(2, T=128, H=256, E=8, k=2, I=256)
    data = generate(cfg)
    out = _forward_stagewise(cfg, data)
    rel, _ = rel_norm_diff(out, dense_bf16_reference(cfg, data))
    assert rel < 0.2


@pytest.mark.timeout(900)
def test_expert_slice_pipeline_config4_stagewise():
    cfg = CONFIGS[4]
    data = generate(cfg)
    out = _forward_stagewise(cfg, data)
    inv = (~np.isin(data["ids"], np.arange(64, 96))).all(axis=1)
    assert inv.any() and not out[inv].any()       # tokens with no local expert: zero partial sums


@pytest.mark.timeout(600)
@pytest.mark.parametrize("fused,transposed", [(True, False), (False, False), (True, True)])
def test_backward_pipeline_config5_stagewise(fused, transposed):
    cfg = CONFIGS[5]
    data = generate(cfg)
    path = BackwardPath(cfg, data, STATIC_ACT_SCALE, STATIC_WEIGHT_SCALE, fused_quantize=fused,
                        transposed_x=transposed)
    print(f"pipeline config 5 backward fused={fused} transposed={transposed}", flush=True)
    path.step()
    torch.cuda.synchronize()
    # the weights: the GPU quantizer's first experts against the oracle's; the later stages take the GPU's
    wq_o, ws_o = quantize_weights(data["weights"]["w_up"][:2], 1, 1, static_scale=STATIC_WEIGHT_SCALE)
    wq, ws_ = host(path.w.q), host(path.w.scale)
    assert_bits_equal(wq[:2], wq_o, "w q")
    assert_bits_equal(ws_[:2], ws_o, "w scale")
    xq, xsc, _ = quantize_rows(data["x"], SCALE_TENSOR_STATIC, static_scale=STATIC_ACT_SCALE)
    if not fused:                      # the fused pass writes no [T, H] codes
        assert_bits_equal(host(path.xq), xq, "xq")
    assert_bits_equal(host(path.xscale), xsc, "xscale")
    srt = sort_by_expert(data["ids"], cfg.E, 0, cfg.E, xq=xq, xscale=xsc, xscale_mode=SCALE_TENSOR_STATIC)
    if transposed:                     # X only in the weight-gradient product's layout (its padded columns)
        want = expected_xt(srt["xs"], srt["group_sizes"], 0, cfg.E, path.M, cfg.E)
        used = int(np.sum((srt["group_sizes"] + 127) // 128)) * 128
        assert_bits_equal(host(path.xt)[:, :used], want[:, :used], "xt")
        for key in ("perm", "inv_pos", "group_sizes"):
            assert_bits_equal(host(getattr(path, key)), srt[key], key)
    else:
        assert_bits_equal(host(path.xs), srt["xs"], "xs")
    dq_r, ds_r, _ = quantize_rows(data["dy"], SCALE_ROW_DYNAMIC)
    dq_t, ds_t, _ = quantize_rows(data["dy"], SCALE_TENSOR_DYNAMIC)
    assert_bits_equal(host(path.dyq_r), dq_r, "dy row q")
    assert_bits_equal(host(path.dys_r), ds_r, "dy row scale")
    assert_bits_equal(host(path.dyq_t), dq_t, "dy tensor q")
    assert_bits_equal(host(path.dys_t), ds_t, "dy tensor scale")
    gs = srt["group_sizes"]
    wT = np.ascontiguousarray(wq.transpose(0, 2, 1))
    _full_gmm_stage(dq_r, ds_r, wT, ws_, gs, 0, cfg.E, host(path.dx), "config 5 dX")
    _full_tgmm(srt["xs"], xsc, dq_t, ds_t, gs, cfg.E, host(path.dw), "config 5 dW")


def _full_tgmm(x, xs, d, ds, gs, El, got, what):
    o = tgmm(x, xs, d, ds, gs, 0, El)
    K, N = x.shape[1], d.shape[1]
    check_f32(got, o["out"], o["abs_sum"], what,
              model=lambda idx: tgmm_samples(x, xs, d, ds, gs, 0, El, idx // (K * N), (idx // N) % K, idx % N))


@pytest.mark.parametrize("shape,fuse,transposed", [("small", True, False), ("small", False, False),
                                                   ("small", True, True), ("config2", True, False),
                                                   ("config2", True, True)])
def test_gated_ffn_backward_stagewise(shape, fuse, transposed):
    """The gated FFN's backward after a forward step, every stage against the
    oracle fed the GPU's own inputs for that stage: the combine backward, the
    quantizations and the activation backward bit-exact, the grouped matmuls
    under the float32 / bf16 rules."""
    cfg = scaled_config(2, T=384, H=512, E=8, k=2, I=256) if shape == "small" else CONFIGS[2]
    data = generate(cfg)
    T, H, E, k, I = cfg.T, cfg.H, cfg.E, cfg.k, cfg.I
    fwd = ForwardPath(cfg, data)
    rng = np.random.default_rng(77)
    dout_bits = to_bf16_bits((rng.standard_normal((T, H)) * 1e-2).astype(np.float32))
    bwd = FFNBackwardPath(fwd, data, dev_bf16(dout_bits), fuse_dy_quant=fuse, transposed_x=transposed)
    print(f"gated ffn backward {shape} fuse_dy_quant={fuse} transposed_x={transposed} T={T} H={H} E={E} k={k} I={I}",
          flush=True)
    fwd.step()
    bwd.step()
    torch.cuda.synchronize()
    for ws in (bwd.ws_q, bwd.ws_qx, bwd.ws_sort, bwd.ws_gmm_h, bwd.ws_gmm_x, bwd.ws_tgmm_o, bwd.ws_tgmm_01) + \
            ((bwd.ws_xt,) if transposed else ()):
        assert m.moe_debug_check(ws) == 0
    inv = host(fwd.inv_pos).reshape(T, k)
    gs = host(fwd.group_sizes)
    Mc, n = fwd.m_cap, int(gs.sum())
    # combine backward from the GPU's forward output y
    o = gather_reduce_backward(dout_bits, host(fwd.y), inv, data["topk_w"], Mc, n)
    dy = host(bwd.dy)
    assert_bits_equal(dy, o["dy"], "dy")
    check_f32(host(bwd.dw_router), o["dw64"], o["dw_abs"], "dw_router")
    # dy quantized per row and per tensor
    q, s_, _ = quantize_rows(dy, SCALE_ROW_DYNAMIC)
    assert_bits_equal(host(bwd.dyq_r), q, "dy row q")
    assert_bits_equal(host(bwd.dys_r), s_, "dy row scale")
    qt, st_, _ = quantize_rows(dy, SCALE_TENSOR_DYNAMIC)
    assert_bits_equal(host(bwd.dyq_t), qt, "dy tensor q")
    assert_bits_equal(host(bwd.dys_t), st_, "dy tensor scale")
    # backward weights: wo^T and [W0 | W1]^T quantized per channel of the backward's output
    # (all experts on the small shape, the first two at full size; the later stages' oracles then take the
    # GPU's weights, verified here)
    ne = E if shape == "small" else 2
    woT_q, woT_s = np.ascontiguousarray(host(bwd.woT.q).transpose(0, 2, 1)), host(bwd.woT.scale)   # [E, H, I]
    oq, os_ = quantize_weights(np.ascontiguousarray(data["weights"]["wo"][:ne].transpose(0, 2, 1)), 1, I)
    assert_bits_equal(woT_q[:ne], oq, "wo^T q")
    assert_bits_equal(woT_s[:ne], os_, "wo^T scale")
    w01T_q, w01T_s = np.ascontiguousarray(host(bwd.w01T.q).transpose(0, 2, 1)), host(bwd.w01T.scale)  # [E, 2I, H]
    w01 = np.concatenate([data["weights"]["wi_0"][:ne], data["weights"]["wi_1"][:ne]], axis=2)
    oq, os_ = quantize_weights(np.ascontiguousarray(w01.transpose(0, 2, 1)), 1, H)
    assert_bits_equal(w01T_q[:ne], oq, "[W0|W1]^T q")
    assert_bits_equal(w01T_s[:ne], os_, "[W0|W1]^T scale")
    # dh = dy wo^T
    dh = host(bwd.dh)
    _full_gmm_stage(q, s_, woT_q, woT_s, gs, 0, E, dh, f"{shape} dh")
    assert not dh[n:].any()
    # dwo = h^T dy, h requantized with one tensor scale from the GPU's a and b
    a, b = host(fwd.a), host(fwd.b)
    hq, hs, _ = quantize_rows(a, SCALE_TENSOR_DYNAMIC, x_up_bits=b)
    assert_bits_equal(host(bwd.hq_t), hq, "h tensor q")
    assert_bits_equal(host(bwd.hs_t), hs, "h tensor scale")
    _full_tgmm(hq, hs, qt, st_, gs, E, host(bwd.dwo), f"{shape} dwo")
    # activation backward
    da, db = silu_mul_backward(a, b, dh)
    dab = host(bwd.dab)
    assert_bits_equal(dab[:, :I], da, "da")
    assert_bits_equal(dab[:, I:], db, "db")
    q2, s2, _ = quantize_rows(dab, SCALE_ROW_DYNAMIC)
    assert_bits_equal(host(bwd.dabq_r), q2, "[da|db] row q")
    assert_bits_equal(host(bwd.dabs_r), s2, "[da|db] row scale")
    q2t, s2t, _ = quantize_rows(dab, SCALE_TENSOR_DYNAMIC)
    assert_bits_equal(host(bwd.dabq_t), q2t, "[da|db] tensor q")
    assert_bits_equal(host(bwd.dabs_t), s2t, "[da|db] tensor scale")
    # dxs = [da|db] [W0|W1]^T
    dxs = host(bwd.dxs)
    _full_gmm_stage(q2, s2, w01T_q, w01T_s, gs, 0, E, dxs, f"{shape} dx sorted")
    # dw01 = x^T [da|db], x requantized with one tensor scale and sorted
    xq, xsc, xam = quantize_rows(data["x"], SCALE_TENSOR_DYNAMIC)
    assert_bits_equal(host(fwd.xamax), xam, "x token maxima (forward's fused pass)")
    assert_bits_equal(host(bwd.xs_scale), xsc, "x tensor scale")
    srt = sort_by_expert(data["ids"], E, 0, E, xq=xq, xscale=xsc, xscale_mode=SCALE_TENSOR_DYNAMIC, m_cap=Mc)
    if transposed:   # [T, H] codes, then the forward's sort gathers them into the product's layout
        assert_bits_equal(host(bwd.xq_t), xq, "x tensor codes")
        used = int(np.sum((gs.astype(np.int64) + 127) // 128)) * 128
        want = expected_xt(srt["xs"], gs, 0, E, Mc, E)
        assert_bits_equal(host(bwd.xt)[:, :used], want[:, :used], "x in the product's layout")
    else:
        assert_bits_equal(host(bwd.xs_t), srt["xs"], "x sorted")
    _full_tgmm(srt["xs"], xsc, q2t, s2t, gs, E, host(bwd.dw01), f"{shape} dw01")
    # dx: unit-weight un-sort of dxs
    o = gather_reduce(dxs, True, inv, np.ones((T, k), np.float32))
    check_bf16(host(bwd.dx), o["out"], o["abs_sum"], "dx")
    # fp8 gradients against an unquantized bf16 backward, next to the pages' TPU figures (context only)
    rdx, rw0, rw1, rwo = dense_bf16_backward_reference(cfg, data, dout_bits)
    dw01 = host(bwd.dw01)
    rel = {"grad_wi_0": rel_norm_diff_f(dw01[:, :, :I], rw0), "grad_wi_1": rel_norm_diff_f(dw01[:, :, I:], rw1),
           "grad_wo": rel_norm_diff_f(host(bwd.dwo), rwo), "dx": rel_norm_diff(host(bwd.dx), rdx)[0]}
    page = accuracy_tables()[("rel", "megablox_fp8_dynamic_ep1")]
    print(f"{shape} backward, fp8 vs bf16 dense relative_norm_diff: grad_wi_0 {rel['grad_wi_0']:.4f} "
          f"grad_wi_1 {rel['grad_wi_1']:.4f} grad_wo {rel['grad_wo']:.4f} dx {rel['dx']:.4f} (pages, TPU v5p-8 "
          f"whole layer, dynamic: grad_wi_0 {page[3]} grad_wi_1 {page[4]} grad_wo {page[5]} state_grad {page[1]})",
          flush=True)
    assert all(v < 0.3 for v in rel.values()), rel


def test_expert_slice_with_no_routed_rows_forward_and_backward():
    """One GPU's expert slice that no token routes to (n = 0) with spare row
    capacity: the sort metadata matches the oracle's, every expert row and
    partial sum is zero, the zero rows requantize to code 0 with scale 1, and
    every gradient of the backward is zero."""
    cfg = scaled_config(4, T=256, H=512, E=16, k=2, I=256, group_offset=4, num_local_experts=4)
    data = generate(cfg)
    rng = np.random.default_rng(11)
    others = np.setdiff1d(np.arange(cfg.E), np.arange(4, 8))
    data["ids"] = np.stack([rng.permutation(others)[:cfg.k] for _ in range(cfg.T)]).astype(np.int32)
    Mc = 256
    fwd = ForwardPath(cfg, data, m_cap=Mc)
    print(f"expert slice with no routed rows: m_cap={Mc} fused={fwd.fused_quantize}", flush=True)
    fwd.step()
    torch.cuda.synchronize()
    assert m.moe_debug_check(fwd.ws_sort) == 0 and m.moe_debug_check(fwd.ws_gmm) == 0
    srt = sort_by_expert(data["ids"], cfg.E, 4, 4, m_cap=Mc)
    assert srt["n"] == 0
    assert_bits_equal(host(fwd.perm), srt["perm"], "perm")
    assert_bits_equal(host(fwd.inv_pos), srt["inv_pos"], "inv_pos")
    assert_bits_equal(host(fwd.group_sizes), srt["group_sizes"], "group_sizes")
    assert not host(fwd.ab).any() and not host(fwd.y).any() and not host(fwd.out).any()
    hq, hs, _ = quantize_rows(host(fwd.a), SCALE_ROW_DYNAMIC, x_up_bits=host(fwd.b))
    assert_bits_equal(host(fwd.hq), hq, "hq")
    assert_bits_equal(host(fwd.hs), hs, "hs")
    assert (hs == 1.0).all()
    dout = dev_bf16(to_bf16_bits(rng.standard_normal((cfg.T, cfg.H)).astype(np.float32)))
    for transposed in (False, True):
        bwd = FFNBackwardPath(fwd, data, dout, transposed_x=transposed)
        bwd.dw01.fill_(7.0)
        bwd.step()
        torch.cuda.synchronize()
        for name in ("dy", "dw_router", "dh", "dwo", "dab", "dxs", "dw01", "dx"):
            assert not host(getattr(bwd, name)).any(), (name, transposed)
    q2, s2, _ = quantize_rows(host(bwd.dab), SCALE_ROW_DYNAMIC)
    assert_bits_equal(host(bwd.dabq_r), q2, "[da|db] row q")
    assert_bits_equal(host(bwd.dabs_r), s2, "[da|db] row scale")
    q2t, s2t, _ = quantize_rows(host(bwd.dab), SCALE_TENSOR_DYNAMIC)
    assert_bits_equal(host(bwd.dabq_t), q2t, "[da|db] tensor q")
    assert_bits_equal(host(bwd.dabs_t), s2t, "[da|db] tensor scale")


@pytest.mark.parametrize("transposed", [False, True])
def test_gated_ffn_backward_hip_graph_replays_match_eager(transposed):
    """The backward step as a HIP graph: every replay, with scribbled outputs
    and eager steps between replays, leaves the eager step's bits in every
    buffer the step writes (of the transposed x layout: the columns up to the
    last group's padded end, all the product reads)."""
    cfg = scaled_config(2, T=384, H=512, E=8, k=2, I=256)
    data = generate(cfg)
    fwd = ForwardPath(cfg, data)
    rng = np.random.default_rng(5)
    dout = dev_bf16(to_bf16_bits((rng.standard_normal((cfg.T, cfg.H)) * 1e-2).astype(np.float32)))
    bwd = FFNBackwardPath(fwd, data, dout, transposed_x=transposed)
    print(f"gated ffn backward graph replays transposed_x={transposed}", flush=True)
    fwd.step()
    bwd.step()
    torch.cuda.synchronize()
    used = int(((host(fwd.group_sizes).astype(np.int64) + 127) // 128).sum()) * 128
    view = lambda k: getattr(bwd, k)[:, :used] if k == "xt" else getattr(bwd, k)
    ref = {k: view(k).clone() for k in bwd.OUTPUTS}
    bwd.capture_graph(warmup=1)
    for rep in range(3):
        for k in bwd.OUTPUTS:
            getattr(bwd, k).view(torch.uint8).fill_(0xA5)
        torch.cuda.synchronize()
        bwd.replay()
        torch.cuda.synchronize()
        for k in bwd.OUTPUTS:
            assert torch.equal(view(k).view(torch.uint8), ref[k].view(torch.uint8)), (rep, k)
        bwd.step()
        torch.cuda.synchronize()


@pytest.mark.parametrize("transposed", [False, True])
def test_backward_config5_hip_graph_replays_match_eager(transposed):
    """The up-projection backward (reduced config-5 shape) as a HIP graph: every
    replay, with scribbled outputs and eager steps between, leaves the eager
    step's bits in every buffer the step writes (of the transposed X layout:
    the columns up to the last group's padded end, all the product reads)."""
    cfg = scaled_config(5, T=512, H=512, E=8, k=4, I=256)
    data = generate(cfg)
    path = BackwardPath(cfg, data, STATIC_ACT_SCALE, STATIC_WEIGHT_SCALE, transposed_x=transposed)
    print(f"config 5 backward graph replays transposed={transposed}", flush=True)
    path.step()
    torch.cuda.synchronize()
    used = int(((host(path.group_sizes).astype(np.int64) + 127) // 128).sum()) * 128
    view = lambda k: getattr(path, k)[:, :used] if k == "xt" else getattr(path, k)
    ref = {k: view(k).clone() for k in path.OUTPUTS}
    path.capture_graph(warmup=1)
    for rep in range(3):
        for k in path.OUTPUTS:
            getattr(path, k).view(torch.uint8).fill_(0xA5)
        torch.cuda.synchronize()
        path.replay()
        torch.cuda.synchronize()
        for k in path.OUTPUTS:
            assert torch.equal(view(k).view(torch.uint8), ref[k].view(torch.uint8)), (rep, k)
        path.step()
        torch.cuda.synchronize()


@pytest.mark.parametrize("cid", [2, 4])
def test_forward_step_hip_graph_replays_match_eager(cid):
    """The bench's timed step is a HIP graph of the forward step: every
    replay, with eager steps and host synchronizations between replays,
    leaves exactly the eager step's bits in every buffer the step writes."""
    cfg = CONFIGS[cid]
    data = generate(cfg)
    n = int(((data["ids"] >= cfg.group_offset) & (data["ids"] < cfg.group_offset + cfg.E_loc)).sum())
    from workloads import m_cap_for
    share = 8 if cfg.E_loc < cfg.E else 1
    path = ForwardPath(cfg, data, m_cap=m_cap_for(cfg, n), share=share)
    names = ([] if path.fused_quantize else ["xq", "xscale"]) + \
        ["perm", "inv_pos", "group_sizes", "xs", "ss", "y", "out"] + \
        (["a", "b", "hq", "hs"] if cfg.pipeline == "ffn" else [])
    path.step()
    torch.cuda.synchronize()
    ref = {k: getattr(path, k).clone() for k in names}
    path.capture_graph(warmup=1)
    for rep in range(3):
        for k in names:                      # scribble over the outputs between replays
            if share > 1 and k in ("xq", "xscale"):
                continue                     # the other GPUs' slots are written once, at set-up
            getattr(path, k).view(torch.uint8).fill_(0xA5)
        torch.cuda.synchronize()
        path.replay()
        torch.cuda.synchronize()
        for k in names:
            assert torch.equal(getattr(path, k).view(torch.uint8), ref[k].view(torch.uint8)), (cid, rep, k)
        path.step()                          # an eager step in between
        torch.cuda.synchronize()
