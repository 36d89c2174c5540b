"""GPU parity of the quantizers and the ragged sort against the oracle:
bit-exact bytes, scales, permutations and group sizes."""

import numpy as np
import pytest
import torch

import moe_fp8_grouped_amd as m
from oracle.quantize import (SCALE_ROW_DYNAMIC, SCALE_TENSOR_DYNAMIC, SCALE_TENSOR_STATIC, quantize_rows,
                             quantize_weights)
from oracle.sort import sort_by_expert
from tests.parity import assert_bits_equal, dev_bf16, dev_f32, dev_i32, dev_u8, host
from workloads import CONFIGS, STATIC_ACT_SCALE, STATIC_WEIGHT_SCALE, generate, scaled_config, to_bf16_bits

pytestmark = pytest.mark.gpu


def gpu_quantize(x_bits, mode, static=0.0, up_bits=None):
    R, C = x_bits.shape
    x = dev_bf16(x_bits)
    up = dev_bf16(up_bits) if up_bits is not None else None
    q = torch.empty((R, C), dtype=torch.uint8, device="cuda")
    s = torch.empty((R if mode == m.MOE_SCALE_ROW_DYNAMIC else 1,), dtype=torch.float32, device="cuda")
    amax = torch.empty((R,), dtype=torch.float32, device="cuda")
    ws = m.workspace(m.MOE_OP_QUANTIZE_ROWS, R, C, mode)
    act = m.MOE_ACT_SILU_MUL if up is not None else m.MOE_ACT_NONE
    print(f"quantize R={R} C={C} mode={mode} act={act}", flush=True)
    m.moe_quantize_rows(x, up, act, R, C, mode, static, q, s, amax, ws)
    torch.cuda.synchronize()
    return host(q), host(s), host(amax)


def _bits(rng, shape, scale=1.0):
    return to_bf16_bits((rng.standard_normal(shape) * scale).astype(np.float32))


@pytest.mark.parametrize("R,C", [(1, 16), (7, 48), (256, 512), (300, 2048), (33, 7168), (5, 8192), (3, 8208),
                                 (5, 256), (9, 768), (3, 1280), (1024, 2064), (2048, 4112), (2049, 4112)])
def test_row_quantize_bit_exact(R, C):
    rng = np.random.default_rng(R * 7 + C)
    x = _bits(rng, (R, C), 3.0)
    x[0, :5] = 0x8000                  # -0.0
    if R > 2:
        x[2] = 0                       # an all-zero row
        x[1, 3] = to_bf16_bits(np.array([1e-39], np.float32))[0]   # subnormal input
    q, s, a = gpu_quantize(x, m.MOE_SCALE_ROW_DYNAMIC)
    qo, so, ao = quantize_rows(x, SCALE_ROW_DYNAMIC)
    assert_bits_equal(q, qo, "q")
    assert_bits_equal(s, so, "scale")
    assert_bits_equal(a, ao, "row_amax")


def test_row_quantize_config_inputs():
    for cid in (1, 2):
        d = generate(CONFIGS[cid], with_weights=False)
        q, s, _ = gpu_quantize(d["x"], m.MOE_SCALE_ROW_DYNAMIC)
        qo, so, _ = quantize_rows(d["x"], SCALE_ROW_DYNAMIC)
        assert_bits_equal(q, qo, f"config {cid} q")
        assert_bits_equal(s, so, f"config {cid} scale")
    # config 4: one GPU's share (1/8 of the tokens) with its outlier rows
    d = generate(CONFIGS[4], with_weights=False)
    share = d["x"][:1024]
    q, s, _ = gpu_quantize(share, m.MOE_SCALE_ROW_DYNAMIC)
    qo, so, _ = quantize_rows(share, SCALE_ROW_DYNAMIC)
    assert_bits_equal(q, qo, "config 4 share q")
    assert_bits_equal(s, so, "config 4 share scale")


def test_tensor_and_static_modes():
    rng = np.random.default_rng(5)
    dy = _bits(rng, (4096, 1536), 1e-3)
    q, s, a = gpu_quantize(dy, m.MOE_SCALE_TENSOR_DYNAMIC)
    qo, so, ao = quantize_rows(dy, SCALE_TENSOR_DYNAMIC)
    assert_bits_equal(q, qo, "tensor q")
    assert_bits_equal(s, so, "tensor scale")
    assert_bits_equal(a, ao, "tensor row_amax")
    x = _bits(rng, (512, 4096), 1.5)         # 1.5 sigma: part of it saturates at +-448
    q, s, _ = gpu_quantize(x, m.MOE_SCALE_TENSOR_STATIC, STATIC_ACT_SCALE)
    qo, so, _ = quantize_rows(x, SCALE_TENSOR_STATIC, static_scale=STATIC_ACT_SCALE)
    assert np.isin(qo, [0x7E, 0xFE]).sum() > 100
    assert_bits_equal(q, qo, "static q")
    assert_bits_equal(s, so, "static scale")


@pytest.mark.parametrize("R,C,act", [(4096, 1536, 0), (300, 7168, 0), (999, 768, 1), (5, 16, 0)])
def test_tensor_scale_from_row_maxima(R, C, act):
    """MOE_SCALE_TENSOR_FROM_ROW_AMAX fed the GPU's own row-mode maxima: the
    tensor-dynamic codes and scale of the oracle, bit for bit."""
    rng = np.random.default_rng(R + C)
    x = _bits(rng, (R, C), 2.0)
    x[R // 2] = 0
    up = _bits(rng, (R, C), 1.0) if act else None
    _, _, amax = gpu_quantize(x, m.MOE_SCALE_ROW_DYNAMIC, up_bits=up)
    xd = dev_bf16(x)
    ud = dev_bf16(up) if act else None
    q = torch.empty((R, C), dtype=torch.uint8, device="cuda")
    sc = torch.empty((1,), dtype=torch.float32, device="cuda")
    print(f"quantize tensor-from-row-amax R={R} C={C} act={act}", flush=True)
    m.moe_quantize_rows(xd, ud, act, R, C, m.MOE_SCALE_TENSOR_FROM_ROW_AMAX, 0.0, q, sc, dev_f32(amax), None)
    torch.cuda.synchronize()
    qo, so, _ = quantize_rows(x, SCALE_TENSOR_DYNAMIC, x_up_bits=up)
    assert_bits_equal(host(q), qo, "q")
    assert_bits_equal(host(sc), so, "scale")


@pytest.mark.parametrize("R,C", [(64, 768), (33, 768), (7, 256), (37, 2048), (2, 16), (37, 4096), (3, 8192)])
def test_silu_mul_requantize_bit_exact(R, C):
    rng = np.random.default_rng(R + C)
    a = _bits(rng, (R, C), 4.0)
    b = _bits(rng, (R, C), 1.0)
    a[0, :4] = to_bf16_bits(np.array([100.0, -100.0, 0.0, -0.0], np.float32))
    q, s, _ = gpu_quantize(a, m.MOE_SCALE_ROW_DYNAMIC, up_bits=b)
    qo, so, _ = quantize_rows(a, SCALE_ROW_DYNAMIC, x_up_bits=b)
    assert_bits_equal(q, qo, "silu q")
    assert_bits_equal(s, so, "silu scale")


@pytest.mark.parametrize("R,C,act,mode", [(37, 768, 1, 0), (4, 256, 1, 0), (9, 2048, 1, 0), (5, 256, 0, 0),
                                          (300, 512, 0, 1), (70, 96 * 8, 0, 2), (5, 3072, 1, 0), (100, 4096, 0, 1),
                                          (64, 7168, 0, 2)])
def test_quantize_rows_strided_bit_exact(R, C, act, mode):
    """Rows read 2C elements apart out of one [R, 2C] buffer (a | b, the
    gated FFN's fused input-projection output): the same bits as the
    oracle on the two halves."""
    rng = np.random.default_rng(R + 3 * C + act)
    ab = _bits(rng, (R, 2 * C), 4.0)
    ab[0, :4] = to_bf16_bits(np.array([100.0, -100.0, 0.0, -0.0], np.float32))
    a_bits, b_bits = np.ascontiguousarray(ab[:, :C]), np.ascontiguousarray(ab[:, C:])
    d = dev_bf16(ab)
    x, up = d[:, :C], (d[:, C:] if act else None)
    static = STATIC_ACT_SCALE if mode == m.MOE_SCALE_TENSOR_STATIC else 0.0
    q = torch.empty((R, C), dtype=torch.uint8, device="cuda")
    sc = torch.empty((R if mode == m.MOE_SCALE_ROW_DYNAMIC else 1,), dtype=torch.float32, device="cuda")
    amax = torch.empty((R,), dtype=torch.float32, device="cuda")
    ws = m.workspace(m.MOE_OP_QUANTIZE_ROWS, R, C, mode)
    print(f"quantize strided R={R} C={C} ld={2 * C} act={act} mode={mode}", flush=True)
    m.moe_quantize_rows_strided(x, up, 2 * C, act, R, C, mode, static, q, sc, amax, ws)
    torch.cuda.synchronize()
    qo, so, ao = quantize_rows(a_bits, mode, static_scale=static if static else None,
                               x_up_bits=b_bits if act else None)
    assert_bits_equal(host(q), qo, "strided q")
    assert_bits_equal(host(sc), so, "strided scale")
    assert_bits_equal(host(amax), ao, "strided row_amax")


def test_silu_mul_backward_every_finite_bf16_gate_value():
    """da, db bit-exact against the oracle for every finite bfloat16 gate a
    (with random b and dh), read from and written to the column halves of
    [R, 2C] buffers as the layer backward lays them out."""
    from oracle.quantize import silu_mul_backward
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    a = bits[(bits & 0x7f80) != 0x7f80]                 # finite values only
    C = 256
    R = -(-a.size // C)
    a = np.concatenate([a, np.zeros(R * C - a.size, np.uint16)]).reshape(R, C)
    rng = np.random.default_rng(21)
    b = _bits(rng, (R, C), 1.0)
    dh = _bits(rng, (R, C), 1e-2)
    dh[0, :8] = to_bf16_bits(np.array([1e-38, -1e-38, 3e38, 0.0, -0.0, 1.0, 1e-30, 5e-39], np.float32))
    ab = np.concatenate([a, b], axis=1)
    d_ab = dev_bf16(ab)
    d_dh = dev_bf16(dh)
    out = torch.full((R, 2 * C), 7, dtype=torch.bfloat16, device="cuda")
    print(f"silu_mul_backward R={R} C={C} lda={2 * C} ldo={2 * C}", flush=True)
    m.moe_silu_mul_backward(d_ab[:, :C], d_ab[:, C:], 2 * C, d_dh, R, C, out[:, :C], out[:, C:], 2 * C)
    torch.cuda.synchronize()
    got = host(out)
    da, db = silu_mul_backward(a, b, dh)
    assert_bits_equal(got[:, :C], da, "da")
    assert_bits_equal(got[:, C:], db, "db")


def test_silu_every_finite_bf16_gate_value():
    """silu(a) for every finite bfloat16 a, observed exactly: row i holds a_i
    and fifteen zeros with b = 1, so its row absmax is |silu(a_i)| in float32
    and its first code is +-448 (the sign) -- bit for bit against the oracle.
    The kernel's SiLU quotient uses a reciprocal, one Newton step and one
    correction instead of the IEEE divide; this covers its whole input set."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = (bits & 0x7F80) != 0x7F80
    a_vals = bits[finite]
    R, C = a_vals.size, 16
    a = np.zeros((R, C), np.uint16)
    a[:, 0] = a_vals
    b = np.full((R, C), 0x3F80, np.uint16)          # 1.0
    q, s, amax = gpu_quantize(a, m.MOE_SCALE_ROW_DYNAMIC, up_bits=b)
    qo, so, ao = quantize_rows(a, SCALE_ROW_DYNAMIC, x_up_bits=b)
    assert_bits_equal(amax, ao, "|silu(a)| over every finite bf16 a")
    assert_bits_equal(s, so, "scale")
    assert_bits_equal(q, qo, "codes")


@pytest.mark.parametrize("T,k,E,g0,El,H,mode,extra,want_scale", [
    (4096, 8, 64, 0, 64, 2048, 0, 0, False),        # the gated FFN's routing shape
    (2000, 8, 256, 64, 32, 7168, 0, 37, True),      # a local expert slice, zero rows after n, every token's scale
    (500, 2, 8, 0, 8, 512, 2, 5, True),             # static scale
    (300, 3, 5, 1, 3, 8208, 0, 3, False),           # rows too long for registers (two passes)
    (0, 4, 8, 0, 8, 64, 0, 4, False),               # no tokens: the window is all zeros
    (4096, 8, 64, 0, 64, 2048, 3, 0, True),         # one tensor scale from the tokens' maxima
    (2000, 8, 256, 64, 32, 7168, 3, 37, True),      # the same on a local slice
])
def test_quantize_sort_fused_bit_exact(T, k, E, g0, El, H, mode, extra, want_scale):
    """moe_quantize_sort_by_expert writes what moe_quantize_rows then
    moe_sort_by_expert write: the oracle's quantization and stable sort."""
    rng = np.random.default_rng(T + H + mode)
    x = _bits(rng, (T, H), 2.0)
    if T > 2:
        x[1] = 0                                     # an all-zero row (scale 1)
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32) if T else \
        np.zeros((0, k), np.int32)
    static = STATIC_ACT_SCALE if mode == m.MOE_SCALE_TENSOR_STATIC else None
    from_rows = mode == m.MOE_SCALE_TENSOR_FROM_ROW_AMAX
    xq, xsc, xam = quantize_rows(x, SCALE_TENSOR_DYNAMIC if from_rows else mode, static_scale=static)
    n = int(((ids >= g0) & (ids < g0 + El)).sum())
    m_cap = n + extra
    o = sort_by_expert(ids, E, g0, El, xq=xq, xscale=xsc, xscale_mode=SCALE_TENSOR_DYNAMIC if from_rows else mode,
                       m_cap=m_cap)
    dev = lambda shape, dt: torch.empty(shape, dtype=dt, device="cuda")
    perm, inv = dev(T * k, torch.int32), dev(T * k, torch.int32)
    gs = dev(E, torch.int32)
    xs = torch.full((m_cap, H), 0x55, dtype=torch.uint8, device="cuda")
    ss = torch.full((m_cap,), 7.0, dtype=torch.float32, device="cuda") if mode == m.MOE_SCALE_ROW_DYNAMIC else None
    sc = dev((T if mode == m.MOE_SCALE_ROW_DYNAMIC else 1,), torch.float32) if want_scale else None
    amax = dev((T,), torch.float32) if mode == m.MOE_SCALE_ROW_DYNAMIC and want_scale else None
    if from_rows:
        amax = dev_f32(xam)                          # the tokens' maxima, as a row-mode pass writes them
    ws = m.workspace(m.MOE_OP_SORT_BY_EXPERT, T * k, 0, 0, E)
    print(f"quantize+sort T={T} k={k} E={E} g0={g0} El={El} H={H} mode={mode} m_cap={m_cap}", flush=True)
    m.moe_quantize_sort_by_expert(dev_bf16(x) if T else dev((0, H), torch.bfloat16), T, H, mode, static or 0.0,
                                  dev_i32(ids), k, E, g0, El, m_cap, perm, inv, gs, xs, ss, sc, ws, row_amax=amax)
    assert m.moe_debug_check(ws) == 0
    assert_bits_equal(host(perm), o["perm"], "perm")
    assert_bits_equal(host(inv), o["inv_pos"], "inv_pos")
    assert_bits_equal(host(gs), o["group_sizes"], "group_sizes")
    assert_bits_equal(host(xs), o["xs"], "xs")
    if ss is not None:
        assert_bits_equal(host(ss), o["ss"], "ss")
    if sc is not None:
        assert_bits_equal(host(sc), xsc, "token scales")
    if amax is not None and mode == m.MOE_SCALE_ROW_DYNAMIC:
        assert_bits_equal(host(amax), xam, "token maxima")


def test_empty_rows_tensor_dynamic():
    ws = m.workspace(m.MOE_OP_QUANTIZE_ROWS, 0, 32, m.MOE_SCALE_TENSOR_DYNAMIC)
    s = torch.zeros(1, dtype=torch.float32, device="cuda")
    dummy = torch.zeros(16, dtype=torch.uint8, device="cuda")
    m.moe_quantize_rows(None, None, 0, 0, 32, m.MOE_SCALE_TENSOR_DYNAMIC, 0.0, None, s, None, ws)
    torch.cuda.synchronize()
    assert host(s)[0] == 1.0
    del dummy


@pytest.mark.parametrize("E,K,N,kb,nb,static,nk", [
    (8, 512, 1024, 1, 1024, None, 0), (8, 512, 1024, 1, 1024, None, 1),      # per channel
    (8, 512, 1024, 4, 1024, None, 1),                                         # 128-row K blocks
    (2, 1024, 512, 8, 4, None, 1), (2, 512, 1024, 4, 8, None, 0),            # 128 x 128 blocks
    (4, 256, 256, 1, 1, STATIC_WEIGHT_SCALE, 0), (4, 256, 256, 2, 256, STATIC_WEIGHT_SCALE, 1)])
def test_weight_quantizer_bit_exact(E, K, N, kb, nb, static, nk):
    rng = np.random.default_rng(E * K + N + kb)
    w = _bits(rng, (E, K, N), 0.02)
    w[0, :K // kb, :N // nb] = 0                                              # an all-zero block
    qd = torch.empty((E, N, K) if nk else (E, K, N), dtype=torch.uint8, device="cuda")
    sd = torch.empty((E, kb, 1, nb), dtype=torch.float32, device="cuda")
    mode = m.MOE_SCALE_TENSOR_STATIC if static else m.MOE_SCALE_ROW_DYNAMIC
    print(f"quantize_weights E={E} K={K} N={N} kb={kb} nb={nb} nk={nk}", flush=True)
    m.moe_quantize_weights(dev_bf16(w), E, K, N, kb, nb, mode, static or 0.0, nk, qd, sd)
    torch.cuda.synchronize()
    qo, so = quantize_weights(w, kb, nb, static_scale=static)
    assert_bits_equal(host(sd), so, "weight scale")
    q = host(qd)
    assert_bits_equal(q.transpose(0, 2, 1) if nk else q, qo, "weight q")


# ------------------------------------------------------------------ sort
def gpu_sort(ids, E, g0, El, xq=None, xscale=None, mode=m.MOE_SCALE_ROW_DYNAMIC, m_cap=None):
    T, k = ids.shape
    M = T * k
    H = xq.shape[1] if xq is not None else 0
    m_cap = M if m_cap is None else m_cap
    perm = torch.full((M,), -7, dtype=torch.int32, device="cuda")
    inv = torch.full((M,), -7, dtype=torch.int32, device="cuda")
    gs = torch.full((E,), -7, dtype=torch.int32, device="cuda")
    xs = torch.full((m_cap, H), 0xAB, dtype=torch.uint8, device="cuda") if xq is not None else None
    row = mode == m.MOE_SCALE_ROW_DYNAMIC and xscale is not None
    ss = torch.full((m_cap,), 7.0, dtype=torch.float32, device="cuda") if row else None
    ws = m.workspace(m.MOE_OP_SORT_BY_EXPERT, M, 0, 0, E)
    print(f"sort T={T} k={k} E={E} g0={g0} El={El} H={H} m_cap={m_cap}", flush=True)
    m.moe_sort_by_expert(dev_i32(ids) if M else torch.zeros(1, dtype=torch.int32, device="cuda"), T, k, E, g0, El,
                         dev_u8(xq) if xq is not None else None,
                         dev_f32(xscale) if xscale is not None else None, mode, H, m_cap, perm, inv, gs, xs, ss, ws)
    err = m.moe_debug_check(ws)
    out = {"perm": host(perm), "inv_pos": host(inv), "group_sizes": host(gs), "err": err}
    if xs is not None:
        out["xs"] = host(xs)
    if ss is not None:
        out["ss"] = host(ss)
    return out


def _check_sort(g, o, with_rows=True):
    assert g["err"] == 0
    assert_bits_equal(g["perm"], o["perm"], "perm")
    assert_bits_equal(g["inv_pos"], o["inv_pos"], "inv_pos")
    assert_bits_equal(g["group_sizes"], o["group_sizes"], "group_sizes")
    assert int(o["group_sizes"].sum()) == len(o["perm"])
    if with_rows and "xs" in g:
        assert_bits_equal(g["xs"], o["xs"], "xs")
    if with_rows and "ss" in g and "ss" in o and o["ss"].shape == g["ss"].shape:
        assert_bits_equal(g["ss"], o["ss"], "ss")


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_sort_config_routing(cid):
    cfg = CONFIGS[cid]
    d = generate(cfg, with_weights=False)
    mode = SCALE_TENSOR_STATIC if cfg.static else SCALE_ROW_DYNAMIC
    st = STATIC_ACT_SCALE if cfg.static else None
    xq, xsc, _ = quantize_rows(d["x"], mode, static_scale=st)
    o = sort_by_expert(d["ids"], cfg.E, cfg.group_offset, cfg.E_loc, xq=xq, xscale=xsc, xscale_mode=mode)
    m_cap = cfg.M if cfg.E_loc == cfg.E else ((o["n"] + 255) // 256) * 256
    o = sort_by_expert(d["ids"], cfg.E, cfg.group_offset, cfg.E_loc, xq=xq, xscale=xsc, xscale_mode=mode,
                       m_cap=m_cap)
    g = gpu_sort(d["ids"], cfg.E, cfg.group_offset, cfg.E_loc, xq, xsc, mode, m_cap)
    _check_sort(g, o)
    if cid == 3:
        assert (o["group_sizes"] == 0).sum() >= 2


@pytest.mark.parametrize("T,k,E,g0,El,extra", [(1, 1, 1, 0, 1, 0), (5, 3, 7, 2, 3, 10), (700, 2, 16, 0, 16, 0),
                                               (1000, 5, 300, 17, 200, 33), (3000, 8, 1024, 512, 512, 0),
                                               (0, 4, 8, 0, 8, 16), (2049, 1, 3, 1, 1, 5)])
def test_sort_edge_cases(T, k, E, g0, El, extra):
    rng = np.random.default_rng(T + E)
    ids = rng.integers(0, E, (T, k)).astype(np.int32)
    if T > 10:
        ids[: T // 2] = g0          # one expert takes half the rows
    H = 32
    xq = rng.integers(0, 256, (T, H)).astype(np.uint8)
    xsc = rng.uniform(0.1, 1.0, T).astype(np.float32)
    o = sort_by_expert(ids, E, g0, El, xq=xq, xscale=xsc)
    m_cap = o["n"] + extra
    o = sort_by_expert(ids, E, g0, El, xq=xq, xscale=xsc, m_cap=m_cap)
    g = gpu_sort(ids, E, g0, El, xq, xsc, m.MOE_SCALE_ROW_DYNAMIC, m_cap)
    _check_sort(g, o)


@pytest.mark.parametrize("H", [16, 1040, 3088, 8192, 8208])
def test_sort_row_widths(H):
    """Rows of 1 .. 9 16-byte segments per lane (the register-staged scatter and
    its loop fallback past 8192 bytes), a local slice and spare capacity."""
    rng = np.random.default_rng(H)
    T, k, E, g0, El = 300, 4, 16, 4, 8
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    xq = rng.integers(0, 256, (T, H)).astype(np.uint8)
    xsc = rng.uniform(0.1, 1.0, T).astype(np.float32)
    o = sort_by_expert(ids, E, g0, El, xq=xq, xscale=xsc)
    m_cap = o["n"] + 40
    o = sort_by_expert(ids, E, g0, El, xq=xq, xscale=xsc, m_cap=m_cap)
    print(f"sort H={H} n={o['n']} m_cap={m_cap}", flush=True)
    g = gpu_sort(ids, E, g0, El, xq, xsc, m.MOE_SCALE_ROW_DYNAMIC, m_cap)
    _check_sort(g, o)


def test_sort_tensor_scale_and_metadata_only():
    rng = np.random.default_rng(9)
    ids = rng.integers(0, 6, (50, 2)).astype(np.int32)
    o = sort_by_expert(ids, 6, 1, 4)
    g = gpu_sort(ids, 6, 1, 4)
    _check_sort(g, o, with_rows=False)


def test_sort_flags_bad_ids_without_faulting():
    ids = np.array([[0, 5], [9, 1], [-2, 3]], np.int32)     # 9 and -2 are out of range for E = 6
    xq = np.arange(3 * 16, dtype=np.uint8).reshape(3, 16)
    g = gpu_sort(ids, 6, 0, 6, xq, np.ones(3, np.float32), m_cap=6)
    assert g["err"] & m.MOE_DEVERR_EXPERT_ID
    assert int(g["group_sizes"].sum()) == 4
    assert sorted(g["perm"].tolist()) == list(range(6))        # still a permutation
    inv = g["inv_pos"]
    assert inv[2] == -1 and inv[4] == -1


def test_sort_flags_rows_beyond_capacity():
    ids = np.zeros((20, 2), np.int32)
    xq = np.ones((20, 16), np.uint8)
    g = gpu_sort(ids, 2, 0, 2, xq, np.ones(20, np.float32), m_cap=10)
    assert g["err"] & m.MOE_DEVERR_ROWS
    assert (g["inv_pos"] >= 10).sum() == 0


@pytest.mark.parametrize("mode", [m.MOE_SCALE_ROW_DYNAMIC, m.MOE_SCALE_TENSOR_STATIC])
def test_sort_metadata_then_gather_rows_equals_one_call(mode):
    """The sort's metadata (no rows) and then moe_sort_gather_rows on its
    workspace: the rows, scales and zero tail of the one-call sort, bit for
    bit, and the oracle's."""
    rng = np.random.default_rng(31 + mode)
    T, k, E, g0, El, H = 700, 4, 40, 6, 20, 512
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    xq = rng.integers(0, 256, (T, H)).astype(np.uint8)
    xscale = (rng.uniform(0.01, 1, T) if mode == m.MOE_SCALE_ROW_DYNAMIC else np.array([0.3])).astype(np.float32)
    M_cap = sort_by_expert(ids, E, g0, El)["n"] + 37      # the local rows and a zero tail
    one = gpu_sort(ids, E, g0, El, xq=xq, xscale=xscale, mode=mode, m_cap=M_cap)
    perm = torch.empty(T * k, dtype=torch.int32, device="cuda")
    inv = torch.empty(T * k, dtype=torch.int32, device="cuda")
    gs = torch.empty(E, dtype=torch.int32, device="cuda")
    xs = torch.full((M_cap, H), 0xAB, dtype=torch.uint8, device="cuda")
    row = mode == m.MOE_SCALE_ROW_DYNAMIC
    ss = torch.full((M_cap,), 7.0, dtype=torch.float32, device="cuda") if row else None
    ws = m.workspace(m.MOE_OP_SORT_BY_EXPERT, T * k, 0, 0, E)
    print(f"sort metadata then gather rows T={T} mode={mode}", flush=True)
    m.moe_sort_by_expert(dev_i32(ids), T, k, E, g0, El, None, None, mode, H, M_cap, perm, inv, gs, None, None, ws)
    m.moe_sort_gather_rows(dev_u8(xq), dev_f32(xscale), mode, inv, T, k, H, M_cap, xs, ss, ws)
    assert m.moe_debug_check(ws) == 0 and one["err"] == 0
    assert_bits_equal(host(xs), one["xs"], "gathered rows")
    if row:
        assert_bits_equal(host(ss), one["ss"], "gathered scales")
    for key, v in (("perm", perm), ("inv_pos", inv), ("group_sizes", gs)):
        assert_bits_equal(host(v), one[key], key)
    o = sort_by_expert(ids, E, g0, El, xq=xq, xscale=xscale, xscale_mode=mode, m_cap=M_cap)
    assert_bits_equal(host(xs), o["xs"], "oracle rows")
