"""GPU parity of the int8 variant against oracle/int8.py: both quantizers bit
for bit; the grouped matmul exactly on its integer sums (unit scales and a
float32 output make every element the exact integer dot product, so one
dropped, doubled or misplaced product fails); with real scales, every element
under the float32 / bf16 rules of tests/parity.py (no matrix-core allowance:
the int8 sums are exact, only the scale arithmetic rounds)."""

import numpy as np
import pytest
import torch

import moe_fp8_grouped_amd as m
from oracle.int8 import (SCALE_ROW_DYNAMIC, SCALE_TENSOR_DYNAMIC, SCALE_TENSOR_FROM_ROW_AMAX, SCALE_TENSOR_STATIC,
                         gmm_int8, quantize_rows_int8, quantize_weights_int8)
from oracle.sort import sort_by_expert
from tests.parity import assert_bits_equal, check_bf16, check_f32, dev_bf16, dev_f32, dev_i32, host
from workloads import CONFIGS, generate, to_bf16_bits

pytestmark = pytest.mark.gpu


def gpu_quantize_rows_i8(x_bits, mode, static=0.0, row_amax_in=None):
    R, C = x_bits.shape
    q = torch.full((R, C), 99, dtype=torch.int8, device="cuda")
    s = torch.full((R if mode == SCALE_ROW_DYNAMIC else 1,), 7.0, dtype=torch.float32, device="cuda")
    if mode == SCALE_TENSOR_FROM_ROW_AMAX:
        ra = dev_f32(row_amax_in)
    else:
        ra = torch.full((max(R, 1),), 7.0, dtype=torch.float32, device="cuda")
    print(f"quantize_rows_i8 R={R} C={C} mode={mode}", flush=True)
    m.moe_quantize_rows_i8(dev_bf16(x_bits) if R else torch.zeros(16, dtype=torch.bfloat16, device="cuda"), R, C,
                           mode, static, q, s, ra)
    torch.cuda.synchronize()
    return host(q), host(s), host(ra)[:R]


def _rows_input(R, C, seed, zero_rows=(), outliers=False):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((R, C)) * rng.uniform(0.01, 20.0, (R, 1))).astype(np.float32)
    if outliers:
        x[rng.random((R, C)) < 0.01] *= 50.0
    for r in zero_rows:
        x[r] = 0.0
    return to_bf16_bits(x)


@pytest.mark.parametrize("R,C", [(1, 16), (5, 48), (333, 2048), (4096, 7168)])
def test_quantize_rows_i8_row_mode_bit_exact(R, C):
    x = _rows_input(R, C, R + C, zero_rows=[0] if R > 3 else (), outliers=True)
    q, s, ra = gpu_quantize_rows_i8(x, SCALE_ROW_DYNAMIC)
    qo, so, rao = quantize_rows_int8(x, SCALE_ROW_DYNAMIC)
    assert_bits_equal(s, so, "row scales")
    assert_bits_equal(ra, rao, "row maxima")
    assert_bits_equal(q, qo, "codes")
    assert (q != -128).all()


@pytest.mark.parametrize("mode", [SCALE_TENSOR_DYNAMIC, SCALE_TENSOR_STATIC, SCALE_TENSOR_FROM_ROW_AMAX])
def test_quantize_rows_i8_tensor_modes_bit_exact(mode):
    x = _rows_input(1000, 512, 11, zero_rows=[3], outliers=True)
    static = float(np.float32(8.0) / np.float32(127.0))      # outliers past 8.0 saturate
    given = quantize_rows_int8(x, SCALE_ROW_DYNAMIC)[2] if mode == SCALE_TENSOR_FROM_ROW_AMAX else None
    q, s, ra = gpu_quantize_rows_i8(x, mode, static=static if mode == SCALE_TENSOR_STATIC else 0.0,
                                    row_amax_in=given)
    qo, so, rao = quantize_rows_int8(x, mode, static_scale=static, row_amax_in=given)
    assert_bits_equal(s, so, "tensor scale")
    assert_bits_equal(q, qo, "codes")
    if mode == SCALE_TENSOR_STATIC:
        assert (np.abs(q) == 127).any()
    if mode == SCALE_TENSOR_DYNAMIC:
        assert_bits_equal(ra, rao, "row maxima")


def test_quantize_rows_i8_empty_writes_the_tensor_scale():
    x = np.zeros((0, 64), np.uint16)
    _, s, _ = gpu_quantize_rows_i8(x, SCALE_TENSOR_STATIC, static=0.25)
    assert s[0] == np.float32(0.25)
    _, s, _ = gpu_quantize_rows_i8(x, SCALE_TENSOR_FROM_ROW_AMAX, row_amax_in=np.zeros(1, np.float32))
    assert s[0] == np.float32(1.0)


def gpu_quantize_weights_i8(w_bits, kb, nb, static=None, transpose_out=0):
    E, K, N = w_bits.shape
    q = torch.full((E, N, K) if transpose_out else (E, K, N), 99, dtype=torch.int8, device="cuda")
    s = torch.empty((E, kb, 1, nb), dtype=torch.float32, device="cuda")
    print(f"quantize_weights_i8 E={E} K={K} N={N} kb={kb} nb={nb} tr={transpose_out}", flush=True)
    m.moe_quantize_weights_i8(dev_bf16(w_bits), E, K, N, kb, nb,
                              SCALE_TENSOR_STATIC if static else SCALE_ROW_DYNAMIC, static or 0.0, transpose_out,
                              q, s)
    torch.cuda.synchronize()
    q = host(q)
    return (np.ascontiguousarray(q.transpose(0, 2, 1)) if transpose_out else q), host(s)


@pytest.mark.parametrize("kb,nb,tr,static", [(1, 1024, 0, None), (1, 1024, 1, None), (4, 8, 1, None),
                                             (2, 2, 0, None), (1, 1, 1, 0.0004)])
def test_quantize_weights_i8_bit_exact(kb, nb, tr, static):
    cfg = CONFIGS[1]
    w = generate(cfg, with_weights=["w_up"])["weights"]["w_up"]
    w = w.copy()
    w[1, :w.shape[1] // kb, :w.shape[2] // nb] = 0                  # an all-zero block
    q, s = gpu_quantize_weights_i8(w, kb, nb, static, tr)
    qo, so = quantize_weights_int8(w, kb, nb, static_scale=static)
    assert_bits_equal(s, so, "weight scales")
    assert_bits_equal(q, qo, "weight codes")


def _dev(a, dtype):
    return a if isinstance(a, torch.Tensor) else torch.from_numpy(np.ascontiguousarray(a, dtype=dtype)).to("cuda")


def gpu_gmm_i8(lhs, ls, ls_mode, rhs, rs, gs, E, g0, El, tr, out_dtype, M=None):
    """rhs and rs: host arrays, or device tensors already in place."""
    M = lhs.shape[0] if M is None else M
    K = lhs.shape[1]
    N = rhs.shape[1] if tr else rhs.shape[2]
    assert rhs.shape[0] == El and tuple(rs.shape) == (El, rs.shape[1], 1, rs.shape[3]) and lhs.shape[0] <= M
    lhs_d = torch.zeros((M, K), dtype=torch.int8, device="cuda")
    lhs_d[:lhs.shape[0]] = torch.from_numpy(np.ascontiguousarray(lhs, dtype=np.int8)).to("cuda")
    out = torch.full((M, N), 3.0, dtype=torch.float32 if out_dtype == m.MOE_F32 else torch.bfloat16, device="cuda")
    ws = m.workspace(m.MOE_OP_GMM, M, K, N, E)
    print(f"gmm_i8 M={M} K={K} N={N} E={E} g0={g0} El={El} Kb={rs.shape[1]} Nb={rs.shape[3]} tr={tr} "
          f"out={out_dtype}", flush=True)
    m.moe_gmm_i8(lhs_d, dev_f32(ls), ls_mode, _dev(rhs, np.int8), _dev(rs, np.float32), rs.shape[1], rs.shape[3], tr,
                 dev_i32(gs), E, g0, El, M, K, N, out_dtype, out, ws)
    err = m.moe_debug_check(ws)
    assert err == 0
    return host(out)


def _codes(rng, shape):
    return rng.integers(-127, 128, shape).astype(np.int8)


@pytest.mark.parametrize("sizes,K,N,Kb,tr", [
    ([0, 5, 0, 130, 1, 0, 257, 0], 512, 384, 1, 1),
    ([0, 5, 0, 130, 1, 0, 257, 0], 512, 384, 4, 0),
    ([300], 1024, 256, 8, 1),
    ([1, 1, 1, 1, 1, 1, 1, 1], 256, 128, 1, 0),
    ([64, 0, 200, 7], 144, 80, 1, 1),                 # sizes that take the 64 x 64 edge kernel
    ([64, 0, 200, 7], 144, 80, 1, 0),
    ([3, 90, 0, 41], 16, 48, 1, 1),
    ([0, 285, 16, 140, 433, 257], 512, 512, 4, 1),    # row blocks of up to 144 rows (absorbing tiles)
    ([0, 285, 16, 140, 433, 257], 512, 384, 1, 1),
])
def test_gmm_i8_integer_sums_exact(sizes, K, N, Kb, tr):
    """Unit scales, float32 output: every element must equal the exact
    integer dot product (the sums stay below 2^24, where float32 is exact)."""
    rng = np.random.default_rng(len(sizes) * 1000 + K + N + Kb + tr)
    El = len(sizes)
    gs = np.array(sizes, np.int32)
    n = int(gs.sum())
    M = n + 37                                        # a tail of rows past the groups
    X = _codes(rng, (n, K))
    W = _codes(rng, (El, K, N))
    ls = np.ones(M, np.float32)
    rs = np.ones((El, Kb, 1, 1 if Kb == 1 else N // 128 if N % 128 == 0 else 1), np.float32)
    o = gmm_int8(np.concatenate([X, np.zeros((M - n, K), np.int8)]), ls, W, rs, gs, 0, El)
    assert np.abs(o["out"]).max() < 2 ** 24
    rhs = np.ascontiguousarray(W.transpose(0, 2, 1)) if tr else W
    g = gpu_gmm_i8(X, ls, SCALE_ROW_DYNAMIC, rhs, rs, gs, El, 0, El, tr, m.MOE_F32, M=M)
    assert_bits_equal(g, o["out"].astype(np.float32), "integer sums")
    assert not g[n:].any()


def test_gmm_i8_split_last_round_rounds_once():
    """Few tiles over many workgroups, K = 2048: each XCD's only round of
    tiles is split along K (four parts of 512).  Codes of one sign push the
    integer sums past 2^24, where float32 is no longer exact: with unit
    scales every element must still be the exact sum rounded once, as
    without the split -- adding the parts' sums as float32 would round up to
    three more times, and does for some elements of these operands (checked
    on the host, so the test cannot pass by accident)."""
    rng = np.random.default_rng(77)
    sizes = [300, 200, 50]
    El, K, N = len(sizes), 2048, 1024
    gs = np.array(sizes, np.int32)
    n = int(gs.sum())
    M = n + 37
    X = rng.integers(96, 128, (n, K)).astype(np.int8)
    W = rng.integers(96, 128, (El, K, N)).astype(np.int8)
    ls = np.ones(M, np.float32)
    rs = np.ones((El, 1, 1, N), np.float32)
    o = gmm_int8(np.concatenate([X, np.zeros((M - n, K), np.int8)]), ls, W, rs, gs, 0, El)
    want = o["out"].astype(np.float32)
    assert np.abs(o["out"]).min(initial=2 ** 25, where=o["out"] != 0) > 2 ** 24
    # the float32 sum of four 512-deep partial sums differs from the single rounding somewhere
    Xg, Wg = X[:300].astype(np.int64), W[0].astype(np.int64)
    parts = [(Xg[:, q * 512:(q + 1) * 512] @ Wg[q * 512:(q + 1) * 512]).astype(np.float32) for q in range(4)]
    fsum = ((parts[0] + parts[1]) + parts[2]) + parts[3]
    assert (fsum != want[:300]).any()
    rhs = np.ascontiguousarray(W.transpose(0, 2, 1))
    g = gpu_gmm_i8(X, ls, SCALE_ROW_DYNAMIC, rhs, rs, gs, El, 0, El, 1, m.MOE_F32, M=M)
    assert_bits_equal(g, want, "int8 split: integer sums rounded once")
    assert not g[n:].any()


def test_gmm_i8_local_slice_exact():
    rng = np.random.default_rng(7)
    E, g0, El, K, N = 16, 4, 8, 384, 256
    gs = rng.integers(0, 90, E).astype(np.int32)
    gs[g0 + 2] = 0
    n = int(gs[g0:g0 + El].sum())
    X = _codes(rng, (n, K))
    W = _codes(rng, (El, K, N))
    ls = np.ones(1, np.float32)
    rs = np.ones((El, 3, 1, 2), np.float32)
    o = gmm_int8(X, ls, W, rs, gs, g0, El)
    g = gpu_gmm_i8(X, ls, SCALE_TENSOR_STATIC, np.ascontiguousarray(W.transpose(0, 2, 1)), rs, gs, E, g0, El, 1,
                   m.MOE_F32)
    assert_bits_equal(g, o["out"].astype(np.float32), "integer sums, local slice")


@pytest.mark.parametrize("cid,weight", [(1, "w_up"), (3, "w_up"), (2, "wi_0")])
def test_int8_forward_stage_small_configs(cid, weight):
    """bf16 tokens and weights through the int8 quantizers, the byte sort and
    the int8 grouped matmul, each stage against the oracle; the matmul on the
    oracle's codes, every output element checked."""
    cfg = CONFIGS[cid]
    d = generate(cfg, with_weights=[weight])
    x, w = d["x"], d["weights"][weight]
    E_loc = w.shape[0]
    q, s, _ = gpu_quantize_rows_i8(x, SCALE_ROW_DYNAMIC)
    qo, so, _ = quantize_rows_int8(x, SCALE_ROW_DYNAMIC)
    assert_bits_equal(q, qo, "token codes")
    assert_bits_equal(s, so, "token scales")
    kb, nb = cfg.scale_blocks(w.shape[1], w.shape[2])
    wq, ws_ = gpu_quantize_weights_i8(w, kb, nb, transpose_out=1)
    wqo, wso = quantize_weights_int8(w, kb, nb)
    assert_bits_equal(wq, wqo, "weight codes")
    assert_bits_equal(ws_, wso, "weight scales")
    srt = sort_by_expert(d["ids"], cfg.E, cfg.group_offset, E_loc, xq=qo.view(np.uint8), xscale=so,
                         xscale_mode=SCALE_ROW_DYNAMIC)
    n = srt["n"]
    xs = srt["xs"][:n].view(np.int8)
    o = gmm_int8(xs, srt["ss"][:n], wqo, wso, srt["group_sizes"], cfg.group_offset, E_loc)
    rhs = np.ascontiguousarray(wqo.transpose(0, 2, 1))
    for od in (m.MOE_F32, m.MOE_BF16):
        g = gpu_gmm_i8(xs, srt["ss"][:n], SCALE_ROW_DYNAMIC, rhs, wso, srt["group_sizes"], cfg.E, cfg.group_offset,
                       E_loc, 1, od)
        if od == m.MOE_F32:
            check_f32(g, o["out"], o["abs_sum"], f"int8 config {cid} f32")
        else:
            check_bf16(g, o["out"], o["abs_sum"], f"int8 config {cid} bf16")


def test_int8_gmm_expert_slice_full():
    """The expert-slice forward's first matmul at its full size and in the
    launch configuration that is timed (8192 tokens, top-8 of 256 experts,
    the 32 local experts of group offset 64, H = 7168 -> 2048, 128 x 128
    weight blocks, weights [E, N, K]) in int8.  Every row of two 128-column
    weight blocks is checked against the oracle; the oracle quantizes only
    those columns (each block's codes depend on its own elements alone), and
    the device's weight codes and scales there must match its bits."""
    cfg = CONFIGS[4]
    d = generate(cfg, with_weights=["wi_0"])
    w = d["weights"]["wi_0"]
    E, K, N = w.shape
    kb, nb = cfg.scale_blocks(cfg.H, cfg.I)
    bn = N // nb
    blocks = [0, 9]
    cols = np.concatenate([np.arange(b * bn, (b + 1) * bn) for b in blocks])
    q_d = torch.empty((E, N, K), dtype=torch.int8, device="cuda")
    s_d = torch.empty((E, kb, 1, nb), dtype=torch.float32, device="cuda")
    print(f"quantize_weights_i8 E={E} K={K} N={N} kb={kb} nb={nb} tr=1", flush=True)
    m.moe_quantize_weights_i8(dev_bf16(w), E, K, N, kb, nb, SCALE_ROW_DYNAMIC, 0.0, 1, q_d, s_d)
    torch.cuda.synchronize()
    wqo, wso = quantize_weights_int8(np.ascontiguousarray(w[:, :, cols]), kb, len(blocks))
    del w
    assert_bits_equal(host(s_d)[:, :, :, blocks], wso, "weight scales (sampled blocks)")
    assert_bits_equal(host(q_d[:, torch.from_numpy(cols).cuda(), :]), np.ascontiguousarray(wqo.transpose(0, 2, 1)),
                      "weight codes (sampled blocks)")
    qo, so, _ = quantize_rows_int8(d["x"], SCALE_ROW_DYNAMIC)
    srt = sort_by_expert(d["ids"], cfg.E, cfg.group_offset, cfg.E_loc, xq=qo.view(np.uint8), xscale=so,
                         xscale_mode=SCALE_ROW_DYNAMIC)
    n = srt["n"]
    m_cap = ((n + 255) // 256) * 256
    xs = srt["xs"][:n].view(np.int8)
    ls = np.zeros(m_cap, np.float32)
    ls[:n] = srt["ss"][:n]
    g = gpu_gmm_i8(xs, ls, SCALE_ROW_DYNAMIC, q_d, s_d, srt["group_sizes"], cfg.E, cfg.group_offset, cfg.E_loc, 1,
                   m.MOE_BF16, M=m_cap)
    assert not g[n:].any()
    o = gmm_int8(xs, ls[:n], wqo, wso, srt["group_sizes"], cfg.group_offset, cfg.E_loc)
    check_bf16(np.ascontiguousarray(g[:n, cols]), o["out"], o["abs_sum"], "int8 expert slice wi_0 bf16 (2 blocks)")
