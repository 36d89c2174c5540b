"""moe_sort_by_expert_noalloc (the sort with its scratch in a library-owned
device array) against moe_sort_by_expert (the same sort on a caller
workspace), through the C ABI: bit-identical perm, inv_pos, group_sizes,
gathered rows and scales, and the same device-error bits, on calls in a row
whose sizes shrink -- the array keeps the previous call's contents."""

import numpy as np
import pytest
import torch

import moe_fp8_grouped_amd as m
from oracle.sort import sort_by_expert
from tests.parity import assert_bits_equal, dev_f32, dev_i32, dev_u8, host
from workloads import CONFIGS, generate

pytestmark = pytest.mark.gpu


def _routing(cid):
    cfg = CONFIGS[cid]
    d = generate(cfg, with_weights=False)
    return cfg, d["ids"]


def _both(ids, E, g0, El, H, m_cap, mode, seed):
    T, k = ids.shape
    rng = np.random.default_rng(seed)
    xq = rng.integers(0, 0x7F, (T, H)).astype(np.uint8)
    xscale = rng.uniform(0.01, 1, T if mode == m.MOE_SCALE_ROW_DYNAMIC else 1).astype(np.float32)
    d_ids, d_xq, d_xs = dev_i32(ids), dev_u8(xq), dev_f32(xscale)

    def outs(fill):
        o = {"perm": torch.full((T * k,), fill, dtype=torch.int32, device="cuda"),
             "inv_pos": torch.full((T * k,), fill, dtype=torch.int32, device="cuda"),
             "group_sizes": torch.full((E,), fill, dtype=torch.int32, device="cuda"),
             "xs": torch.full((m_cap, H), fill & 0xFF, dtype=torch.uint8, device="cuda")}
        if mode == m.MOE_SCALE_ROW_DYNAMIC:          # a tensor scale passes through: no gathered scales
            o["ss"] = torch.full((m_cap,), float(fill), dtype=torch.float32, device="cuda")
        return o

    a = outs(-3)
    ws = m.workspace(m.MOE_OP_SORT_BY_EXPERT, T * k, 0, 0, E)
    m.moe_sort_by_expert(d_ids, T, k, E, g0, El, d_xq, d_xs, mode, H, m_cap, a["perm"], a["inv_pos"],
                         a["group_sizes"], a["xs"], a.get("ss"), ws)
    b = outs(77)
    derr = torch.zeros(1, dtype=torch.int32, device="cuda")
    print(f"noalloc sort T={T} k={k} E={E} g0={g0} El={El} H={H} m_cap={m_cap}", flush=True)
    m.moe_sort_by_expert_noalloc(d_ids, T, k, E, g0, El, d_xq, d_xs, mode, H, m_cap, b["perm"], b["inv_pos"],
                                 b["group_sizes"], b["xs"], b.get("ss"), derr)
    torch.cuda.synchronize()
    for key in a:
        assert_bits_equal(host(b[key]), host(a[key]), f"noalloc {key}")
    assert int(derr.item()) == m.moe_debug_check(ws)
    return {key: host(b[key]) for key in b}, int(derr.item()), xq, xscale


def test_noalloc_sort_matches_the_workspace_sort_on_calls_in_a_row():
    # 1: one GPU's expert slice (65536 routed slots, 256 experts, rows of 7168 bytes)
    cfg, ids = _routing(4)
    n = int(((ids >= 64) & (ids < 96)).sum())
    m_cap = (n + 255) // 256 * 256
    got, err, xq, xs = _both(ids, cfg.E, 64, 32, cfg.H, m_cap, m.MOE_SCALE_ROW_DYNAMIC, 1)
    assert err == 0
    o = sort_by_expert(ids, cfg.E, 64, 32, xq=xq, xscale=xs, xscale_mode=m.MOE_SCALE_ROW_DYNAMIC, m_cap=m_cap)
    for key in ("perm", "inv_pos", "group_sizes", "xs", "ss"):
        assert_bits_equal(got[key], o[key], f"noalloc vs oracle {key}")
    # 2: a smaller call right after (512 slots, 8 experts): nothing of the first call's table leaks in
    cfg, ids = _routing(1)
    got, err, xq, xs = _both(ids, cfg.E, 0, cfg.E, cfg.H, cfg.M, m.MOE_SCALE_TENSOR_STATIC, 2)
    assert err == 0
    o = sort_by_expert(ids, cfg.E, 0, cfg.E, xq=xq, xscale=xs, xscale_mode=m.MOE_SCALE_TENSOR_STATIC, m_cap=cfg.M)
    for key in ("perm", "inv_pos", "group_sizes", "xs"):
        assert_bits_equal(got[key], o[key], f"noalloc vs oracle {key} (second call)")


def test_noalloc_sort_reports_device_errors_and_the_size_limit():
    rng = np.random.default_rng(3)
    T, k, E = 300, 2, 16
    ids = rng.integers(0, E, (T, k)).astype(np.int32)
    ids[5, 1] = 99                                     # an expert id out of range
    _, err, _, _ = _both(ids, E, 0, E, 32, T * k, m.MOE_SCALE_ROW_DYNAMIC, 4)
    assert err & m.MOE_DEVERR_EXPERT_ID
    # more slots than the array's table holds: rejected before any launch
    big = torch.zeros(300000, dtype=torch.int32, device="cuda")
    with pytest.raises(m.MoeError) as e:
        m.moe_sort_by_expert_noalloc(big, 300000, 1, 1024, 0, 1024, None, None, 0, 0, 0, big, big,
                                     big[:1024], None, None)
    assert e.value.status == m.MOE_ERR_WORKSPACE
    # and a last, small call is still right
    ids = rng.integers(0, 4, (10, 1)).astype(np.int32)
    got, err, _, _ = _both(ids, 4, 1, 2, 16, 10, m.MOE_SCALE_ROW_DYNAMIC, 5)
    assert err == 0
