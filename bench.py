"""Benchmark of the fp8 MoE hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--config 4] [--no-cpu-baseline] [--no-secondary]

Line of record (config 4): one GPU's expert slice of a large MoE layer's gated
FFN forward -- T=8192 tokens, H=7168, E=256 experts, top-8, I=2048, this
GPU's experts 64..95 (group_offset 64), 128x128 blockwise weight scales, 1 %
outlier token rows.  A step is one pass of the whole hot path with every input
resident in HBM: quantize this GPU's own 1024 tokens, sort the 65536 routed
slots and gather the fp8 rows of the local window, the two input projections
as one grouped matmul over [W0 | W1], SiLU*mul requantized per row, the down
projection, and the weighted gather-reduce (local partial sums).  The 1.4 GB
of fp8 weights exceed the 256 MB Infinity Cache, so each step reads them
from HBM.

Prints one JSON line:

  value      whole-step throughput: algorithmic GMM flops of a step / step
             time, the step replayed as a HIP graph (K timed replays after W)
  settle     directly before each timed region (and its W warm-up steps),
             untimed steps for --settle-s seconds (0.3 by default): after any
             host-side pause the first ~50 steps run slower while the clocks
             ramp up; the record keeps the ms per step of the first K steps
  roofline   the dominant kernel, the fused input projections' moe_gmm_fp8
             launch: its algorithmic bytes (and flops) per launch / its
             average duration by HIP events around each launch on its own
             stream over K eager steps; HBM-bound (its flop/byte sits below
             the fp8 ridge, 5.0 PFLOP/s / 8 TB/s = 629), so `frac` is of 8 TB/s;
             `traffic` = HBM bytes per launch from the committed rocprofv3
             counter summary (while the kernel sources match it)
  kernels    every stage of the step: mean / median / min duration, GB/s,
             TFLOP/s
  secondary  the other workloads: the gated FFN forward (config 2, one and
             three rotating buffer sets), the MoE backward (config 5, one and
             three sets), the gated FFN's backward, the tiny and skewed
             up-projections (configs 1, 3 and the large skewed variant), and
             the line of record's two grouped matmuls in the int8 variant
  cpu_baseline  the CPU oracle on a bounded sample of the same workload, timed
             stage by stage on the host's cores (plus configs 1 and 3 whole,
             single-threaded and on every core)
"""

import argparse
import dataclasses
import hashlib
import json
import os
import re
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fp8 MoE GMM TFLOP/s (% fp8 MFMA peak) + sort/gather HBM GB/s, 1×MI355X"
PEAK_FP8_TFLOPS = 5000.0      # dense fp8 MFMA, MI355X
PEAK_HBM_GBPS = 8000.0        # HBM3E
RIDGE = PEAK_FP8_TFLOPS * 1e12 / (PEAK_HBM_GBPS * 1e9)
# sources of the dominant kernel; a counter summary applies only to the build it was taken on
GMM_SOURCES = ("moe_fp8_grouped_amd/csrc/gmm.hip", "moe_fp8_grouped_amd/csrc/tile_common.hpp",
               "moe_fp8_grouped_amd/csrc/common.hpp")
GMM_COUNTERS = "profiles/moe_gmm_fp8__ep-slice-ffn-fwd__hbm_counters.md"


def gmm_source_hash():
    h = hashlib.sha256()
    for rel in GMM_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes of the dominant launch from the committed rocprofv3 counter
    summary (FETCH_SIZE + WRITE_SIZE, calibrated on a plain copy), or None when
    the summary is missing or was taken on other kernel sources."""
    path = os.path.join(ROOT, GMM_COUNTERS)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"^- source_hash: (\w+)", text, re.M)
    m_bytes = re.search(r"^- hbm_bytes_per_launch: (\d+)", text, re.M)
    if not m_hash or not m_bytes or m_hash.group(1) != gmm_source_hash():
        return None
    return int(m_bytes.group(1))


# ------------------------------------------------------------------ timing
def _stats(durs_ms):
    d = np.asarray(durs_ms, np.float64) * 1e3
    return {"avg_us": round(float(d.mean()), 2), "median_us": round(float(np.median(d)), 2),
            "min_us": round(float(d.min()), 2)}


SETTLE_S = 0.3     # --settle-s


def eager_step(calls):
    def run():
        for _, fn in calls:
            fn()
    return run


def settle(step, steps):
    """Untimed runs of ``step`` (a callable doing one whole step) for
    SETTLE_S seconds, directly before a timed region.  After any pause --
    the host-side gaps of data generation, graph capture or event
    read-back, even ~1 ms -- the device runs the next ~50 expert-slice steps
    (~40 ms) up to 15-40 % slower while its clocks ramp up again, and a
    default window of warm-up plus timed steps would fall inside that ramp.
    Returns the settle record: seconds, steps run, and the ms per step of
    its first ``steps`` runs (the unsettled figure)."""
    if SETTLE_S <= 0:
        return {"s": 0.0, "steps": 0}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    first = (time.perf_counter() - t0) * 1e3 / steps
    n = steps
    while time.perf_counter() - t0 < SETTLE_S:
        for _ in range(10):
            step()
        n += 10
        torch.cuda.synchronize()
    return {"s": SETTLE_S, "steps": n, "ms_per_step_first_steps": round(first, 4)}


def rotation(paths):
    state = {"i": 0}

    def run():
        paths[state["i"] % len(paths)].replay()
        state["i"] += 1
    return run


def time_back_to_back(calls, steps):
    """ms per step of ``steps`` eager steps launched back to back (no events
    between launches), bracketed by device synchronisations."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        for _, fn in calls:
            fn()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def time_calls(calls, steps, warmup):
    """Eager timing of a list of (name, fn) launches: a HIP event pair around
    each launch, recorded on torch's current stream -- the stream every call
    of the binding launches on.  Returns per-name duration lists (ms) and
    the eager ms per step."""
    for _ in range(warmup):
        for _, fn in calls:
            fn()
    torch.cuda.synchronize()
    ev = {nm: [] for nm, _ in calls}
    t0 = time.perf_counter()
    for _ in range(steps):
        for nm, fn in calls:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            ev[nm].append((a, b))
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    return {nm: [a.elapsed_time(b) for a, b in lst] for nm, lst in ev.items()}, ms


def time_replays(paths, steps, warmup):
    """ms per step of HIP graph replays, rotating over ``paths`` (each with a
    captured graph): the timed region is exactly ``steps`` replays bracketed
    by device synchronisations."""
    n = len(paths)
    for i in range(warmup * n):
        paths[i % n].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        paths[i % n].replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def kern_entry(durs, nbytes, flops=0):
    e = _stats(durs)
    us = e["avg_us"]
    e.update({"alg_bytes": int(nbytes), "GB_s": round(nbytes / (us * 1e-6) / 1e9, 1),
              "frac_hbm": round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4)})
    if flops:
        tf = flops / (us * 1e-6) / 1e12
        e.update({"alg_flops": int(flops), "TFLOP_s": round(tf, 1), "frac_fp8_peak": round(tf / PEAK_FP8_TFLOPS, 4)})
    return e


# ------------------------------------------------------------------ forward workloads
def forward_path(cid, static=False, seed=None):
    """A ForwardPath for config ``cid`` with its accounting inputs."""
    from moe_fp8_grouped_amd.pipeline import ForwardPath
    from workloads import CONFIGS, STATIC_ACT_SCALE, STATIC_WEIGHT_SCALE, generate, m_cap_for

    cfg = CONFIGS[cid]
    data = generate(cfg, seed=seed)
    ids = data["ids"]
    local = (ids >= cfg.group_offset) & (ids < cfg.group_offset + cfg.E_loc)
    n, U = int(local.sum()), int(local.any(axis=1).sum())
    share = 8 if cfg.E_loc < cfg.E else 1
    path = ForwardPath(cfg, data, m_cap=m_cap_for(cfg, n), share=share,
                       static_act=STATIC_ACT_SCALE if static else None,
                       static_weight=STATIC_WEIGHT_SCALE if static else None)
    gs = np.bincount(ids.ravel(), minlength=cfg.E)[cfg.group_offset:cfg.group_offset + cfg.E_loc]
    path.nonempty_local = int((gs > 0).sum())
    path.n_local, path.U = n, U
    path.largest_group, path.empty_groups = int(gs.max()), int((gs == 0).sum())
    return path, data


def step_accounting(path):
    """Algorithmic bytes / flops of each launch of one forward step."""
    cfg = path.cfg
    T, H, k, E, I = cfg.T, cfg.H, cfg.k, cfg.E, cfg.I
    n, U, M_cap = path.n_local, path.U, path.m_cap
    acc = {}
    if path.fused_quantize:
        # one pass: ids, perm and inv_pos, the bf16 rows of the U tokens with a local row, the fp8 rows
        # and scales of the n local rows
        acc["quantize_sort"] = {"bytes": T * k * 4 + 2 * T * k * 4 + E * 4 + U * H * 2 + n * H + 4 * n, "flops": 0}
    else:
        own = T // path.share
        acc["quantize"] = {"bytes": own * H * 3 + own * 4, "flops": 0}
        acc["sort"] = {"bytes": T * k * 4 + 2 * T * k * 4 + E * 4 + U * H + n * H + 8 * n, "flops": 0}
    nonempty = path.nonempty_local
    launches = [("wi_01", path.w01), ("wo", path.w["wo"])] if cfg.pipeline == "ffn" else [("w_up", path.w["w_up"])]
    for name, w in launches:
        K, N = w.K, w.N
        by = n * K + nonempty * K * N + n * N * 2 + (M_cap - n) * N * 2 + n * 4 + nonempty * w.kb * w.nb * 4
        acc["gmm_" + name] = {"bytes": by, "flops": 2 * n * K * N}
    if cfg.pipeline == "ffn":
        acc["silu_quant"] = {"bytes": M_cap * I * 5 + M_cap * 4, "flops": 0}
    N_out = path.N_out
    acc["gather_reduce"] = {"bytes": n * N_out * 2 + T * N_out * 2 + T * k * 8, "flops": 0}
    return acc


def step_calls(path):
    import moe_fp8_grouped_amd as m
    cfg = path.cfg
    calls = [("quantize_sort", path.sort)] if path.fused_quantize else [("quantize", path.quantize),
                                                                       ("sort", path.sort)]
    ls = path.ss if path.act_mode == m.MOE_SCALE_ROW_DYNAMIC else path.xscale
    if cfg.pipeline == "up":
        calls.append(("gmm_w_up", lambda: path.gmm(path.xs, ls, path.act_mode, path.w["w_up"], path.y)))
    else:
        calls += [("gmm_wi_01", lambda: path.gmm_gate_up(ls)), ("silu_quant", path.silu_quant),
                  ("gmm_wo", lambda: path.gmm(path.hq, path.hs, m.MOE_SCALE_ROW_DYNAMIC, path.w["wo"], path.y))]
    calls.append(("gather_reduce", path.combine))
    return calls


def measure_forward(path, steps, warmup):
    """Per-launch HIP-event durations over ``steps`` eager steps, then the
    step as a HIP graph: ``steps`` timed replays after ``warmup``."""
    acc = step_accounting(path)
    calls = step_calls(path)
    st = settle(eager_step(calls), steps)
    durs, ms_eager = time_calls(calls, steps, warmup)
    kern = {nm: kern_entry(d, acc[nm]["bytes"], acc[nm]["flops"]) for nm, d in durs.items()}
    settle(eager_step(calls), steps)
    ms_b2b = time_back_to_back(calls, steps)
    path.capture_graph(warmup=1)
    settle(path.replay, steps)
    ms = time_replays([path], steps, warmup)
    flops = sum(a["flops"] for a in acc.values())
    cfg = path.cfg
    return {"workload": workload_name(cfg), "routed_local_rows": path.n_local, "m_cap": path.m_cap,
            "ms_per_step": round(ms, 4), "ms_per_step_eager": round(ms_eager, 4),
            "ms_per_step_eager_back_to_back": round(ms_b2b, 4), "settle": st,
            "gmm_flops_per_step": int(flops), "gmm_TFLOP_s_whole_step": round(flops / (ms * 1e-3) / 1e12, 1),
            "kernels": kern}, durs, acc


def int8_gmm_timing(path, acc, steps, warmup):
    """The two grouped matmuls of the expert-slice step in the int8 variant
    (moe_gmm_i8, int8 codes, int32 accumulation), on the step's own group
    sizes and row capacity, with random codes and scales (the int8 matrix
    cores' speed does not depend on the values).  Same algorithmic bytes and
    operations as the fp8 launches (one byte per code); int8 dense peak 5.0
    POP/s, the fp8 one."""
    import moe_fp8_grouped_amd as m
    cfg = path.cfg
    g = torch.Generator(device="cuda").manual_seed(11)
    El, H, I, m_cap = cfg.E_loc, cfg.H, cfg.I, path.m_cap
    lhs = torch.randint(-127, 128, (m_cap, H), dtype=torch.int8, device="cuda", generator=g)
    h = torch.randint(-127, 128, (m_cap, I), dtype=torch.int8, device="cuda", generator=g)
    ls = torch.rand(m_cap, device="cuda", generator=g) + 0.5
    w01 = torch.randint(-127, 128, (El, 2 * I, H), dtype=torch.int8, device="cuda", generator=g)
    wo = torch.randint(-127, 128, (El, H, I), dtype=torch.int8, device="cuda", generator=g)
    s01 = torch.rand((El, H // 128, 1, 2 * I // 128), device="cuda", generator=g) * 1e-3
    so = torch.rand((El, I // 128, 1, H // 128), device="cuda", generator=g) * 1e-3
    y01 = torch.empty((m_cap, 2 * I), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((m_cap, H), dtype=torch.bfloat16, device="cuda")
    ws = m.workspace(m.MOE_OP_GMM, m_cap, H, max(H, 2 * I), cfg.E)

    def gmm(a, w, s, out, K, N):
        m.moe_gmm_i8(a, ls, m.MOE_SCALE_ROW_DYNAMIC, w, s, s.shape[1], s.shape[3], 1, path.group_sizes, cfg.E,
                     cfg.group_offset, El, m_cap, K, N, m.MOE_BF16, out, ws)

    calls = [("gmm_wi_01", lambda: gmm(lhs, w01, s01, y01, H, 2 * I)), ("gmm_wo", lambda: gmm(h, wo, so, y, I, H))]
    settle(eager_step(calls), steps)
    durs, _ = time_calls(calls, steps, warmup)
    if m.moe_debug_check(ws) != 0:
        raise RuntimeError("moe_gmm_i8 flagged a device error")
    res = {"workload": workload_name(cfg) + ", int8 operands (moe_gmm_i8) on the step's group sizes",
           "kernels": {}}
    for nm, d in durs.items():
        e = kern_entry(d, acc[nm]["bytes"])
        tops = acc[nm]["flops"] / (e["avg_us"] * 1e-6) / 1e12
        e.update({"alg_ops": int(acc[nm]["flops"]), "TOP_s": round(tops, 1),
                  "frac_int8_peak": round(tops / PEAK_FP8_TFLOPS, 4)})
        res["kernels"]["i8_" + nm] = e
    del lhs, h, w01, wo, y01, y
    torch.cuda.empty_cache()
    return res


def workload_name(cfg, static=False):
    s = f"{cfg.name}{' static scales' if static else ''}: T={cfg.T} H={cfg.H} E={cfg.E} top-{cfg.k} " \
        f"{'I' if cfg.pipeline == 'ffn' else 'N'}={cfg.I}"
    if cfg.E_loc < cfg.E:
        s += f", local experts {cfg.group_offset}..{cfg.group_offset + cfg.E_loc - 1}"
    if cfg.weight_block_k:
        s += ", 128x128 weight blocks" if cfg.weight_block_n > 1 else ", [E, K/128, 1, N] weight scales"
    return s


def roofline(durs, info):
    """The dominant launch against the roofline that bounds it."""
    st = _stats(durs)
    us = st["avg_us"]
    gbps = info["bytes"] / (us * 1e-6) / 1e9
    tf = info["flops"] / (us * 1e-6) / 1e12
    intensity = info["flops"] / info["bytes"]
    r = {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
         "frac": round(gbps / PEAK_HBM_GBPS, 4), "traffic": measured_traffic(),
         "kernel": "moe_gmm_fp8, the fused input projections (one grouped matmul over [W0 | W1], N = 4096)",
         "alg_bytes_per_launch": int(info["bytes"]), "alg_flops_per_launch": int(info["flops"]),
         "avg_launch_us": st["avg_us"], "median_launch_us": st["median_us"], "min_launch_us": st["min_us"],
         "launches_timed": len(durs), "alg_intensity_flop_per_byte": round(intensity, 1),
         "mfma_TFLOP_s": round(tf, 1), "mfma_frac_fp8_peak": round(tf / PEAK_FP8_TFLOPS, 4),
         "source_hash": gmm_source_hash(),
         "timing": "HIP events around each launch, on the stream it runs on, over the timed eager steps"}
    if intensity > RIDGE:
        r.update({"bound": "mfma", "achieved": round(tf, 1), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                  "frac": round(tf / PEAK_FP8_TFLOPS, 4)})
    return r


def secondary_forward(cid, steps, warmup, static=False):
    path, data = forward_path(cid, static=static)
    del data
    res, _, _ = measure_forward(path, steps, warmup)
    res["workload"] = workload_name(path.cfg, static)
    if path.cfg.pipeline == "up":
        res.update({"empty_experts": path.empty_groups, "largest_group": path.largest_group})
    del path
    torch.cuda.empty_cache()
    return res


def rotating_forward(cid, steps, warmup, nsets=3):
    """The forward step with ``nsets`` independent weight and buffer sets
    (own seeds), each in its own HIP graph, replayed in rotation, so every
    step's weights and activations were last touched ``nsets`` steps earlier
    (together far beyond the 256 MB Infinity Cache)."""
    paths = []
    for i in range(nsets):
        p, data = forward_path(cid, seed=7000 + i)
        del data
        p.capture_graph(warmup=1)
        paths.append(p)
    nrep = max(steps, nsets) // nsets * nsets
    settle(rotation(paths), nrep)
    ms = time_replays(paths, nrep, warmup)
    flops = sum(a["flops"] for a in step_accounting(paths[0]).values())
    res = {"workload": workload_name(paths[0].cfg) + f", {nsets} independent weight and buffer sets in rotation",
           "steps": nrep, "ms_per_step": round(ms, 4), "gmm_TFLOP_s_whole_step": round(flops / (ms * 1e-3) / 1e12, 1)}
    del paths
    torch.cuda.empty_cache()
    return res


# ------------------------------------------------------------------ backward workloads
def backward_path(seed=None):
    from moe_fp8_grouped_amd.pipeline import BackwardPath
    from workloads import CONFIGS, STATIC_ACT_SCALE, STATIC_WEIGHT_SCALE, generate
    cfg = CONFIGS[5]
    data = generate(cfg, seed=seed)
    # X: the [T, H] codes, the sort's metadata, then the codes gathered straight into the weight-gradient
    # product's transposed layout (no sorted rows, no transpose pass of X)
    p = BackwardPath(cfg, data, STATIC_ACT_SCALE, STATIC_WEIGHT_SCALE, fused_quantize=False, transposed_x=True)
    del data
    return p


def secondary_backward(steps, warmup, nsets=3):
    """Config 5: the backward of an up projection (T=8192 H=4096 E=64 top-4
    I=1536, static X and W scales): dX = gmm(dY, W^T), dW = tgmm(X_sorted, dY) with X gathered into the
    product's transposed layout -- eager per-call times, one graph-replayed set, then ``nsets`` rotating sets."""
    path = backward_path()
    cfg = path.cfg
    T, H, E, k, I = cfg.T, cfg.H, cfg.E, cfg.k, cfg.I
    M = T * k
    calls = [("quantize_x_and_sort", path.quantize_and_sort), ("quantize_dy_row_and_tensor", path.quantize_dy),
             ("gmm_dx", path.grad_input), ("tgmm_dw", path.grad_weight)]
    settle(eager_step(calls), steps)
    durs, ms_eager = time_calls(calls, steps, warmup)
    path.capture_graph(warmup=1)
    settle(path.replay, steps)
    ms = time_replays([path], steps, warmup)
    qx = T * H * 2 + 4 if path.fused_quantize else T * H * 3 + 4 + T * H
    by = {"quantize_x_and_sort": qx + (M * 4 + 2 * M * 4 + E * 4 + M * H),
          "quantize_dy_row_and_tensor": (M * I * 3 + M * 4) + (M * I * 2 + M * I * 3 + 4),
          "gmm_dx": M * I + E * I * H + M * H * 2 + M * 4 + E * 4,
          "tgmm_dw": M * H + M * I + E * H * I * 4}
    fl = {"gmm_dx": 2 * M * I * H, "tgmm_dw": 2 * M * H * I}
    kern = {nm: kern_entry(d, by[nm], fl.get(nm, 0)) for nm, d in durs.items()}
    flops = fl["gmm_dx"] + fl["tgmm_dw"]
    res = {"workload": f"{cfg.name}: T={T} H={H} E={E} top-{k} I={I}, static activation and weight scales",
           "ms_per_step": round(ms, 4), "ms_per_step_eager": round(ms_eager, 4),
           "gmm_TFLOP_s_whole_step": round(flops / (ms * 1e-3) / 1e12, 1), "kernels": kern}
    paths = [path] + [backward_path(seed=7100 + i) for i in range(nsets - 1)]
    for p in paths[1:]:
        p.capture_graph(warmup=1)
    nrep = max(steps, nsets) // nsets * nsets
    settle(rotation(paths), nrep)
    msr = time_replays(paths, nrep, warmup)
    res["rotating_sets"] = {"sets": nsets, "steps": nrep, "ms_per_step": round(msr, 4),
                            "gmm_TFLOP_s_whole_step": round(flops / (msr * 1e-3) / 1e12, 1)}
    del paths, path
    torch.cuda.empty_cache()
    return res


def secondary_ffn_backward(steps, warmup):
    """The gated FFN's whole backward after a config-2 forward step: every
    call timed eagerly with HIP events, then the backward step as a graph.
    dW01's x is gathered by the forward's sort into the weight-gradient
    product's transposed layout."""
    from moe_fp8_grouped_amd.pipeline import FFNBackwardPath
    path, data = forward_path(2)
    weights = dict(data["weights"])
    del data
    cfg = path.cfg
    T, H, I, n = cfg.T, cfg.H, cfg.I, path.n_local
    path.step()
    g = torch.Generator(device="cuda").manual_seed(99)
    dout = (torch.randn((T, H), generator=g, device="cuda") * 1e-2).to(torch.bfloat16)
    b = FFNBackwardPath(path, {"weights": weights}, dout, transposed_x=True)
    del weights
    names = ("combine_backward", "quantize_dy", "grad_h", "grad_wo", "silu_backward", "quantize_dab",
             "grad_x_sorted", "grad_w01", "grad_x")
    calls = [(nm, getattr(b, nm)) for nm in names]
    settle(eager_step(calls), min(steps, 10))
    durs, ms_eager = time_calls(calls, min(steps, 10), warmup)
    b.capture_graph(warmup=1)
    settle(b.replay, steps)
    ms = time_replays([b], steps, warmup)
    fl = {"grad_h": 2 * n * H * I, "grad_wo": 2 * n * I * H, "grad_x_sorted": 2 * n * 2 * I * H,
          "grad_w01": 2 * n * H * 2 * I}
    kern = {}
    for nm, d in durs.items():
        e = _stats(d)
        if nm in fl:
            e["alg_flops"] = int(fl[nm])
            e["TFLOP_s"] = round(fl[nm] / (e["avg_us"] * 1e-6) / 1e12, 1)
        kern[nm] = e
    total = sum(fl.values())
    del b, path
    torch.cuda.empty_cache()
    return {"workload": workload_name(cfg) + ", backward after the forward step", "ms_per_step": round(ms, 4),
            "ms_per_step_eager": round(ms_eager, 4), "gmm_tgmm_flops": int(total),
            "gmm_TFLOP_s_whole_step": round(total / (ms * 1e-3) / 1e12, 1),
            "launch": "HIP graph replay of the backward step (per-call times from eager calls with HIP events)",
            "kernels": kern}


# ------------------------------------------------------------------ CPU oracle baseline
def oracle_forward_stages(cfg, data, qw, own_rows, m_cap, act_static=None):
    """The oracle's forward step stage by stage, each timed with perf_counter
    from inputs in host RAM to its output array: quantize this GPU's own rows
    (the rest of the token buffer stands for the all-gathered rows and is
    quantized beforehand), sort/gather, the grouped matmuls, the SiLU*mul
    requantization, the gather-reduce.  Returns (seconds per stage, GMM flops)."""
    from oracle.gather_reduce import gather_reduce
    from oracle.gmm import gmm
    from oracle.quantize import SCALE_ROW_DYNAMIC, SCALE_TENSOR_STATIC, quantize_rows
    from oracle.sort import sort_by_expert

    mode = SCALE_TENSOR_STATIC if act_static else SCALE_ROW_DYNAMIC
    T = cfg.T
    t = {}
    if own_rows < T:
        rest_q, rest_s, _ = quantize_rows(data["x"][own_rows:], mode, static_scale=act_static)
    c0 = time.perf_counter()
    q, s, _ = quantize_rows(data["x"][:own_rows], mode, static_scale=act_static)
    t["quantize"] = time.perf_counter() - c0
    if own_rows < T:
        q = np.concatenate([q, rest_q])
        s = np.concatenate([s, rest_s]) if mode == SCALE_ROW_DYNAMIC else s
    c0 = time.perf_counter()
    srt = sort_by_expert(data["ids"], cfg.E, cfg.group_offset, cfg.E_loc, xq=q, xscale=s, xscale_mode=mode,
                         m_cap=m_cap)
    t["sort"] = time.perf_counter() - c0
    gs, g0, El = srt["group_sizes"], cfg.group_offset, cfg.E_loc
    ls = srt["ss"] if mode == SCALE_ROW_DYNAMIC else s
    n = int(srt["n"])
    flops = 0
    if cfg.pipeline == "up":
        w, ws = qw["w_up"]
        c0 = time.perf_counter()
        y = gmm(srt["xs"], ls, w, ws, gs, g0, El)
        t["gmm_w_up"] = time.perf_counter() - c0
        flops += 2 * n * w.shape[1] * w.shape[2]
    else:
        (w0, s0), (w1, s1), (wo, so) = qw["wi_0"], qw["wi_1"], qw["wo"]
        c0 = time.perf_counter()
        a = gmm(srt["xs"], ls, w0, s0, gs, g0, El)
        b = gmm(srt["xs"], ls, w1, s1, gs, g0, El)
        t["gmm_wi_01"] = time.perf_counter() - c0
        c0 = time.perf_counter()
        hq, hs, _ = quantize_rows(a["bf16"], SCALE_ROW_DYNAMIC, x_up_bits=b["bf16"])
        t["silu_quant"] = time.perf_counter() - c0
        c0 = time.perf_counter()
        y = gmm(hq, hs, wo, so, gs, g0, El)
        t["gmm_wo"] = time.perf_counter() - c0
        flops += 2 * n * (w0.shape[1] * w0.shape[2] * 2 + wo.shape[1] * wo.shape[2])
    c0 = time.perf_counter()
    gather_reduce(y["bf16"], True, srt["inv_pos"].reshape(T, cfg.k), data["topk_w"])
    t["gather_reduce"] = time.perf_counter() - c0
    return t, flops, n


def cpu_baseline(cfg4_data, n_local_experts=8, reps_small=5):
    """The oracle on the host's cores.  Line of record: config 4's step
    restricted to ``n_local_experts`` of the 32 local experts (64, 65, ...):
    the same tokens, quantization of the own 1024 rows, sort and gather-reduce
    over all 8192 tokens, the grouped matmuls on the rows routed to those
    experts.  Also configs 1 and 3 whole, on every core and single-threaded,
    median of ``reps_small`` runs per stage."""
    from threadpoolctl import threadpool_info, threadpool_limits
    from oracle.pipeline import quantize_config_weights
    from workloads import CONFIGS, STATIC_ACT_SCALE, STATIC_WEIGHT_SCALE, generate

    blas = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
    cores = max(blas) if blas else 1
    cfg = dataclasses.replace(CONFIGS[4], num_local_experts=n_local_experts)
    data = dict(cfg4_data)
    data["weights"] = {nm: w[:n_local_experts] for nm, w in cfg4_data["weights"].items()}
    qw = quantize_config_weights(cfg, data["weights"])           # pre-quantized weights (set-up, not timed)
    n = int(((data["ids"] >= cfg.group_offset) & (data["ids"] < cfg.group_offset + cfg.E_loc)).sum())
    m_cap = (n + 255) // 256 * 256
    c0 = time.perf_counter()
    t, flops, n = oracle_forward_stages(cfg, data, qw, cfg.T // 8, m_cap)
    wall = time.perf_counter() - c0
    res = {"value": round(flops / wall / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
           "sample": f"config 4's step restricted to local experts {cfg.group_offset}..{cfg.group_offset + n_local_experts - 1} "
                     f"({n} of the slice's routed rows; GMM flops {flops}): quantize the own {cfg.T // 8} tokens, "
                     f"sort and gather-reduce all {cfg.T} tokens, the three grouped matmuls and the SiLU "
                     f"requantization on those rows; numpy float64, {wall:.1f} s",
           "stages_s": {k: round(v, 3) for k, v in t.items()},
           "affinity_cpus": len(os.sched_getaffinity(0)), "blas_threads": int(cores)}
    small = {}
    for cid, static in ((1, False), (3, False), (3, True)):
        c = CONFIGS[cid]
        d = generate(c)
        q = quantize_config_weights(c, d["weights"], static_scale=STATIC_WEIGHT_SCALE if static else None)
        key = f"config {cid}{' static' if static else ''}"
        for label, limit in (("all_cores", None), ("single_thread", 1)):
            per = []
            with threadpool_limits(limits=limit):
                for _ in range(reps_small):
                    tt, fl, _ = oracle_forward_stages(c, d, q, c.T, c.M, act_static=STATIC_ACT_SCALE if static else None)
                    per.append(tt)
            med = {k: float(np.median([p[k] for p in per])) for k in per[0]}
            tot = sum(med.values())
            small.setdefault(key, {})[label] = {"stages_ms": {k: round(v * 1e3, 3) for k, v in med.items()},
                                               "step_ms": round(tot * 1e3, 3),
                                               "gmm_TFLOP_s": round(fl / tot / 1e12, 6)}
    res["small_configs"] = small
    return res


def main():
    global SETTLE_S
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the other workloads measured beside the line of record")
    ap.add_argument("--settle-s", type=float, default=SETTLE_S,
                    help="seconds of untimed steps before each timed region (clock ramp; 0 to skip)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="run a plain copy of this many MiB first (profiler byte-counter calibration)")
    ap.add_argument("--only", default="",
                    help="comma-separated names of the other workloads to run alone (no line of record), "
                         "e.g. moe_backward; for profiling one workload")
    a = ap.parse_args()
    SETTLE_S = a.settle_s
    if a.gpus != 1:
        print(f"bench.py: the benchmark runs on one GPU only (asked for {a.gpus}); expert parallelism is modelled "
              f"as one GPU's expert slice", file=sys.stderr)
        sys.exit(2)
    import moe_fp8_grouped_amd as m
    m.load_library()
    if a.calib_copy_mib:
        # a plain copy kernel of known size: its HBM counters calibrate the profiler's byte counts
        src = torch.ones(a.calib_copy_mib << 18, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.add(src, 0.0, out=dst)
        torch.cuda.synchronize()
        del src, dst
    secondaries = (("gated_ffn_fwd", lambda: secondary_forward(2, a.steps, a.warmup)),
                   ("gated_ffn_fwd_cold", lambda: rotating_forward(2, a.steps, a.warmup)),
                   ("moe_backward", lambda: secondary_backward(min(a.steps, 50), a.warmup)),
                   ("gated_ffn_backward", lambda: secondary_ffn_backward(a.steps, a.warmup)),
                   ("tiny_up_proj", lambda: secondary_forward(1, a.steps, a.warmup)),
                   ("tiny_zipf_blockwise", lambda: secondary_forward(3, a.steps, a.warmup)),
                   ("tiny_zipf_blockwise_static", lambda: secondary_forward(3, a.steps, a.warmup, True)),
                   ("skewed_large_blockwise", lambda: secondary_forward(6, a.steps, a.warmup)),
                   ("skewed_large_blockwise_static", lambda: secondary_forward(6, a.steps, a.warmup, True)))
    if a.only:
        names = a.only.split(",")
        unknown = sorted(set(names) - {k for k, _ in secondaries})
        if unknown:
            print(f"bench.py: unknown workload(s) {unknown}", file=sys.stderr)
            sys.exit(2)
        sec = {}
        for key, fn in secondaries:
            if key in names:
                print(f"bench: {key} alone", file=sys.stderr, flush=True)
                sec[key] = fn()
        print(json.dumps({"only": names, "steps": a.steps, "warmup": a.warmup, "secondary": sec}), flush=True)
        return
    print(f"bench: config {a.config}, {a.steps} timed steps after {a.warmup}", file=sys.stderr, flush=True)
    path, data = forward_path(a.config)
    cfg = path.cfg
    keep = data if (a.config == 4 and not a.no_cpu_baseline) else None
    del data
    head, durs, acc = measure_forward(path, a.steps, a.warmup)
    dominant = "gmm_wi_01" if cfg.pipeline == "ffn" else "gmm_w_up"
    roof = roofline(durs[dominant], acc[dominant])
    if a.config != 4:
        roof["traffic"] = None     # the committed counter summary covers config 4's dominant launch
    int8 = None
    if not a.no_secondary and cfg.pipeline == "ffn" and cfg.weight_block_k and cfg.weight_block_n > 1:
        print("bench: int8 grouped matmuls", file=sys.stderr, flush=True)
        int8 = int8_gmm_timing(path, acc, a.steps, a.warmup)
    del path
    torch.cuda.empty_cache()
    value = head["gmm_TFLOP_s_whole_step"]
    res = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": head["ms_per_step"], "ms_per_step_eager": head["ms_per_step_eager"],
        "ms_per_step_eager_back_to_back": head["ms_per_step_eager_back_to_back"],
        "settle": head["settle"],
        "launch": "HIP graph replay of the whole step (per-launch times from eager steps with HIP events)",
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8 (e4m3fn operands, f32 accumulate)", "data": "synthetic (seeded; random-init weights)",
        "config": {"workload": head["workload"], "routed_local_rows": head["routed_local_rows"],
                   "m_cap": head["m_cap"], "gmm_flops_per_step": head["gmm_flops_per_step"]},
        "frac_fp8_peak_whole_step": round(value / PEAK_FP8_TFLOPS, 4),
        "sort_gather_GB_s": {nm: head["kernels"][nm]["GB_s"] for nm in ("quantize", "sort", "quantize_sort",
                                                                        "gather_reduce") if nm in head["kernels"]},
        "roofline": roof,
        "kernels": head["kernels"],
        "device": torch.cuda.get_device_name(0),
    }
    if not a.no_secondary:
        sec = {}
        for key, fn in secondaries:
            print(f"bench: secondary {key}", file=sys.stderr, flush=True)
            sec[key] = fn()
        if int8 is not None:
            sec["int8_gmm_expert_slice"] = int8
        res["secondary"] = sec
    if keep is not None:
        print("bench: cpu baseline", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(keep)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
