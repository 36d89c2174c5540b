"""End-to-end context for the oracle: the fp8 pipelines against the
unquantized bf16 dense reference, compared with the pages' own accuracy
ordering (dynamic absmax closer to bf16 than static scales) and magnitude."""

import numpy as np

from oracle.pipeline import (dense_bf16_reference, forward_pipeline, quantize_config_weights,
                             rel_norm_diff)
from oracle.quantize import SCALE_ROW_DYNAMIC, SCALE_TENSOR_STATIC
from tests.golden import accuracy_tables
from workloads import CONFIGS, STATIC_ACT_SCALE, STATIC_WEIGHT_SCALE, generate, scaled_config


def _run(cfg, static):
    data = generate(cfg)
    qw = quantize_config_weights(cfg, data["weights"], static_scale=STATIC_WEIGHT_SCALE if static else None)
    mode = SCALE_TENSOR_STATIC if static else SCALE_ROW_DYNAMIC
    st = forward_pipeline(cfg, data, qw, act_mode=mode, act_static=STATIC_ACT_SCALE if static else None)
    ref = dense_bf16_reference(cfg, data)
    return rel_norm_diff(st["out"]["bf16"], ref), st


def test_up_projection_dynamic_better_than_static_like_the_pages():
    tables = accuracy_tables()
    dyn_page = tables[("rel", "megablox_fp8_dynamic_ep1")][0]
    sta_page = tables[("rel", "megablox_fp8_static_ep1")][0]
    assert dyn_page < sta_page
    (dyn, _), _ = _run(CONFIGS[1], static=False)
    (sta, _), _ = _run(CONFIGS[3], static=True)
    (dyn3, _), _ = _run(CONFIGS[3], static=False)
    # e4m3 keeps 3 mantissa bits: a few percent of relative error, never order one
    assert 0.005 < dyn < 0.2 and 0.005 < dyn3 < 0.2
    assert dyn < sta < 1.0
    assert dyn3 < sta


def test_small_gated_ffn_and_expert_slice_context():
    cfg = scaled_config(2, T=64, H=256, E=8, k=2, I=128)
    (dyn, mx), st = _run(cfg, static=False)
    assert 0.005 < dyn < 0.2
    # local expert slice: tokens with no local expert come out exactly zero
    cfg4 = scaled_config(4, T=64, H=256, E=16, k=2, I=128, group_offset=4, num_local_experts=4,
                         outlier_frac=0.05)
    (d4, _), st4 = _run(cfg4, static=False)
    inv = st4["sort"]["inv_pos"].reshape(cfg4.T, cfg4.k)
    none = np.all(inv < 0, axis=1)
    assert none.any()
    assert not st4["out"]["bf16"][none].any()
    assert 0.005 < d4 < 0.2
