"""Seeded generator checks (CPU only): determinism, shapes and the load skew."""

import numpy as np

from mxfp4_quantized_expert_amd import workloads as W
from oracle import mxfp4_moe as O


def test_same_seed_same_bytes():
    a = W.make_layer(W.LAYERS["tiny"])
    b = W.make_layer(W.LAYERS["tiny"])
    for k in a:
        assert np.array_equal(a[k], b[k]), k
    c = W.make_layer(W.LAYERS["tiny"], seed=1)
    assert not np.array_equal(a["w13_blocks"], c["w13_blocks"])


def test_shapes_and_ranges():
    spec = W.LAYERS["tiny"]
    L = W.make_layer(spec)
    E, H, I, T = spec.E, spec.H, spec.I, spec.T
    assert L["x"].shape == (T, H) and L["x"].dtype == np.uint16
    assert L["router_logits"].shape == (T, E) and L["router_logits"].dtype == np.float32
    assert L["w13_blocks"].shape == (E, 2 * I, H // 2)
    assert L["w13_scales"].shape == (E, 2 * I, H // 32)
    assert L["w2_blocks"].shape == (E, H, I // 2)
    assert L["w2_scales"].shape == (E, H, I // 32)
    assert L["w13_bias"].shape == (E, 2 * I) and L["w2_bias"].shape == (E, H)
    assert L["w13_scales"].min() >= 123 and L["w13_scales"].max() <= 129


def test_routing_inputs_replay_the_layer_draws():
    spec = W.LAYERS["tiny"]
    x, lg = W.make_routing_inputs(spec)
    L = W.make_layer(spec)
    assert np.array_equal(x, L["x"]) and np.array_equal(lg, L["router_logits"])


def test_zipf_layer_leaves_experts_empty():
    # The 120b long-prefill layer: Zipf-skewed routing leaves some experts with no token.
    spec = W.LAYERS["120b_prefill"]
    _, logits = W.make_routing_inputs(spec)
    ids, _ = O.route(logits, spec.top_k)
    counts = np.bincount(ids.ravel(), minlength=spec.E)
    assert (counts == 0).sum() >= 1
    assert counts.max() > 8 * np.median(counts[counts > 0])
