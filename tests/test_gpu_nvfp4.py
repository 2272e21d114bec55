"""moe_nvfp4_forward (NVFP4 experts: E4M3 block scales per 16, a float32
second-level scale per expert and projection, multiplied before the bias) on
the GPU against the float64 oracle; same bar as the MXFP4 layer."""

import numpy as np
import pytest
import torch

from mxfp4_quantized_expert_amd import workloads as W
from oracle import mxfp4_moe as O
from tests.helpers import assert_layer_parity

pytestmark = pytest.mark.gpu


def _forward(gpu, L, k):
    d = gpu.layer_to_device(L)
    y = gpu.moe_nvfp4_forward(d["x"], d["router_logits"], d["w13_blocks"], d["w13_scales"], d["w13_scale2"],
                              d["w13_bias"], d["w2_blocks"], d["w2_scales"], d["w2_scale2"], d["w2_bias"], k)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("name", ["20b_decode", "20b_prefill"])
def test_gpt_oss_20b_shapes(gpu, name):
    spec = W.LAYERS[name]
    L = W.make_nvfp4_layer(spec)
    assert_layer_parity(_forward(gpu, L, spec.top_k), O.moe_forward_nvfp4(L, spec.top_k), f"nvfp4 {name}")


@pytest.mark.parametrize("T,H,I,E,k", [(5, 96, 160, 7, 3), (300, 128, 64, 2, 1), (3, 32, 32, 1, 1),
                                       (40, 4096, 64, 4, 2)])
def test_ragged_shapes(gpu, T, H, I, E, k):
    # odd numbers of 16- and 32-element blocks, experts with several mid
    # tiles, a single expert, the largest hidden size
    spec = W.LAYERS["20b_live"].with_(T=T, H=H, I=I, E=E, top_k=k)
    L = W.make_nvfp4_layer(spec, seed=T + H)
    assert_layer_parity(_forward(gpu, L, k), O.moe_forward_nvfp4(L, k), f"nvfp4 {(T, H, I, E, k)}")


def test_second_level_scale_before_the_bias(gpu):
    # A layer where the down bias is a large part of z: the GPU must follow
    # sum w*(s*y + b) and miss the folded form sum w*s*(y + b) by far.
    spec = W.LAYERS["20b_live"].with_(T=64, H=256, I=128, E=8, top_k=2, bias_std=2.0)
    L = W.make_nvfp4_layer(spec, seed=4, scale_lo=0x18, scale_hi=0x20)
    L["w2_scale2"][:] = 0.125
    ref = O.moe_forward_nvfp4(L, spec.top_k)
    y = _forward(gpu, L, spec.top_k)
    assert_layer_parity(y, ref, "nvfp4 bias after scale")
    L1 = dict(L, w2_scale2=np.ones_like(L["w2_scale2"]), w2_bias=np.zeros_like(L["w2_bias"]))
    y1 = O.moe_forward_nvfp4(L1, spec.top_k)
    ids, w = O.route(L["router_logits"], spec.top_k)
    b2 = O.bf16_decode(L["w2_bias"])
    folded = 0.125 * (y1 + sum(w[:, j:j + 1] * b2[ids[:, j]] for j in range(spec.top_k)))
    assert O.parity_errors(folded, ref)[0] > 10 * 1e-2
