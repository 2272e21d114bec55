"""moe_nvfp4_forward (NVFP4 experts: E4M3 block scales per 16, a float32
second-level scale per expert and projection, multiplied before the bias) on
the GPU against the float64 oracle; same bar as the MXFP4 layer.  Experts with
at least 128 pairs take full tiles when H and I are multiples of 64, else mid
tiles; both are covered."""

import numpy as np
import pytest
import torch

from mxfp4_quantized_expert_amd import workloads as W
from oracle import mxfp4_moe as O
from tests.helpers import assert_layer_parity, assert_layer_parity_nan, long_prefill_120b_nvfp4

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
                                       (40, 4096, 64, 4, 2), (600, 96, 160, 3, 2), (700, 4096, 64, 2, 1),
                                       (900, 192, 320, 3, 2)])
def test_ragged_shapes(gpu, T, H, I, E, k):
    # odd numbers of 16- and 32-element blocks, experts with several mid
    # tiles, a single expert, the largest hidden size; experts with full
    # tiles and remainders (H, I multiples of 64), and with 128+ pairs where
    # H = 96 keeps them on mid tiles
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


def _owned_layer(counts, H, I, seed):
    """A top-1 NVFP4 layer whose expert e gets exactly counts[e] tokens."""
    E = len(counts)
    T = sum(counts)
    spec = W.LAYERS["20b_live"].with_(T=T, H=H, I=I, E=E, top_k=1)
    L = W.make_nvfp4_layer(spec, seed=seed)
    rng = np.random.default_rng(seed + 1)
    owner = rng.permutation(np.repeat(np.arange(E), counts))
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[np.arange(T), owner] += 20.0
    L["router_logits"] = logits
    return L


def test_tile_boundaries(gpu):
    # experts on both sides of the 128-pair full-tile threshold, the 4-pair
    # streaming limit and the 48-pair mid-tile size
    counts = [128, 127, 129, 4, 5, 16, 17, 32, 33, 48, 49, 64, 65, 96, 97, 1, 0, 259, 256]
    L = _owned_layer(counts, H=128, I=192, seed=51)
    assert_layer_parity(_forward(gpu, L, 1), O.moe_forward_nvfp4(L, 1), "nvfp4 tile boundaries")


def test_scale_bytes_full_range(gpu):
    # every finite E4M3 value as a block scale (both signs, the subnormals and
    # zero) on experts with full, mid and streaming tiles: the full tiles' f16
    # down GEMM builds code x scale from the scale's power of two and its
    # significand, exact for all of them, as the bf16 tiles' float32 product is
    counts = [259, 128, 130, 60, 17, 3, 1, 0]
    L = _owned_layer(counts, H=128, I=192, seed=71)
    rng = np.random.default_rng(72)
    finite = np.array([b for b in range(256) if b & 0x7F != 0x7F], dtype=np.uint8)
    for k in ("w13_scales", "w2_scales"):
        L[k] = rng.choice(finite, size=L[k].shape)
    assert_layer_parity(_forward(gpu, L, 1), O.moe_forward_nvfp4(L, 1), "nvfp4 full-range scale bytes")


def test_nan_scale_byte(gpu):
    # E4M3 NaN scale bytes (0x7F, 0xFF) in one block of a gate_up row and of a
    # down row of an expert on each kind of tile (full, mid, streaming): the
    # output NaNs sit exactly where the oracle's do, every other element meets
    # the bar
    counts = [128, 127, 129, 4, 5, 16, 17, 32, 33, 64, 65, 1, 0, 259]
    L = _owned_layer(counts, H=64, I=128, seed=61)
    L["w13_scales"][13, 7, 1] = 0x7F    # full tiles (259 pairs), a gate row
    L["w13_scales"][8, 130, 2] = 0xFF   # mid tile (33 pairs)
    L["w13_scales"][3, 191, 3] = 0x7F   # streaming tile (4 pairs), an up row
    L["w2_scales"][0, 5, 2] = 0xFF      # full tile (128 pairs)
    L["w2_scales"][10, 40, 0] = 0x7F    # mid tiles (65 pairs)
    L["w2_scales"][11, 63, 7] = 0xFF    # streaming tile (1 pair), the last block of the row
    assert_layer_parity_nan(_forward(gpu, L, 1), O.moe_forward_nvfp4(L, 1), "nvfp4 NaN scale bytes")


def test_120b_long_prefill(gpu):
    # every output of the gpt-oss-120b shaped long prefill with NVFP4 experts
    spec, L, ref = long_prefill_120b_nvfp4()
    ids, _ = O.route(L["router_logits"], spec.top_k)
    counts = np.bincount(ids.ravel(), minlength=spec.E)
    assert (counts >= 128).any() and ((counts > 4) & (counts < 128)).any() and ((counts > 0) & (counts <= 4)).any()
    assert_layer_parity(_forward(gpu, L, spec.top_k), ref, "nvfp4 120b (all tokens)")
