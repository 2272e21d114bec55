"""The opt-in FP4 scaled-MFMA path (MXFP4MOE_ACT_MXFP8[_SPLIT]) on the GPU.

The activation quantizer decides integers (E4M3 codes and E8M0 scale bytes)
from exact bf16 inputs with exact power-of-two scaling, so its output must
equal the oracle's bit for bit.  The layer is compared with the oracle of the
same mode (experts with at least 128 pairs quantized, the rest exact) at the
layer's bar; its distance from the exact layer is printed, and for the split
mode must also be inside the bar.
"""

import numpy as np
import pytest
import torch

from mxfp4_quantized_expert_amd import workloads as W
from oracle import mxfp4_moe as O
from tests.helpers import assert_layer_parity, bf16_to_f64, long_prefill_120b

pytestmark = pytest.mark.gpu


def _expected_quant(v: np.ndarray, split: bool):
    """Oracle codes/scales in the quantizer's chunk-interleaved layout."""
    rows, K = v.shape
    nc = (K + 63) // 64
    Kp = 64 * nc
    vp = np.zeros((rows, Kp))
    vp[:, :K] = v
    hc, hs = O.mxfp8_quantize(vp)
    if split:
        lc, ls = O.mxfp8_quantize(vp - O.mxfp8_dequantize(hc, hs))
    else:
        lc, ls = np.zeros_like(hc), np.full_like(hs, 127)
    # pad groups (past K) carry zero codes and scale 127
    pad = np.arange(Kp // 32) * 32 >= K
    hs[:, pad] = 127
    ls[:, pad] = 127
    codes = np.concatenate([hc.reshape(rows, nc, 64), lc.reshape(rows, nc, 64)], axis=2).reshape(rows, 128 * nc)
    scales = np.stack([hs[:, 0::2], hs[:, 1::2], ls[:, 0::2], ls[:, 1::2]], axis=2).reshape(rows, 4 * nc)
    return codes.astype(np.uint8), scales.astype(np.uint8)


@pytest.mark.parametrize("K", [64, 96, 2880])
@pytest.mark.parametrize("split", [True, False])
def test_quantizer_bit_exact(gpu, K, split):
    rng = np.random.default_rng(K)
    rows = 37
    v = rng.standard_normal((rows, K)).astype(np.float32) * np.float32(3.0)
    v[0, :] = 0.0                        # all-zero row
    v[1, :32] = -0.0                     # negative zeros
    v[2, :] *= np.float32(1e-30)         # tiny blocks
    v[3, ::7] = np.float32(250.0)        # large values
    v[4, :32] = np.float32(2.0 ** -140)  # below the bf16 normal range
    bits = W.to_bf16_bits(v)
    exp_codes, exp_scales = _expected_quant(O.bf16_decode(bits), split)
    src = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    codes, scales = gpu.moe_mxfp8_quantize(src, split)
    torch.cuda.synchronize()
    got_c, got_s = codes.cpu().numpy(), scales.cpu().numpy()
    assert np.array_equal(got_s, exp_scales), np.argwhere(got_s != exp_scales)[:5]
    assert np.array_equal(got_c, exp_codes), np.argwhere(got_c != exp_codes)[:5]


def _quantized_experts(L, k):
    ids, _ = O.route(L["router_logits"], k)
    E = L["router_logits"].shape[1]
    return np.bincount(ids.ravel(), minlength=E) >= 128


def _run(gpu, L, k, act, tokens=None):
    d = gpu.layer_to_device(L)
    y = gpu.moe_mxfp4_forward(d["x"], d["router_logits"], d["w13_blocks"], d["w13_scales"], d["w13_bias"],
                              d["w2_blocks"], d["w2_scales"], d["w2_bias"], k, act=act)
    torch.cuda.synchronize()
    if tokens is not None:
        y = y[torch.from_numpy(np.asarray(tokens)).to(y.device)]
    return y


def _check(gpu, L, k, act, label, tokens=None, exact=None):
    mode = "split" if act == "mxfp8_split" else "single"
    q = _quantized_experts(L, k)
    assert q.any(), "the case must have experts on the FP4 path"
    y = _run(gpu, L, k, act, tokens)
    ref = O.moe_forward_fp8act(L, k, q, mode, tokens=tokens)
    assert_layer_parity(y, ref, f"{label}/{act} vs its oracle")
    if exact is None:
        exact = O.moe_forward(L, k, tokens=tokens)
    rel, mx = O.parity_errors(bf16_to_f64(y), exact)
    print(f"[fp4mma] {label}/{act}: vs the exact layer normwise {rel:.3e}, max-element {mx:.3e}", flush=True)
    if act == "mxfp8_split":
        assert rel <= 1e-2 and mx <= 2e-2


@pytest.mark.parametrize("act", ["mxfp8_split", "mxfp8"])
@pytest.mark.parametrize("case", [(600, 96, 160, 3, 2), (300, 128, 64, 2, 1), (700, 4096, 64, 2, 1)])
def test_layer_against_oracle(gpu, act, case):
    # experts with several full 128-pair tiles plus remainders; K tails (96 and
    # 160 are odd numbers of 32-groups); the largest hidden size
    T, H, I, E, k = case
    spec = W.LAYERS["20b_live"].with_(T=T, H=H, I=I, E=E, top_k=k)
    L = W.make_layer(spec, seed=T + H)
    _check(gpu, L, k, act, f"{case}")


def test_tile_boundaries_split(gpu):
    # experts on both sides of the 128-pair threshold in one batch
    counts = [128, 127, 129, 4, 5, 16, 17, 32, 33, 64, 65, 1, 0, 259]
    E = len(counts)
    T = sum(counts)
    spec = W.LAYERS["20b_live"].with_(T=T, H=64, I=96, E=E, top_k=1)
    L = W.make_layer(spec, seed=31)
    rng = np.random.default_rng(32)
    owner = rng.permutation(np.repeat(np.arange(E), counts))
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[np.arange(T), owner] += 20.0
    L["router_logits"] = logits
    _check(gpu, L, 1, "mxfp8_split", "tile boundaries")


@pytest.mark.parametrize("act", ["mxfp8_split", "mxfp8"])
def test_120b_long_prefill(gpu, act):
    # every output of the 120b long prefill: against the oracle of the same
    # mode at the bar, and (split) against the exact oracle at the bar
    spec, L, exact = long_prefill_120b()
    _check(gpu, L, spec.top_k, act, "120b (all tokens)", exact=exact)
