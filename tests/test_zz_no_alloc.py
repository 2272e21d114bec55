"""moe_mxfp4_forward_noalloc - the entry point whose scratch is a fixed device
array of the library - against moe_mxfp4_forward with a caller's workspace,
through the C ABI, on calls in a row of decreasing size (each call leaves the
scratch to the next): the same kernels must give the same bits, and the
layer must meet the bar against the oracle."""

import numpy as np
import pytest
import torch

from mxfp4_quantized_expert_amd import workloads as W
from oracle import mxfp4_moe as O
from tests.helpers import assert_layer_parity, bits_u16

pytestmark = pytest.mark.gpu


def test_noalloc_matches_workspace_entry_calls_in_a_row(gpu):
    cases = [
        # gpt-oss shapes, four experts with 256 pairs each: full 128-pair tiles (about 12 MB of scratch)
        ("full tiles", W.LAYERS["20b_prefill"].with_(T=512, E=4, top_k=2), 31),
        # the 20b prefill batch: mid and streaming tiles
        ("mid tiles", W.LAYERS["20b_prefill"], 32),
        # a decode batch, much smaller than the calls before it
        ("decode", W.LAYERS["20b_live"], 33),
    ]
    for label, spec, seed in cases:
        L = W.make_layer(spec, seed=seed)
        d = gpu.layer_to_device(L)
        args = (d["x"], d["router_logits"], d["w13_blocks"], d["w13_scales"], d["w13_bias"], d["w2_blocks"],
                d["w2_scales"], d["w2_bias"], spec.top_k)
        need = gpu.workspace_bytes(spec.T, spec.H, spec.I, spec.E, spec.top_k)
        assert need <= gpu.NOALLOC_SCRATCH_BYTES
        y_na = gpu.moe_mxfp4_forward_noalloc(*args)
        y_ws = gpu.moe_mxfp4_forward(*args)
        torch.cuda.synchronize()
        print(f"[noalloc] {label}: T={spec.T} E={spec.E} k={spec.top_k}, {need / 2**20:.1f} MiB of scratch",
              flush=True)
        assert np.array_equal(bits_u16(y_na), bits_u16(y_ws)), f"{label}: differs from the workspace entry point"
        assert_layer_parity(y_na, O.moe_forward(L, spec.top_k), f"noalloc {label}")


def test_noalloc_rejects_layers_beyond_the_scratch(gpu):
    spec = W.LAYERS["tiny"].with_(T=4096, H=2880, I=2880, E=8, top_k=4)
    assert gpu.workspace_bytes(spec.T, spec.H, spec.I, spec.E, spec.top_k) > gpu.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((spec.T, spec.H), dtype=torch.bfloat16, device="cuda")
    lg = torch.zeros((spec.T, spec.E), dtype=torch.float32, device="cuda")
    w13b = torch.zeros((spec.E, 2 * spec.I, spec.H // 2), dtype=torch.uint8, device="cuda")
    w13s = torch.zeros((spec.E, 2 * spec.I, spec.H // 32), dtype=torch.uint8, device="cuda")
    b13 = torch.zeros((spec.E, 2 * spec.I), dtype=torch.bfloat16, device="cuda")
    w2b = torch.zeros((spec.E, spec.H, spec.I // 2), dtype=torch.uint8, device="cuda")
    w2s = torch.zeros((spec.E, spec.H, spec.I // 32), dtype=torch.uint8, device="cuda")
    b2 = torch.zeros((spec.E, spec.H), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(gpu.MXFP4MoEError) as err:
        gpu.moe_mxfp4_forward_noalloc(x, lg, w13b, w13s, b13, w2b, w2s, b2, spec.top_k)
    assert err.value.status == -6
