"""moe_mxfp4_forward, moe_mxfp4_forward_router and mxfp4_dequantize captured
in a HIP graph (torch.cuda.CUDAGraph) and replayed.

The library makes no allocation, memset or host synchronization inside a
call, so a call is capturable after a first eager call (which sets the
kernels' LDS attributes).  Each replay runs on new inputs copied into the
captured buffers, with eager library calls and synchronizations between the
replays, and must give the bits of the eager call on the same inputs (the
path is deterministic).
"""

import numpy as np
import pytest
import torch

from mxfp4_quantized_expert_amd import workloads as W
from tests.helpers import bits_u16

pytestmark = pytest.mark.gpu


def _bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


@pytest.mark.parametrize("name,T", [("tiny", 16), ("20b_decode", 4), ("20b_prefill", 64), ("20b_prefill", 256)])
@pytest.mark.parametrize("router", [False, True])
def test_forward_graph_replays(gpu, name, T, router):
    spec = W.LAYERS[name].with_(T=T)
    L = dict(W.make_layer(spec), **W.make_router(spec))
    d = gpu.layer_to_device(L)
    k = spec.top_k
    ws = torch.empty((gpu.workspace_bytes(T, spec.H, spec.I, spec.E, k),), dtype=torch.uint8, device="cuda")
    x = d["x"].clone()
    logits = d["router_logits"].clone()
    y = torch.empty((T, spec.H), dtype=torch.bfloat16, device="cuda")

    def call(xx, lg, out, workspace=ws):
        if router:
            return gpu.moe_mxfp4_forward_router(xx, d["router_w"], d["router_b"], d["w13_blocks"], d["w13_scales"],
                                                d["w13_bias"], d["w2_blocks"], d["w2_scales"], d["w2_bias"], k,
                                                out=out, workspace=workspace)
        return gpu.moe_mxfp4_forward(xx, lg, d["w13_blocks"], d["w13_scales"], d["w13_bias"], d["w2_blocks"],
                                     d["w2_scales"], d["w2_bias"], k, out=out, workspace=workspace)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call(x, logits, y)  # eager first call on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(x, logits, y)
    rng = np.random.default_rng(3)
    for rep in range(4):
        xn = _bf16(W.to_bf16_bits(rng.standard_normal((T, spec.H)).astype(np.float32)))
        ln = torch.from_numpy((rng.standard_normal((T, spec.E)) * 2).astype(np.float32)).cuda()
        x.copy_(xn)
        logits.copy_(ln)
        g.replay()
        torch.cuda.synchronize()
        got = bits_u16(y)
        # eager reference on the same inputs, with its own workspace and output
        ws2 = torch.empty_like(ws)
        ref = call(xn, ln, torch.empty_like(y), ws2)
        torch.cuda.synchronize()
        assert np.array_equal(got, bits_u16(ref)), f"replay {rep} differs from the eager call"


def test_dequant_graph_replays(gpu):
    bank = W.DequantBankSpec("small", E=2, N=96, K=160)
    blocks, scales = W.make_bank(bank)
    b = torch.from_numpy(blocks).cuda()
    sc = torch.from_numpy(scales).cuda()
    out = torch.empty(blocks.shape[:-1] + (2 * blocks.shape[-1],), dtype=torch.bfloat16, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        gpu.mxfp4_dequantize(b, sc, out=out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gpu.mxfp4_dequantize(b, sc, out=out)
    rng = np.random.default_rng(4)
    for rep in range(3):
        b.copy_(torch.from_numpy(np.frombuffer(rng.bytes(blocks.size), dtype=np.uint8).reshape(blocks.shape).copy()))
        g.replay()
        torch.cuda.synchronize()
        ref = gpu.mxfp4_dequantize(b, sc)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"replay {rep}"


@pytest.mark.parametrize("act", ["bf16", "mxfp8_split"])
def test_forward_graph_replays_full_tiles(gpu, act):
    # Experts with several full 128-pair tiles, so the full-tile kernels (LDS
    # staging by the load unit; the FP4 kernel's dynamic LDS) run inside the
    # graph; a small hidden size keeps the layer cheap.
    spec = W.LAYERS["20b_live"].with_(T=1024, H=256, I=192, E=4, top_k=2)
    L = W.make_layer(spec, seed=11)
    d = gpu.layer_to_device(L)
    k = spec.top_k
    flags = gpu.ACT_FLAGS[act]
    ws = torch.empty((gpu.workspace_bytes(spec.T, spec.H, spec.I, spec.E, k, flags),), dtype=torch.uint8,
                     device="cuda")
    x = d["x"].clone()
    logits = d["router_logits"].clone()
    y = torch.empty((spec.T, spec.H), dtype=torch.bfloat16, device="cuda")

    def call(xx, lg, out, workspace=ws):
        return gpu.moe_mxfp4_forward(xx, lg, d["w13_blocks"], d["w13_scales"], d["w13_bias"], d["w2_blocks"],
                                     d["w2_scales"], d["w2_bias"], k, out=out, workspace=workspace, act=act)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call(x, logits, y)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(x, logits, y)
    rng = np.random.default_rng(12)
    for rep in range(3):
        xn = _bf16(W.to_bf16_bits(rng.standard_normal((spec.T, spec.H)).astype(np.float32)))
        ln = torch.from_numpy((rng.standard_normal((spec.T, spec.E)) * 2).astype(np.float32)).cuda()
        x.copy_(xn)
        logits.copy_(ln)
        g.replay()
        torch.cuda.synchronize()
        got = bits_u16(y)
        ref = call(xn, ln, torch.empty_like(y), torch.empty_like(ws))
        torch.cuda.synchronize()
        assert np.array_equal(got, bits_u16(ref)), f"replay {rep} differs from the eager call"
