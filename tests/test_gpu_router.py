"""The router projection fused ahead of the top-k (moe_mxfp4_router and
moe_mxfp4_forward_router) on the GPU against the float64 oracle.

The logits are a float computation (fp32 accumulation on the GPU, float64 in
the oracle), so they are compared within a bound derived from the
accumulation: |error| <= 2e-5 * sum_h |x_h W_eh| + 1e-6 (about a hundred
times the typical fp32 error over 2880 terms; a dropped 32-wide K step alone
is about 1e-2 of that sum).  The top-k choice is an integer
decided by those floats: on every token whose oracle gap between the k-th and
the (k+1)-th logit exceeds twice that bound the ids must equal the oracle's
exactly, and on the others the GPU's picks must be a valid top-k within the
bound.  Layer outputs are compared on the unambiguous tokens at the layer's
bar.
"""

import numpy as np
import pytest
import torch

from mxfp4_quantized_expert_amd import workloads as W
from oracle import mxfp4_moe as O
from tests.helpers import assert_layer_parity

pytestmark = pytest.mark.gpu


def _layer(spec, seed=None):
    return dict(W.make_layer(spec, seed=seed), **W.make_router(spec, seed=seed))


def _logit_bound(L):
    x = np.abs(O.bf16_decode(L["x"]))
    w = np.abs(O.bf16_decode(L["router_w"]))
    return 2e-5 * (x @ w.T) + 1e-6


def _check_router(L, top_k, logits, ids, weights, label):
    """Checks the GPU router outputs; returns the mask of unambiguous tokens."""
    ref = O.router_logits(L["x"], L["router_w"], L["router_b"])
    bound = _logit_bound(L)
    err = np.abs(logits - ref)
    assert np.all(err <= bound), f"{label}: logits off by {err.max():.3e} (bound {bound.min():.3e}..)"
    ref_ids, ref_w = O.route(ref, top_k)
    srt = -np.sort(-ref, axis=1)
    E = ref.shape[1]
    if top_k < E:
        gap = srt[:, top_k - 1] - srt[:, top_k]
        clear = gap > 2 * bound.max(axis=1)
    else:
        clear = np.ones(ref.shape[0], dtype=bool)
    # ties inside the selected set order by value too: require those gaps as well
    for j in range(top_k - 1):
        clear &= (srt[:, j] - srt[:, j + 1]) > 2 * bound.max(axis=1)
    assert np.array_equal(ids[clear], ref_ids[clear]), f"{label}: top-k ids differ on unambiguous tokens"
    np.testing.assert_allclose(weights[clear], ref_w[clear], rtol=1e-4, atol=1e-6)
    # elsewhere: every pick is within the bound of the k-th largest oracle logit
    kth = srt[:, top_k - 1]
    picked = np.take_along_axis(ref, ids.astype(np.int64), axis=1)
    assert np.all(picked >= kth[:, None] - 2 * bound.max(axis=1)[:, None]), f"{label}: an invalid top-k pick"
    for t in range(ids.shape[0]):
        assert len(set(ids[t].tolist())) == top_k, f"{label}: repeated expert in token {t}"
    print(f"[router] {label}: logits max err {err.max():.2e}, unambiguous tokens {clear.sum()}/{clear.size}",
          flush=True)
    return clear


def _bf16_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


@pytest.mark.parametrize("name,T,H,E,k", [("tiny", 16, 64, 4, 2), ("20b", 4, 2880, 32, 4), ("20b", 256, 2880, 32, 4),
                                          ("120b", 4096, 2880, 128, 4), ("ragged", 37, 96, 9, 3),
                                          ("wide", 33, 64, 512, 32), ("one", 1, 32, 1, 1)])
def test_router_against_oracle(gpu, name, T, H, E, k):
    # Token tiles of 16 with a ragged last one, expert blocks of 16 with a
    # ragged last one, the most experts and the largest top_k, one expert.
    base = {"tiny": "tiny", "20b": "20b_prefill", "120b": "120b_prefill"}.get(name, "tiny")
    spec = W.LAYERS[base].with_(T=T, H=H, E=E, top_k=k)
    L = {"x": W.make_routing_inputs(spec)[0], **W.make_router(spec)}
    logits, ids, w = gpu.moe_mxfp4_router(_bf16_dev(L["x"]), _bf16_dev(L["router_w"]), _bf16_dev(L["router_b"]), k)
    torch.cuda.synchronize()
    clear = _check_router(L, k, logits.cpu().numpy().astype(np.float64), ids.cpu().numpy(),
                          w.cpu().numpy().astype(np.float64), f"{name}{(T, H, E, k)}")
    assert clear.any()
    if k <= 4:
        assert clear.mean() > 0.9


@pytest.mark.parametrize("name", ["tiny", "20b_decode", "20b_prefill"])
def test_forward_router_layer(gpu, name):
    spec = W.LAYERS[name]
    L = _layer(spec)
    d = gpu.layer_to_device(L)
    y = gpu.moe_mxfp4_forward_router(d["x"], d["router_w"], d["router_b"], d["w13_blocks"], d["w13_scales"],
                                     d["w13_bias"], d["w2_blocks"], d["w2_scales"], d["w2_bias"], spec.top_k)
    logits, ids, w = gpu.moe_mxfp4_router(d["x"], d["router_w"], d["router_b"], spec.top_k)
    torch.cuda.synchronize()
    clear = _check_router(L, spec.top_k, logits.cpu().numpy().astype(np.float64), ids.cpu().numpy(),
                          w.cpu().numpy().astype(np.float64), name)
    tokens = np.nonzero(clear)[0]
    ref = O.moe_forward_router(L, spec.top_k, tokens=tokens)
    assert_layer_parity(y[torch.from_numpy(tokens).to(y.device)], ref, f"forward_router {name}")


def test_forward_router_120b(gpu):
    # The 120b layer with its Zipf skew carried by the router bias, checked on
    # every token whose top-k is unambiguous (a tie within the fp32 bound has
    # more than one valid answer; those tokens' picks are checked for validity
    # by _check_router).
    spec = W.LAYERS["120b_prefill"]
    L = _layer(spec)
    d = gpu.layer_to_device(L)
    y = gpu.moe_mxfp4_forward_router(d["x"], d["router_w"], d["router_b"], d["w13_blocks"], d["w13_scales"],
                                     d["w13_bias"], d["w2_blocks"], d["w2_scales"], d["w2_bias"], spec.top_k)
    logits, ids, w = gpu.moe_mxfp4_router(d["x"], d["router_w"], d["router_b"], spec.top_k)
    torch.cuda.synchronize()
    clear = _check_router(L, spec.top_k, logits.cpu().numpy().astype(np.float64), ids.cpu().numpy(),
                          w.cpu().numpy().astype(np.float64), "120b")
    tokens = np.nonzero(clear)[0]
    assert tokens.size > 0.9 * spec.T
    ref = O.moe_forward_router(L, spec.top_k, tokens=tokens)
    assert_layer_parity(y[torch.from_numpy(tokens).to(y.device)], ref,
                        f"forward_router 120b ({tokens.size} unambiguous tokens)")


@pytest.mark.parametrize("T", [64, 4, 1])
def test_forward_router_matches_logits_entry(gpu, T):
    # The same layer through moe_mxfp4_forward with the logits the router
    # entry returned gives the same bits (the projection only replaces the
    # logits input; decode batches are routed inside the gate_up launch from
    # the projected logits).
    spec = W.LAYERS["20b_prefill"].with_(T=T)
    L = _layer(spec)
    d = gpu.layer_to_device(L)
    y = gpu.moe_mxfp4_forward_router(d["x"], d["router_w"], d["router_b"], d["w13_blocks"], d["w13_scales"],
                                     d["w13_bias"], d["w2_blocks"], d["w2_scales"], d["w2_bias"], spec.top_k)
    logits, _, _ = gpu.moe_mxfp4_router(d["x"], d["router_w"], d["router_b"], spec.top_k)
    y2 = gpu.moe_mxfp4_forward(d["x"], logits, d["w13_blocks"], d["w13_scales"], d["w13_bias"], d["w2_blocks"],
                               d["w2_scales"], d["w2_bias"], spec.top_k)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
