"""moe_mxfp4_route on the GPU against the oracle: ids, offsets and the
expert-ordered pair list bit-exact, weights within 1e-6."""

import numpy as np
import pytest
import torch

from mxfp4_quantized_expert_amd import workloads as W
from oracle import mxfp4_moe as O

pytestmark = pytest.mark.gpu


def _check(gpu, logits: np.ndarray, k: int):
    T, E = logits.shape
    ids, w, offsets, pairs = gpu.moe_mxfp4_route(torch.from_numpy(logits).cuda(), k)
    torch.cuda.synchronize()
    rids, rw = O.route(logits, k)
    counts, roff, rperm = O.group_by_expert(rids, E)
    assert np.array_equal(ids.cpu().numpy(), rids)
    assert np.max(np.abs(w.cpu().numpy() - rw), initial=0.0) <= 1e-6
    assert np.array_equal(offsets.cpu().numpy(), roff)
    assert np.array_equal(pairs.cpu().numpy(), rperm)


@pytest.mark.parametrize("name", ["tiny", "20b_decode", "20b_prefill", "120b_prefill"])
def test_route_layers(gpu, name):
    spec = W.LAYERS[name]
    _, logits = W.make_routing_inputs(spec)
    _check(gpu, logits, spec.top_k)


@pytest.mark.parametrize("T,E,k", [(1, 1, 1), (3, 7, 7), (77, 512, 32), (5000, 64, 1), (2048, 128, 8),
                                   (1, 65, 4), (40, 64, 4), (300, 129, 4), (100, 200, 2), (64, 256, 8),
                                   (33, 257, 16)])
def test_route_shapes(gpu, T, E, k):
    # every keys-per-lane form of the top-k (E up to 64, 128, 256, 512) and its edges
    rng = np.random.default_rng(T + E + k)
    _check(gpu, rng.standard_normal((T, E)).astype(np.float32), k)


def test_route_ties_go_to_lower_index(gpu):
    rng = np.random.default_rng(1)
    logits = np.round(rng.standard_normal((300, 40)) * 2).astype(np.float32)  # many equal logits
    _check(gpu, logits, 6)


def test_route_empty(gpu):
    logits = torch.zeros((0, 8), dtype=torch.float32, device="cuda")
    ids, w, offsets, pairs = gpu.moe_mxfp4_route(logits, 2)
    torch.cuda.synchronize()
    assert np.array_equal(offsets.cpu().numpy(), np.zeros(9, np.int32))


@pytest.mark.parametrize("P", [1023, 1024, 1025, 2047, 2048, 2049, 3072])
@pytest.mark.parametrize("skew", ["uniform", "one_expert", "two_alternating"])
def test_group_chunk_boundaries(gpu, P, skew):
    # The grouping splits the pairs into chunks of 1024, one block each; every
    # block counts the pairs before its chunk itself.  Pair counts on and
    # around chunk edges, with the pairs spread evenly, all on one expert
    # (its run crosses every chunk edge) or alternating between two experts.
    E, k = 24, 1
    rng = np.random.default_rng(P)
    logits = rng.standard_normal((P, E)).astype(np.float32)
    if skew == "one_expert":
        logits[:, 17] += 50.0
    elif skew == "two_alternating":
        logits[0::2, 3] += 50.0
        logits[1::2, 20] += 50.0
    _check(gpu, logits, k)


def test_group_chunk_boundaries_top_k(gpu):
    # pairs of one token straddle a chunk edge (P = 3 * 683 = 2049)
    rng = np.random.default_rng(7)
    _check(gpu, rng.standard_normal((683, 96)).astype(np.float32), 3)


def test_route_signed_zero_ties(gpu):
    # -0 and +0 compare equal: the lower expert index wins either way round
    logits = np.full((4, 8), -1.0, dtype=np.float32)
    logits[0, 2], logits[0, 5] = 0.0, -0.0
    logits[1, 2], logits[1, 5] = -0.0, 0.0
    logits[2, 0], logits[2, 7] = -0.0, -0.0
    logits[3, :] = -0.0
    _check(gpu, logits, 2)
