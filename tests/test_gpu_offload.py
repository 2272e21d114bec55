"""mxfp4_dequantize_from_host (dequant-on-copy from host memory) on the GPU
against the oracle: bit-exact (uint16 compare)."""

import numpy as np
import pytest
import torch

from mxfp4_quantized_expert_amd import workloads as W
from oracle import mxfp4_moe as O
from tests.helpers import bits_u16

pytestmark = pytest.mark.gpu


def _host(a: np.ndarray, pinned: bool) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    return t.pin_memory() if pinned else t


def test_multi_chunk_bank_pinned(gpu):
    # six 120b-shaped w13 experts: 53 MB of packed rows, several chunks
    # through both staging slots
    bank = W.DEQUANT_BANK_120B[0]
    blocks, scales = W.make_bank(bank)
    blocks, scales = blocks[:6], scales[:6]
    out = gpu.mxfp4_dequantize_from_host(_host(blocks, True), _host(scales, True))
    torch.cuda.synchronize()
    got = bits_u16(out)
    for e in range(blocks.shape[0]):
        assert np.array_equal(got[e], O.mxfp4_dequantize(blocks[e], scales[e])), e


@pytest.mark.parametrize("N,K,pinned", [(1, 32, True), (100, 96, False), (33, 4096, True), (7000, 2880, False)])
def test_shapes_pinned_and_pageable(gpu, N, K, pinned):
    rng = np.random.default_rng(N + K)
    blocks = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    scales = rng.integers(0, 256, size=(N, K // 32), dtype=np.uint8)
    out = gpu.mxfp4_dequantize_from_host(_host(blocks, pinned), _host(scales, pinned))
    torch.cuda.synchronize()
    assert np.array_equal(bits_u16(out), O.mxfp4_dequantize(blocks, scales))


def test_back_to_back_calls_share_staging(gpu):
    rng = np.random.default_rng(5)
    a_b = rng.integers(0, 256, size=(9000, 1440), dtype=np.uint8)
    a_s = rng.integers(118, 133, size=(9000, 90), dtype=np.uint8)
    b_b = rng.integers(0, 256, size=(300, 1440), dtype=np.uint8)
    b_s = rng.integers(118, 133, size=(300, 90), dtype=np.uint8)
    staging = torch.empty((gpu.offload_staging_bytes(9000, 2880),), dtype=torch.uint8, device="cuda")
    out_a = gpu.mxfp4_dequantize_from_host(_host(a_b, True), _host(a_s, True), staging=staging)
    out_b = gpu.mxfp4_dequantize_from_host(_host(b_b, True), _host(b_s, True), staging=staging)
    torch.cuda.synchronize()
    assert np.array_equal(bits_u16(out_a), O.mxfp4_dequantize(a_b, a_s))
    assert np.array_equal(bits_u16(out_b), O.mxfp4_dequantize(b_b, b_s))


def test_empty_is_noop(gpu):
    out = gpu.mxfp4_dequantize_from_host(torch.zeros((0, 16), dtype=torch.uint8),
                                         torch.zeros((0, 1), dtype=torch.uint8))
    assert out.shape == (0, 32)
