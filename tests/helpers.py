"""Shared helpers of the GPU parity tests: host <-> device, tolerances, and the
oracle's reference for the 120b long prefill, computed once per session."""

import functools
import time

import numpy as np
import torch

from mxfp4_quantized_expert_amd import workloads as W
from oracle import mxfp4_moe as O

# Acceptance bar for the fused layer (bf16 output, fp32 accumulation):
# normwise relative error and the largest element error relative to max|y_ref|.
REL_TOL = 1e-2
MAX_TOL = 2e-2


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    bits = t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return O.bf16_decode(bits)


def bits_u16(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def assert_layer_parity(y_gpu: torch.Tensor, y_ref: np.ndarray, label: str):
    y = bf16_to_f64(y_gpu)
    bad = np.argwhere(~np.isfinite(y))
    assert bad.size == 0, (f"{label}: {len(bad)} non-finite outputs, first at {bad[:4].tolist()}, "
                           f"rows {np.unique(bad[:, 0])[:8].tolist() if y.ndim == 2 else ''}")
    rel, mx = O.parity_errors(y, y_ref)
    print(f"[parity] {label}: normwise {rel:.3e}, max-element {mx:.3e} over {y.size} elements", flush=True)
    assert rel <= REL_TOL, f"{label}: normwise relative error {rel:.3e} > {REL_TOL}"
    assert mx <= MAX_TOL, f"{label}: max element error {mx:.3e} > {MAX_TOL} * max|y_ref|"
    return rel, mx


def assert_layer_parity_nan(y_gpu: torch.Tensor, y_ref: np.ndarray, label: str):
    """As assert_layer_parity for outputs with NaN elements: the NaNs must sit
    exactly where the oracle's are, and the other elements meet the bar."""
    y = bf16_to_f64(y_gpu)
    nan_ref = np.isnan(y_ref)
    assert nan_ref.any(), f"{label}: the case must produce NaN outputs"
    assert np.array_equal(np.isnan(y), nan_ref), \
        f"{label}: NaN at {np.argwhere(np.isnan(y) != nan_ref)[:5].tolist()} differs from the oracle"
    assert np.all(np.isfinite(y[~nan_ref])), f"{label}: infinite output"
    rel, mx = O.parity_errors(y[~nan_ref], y_ref[~nan_ref])
    print(f"[parity] {label}: {int(nan_ref.sum())} NaN as the oracle; others normwise {rel:.3e}, "
          f"max-element {mx:.3e}", flush=True)
    assert rel <= REL_TOL and mx <= MAX_TOL, f"{label}: normwise {rel:.3e}, max {mx:.3e}"


@functools.lru_cache(maxsize=None)
def long_prefill_120b():
    """The gpt-oss-120b shaped long-prefill layer (T=4096, E=128, top-4, Zipf
    routing) and the oracle's output on every one of its 4096 x 2880 elements."""
    spec = W.LAYERS["120b_prefill"]
    L = W.make_layer(spec)
    t0 = time.perf_counter()
    ref = O.moe_forward(L, spec.top_k)
    print(f"[oracle] 120b long prefill, all {spec.T} tokens: {time.perf_counter() - t0:.1f} s", flush=True)
    return spec, L, ref


@functools.lru_cache(maxsize=None)
def long_prefill_120b_nvfp4():
    """The same long-prefill shapes with NVFP4 experts, and the oracle's output
    on every element."""
    spec = W.LAYERS["120b_prefill"]
    L = W.make_nvfp4_layer(spec)
    t0 = time.perf_counter()
    ref = O.moe_forward_nvfp4(L, spec.top_k)
    print(f"[oracle] NVFP4 120b long prefill, all {spec.T} tokens: {time.perf_counter() - t0:.1f} s", flush=True)
    return spec, L, ref
