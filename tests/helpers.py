"""Shared helpers of the GPU parity tests: host <-> device, tolerances."""

import numpy as np
import torch

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
    assert np.all(np.isfinite(y)), f"{label}: non-finite output"
    rel, mx = O.parity_errors(y, y_ref)
    print(f"[parity] {label}: normwise {rel:.3e}, max-element {mx:.3e}", flush=True)
    assert rel <= REL_TOL, f"{label}: normwise relative error {rel:.3e} > {REL_TOL}"
    assert mx <= MAX_TOL, f"{label}: max element error {mx:.3e} > {MAX_TOL} * max|y_ref|"
    return rel, mx
