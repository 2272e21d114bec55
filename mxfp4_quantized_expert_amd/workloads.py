"""Seeded synthetic MXFP4 mixture-of-experts layers.

This module only draws random inputs.  It holds none of the arithmetic of the
method (no decoding, routing, GEMM or activation), so both the CPU oracle and
the HIP path can consume the same inputs without sharing any computation.

Shapes and value ranges follow the gpt-oss expert layers discussed in
"feat(gpt-oss): expert offloading Phase 3" (MoE-Infinity PR #153, description:
six packed components per layer) and "feat(gguf): serve gpt-oss gguf
checkpoints" (FreeToken PR #838, "What it does": gate_up_bias[E, 2I] and
down_bias[E, H] in bf16).  Packed blocks are [E, N, K/2] uint8 (two E2M1
nibbles per byte) and scales are [E, N, K/32] uint8 E8M0 bytes ("Add native
GPT-OSS MXFP4 QMoE export", mobius PR #719, Summary: blocks [E, N, K/32, 16]).

Draw order is fixed for every layer: x, logits, the Zipf expert-rank
permutation (skewed layers only), w13_blocks, w13_scales, w13_bias,
w2_blocks, w2_scales, w2_bias.  Routing therefore depends only on the first
draws, and ``make_routing_inputs`` replays them without drawing the weights.
bf16 tensors are drawn in float32 and rounded to nearest-even by torch's float32 -> bfloat16 conversion; they are returned as
uint16 bit patterns.
"""

from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Dict, Optional

import numpy as np

__all__ = [
    "LayerSpec",
    "LAYERS",
    "DequantBankSpec",
    "DEQUANT_BANK_120B",
    "make_layer",
    "make_nvfp4_layer",
    "make_routing_inputs",
    "make_router",
    "make_bank",
    "to_bf16_bits",
]


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 array -> bf16 bit patterns (uint16), round-to-nearest-even by torch."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


@dataclass(frozen=True)
class LayerSpec:
    """One synthetic MoE expert layer.

    T tokens, hidden H, intermediate I, E experts, top_k experts per token.
    w13 is [E, 2I, H] (gate and up rows interleaved), w2 is [E, H, I].
    """

    name: str
    T: int
    H: int
    I: int
    E: int
    top_k: int
    x_std: float = 1.0
    logit_std: float = 1.0
    zipf_s: Optional[float] = None  # per-expert logit offset -s*ln(rank)
    scale_lo: int = 118
    scale_hi: int = 132
    bias_std: float = 0.02
    seed: int = 0

    @property
    def pairs(self) -> int:
        return self.T * self.top_k

    def with_(self, **kw) -> "LayerSpec":
        return replace(self, **kw)


LAYERS: Dict[str, LayerSpec] = {
    # Tiny layer: T=16, H=I=64, E=4, top-2; scales in [123,129]; biases N(0,0.1).
    "tiny": LayerSpec("tiny", T=16, H=64, I=64, E=4, top_k=2, logit_std=1.0,
                      scale_lo=123, scale_hi=129, bias_std=0.1),
    # gpt-oss-20b shaped decode: T=4, H=I=2880, E=32, top-4, logits N(0,2).
    "20b_decode": LayerSpec("20b_decode", T=4, H=2880, I=2880, E=32, top_k=4,
                            logit_std=2.0),
    # gpt-oss-20b shaped prefill: T=256, same distributions, non-zero biases.
    "20b_prefill": LayerSpec("20b_prefill", T=256, H=2880, I=2880, E=32, top_k=4,
                             logit_std=2.0),
    # gpt-oss-120b shaped long prefill: T=4096, E=128, top-4, Zipf(1.1) skew.
    "120b_prefill": LayerSpec("120b_prefill", T=4096, H=2880, I=2880, E=128, top_k=4,
                              logit_std=1.0, zipf_s=1.1),
    # Live-region case: the decode shapes with small scales so the clamped
    # SwiGLU is not saturated and the biases move the output measurably.
    "20b_live": LayerSpec("20b_live", T=4, H=2880, I=2880, E=32, top_k=4,
                          logit_std=2.0, scale_lo=112, scale_hi=120, bias_std=0.02),
}


def _uniform_bytes(rng: np.random.Generator, shape) -> np.ndarray:
    n = int(np.prod(shape))
    return np.frombuffer(rng.bytes(n), dtype=np.uint8).reshape(shape).copy()


def _scale_bytes(rng: np.random.Generator, shape, lo: int, hi: int) -> np.ndarray:
    return rng.integers(lo, hi + 1, size=shape, dtype=np.uint8)


def _draw_x_logits(rng: np.random.Generator, spec: LayerSpec):
    x = to_bf16_bits(rng.standard_normal((spec.T, spec.H), dtype=np.float32) * np.float32(spec.x_std))
    logits = rng.standard_normal((spec.T, spec.E), dtype=np.float32) * np.float32(spec.logit_std)
    if spec.zipf_s is not None:
        # Zipf(s) expert popularity expressed as a log-offset on the logits:
        # the expert of popularity rank r gets -s*ln(r); ranks are a seeded permutation.
        rank = rng.permutation(spec.E).astype(np.float64) + 1.0
        offset = (-spec.zipf_s * np.log(rank)).astype(np.float32)
        logits = logits + offset[None, :]
    return x, np.ascontiguousarray(logits, dtype=np.float32)


def make_routing_inputs(spec: LayerSpec, seed: Optional[int] = None):
    """(x, router_logits) exactly as ``make_layer`` draws them, without the weights."""
    rng = np.random.default_rng(spec.seed if seed is None else seed)
    return _draw_x_logits(rng, spec)


def make_layer(spec: LayerSpec, seed: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Draw one layer.  Returns host numpy arrays keyed by the boundary's names.

    x [T,H] uint16 (bf16 bits), router_logits [T,E] float32,
    w13_blocks [E,2I,H/2] uint8, w13_scales [E,2I,H/32] uint8, w13_bias [E,2I] uint16,
    w2_blocks [E,H,I/2] uint8, w2_scales [E,H,I/32] uint8, w2_bias [E,H] uint16.
    """
    rng = np.random.default_rng(spec.seed if seed is None else seed)
    H, I, E = spec.H, spec.I, spec.E
    if H % 32 or I % 32:
        raise ValueError("H and I must be multiples of 32")
    out: Dict[str, np.ndarray] = {}
    out["x"], out["router_logits"] = _draw_x_logits(rng, spec)
    out["w13_blocks"] = _uniform_bytes(rng, (E, 2 * I, H // 2))
    out["w13_scales"] = _scale_bytes(rng, (E, 2 * I, H // 32), spec.scale_lo, spec.scale_hi)
    out["w13_bias"] = to_bf16_bits(rng.standard_normal((E, 2 * I), dtype=np.float32) * np.float32(spec.bias_std))
    out["w2_blocks"] = _uniform_bytes(rng, (E, H, I // 2))
    out["w2_scales"] = _scale_bytes(rng, (E, H, I // 32), spec.scale_lo, spec.scale_hi)
    out["w2_bias"] = to_bf16_bits(rng.standard_normal((E, H), dtype=np.float32) * np.float32(spec.bias_std))
    return out


def make_router(spec: LayerSpec, seed: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Router weights for the layer of ``spec``: router_w [E, H] and router_b [E]
    as bf16 bits, from a stream of their own (seed sequence [seed, 1]), so that
    adding a router leaves every other tensor of the layer unchanged.

    W_r is N(0, logit_std^2 / H), which gives logits of about logit_std on
    x ~ N(0, x_std^2) rows of std 1; the bias is the Zipf(s) log-offset
    -s*ln(rank) over a seeded rank permutation for skewed layers, else
    N(0, (logit_std / 4)^2)."""
    rng = np.random.default_rng([spec.seed if seed is None else seed, 1])
    w = rng.standard_normal((spec.E, spec.H), dtype=np.float32) * np.float32(spec.logit_std / np.sqrt(spec.H))
    if spec.zipf_s is not None:
        rank = rng.permutation(spec.E).astype(np.float64) + 1.0
        b = (-spec.zipf_s * np.log(rank)).astype(np.float32)
    else:
        b = rng.standard_normal(spec.E, dtype=np.float32) * np.float32(spec.logit_std / 4)
    return {"router_w": to_bf16_bits(w), "router_b": to_bf16_bits(b)}


def make_nvfp4_layer(spec: LayerSpec, seed: Optional[int] = None, scale_lo: int = 0x30,
                     scale_hi: int = 0x48) -> Dict[str, np.ndarray]:
    """An NVFP4 expert layer of the same shapes: blocks [E,N,K/2] uint8, E4M3
    block scales [E,N,K/16] uint8 drawn uniform in [scale_lo, scale_hi] (positive
    values 0.5 .. 4 by default), second-level scales w13_scale2 / w2_scale2 [E]
    float32 drawn uniform in [1/16, 1/4], biases bf16 N(0, bias_std).  Draw
    order: x, logits, (Zipf permutation), w13 blocks, w13 scales, w13 scale2,
    w13 bias, w2 blocks, w2 scales, w2 scale2, w2 bias."""
    rng = np.random.default_rng(spec.seed if seed is None else seed)
    H, I, E = spec.H, spec.I, spec.E
    if H % 32 or I % 32:
        raise ValueError("H and I must be multiples of 32")
    out: Dict[str, np.ndarray] = {}
    out["x"], out["router_logits"] = _draw_x_logits(rng, spec)
    out["w13_blocks"] = _uniform_bytes(rng, (E, 2 * I, H // 2))
    out["w13_scales"] = _scale_bytes(rng, (E, 2 * I, H // 16), scale_lo, scale_hi)
    out["w13_scale2"] = rng.uniform(1 / 16, 1 / 4, size=E).astype(np.float32)
    out["w13_bias"] = to_bf16_bits(rng.standard_normal((E, 2 * I), dtype=np.float32) * np.float32(spec.bias_std))
    out["w2_blocks"] = _uniform_bytes(rng, (E, H, I // 2))
    out["w2_scales"] = _scale_bytes(rng, (E, H, I // 16), scale_lo, scale_hi)
    out["w2_scale2"] = rng.uniform(1 / 16, 1 / 4, size=E).astype(np.float32)
    out["w2_bias"] = to_bf16_bits(rng.standard_normal((E, H), dtype=np.float32) * np.float32(spec.bias_std))
    return out


@dataclass(frozen=True)
class DequantBankSpec:
    """A full expert bank for the standalone dequant: [E, N, K/2] blocks, [E, N, K/32] scales."""

    name: str
    E: int
    N: int
    K: int
    scale_lo: int = 118
    scale_hi: int = 132
    seed: int = 0


# gpt-oss-120b shaped banks: w13 [128, 5760, 2880] and w2 [128, 2880, 2880].
DEQUANT_BANK_120B = (
    DequantBankSpec("w13_120b", E=128, N=5760, K=2880, seed=0),
    DequantBankSpec("w2_120b", E=128, N=2880, K=2880, seed=1),
)


def make_bank(spec: DequantBankSpec, seed: Optional[int] = None, experts: Optional[int] = None):
    """Draw (blocks [E,N,K/2] uint8, scales [E,N,K/32] uint8). ``experts`` truncates E."""
    s = spec.seed if seed is None else seed
    rng = np.random.default_rng(s)
    E = spec.E if experts is None else experts
    blocks = _uniform_bytes(rng, (E, spec.N, spec.K // 2))
    scales = _scale_bytes(rng, (E, spec.N, spec.K // 32), spec.scale_lo, spec.scale_hi)
    return blocks, scales
