"""CPU oracle for the MXFP4 mixture-of-experts expert FFN and the MXFP4 dequant.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or links
this module; only the tests, the smoke check and the benchmark's CPU baseline
do.  It shares no code with the HIP kernels.

Plain, slow, obviously correct numpy in float64.  Every function follows a
passage of the pages it cites (page title, then section):

* "feat(gpt-oss): expert offloading Phase 2 — MXFP4 dequant-on-copy execution"
  (MoE-Infinity PR #152): Changes (packed experts dequantized to bf16,
  golden test at relative error 0.0) and the numerical review (scales, bias,
  the [N, K//2] layout, gate/up split, clamped SwiGLU, fp32 accumulation).
* "feat(gguf): serve gpt-oss gguf checkpoints on gpt_oss" (FreeToken PR #838):
  "What it does" (alpha 1.702 / limit 7 family constants; interleaved gate/up;
  gate/up bias added before the gated activation, down bias before the routing
  weight; the second-level scale multiplies before the bias) and review items
  3 and 4 (sum_k w*(s*y + b), never sum_k w*s*(y + b); router weight on the
  output, never on the input, when biases exist).
* "Restore GPT-OSS's router-masked expert-parallel plan" (transformers PR
  #49431), description: MXFP4 experts consume routing data (top-k ids and
  weights) and group their tokens themselves.
* FreeToken PR #838, review item 3, for the NVFP4 variant: the second-level
  weight_scale_2 multiplies the expert output before its bias.
* FreeToken PR #838, the cleanups (the router is mlp.router) and "What it
  does" (the router bias is loaded, the router input's bias is required), for
  the router projection: logits = x W_r^T + b_r ahead of the top-k.
* "Add native GPT-OSS MXFP4 QMoE export" (mobius PR #719): Summary (blocks
  [E, N, K/32, 16], one E8M0 scale byte per 16-byte block) and Validation
  (scale bytes 0x00..0xfe are valid, 0xff is not).

The element encodings come from the OCP Microscaling Formats (MX) v1.0
specification: E2M1 (1 sign, 2 exponent bits with bias 1, 1 mantissa bit) and
E8M0 (an unsigned power-of-two exponent with bias 127, 0xFF = NaN).

Readings where the pages are silent (each is listed in the design notes):
nibble order (low nibble = even k), gate = even rows of w13 and up = odd rows,
the gate clamp is one-sided (min(gate, 7)) and the up clamp two-sided,
top-k ties go to the lower expert index, and the softmax runs over the k
selected logits.
"""

from __future__ import annotations

from typing import Dict, Optional, Sequence, Tuple

import numpy as np

SWIGLU_ALPHA = 1.702
SWIGLU_LIMIT = 7.0
GROUP = 32  # elements per E8M0 scale (one 16-byte block of nibbles)


# --------------------------------------------------------------------------
# Element encodings (OCP MX v1.0)
# --------------------------------------------------------------------------

def _e2m1_from_fields(code: int) -> float:
    """E2M1: bit 3 sign, bits 2..1 exponent (bias 1), bit 0 mantissa.

    Exponent field 0 is subnormal: value = mantissa * 2^(1-1) * 0.5.
    """
    sign = -1.0 if (code >> 3) & 1 else 1.0
    exp_field = (code >> 1) & 0x3
    man = code & 0x1
    if exp_field == 0:
        mag = man * 0.5
    else:
        mag = (1.0 + man * 0.5) * 2.0 ** (exp_field - 1)
    return sign * mag


# Value of each of the 16 codes (code 0x8 is -0.0).
E2M1_VALUES = np.array([_e2m1_from_fields(c) for c in range(16)], dtype=np.float64)


def e8m0_value(s) -> np.ndarray:
    """E8M0 scale byte -> 2^(s-127); byte 0xFF is NaN."""
    s = np.asarray(s, dtype=np.int64)
    v = np.ldexp(np.ones(s.shape, dtype=np.float64), s - 127)
    return np.where(s == 255, np.nan, v)


# --------------------------------------------------------------------------
# bf16 (1 sign, 8 exponent bits with bias 127, 7 mantissa bits)
# --------------------------------------------------------------------------

def bf16_decode(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64 (exact: bf16 is the top half of a float32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def bf16_encode_rne(v: np.ndarray) -> np.ndarray:
    """float64 -> bf16 bits, round to nearest, ties to even, from the format itself.

    Finite magnitudes are rounded to a multiple of the quantum
    q = 2^(max(floor(log2|v|), -126) - 7); results reaching 2^128 overflow to
    infinity; NaN becomes the quiet NaN 0x7FC0.
    """
    v = np.asarray(v, dtype=np.float64)
    flat = v.ravel()
    out = np.zeros(flat.shape, dtype=np.uint32)
    sign = np.signbit(flat).astype(np.uint32) << np.uint32(15)
    a = np.abs(flat)
    nan = np.isnan(flat)
    inf = np.isinf(a)
    fin = ~(nan | inf) & (a > 0)
    af = a[fin]
    _, e = np.frexp(af)  # af = m * 2^e with m in [0.5, 1): floor(log2 af) = e - 1
    ee = np.maximum(e - 1, -126)
    q = np.ldexp(1.0, ee - 7)
    r = np.rint(af / q)  # af / q is exact (power-of-two divide); rint ties to even
    val = r * q
    bits = np.zeros(af.shape, dtype=np.uint32)
    over = val >= 2.0 ** 128
    sub = val < 2.0 ** -126
    nrm = ~over & ~sub
    bits[over] = 0x7F80
    bits[sub] = (val[sub] / 2.0 ** -133).astype(np.uint32)
    m2, e2 = np.frexp(val[nrm])
    bexp = (e2 - 1 + 127).astype(np.uint32)
    man = ((m2 * 2.0 - 1.0) * 128.0).astype(np.uint32)
    bits[nrm] = (bexp << np.uint32(7)) | man
    out[fin] = bits
    out[inf] = 0x7F80
    out = out | sign
    out[nan] = 0x7FC0
    return out.astype(np.uint16).reshape(v.shape)


# --------------------------------------------------------------------------
# MXFP4 dequant ("dequant-on-copy"), MoE-Infinity PR #152, Changes
# --------------------------------------------------------------------------

def unpack_codes(blocks: np.ndarray) -> np.ndarray:
    """[..., K/2] bytes -> [..., K] 4-bit codes; element 2i is the low nibble of byte i."""
    b = np.asarray(blocks, dtype=np.uint8)
    codes = np.empty(b.shape[:-1] + (b.shape[-1] * 2,), dtype=np.uint8)
    codes[..., 0::2] = b & 0x0F
    codes[..., 1::2] = b >> 4
    return codes


def dequantize_f64(blocks: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Exact real value of every element: E2M1(code) * 2^(scale-127).

    blocks [..., N, K/2] uint8, scales [..., N, K/32] uint8 -> [..., N, K] float64.
    Element k of a row uses the scale byte of its 32-element group, k // 32.
    """
    codes = unpack_codes(blocks)
    K = codes.shape[-1]
    if scales.shape[-1] * GROUP != K:
        raise ValueError("scales must have K/32 entries per row")
    s = np.repeat(e8m0_value(scales), GROUP, axis=-1)
    return E2M1_VALUES[codes] * s


def _dequant_table() -> np.ndarray:
    """bf16 bits of every (scale byte, code) pair: [256, 16].

    The dequantized element depends only on its code and its group's scale, so
    evaluating the definition once per pair gives every element's output.
    """
    s = np.arange(256)[:, None]
    c = np.arange(16)[None, :]
    return bf16_encode_rne(E2M1_VALUES[c] * e8m0_value(s))


_DQ_TABLE: Optional[np.ndarray] = None


def mxfp4_dequantize(blocks: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """MXFP4 -> bf16 bits, [..., N, K/2] + [..., N, K/32] -> [..., N, K] uint16.

    Each output is the bf16 round-to-nearest-even of E2M1(code) * 2^(s-127);
    for scale bytes up to 252 this is exact.  Scale byte 0xFF gives NaN (0x7FC0)
    for all 32 elements of its group.
    """
    global _DQ_TABLE
    if _DQ_TABLE is None:
        _DQ_TABLE = _dequant_table()
    codes = unpack_codes(blocks)
    s = np.repeat(np.asarray(scales, dtype=np.uint8), GROUP, axis=-1)
    return _DQ_TABLE[s, codes]


# --------------------------------------------------------------------------
# NVFP4 experts ("feat(gguf): serve gpt-oss gguf checkpoints on gpt_oss",
# FreeToken PR #838, review item 3: NVFP4 experts carry a second-level
# weight_scale_2 that multiplies the expert output before the bias,
# sum_k w*(s*y + b)).  Element format, as publicly described for NVFP4: E2M1
# codes in blocks of 16 with one FP8 E4M3 scale byte each, times one float32
# second-level scale per expert and projection.
# --------------------------------------------------------------------------

NV_GROUP = 16


def e4m3_value(b) -> np.ndarray:
    """FP8 E4M3 (OCP, no infinities): 1 sign, 4 exponent bits (bias 7), 3
    mantissa bits; exponent field 0 is subnormal (m * 2^-9); S.1111.111 is NaN."""
    b = np.asarray(b, dtype=np.int64)
    sign = np.where((b >> 7) & 1, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = b & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.ldexp(1.0, e - 7))
    return np.where((b & 0x7F) == 0x7F, np.nan, sign * mag)


def nvfp4_dequantize_f64(blocks: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Exact value of every element before the second-level scale:
    E2M1(code) * E4M3(scale of its 16-element block).

    blocks [..., N, K/2] uint8, scales [..., N, K/16] uint8 -> [..., N, K] float64.
    """
    codes = unpack_codes(blocks)
    K = codes.shape[-1]
    if scales.shape[-1] * NV_GROUP != K:
        raise ValueError("scales must have K/16 entries per row")
    return E2M1_VALUES[codes] * np.repeat(e4m3_value(scales), NV_GROUP, axis=-1)


def expert_ffn_nvfp4(xrows: np.ndarray, w13_blocks, w13_scales, w13_scale2, w13_bias_bits,
                     w2_blocks, w2_scales, w2_scale2, w2_bias_bits) -> np.ndarray:
    """One NVFP4 expert: h = s2_13 * (x W13^T) + b13, a = clamped SwiGLU,
    z = s2_2 * (a W2^T) + b2.  Each second-level scale multiplies its GEMM
    result before that GEMM's bias is added."""
    W13 = nvfp4_dequantize_f64(w13_blocks, w13_scales)
    h = float(w13_scale2) * (xrows @ W13.T) + bf16_decode(w13_bias_bits)[None, :]
    a = swiglu_clamped(h[:, 0::2], h[:, 1::2])
    W2 = nvfp4_dequantize_f64(w2_blocks, w2_scales)
    return float(w2_scale2) * (a @ W2.T) + bf16_decode(w2_bias_bits)[None, :]


def moe_forward_nvfp4(layer: Dict[str, np.ndarray], top_k: int,
                      tokens: Optional[Sequence[int]] = None) -> np.ndarray:
    """Routed NVFP4 layer: y_t = sum_j w_tj * z_{e_tj}(x_t) with z as in
    expert_ffn_nvfp4 (the routing weight multiplies s*y + b)."""
    x = bf16_decode(layer["x"])
    logits = np.asarray(layer["router_logits"])
    if tokens is not None:
        tokens = np.asarray(tokens, dtype=np.int64)
        x = x[tokens]
        logits = logits[tokens]
    T, H = x.shape
    E = logits.shape[1]
    ids, w = route(logits, top_k)
    counts, offsets, perm = group_by_expert(ids, E)
    z = np.zeros((T * top_k, H), dtype=np.float64)
    for e in range(E):
        if counts[e] == 0:
            continue
        pairs = perm[offsets[e]:offsets[e + 1]]
        z[pairs] = expert_ffn_nvfp4(
            x[pairs // top_k],
            layer["w13_blocks"][e], layer["w13_scales"][e], layer["w13_scale2"][e], layer["w13_bias"][e],
            layer["w2_blocks"][e], layer["w2_scales"][e], layer["w2_scale2"][e], layer["w2_bias"][e])
    z = z.reshape(T, top_k, H)
    y = np.zeros((T, H), dtype=np.float64)
    for j in range(top_k):
        y += w[:, j:j + 1] * z[:, j, :]
    return y


# --------------------------------------------------------------------------
# Routing (top-k, softmax over the selected logits) and grouping by expert
# --------------------------------------------------------------------------

def route(logits: np.ndarray, top_k: int) -> Tuple[np.ndarray, np.ndarray]:
    """Top-k experts per token, then softmax over the k selected logits.

    Order within a token: descending logit, equal logits by lower expert index.
    Returns ids [T, k] int32 and weights [T, k] float64.
    """
    lg = np.asarray(logits, dtype=np.float64)
    order = np.argsort(-lg, axis=1, kind="stable")
    ids = order[:, :top_k]
    sel = np.take_along_axis(lg, ids, axis=1)
    ex = np.exp(sel - sel[:, :1])
    w = ex / ex.sum(axis=1, keepdims=True)
    return ids.astype(np.int32), w


def group_by_expert(ids: np.ndarray, E: int):
    """Counting sort of pairs p = t*k + j by expert (stable in p).

    Returns counts [E], offsets [E+1] and perm [T*k] (pair ids in expert order).
    """
    flat = np.asarray(ids).ravel()
    counts = np.bincount(flat, minlength=E).astype(np.int64)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    perm = np.argsort(flat, kind="stable").astype(np.int64)
    return counts, offsets, perm


# --------------------------------------------------------------------------
# Router projection ("feat(gguf): serve gpt-oss gguf checkpoints on gpt_oss",
# FreeToken PR #838: the cleanups name the router mlp.router, and "What it
# does" loads the router bias with the dense weights and lists the router
# input's bias among the tensors a file must carry).  The router is a linear
# layer with a bias over the hidden state; its output is the logits that
# route() consumes.
# --------------------------------------------------------------------------

def router_logits(x_bits: np.ndarray, w_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    """logits[t, e] = sum_h x[t, h] * W_r[e, h] + b_r[e], in float64.

    x [T, H], W_r [E, H] and b_r [E] are bf16 bit patterns.
    """
    x = bf16_decode(x_bits)
    w = bf16_decode(w_bits)
    b = bf16_decode(b_bits)
    return x @ w.T + b[None, :]


def moe_forward_router(layer: Dict[str, np.ndarray], top_k: int,
                       tokens: Optional[Sequence[int]] = None) -> np.ndarray:
    """moe_forward with the logits produced by the router projection of the
    layer's own x (layer["router_w"], layer["router_b"])."""
    logits = router_logits(layer["x"], layer["router_w"], layer["router_b"])
    return moe_forward(dict(layer, router_logits=logits), top_k, tokens=tokens)


# --------------------------------------------------------------------------
# Clamped SwiGLU (gpt-oss), FreeToken PR #838 "What it does"
# --------------------------------------------------------------------------

def swiglu_clamped(gate: np.ndarray, up: np.ndarray,
                   alpha: float = SWIGLU_ALPHA, limit: float = SWIGLU_LIMIT) -> np.ndarray:
    """a = g * sigmoid(alpha * g) * (u + 1) with g = min(gate, limit), u = clip(up, -limit, limit)."""
    g = np.minimum(np.asarray(gate, dtype=np.float64), limit)
    u = np.clip(np.asarray(up, dtype=np.float64), -limit, limit)
    with np.errstate(over="ignore"):
        sig = 1.0 / (1.0 + np.exp(-alpha * g))
    return g * sig * (u + 1.0)


# --------------------------------------------------------------------------
# Expert FFN and the routed layer
# --------------------------------------------------------------------------

def expert_ffn(xrows: np.ndarray, w13_blocks, w13_scales, w13_bias_bits,
               w2_blocks, w2_scales, w2_bias_bits) -> np.ndarray:
    """One expert on a set of token rows (float64 [n, H]) -> z [n, H].

    h = x W13^T + b13 (bias before the activation); gate = h[:, 0::2],
    up = h[:, 1::2]; a = clamped SwiGLU; z = a W2^T + b2 (bias before the
    routing weight).
    """
    W13 = dequantize_f64(w13_blocks, w13_scales)  # [2I, H]
    h = xrows @ W13.T + bf16_decode(w13_bias_bits)[None, :]
    a = swiglu_clamped(h[:, 0::2], h[:, 1::2])
    W2 = dequantize_f64(w2_blocks, w2_scales)  # [H, I]
    return a @ W2.T + bf16_decode(w2_bias_bits)[None, :]


def moe_forward(layer: Dict[str, np.ndarray], top_k: int,
                tokens: Optional[Sequence[int]] = None) -> np.ndarray:
    """Routed MoE layer output y [T, H] float64 (or only the rows ``tokens``).

    y_t = sum_j w_tj * z_{e_tj}(x_t), where z_e = W2_e a + b2_e: the routing
    weight multiplies the biased expert output (sum_k w*(s*y + b)).
    Pairs are processed grouped by expert, each expert's weights dequantized
    once; the k terms of a token are summed in j order.
    """
    x = bf16_decode(layer["x"])
    logits = np.asarray(layer["router_logits"])
    if tokens is not None:
        tokens = np.asarray(tokens, dtype=np.int64)
        x = x[tokens]
        logits = logits[tokens]
    T = x.shape[0]
    H = x.shape[1]
    E = logits.shape[1]
    ids, w = route(logits, top_k)
    counts, offsets, perm = group_by_expert(ids, E)
    z = np.zeros((T * top_k, H), dtype=np.float64)
    for e in range(E):
        if counts[e] == 0:
            continue
        pairs = perm[offsets[e]:offsets[e + 1]]
        z[pairs] = expert_ffn(
            x[pairs // top_k],
            layer["w13_blocks"][e], layer["w13_scales"][e], layer["w13_bias"][e],
            layer["w2_blocks"][e], layer["w2_scales"][e], layer["w2_bias"][e])
    z = z.reshape(T, top_k, H)
    y = np.zeros((T, H), dtype=np.float64)
    for j in range(top_k):
        y += w[:, j:j + 1] * z[:, j, :]
    return y


# --------------------------------------------------------------------------
# Block-scaled FP8 activations for the opt-in FP4 scaled-MFMA path.  This is
# an approximation of this implementation's own (the pages fix fp32
# accumulation of exact bf16 products only); it is defined here so that the
# GPU's quantized codes can be checked exactly.  Encodings from the OCP
# Microscaling Formats v1.0 specification: MXFP8 E4M3 elements in blocks of
# 32 along K sharing one E8M0 scale.  The shared exponent is this
# implementation's own choice, floor(log2(max|v|)) - 7: the specification
# subtracts the element format's emax (8 for E4M3), which puts the scaled
# block maximum in [256, 512) and clamps what exceeds 448; subtracting 7 keeps every
# scaled magnitude below 256, so no element is clamped.  An all-zero block
# takes scale byte 127.  "split" activations add a second MXFP8 tensor that
# quantizes the residual v - hi the same way.
# --------------------------------------------------------------------------

def e4m3_encode_rne(v) -> np.ndarray:
    """float64 -> FP8 E4M3 code, round to nearest, ties to even.  |v| <= 448."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    if np.any(a > 448.0):
        raise ValueError("E4M3 magnitude above 448")
    _, ex = np.frexp(np.where(a > 0, a, 1.0))   # a = m * 2^ex, m in [0.5, 1)
    e = np.maximum(ex - 1, -6)                   # binade; below 2^-6 the subnormal quantum 2^-9
    q = np.ldexp(1.0, e - 3)                     # three mantissa bits
    r = np.round(a / q) * q                      # numpy rounds halves to even
    _, ex2 = np.frexp(np.where(r > 0, r, 1.0))
    e2 = ex2 - 1
    normal = r >= 2.0 ** -6
    expf = np.where(normal, e2 + 7, 0)
    mant = np.where(normal, np.round(r / np.ldexp(1.0, e2) * 8 - 8), np.round(r / 2.0 ** -9))
    code = (np.signbit(v).astype(np.int64) << 7) | (expf.astype(np.int64) << 3) | mant.astype(np.int64)
    return code.astype(np.uint8)


def mxfp8_quantize(v: np.ndarray):
    """[..., K] float64 -> (E4M3 codes [..., K] uint8, E8M0 scale bytes [..., K/32] uint8)."""
    v = np.asarray(v, dtype=np.float64)
    K = v.shape[-1]
    if K % GROUP:
        raise ValueError("K must be a multiple of 32")
    blk = v.reshape(v.shape[:-1] + (K // GROUP, GROUP))
    amax = np.abs(blk).max(axis=-1)
    _, ex = np.frexp(np.where(amax > 0, amax, 1.0))
    X = np.where(amax > 0, ex - 1 - 7, 0)
    sbyte = np.clip(X + 127, 0, 254)
    scaled = blk / np.ldexp(1.0, (sbyte - 127).astype(np.int64))[..., None]
    codes = e4m3_encode_rne(scaled).reshape(v.shape)
    return codes, sbyte.astype(np.uint8)


def mxfp8_dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    vals = e4m3_value(codes)
    return vals * np.repeat(np.ldexp(1.0, scales.astype(np.int64) - 127), GROUP, axis=-1)


def mxfp8_activations(v: np.ndarray, mode: str) -> np.ndarray:
    """The value the FP4 scaled-MFMA path multiplies in place of v: one MXFP8
    tensor ("single") or an MXFP8 tensor plus the MXFP8 tensor of its
    residual ("split")."""
    hi_c, hi_s = mxfp8_quantize(v)
    hi = mxfp8_dequantize(hi_c, hi_s)
    if mode == "single":
        return hi
    if mode != "split":
        raise ValueError(mode)
    lo_c, lo_s = mxfp8_quantize(np.asarray(v, dtype=np.float64) - hi)
    return hi + mxfp8_dequantize(lo_c, lo_s)


def expert_ffn_fp8act(xrows: np.ndarray, w13_blocks, w13_scales, w13_bias_bits,
                      w2_blocks, w2_scales, w2_bias_bits, mode: str) -> np.ndarray:
    """expert_ffn with block-scaled FP8 activations feeding both GEMMs: x
    quantized as above; the SwiGLU output rounded to bf16 (the path's
    intermediate), then quantized the same way."""
    W13 = dequantize_f64(w13_blocks, w13_scales)
    h = mxfp8_activations(xrows, mode) @ W13.T + bf16_decode(w13_bias_bits)[None, :]
    a = bf16_decode(bf16_encode_rne(swiglu_clamped(h[:, 0::2], h[:, 1::2])))
    W2 = dequantize_f64(w2_blocks, w2_scales)
    return mxfp8_activations(a, mode) @ W2.T + bf16_decode(w2_bias_bits)[None, :]


def moe_forward_fp8act(layer: Dict[str, np.ndarray], top_k: int, quantized: np.ndarray, mode: str,
                       tokens: Optional[Sequence[int]] = None) -> np.ndarray:
    """moe_forward where the experts with quantized[e] run expert_ffn_fp8act
    (the FP4 scaled-MFMA path applies to whole experts) and the rest expert_ffn."""
    x = bf16_decode(layer["x"])
    logits = np.asarray(layer["router_logits"])
    if tokens is not None:
        tokens = np.asarray(tokens, dtype=np.int64)
        x = x[tokens]
        logits = logits[tokens]
    T, H = x.shape
    E = logits.shape[1]
    ids, w = route(logits, top_k)
    counts, offsets, perm = group_by_expert(ids, E)
    z = np.zeros((T * top_k, H), dtype=np.float64)
    for e in range(E):
        if counts[e] == 0:
            continue
        pairs = perm[offsets[e]:offsets[e + 1]]
        args = (x[pairs // top_k], layer["w13_blocks"][e], layer["w13_scales"][e], layer["w13_bias"][e],
                layer["w2_blocks"][e], layer["w2_scales"][e], layer["w2_bias"][e])
        z[pairs] = expert_ffn_fp8act(*args, mode) if quantized[e] else expert_ffn(*args)
    z = z.reshape(T, top_k, H)
    y = np.zeros((T, H), dtype=np.float64)
    for j in range(top_k):
        y += w[:, j:j + 1] * z[:, j, :]
    return y


def moe_forward_dense(layer: Dict[str, np.ndarray], top_k: int) -> np.ndarray:
    """Brute force for tiny layers: every expert on every token, then a dense
    routing matrix R[T, E] (softmax weight at the selected experts, 0 elsewhere)
    combines them.  Shares no loop with moe_forward."""
    x = bf16_decode(layer["x"])
    logits = np.asarray(layer["router_logits"])
    T, E = logits.shape
    ids, w = route(logits, top_k)
    R = np.zeros((T, E), dtype=np.float64)
    for t in range(T):
        for j in range(top_k):
            R[t, ids[t, j]] += w[t, j]
    y = np.zeros((T, x.shape[1]), dtype=np.float64)
    for e in range(E):
        Ze = expert_ffn(x, layer["w13_blocks"][e], layer["w13_scales"][e], layer["w13_bias"][e],
                        layer["w2_blocks"][e], layer["w2_scales"][e], layer["w2_bias"][e])
        y += R[:, e:e + 1] * Ze
    return y


def parity_errors(y_test: np.ndarray, y_ref: np.ndarray) -> Tuple[float, float]:
    """Normwise relative error ||y - y_ref||_2 / ||y_ref||_2 and the max element
    error relative to max|y_ref|, both in float64."""
    a = np.asarray(y_test, dtype=np.float64)
    b = np.asarray(y_ref, dtype=np.float64)
    nref = float(np.linalg.norm(b.ravel()))
    rel = float(np.linalg.norm((a - b).ravel())) / max(nref, 1e-300)
    mref = float(np.max(np.abs(b))) if b.size else 0.0
    mx = float(np.max(np.abs(a - b))) / max(mref, 1e-300) if b.size else 0.0
    return rel, mx


def flops_per_pair(H: int, I: int) -> int:
    """Multiply-adds counted as 2 FLOPs: gate_up 2*H*2I plus down 2*I*H."""
    return 6 * H * I


__all__ = [
    "E2M1_VALUES", "SWIGLU_ALPHA", "SWIGLU_LIMIT", "GROUP",
    "e8m0_value", "bf16_decode", "bf16_encode_rne", "unpack_codes",
    "dequantize_f64", "mxfp4_dequantize", "route", "group_by_expert",
    "swiglu_clamped", "expert_ffn", "moe_forward", "moe_forward_dense",
    "parity_errors", "flops_per_pair",
    "NV_GROUP", "e4m3_value", "nvfp4_dequantize_f64", "expert_ffn_nvfp4", "moe_forward_nvfp4",
    "router_logits", "moe_forward_router",
    "e4m3_encode_rne", "mxfp8_quantize", "mxfp8_dequantize", "mxfp8_activations", "expert_ffn_fp8act",
    "moe_forward_fp8act",
]

