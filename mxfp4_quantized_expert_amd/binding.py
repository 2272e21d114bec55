"""ctypes binding of libmxfp4moe.so.

Argument marshalling only: dtype/device/shape checks, output allocation with
torch, and the raw C call on torch's current HIP stream.  Every step of the
computation runs in the library's HIP kernels; there is no other code path.
The C ABI is declared in include/mxfp4moe.h.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmxfp4moe.so")

STATUS = {
    0: "ok",
    -1: "invalid argument",
    -2: "unsupported shape",
    -3: "workspace too small",
    -4: "pointer not aligned as required",
    -5: "HIP launch error",
    -6: "layer needs more than the no-allocation scratch",
}

STAGES = {"route": 1, "group": 2, "gate_up": 3, "down": 4, "combine": 5, "dequant": 6,
          "gate_up_wide": 7, "gate_up_stream": 8, "down_wide": 9, "down_stream": 10,
          "gate_up_mid": 11, "down_mid": 12, "act_quant": 13}

_lib: Optional[ctypes.CDLL] = None

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64


class MXFP4MoEError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: status {status} ({STATUS.get(status, 'unknown')})")
        self.status = status


def load() -> ctypes.CDLL:
    """Load the HIP library; raises if it has not been built (no fallback exists)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                           "or python -m mxfp4_quantized_expert_amd.build")
    lib = ctypes.CDLL(LIB_PATH)
    lib.mxfp4_dequantize.argtypes = [_vp, _vp, _vp, _i64, _i64, _vp]
    lib.mxfp4_dequantize.restype = ctypes.c_int
    lib.mxfp4_dequantize_from_host.argtypes = [_vp, _vp, _vp, _i64, _i64, _vp, ctypes.POINTER(ctypes.c_size_t), _vp]
    lib.mxfp4_dequantize_from_host.restype = ctypes.c_int
    lib.moe_mxfp4_route.argtypes = [_vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp]
    lib.moe_mxfp4_route.restype = ctypes.c_int
    lib.moe_mxfp4_forward.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                      _i64, _i64, _i64, _i64, _i64, _vp,
                                      ctypes.POINTER(ctypes.c_size_t), _vp]
    lib.moe_mxfp4_forward.restype = ctypes.c_int
    lib.moe_mxfp4_forward_noalloc.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                              _i64, _i64, _i64, _i64, _i64, _vp]
    lib.moe_mxfp4_forward_noalloc.restype = ctypes.c_int
    lib.moe_mxfp4_forward_ex.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                         _i64, _i64, _i64, _i64, _i64, ctypes.c_uint32, _vp,
                                         ctypes.POINTER(ctypes.c_size_t), _vp]
    lib.moe_mxfp4_forward_ex.restype = ctypes.c_int
    lib.moe_nvfp4_forward.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                      _i64, _i64, _i64, _i64, _i64, _vp, ctypes.POINTER(ctypes.c_size_t), _vp]
    lib.moe_nvfp4_forward.restype = ctypes.c_int
    lib.moe_mxfp4_router.argtypes = [_vp, _vp, _vp, _i64, _i64, _i64, _i64, _vp, _vp, _vp, _vp]
    lib.moe_mxfp4_router.restype = ctypes.c_int
    lib.moe_mxfp4_forward_router.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                             _i64, _i64, _i64, _i64, _i64, ctypes.c_uint32, _vp,
                                             ctypes.POINTER(ctypes.c_size_t), _vp]
    lib.moe_mxfp4_forward_router.restype = ctypes.c_int
    lib.moe_mxfp8_quantize.argtypes = [_vp, _i64, _i64, ctypes.c_int, _vp, _vp, _vp]
    lib.moe_mxfp8_quantize.restype = ctypes.c_int
    lib.mxfp4moe_status_string.argtypes = [ctypes.c_int]
    lib.mxfp4moe_status_string.restype = ctypes.c_char_p
    lib.mxfp4moe_profile_begin.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.mxfp4moe_profile_begin.restype = ctypes.c_int
    lib.mxfp4moe_profile_end.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_int]
    lib.mxfp4moe_profile_end.restype = ctypes.c_int
    _lib = lib
    return lib


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _check(t: torch.Tensor, name: str, dtype: torch.dtype, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and t.shape != shape:  # torch.Size is a tuple
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _raise(fn: str, st: int):
    if st != 0:
        raise MXFP4MoEError(fn, st)


def mxfp4_dequantize(blocks: torch.Tensor, scales: torch.Tensor, out: Optional[torch.Tensor] = None,
                     stream=None) -> torch.Tensor:
    """blocks [..., N, K/2] uint8 + scales [..., N, K/32] uint8 -> [..., N, K] bfloat16."""
    lib = load()
    half_k = blocks.shape[-1]
    K = 2 * half_k
    lead = tuple(blocks.shape[:-1])
    _check(blocks, "blocks", torch.uint8)
    _check(scales, "scales", torch.uint8, lead + (K // 32,))
    if out is None:
        out = torch.empty(lead + (K,), dtype=torch.bfloat16, device=blocks.device)
    _check(out, "out", torch.bfloat16, lead + (K,))
    N = 1
    for d in lead:
        N *= d
    st = lib.mxfp4_dequantize(blocks.data_ptr(), scales.data_ptr(), out.data_ptr(), N, K, _stream(stream))
    _raise("mxfp4_dequantize", st)
    return out


def offload_staging_bytes(N: int, K: int) -> int:
    """Device staging mxfp4_dequantize_from_host needs for N rows of K elements."""
    n = ctypes.c_size_t(0)
    st = load().mxfp4_dequantize_from_host(None, None, None, N, K, None, ctypes.byref(n), None)
    _raise("mxfp4_dequantize_from_host(staging query)", st)
    return int(n.value)


def mxfp4_dequantize_from_host(blocks: torch.Tensor, scales: torch.Tensor, out: Optional[torch.Tensor] = None,
                               staging: Optional[torch.Tensor] = None, device="cuda",
                               stream=None) -> torch.Tensor:
    """Host blocks [..., N, K/2] + host scales [..., N, K/32] (uint8, CPU; pinned memory copies
    asynchronously) -> device bf16 [..., N, K], copied in chunks and dequantized on arrival."""
    lib = load()
    half_k = blocks.shape[-1]
    K = 2 * half_k
    lead = tuple(blocks.shape[:-1])
    for t, name, shape in ((blocks, "blocks", None), (scales, "scales", lead + (K // 32,))):
        if t.dtype != torch.uint8 or t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous uint8 host tensor")
        if shape is not None and tuple(t.shape) != shape:
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shape}")
    N = 1
    for d in lead:
        N *= d
    if out is None:
        out = torch.empty(lead + (K,), dtype=torch.bfloat16, device=device)
    _check(out, "out", torch.bfloat16, lead + (K,))
    need = offload_staging_bytes(N, K)
    if staging is None:
        staging = torch.empty((max(need, 1),), dtype=torch.uint8, device=out.device)
    _check(staging, "staging", torch.uint8)
    n = ctypes.c_size_t(staging.numel())
    st = lib.mxfp4_dequantize_from_host(blocks.data_ptr(), scales.data_ptr(), out.data_ptr(), N, K,
                                        staging.data_ptr(), ctypes.byref(n), _stream(stream))
    _raise("mxfp4_dequantize_from_host", st)
    return out


def moe_mxfp4_route(router_logits: torch.Tensor, top_k: int, stream=None):
    """Returns (topk_ids [T,k] int32, topk_weights [T,k] float32, expert_offsets [E+1] int32,
    sorted_pairs [T*k] int32)."""
    lib = load()
    _check(router_logits, "router_logits", torch.float32)
    T, E = router_logits.shape
    dev = router_logits.device
    ids = torch.empty((T, top_k), dtype=torch.int32, device=dev)
    w = torch.empty((T, top_k), dtype=torch.float32, device=dev)
    offsets = torch.empty((E + 1,), dtype=torch.int32, device=dev)
    pairs = torch.empty((T * top_k,), dtype=torch.int32, device=dev)
    st = lib.moe_mxfp4_route(router_logits.data_ptr(), T, E, top_k, ids.data_ptr(), w.data_ptr(),
                             offsets.data_ptr(), pairs.data_ptr(), _stream(stream))
    _raise("moe_mxfp4_route", st)
    return ids, w, offsets, pairs


def moe_mxfp8_quantize(src: torch.Tensor, split: bool = True, stream=None):
    """bf16 [rows, K] -> (codes [rows, 128*ceil(K/64)] uint8, scales [rows, 4*ceil(K/64)] uint8)
    in the chunk-interleaved layout of the FP4 scaled-MFMA path."""
    lib = load()
    rows, K = src.shape
    _check(src, "src", torch.bfloat16)
    nc = (K + 63) // 64
    codes = torch.empty((rows, 128 * nc), dtype=torch.uint8, device=src.device)
    scales = torch.empty((rows, 4 * nc), dtype=torch.uint8, device=src.device)
    st = lib.moe_mxfp8_quantize(src.data_ptr(), rows, K, 1 if split else 0, codes.data_ptr(), scales.data_ptr(),
                                _stream(stream))
    _raise("moe_mxfp8_quantize", st)
    return codes, scales


def moe_mxfp4_router(x: torch.Tensor, router_w: torch.Tensor, router_b: torch.Tensor, top_k: int, stream=None):
    """Router projection fused ahead of the top-k.  Returns (logits [T,E] float32,
    topk_ids [T,k] int32, topk_weights [T,k] float32)."""
    lib = load()
    T, H = x.shape
    E = router_w.shape[0]
    _check(x, "x", torch.bfloat16, (T, H))
    _check(router_w, "router_w", torch.bfloat16, (E, H))
    _check(router_b, "router_b", torch.bfloat16, (E,))
    dev = x.device
    logits = torch.empty((T, E), dtype=torch.float32, device=dev)
    ids = torch.empty((T, top_k), dtype=torch.int32, device=dev)
    w = torch.empty((T, top_k), dtype=torch.float32, device=dev)
    st = lib.moe_mxfp4_router(x.data_ptr(), router_w.data_ptr(), router_b.data_ptr(), T, H, E, top_k,
                              logits.data_ptr(), ids.data_ptr(), w.data_ptr(), _stream(stream))
    _raise("moe_mxfp4_router", st)
    return logits, ids, w


FLAG_GATE_UP_SPLIT = 1
ACT_FLAGS = {"bf16": 0, "mxfp8": 2, "mxfp8_split": 4}
FLAG_TILES_STREAM = 8


def workspace_bytes(T: int, H: int, I: int, E: int, top_k: int, flags: int = 0) -> int:
    """Device workspace moe_mxfp4_forward needs for these sizes (and layout/activation flags)."""
    lib = load()
    n = ctypes.c_size_t(0)
    st = lib.moe_mxfp4_forward_ex(None, None, None, None, None, None, None, None, None,
                                  T, H, I, E, top_k, flags, None, ctypes.byref(n), None)
    _raise("moe_mxfp4_forward(workspace query)", st)
    return int(n.value)


def moe_mxfp4_forward(x: torch.Tensor, router_logits: torch.Tensor,
                      w13_blocks: torch.Tensor, w13_scales: torch.Tensor, w13_bias: torch.Tensor,
                      w2_blocks: torch.Tensor, w2_scales: torch.Tensor, w2_bias: torch.Tensor,
                      top_k: int, out: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None, stream=None,
                      gate_up_split: bool = False, act: str = "bf16",
                      stream_tiles_only: bool = False) -> torch.Tensor:
    """One MXFP4 MoE expert layer; returns y [T, H] bfloat16.  gate_up_split: w13 rows are
    [I gate rows; I up rows] instead of interleaved.  act: "bf16" (exact), or the opt-in
    FP4 scaled-MFMA path for experts with at least 128 pairs over MXFP8 activations,
    "mxfp8_split" (high part + residual) or "mxfp8" (one tensor).  stream_tiles_only:
    every pair through the streaming kernels (MXFP4MOE_TILES_STREAM)."""
    lib = load()
    T, H = x.shape
    E = router_logits.shape[1]
    I = w2_blocks.shape[-1] * 2
    _check(x, "x", torch.bfloat16, (T, H))
    _check(router_logits, "router_logits", torch.float32, (T, E))
    _check(w13_blocks, "w13_blocks", torch.uint8, (E, 2 * I, H // 2))
    _check(w13_scales, "w13_scales", torch.uint8, (E, 2 * I, H // 32))
    _check(w13_bias, "w13_bias", torch.bfloat16, (E, 2 * I))
    _check(w2_blocks, "w2_blocks", torch.uint8, (E, H, I // 2))
    _check(w2_scales, "w2_scales", torch.uint8, (E, H, I // 32))
    _check(w2_bias, "w2_bias", torch.bfloat16, (E, H))
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    _check(out, "out", torch.bfloat16, (T, H))
    flags = (FLAG_GATE_UP_SPLIT if gate_up_split else 0) | ACT_FLAGS[act] | (FLAG_TILES_STREAM if stream_tiles_only else 0)
    if workspace is None:  # a caller's workspace is size-checked by the library
        workspace = torch.empty((max(workspace_bytes(T, H, I, E, top_k, flags), 1),), dtype=torch.uint8, device=x.device)
    _check(workspace, "workspace", torch.uint8)
    n = ctypes.c_size_t(workspace.numel())
    st = lib.moe_mxfp4_forward_ex(x.data_ptr(), router_logits.data_ptr(),
                                  w13_blocks.data_ptr(), w13_scales.data_ptr(), w13_bias.data_ptr(),
                                  w2_blocks.data_ptr(), w2_scales.data_ptr(), w2_bias.data_ptr(),
                                  out.data_ptr(), T, H, I, E, top_k, flags,
                                  workspace.data_ptr(), ctypes.byref(n), _stream(stream))
    _raise("moe_mxfp4_forward", st)
    return out


NOALLOC_SCRATCH_BYTES = 32 << 20


def moe_mxfp4_forward_noalloc(x: torch.Tensor, router_logits: torch.Tensor,
                              w13_blocks: torch.Tensor, w13_scales: torch.Tensor, w13_bias: torch.Tensor,
                              w2_blocks: torch.Tensor, w2_scales: torch.Tensor, w2_bias: torch.Tensor,
                              top_k: int, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """moe_mxfp4_forward through the entry point that takes no workspace (its scratch
    is a fixed device array of the library); returns y [T, H] bfloat16."""
    lib = load()
    T, H = x.shape
    E = router_logits.shape[1]
    I = w2_blocks.shape[-1] * 2
    _check(x, "x", torch.bfloat16, (T, H))
    _check(router_logits, "router_logits", torch.float32, (T, E))
    _check(w13_blocks, "w13_blocks", torch.uint8, (E, 2 * I, H // 2))
    _check(w13_scales, "w13_scales", torch.uint8, (E, 2 * I, H // 32))
    _check(w13_bias, "w13_bias", torch.bfloat16, (E, 2 * I))
    _check(w2_blocks, "w2_blocks", torch.uint8, (E, H, I // 2))
    _check(w2_scales, "w2_scales", torch.uint8, (E, H, I // 32))
    _check(w2_bias, "w2_bias", torch.bfloat16, (E, H))
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    _check(out, "out", torch.bfloat16, (T, H))
    st = lib.moe_mxfp4_forward_noalloc(x.data_ptr(), router_logits.data_ptr(),
                                       w13_blocks.data_ptr(), w13_scales.data_ptr(), w13_bias.data_ptr(),
                                       w2_blocks.data_ptr(), w2_scales.data_ptr(), w2_bias.data_ptr(),
                                       out.data_ptr(), T, H, I, E, top_k, _stream(stream))
    _raise("moe_mxfp4_forward_noalloc", st)
    return out


def moe_mxfp4_forward_router(x: torch.Tensor, router_w: torch.Tensor, router_b: torch.Tensor,
                             w13_blocks: torch.Tensor, w13_scales: torch.Tensor, w13_bias: torch.Tensor,
                             w2_blocks: torch.Tensor, w2_scales: torch.Tensor, w2_bias: torch.Tensor,
                             top_k: int, out: Optional[torch.Tensor] = None,
                             workspace: Optional[torch.Tensor] = None, stream=None,
                             gate_up_split: bool = False) -> torch.Tensor:
    """One MXFP4 MoE expert layer whose logits come from the router projection
    x W_r^T + b_r (router_w [E,H], router_b [E] bfloat16); returns y [T, H] bfloat16."""
    lib = load()
    T, H = x.shape
    E = router_w.shape[0]
    I = w2_blocks.shape[-1] * 2
    _check(x, "x", torch.bfloat16, (T, H))
    _check(router_w, "router_w", torch.bfloat16, (E, H))
    _check(router_b, "router_b", torch.bfloat16, (E,))
    _check(w13_blocks, "w13_blocks", torch.uint8, (E, 2 * I, H // 2))
    _check(w13_scales, "w13_scales", torch.uint8, (E, 2 * I, H // 32))
    _check(w13_bias, "w13_bias", torch.bfloat16, (E, 2 * I))
    _check(w2_blocks, "w2_blocks", torch.uint8, (E, H, I // 2))
    _check(w2_scales, "w2_scales", torch.uint8, (E, H, I // 32))
    _check(w2_bias, "w2_bias", torch.bfloat16, (E, H))
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    _check(out, "out", torch.bfloat16, (T, H))
    if workspace is None:  # a caller's workspace is size-checked by the library
        workspace = torch.empty((max(workspace_bytes(T, H, I, E, top_k), 1),), dtype=torch.uint8, device=x.device)
    _check(workspace, "workspace", torch.uint8)
    n = ctypes.c_size_t(workspace.numel())
    st = lib.moe_mxfp4_forward_router(x.data_ptr(), router_w.data_ptr(), router_b.data_ptr(),
                                      w13_blocks.data_ptr(), w13_scales.data_ptr(), w13_bias.data_ptr(),
                                      w2_blocks.data_ptr(), w2_scales.data_ptr(), w2_bias.data_ptr(),
                                      out.data_ptr(), T, H, I, E, top_k, 1 if gate_up_split else 0,
                                      workspace.data_ptr(), ctypes.byref(n), _stream(stream))
    _raise("moe_mxfp4_forward_router", st)
    return out


def moe_nvfp4_forward(x: torch.Tensor, router_logits: torch.Tensor,
                      w13_blocks: torch.Tensor, w13_scales: torch.Tensor, w13_scale2: torch.Tensor,
                      w13_bias: torch.Tensor, w2_blocks: torch.Tensor, w2_scales: torch.Tensor,
                      w2_scale2: torch.Tensor, w2_bias: torch.Tensor, top_k: int,
                      out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                      stream=None) -> torch.Tensor:
    """One NVFP4 MoE expert layer (E4M3 block scales per 16, float32 second-level
    scales [E]); returns y [T, H] bfloat16."""
    lib = load()
    T, H = x.shape
    E = router_logits.shape[1]
    I = w2_blocks.shape[-1] * 2
    _check(x, "x", torch.bfloat16, (T, H))
    _check(router_logits, "router_logits", torch.float32, (T, E))
    _check(w13_blocks, "w13_blocks", torch.uint8, (E, 2 * I, H // 2))
    _check(w13_scales, "w13_scales", torch.uint8, (E, 2 * I, H // 16))
    _check(w13_scale2, "w13_scale2", torch.float32, (E,))
    _check(w13_bias, "w13_bias", torch.bfloat16, (E, 2 * I))
    _check(w2_blocks, "w2_blocks", torch.uint8, (E, H, I // 2))
    _check(w2_scales, "w2_scales", torch.uint8, (E, H, I // 16))
    _check(w2_scale2, "w2_scale2", torch.float32, (E,))
    _check(w2_bias, "w2_bias", torch.bfloat16, (E, H))
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    _check(out, "out", torch.bfloat16, (T, H))
    if workspace is None:  # a caller's workspace is size-checked by the library
        workspace = torch.empty((max(workspace_bytes(T, H, I, E, top_k), 1),), dtype=torch.uint8, device=x.device)
    _check(workspace, "workspace", torch.uint8)
    n = ctypes.c_size_t(workspace.numel())
    st = lib.moe_nvfp4_forward(x.data_ptr(), router_logits.data_ptr(), w13_blocks.data_ptr(),
                               w13_scales.data_ptr(), w13_scale2.data_ptr(), w13_bias.data_ptr(),
                               w2_blocks.data_ptr(), w2_scales.data_ptr(), w2_scale2.data_ptr(),
                               w2_bias.data_ptr(), out.data_ptr(), T, H, I, E, top_k, workspace.data_ptr(),
                               ctypes.byref(n), _stream(stream))
    _raise("moe_nvfp4_forward", st)
    return out


def profile_begin(stage: str, max_calls: int) -> None:
    """Record HIP events around the next ``max_calls`` launches of one kernel stage."""
    st = load().mxfp4moe_profile_begin(STAGES[stage], max_calls)
    _raise("mxfp4moe_profile_begin", st)


def profile_end(capacity: int):
    """Per-launch durations (ms) recorded since profile_begin."""
    buf = (ctypes.c_float * max(capacity, 1))()
    n = load().mxfp4moe_profile_end(buf, capacity)
    if n < 0:
        raise MXFP4MoEError("mxfp4moe_profile_end", n)
    return [float(buf[i]) for i in range(n)]


def layer_to_device(layer, device="cuda"):
    """Host numpy layer (workloads.make_layer) -> device tensors with the binding's dtypes."""
    import numpy as np

    def dev(a, dtype):
        a = np.ascontiguousarray(a)
        if dtype == torch.bfloat16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
        return torch.from_numpy(a).to(device)

    out = {
        "x": dev(layer["x"], torch.bfloat16),
        "router_logits": dev(layer["router_logits"], torch.float32),
        "w13_blocks": dev(layer["w13_blocks"], torch.uint8),
        "w13_scales": dev(layer["w13_scales"], torch.uint8),
        "w13_bias": dev(layer["w13_bias"], torch.bfloat16),
        "w2_blocks": dev(layer["w2_blocks"], torch.uint8),
        "w2_scales": dev(layer["w2_scales"], torch.uint8),
        "w2_bias": dev(layer["w2_bias"], torch.bfloat16),
    }
    for k in ("w13_scale2", "w2_scale2"):  # NVFP4 layers
        if k in layer:
            out[k] = dev(np.asarray(layer[k], dtype=np.float32), torch.float32)
    for k in ("router_w", "router_b"):  # layers with a router projection
        if k in layer:
            out[k] = dev(layer[k], torch.bfloat16)
    return out
