"""The C-ABI library: it loads, exports every declared entry point, and
rejects bad arguments on the host before any HIP call (CPU only; no kernel runs)."""

import ctypes
import os
import re

import pytest

from mxfp4_quantized_expert_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxfp4moe.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        from mxfp4_quantized_expert_amd import build
        build.build(verbose=False)
    return binding.load()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)


def test_exports_every_declared_function(lib):
    names = _declared()
    assert {"mxfp4_dequantize", "moe_mxfp4_route", "moe_mxfp4_forward"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    assert lib.mxfp4moe_status_string(0) == b"ok"
    assert b"shape" in lib.mxfp4moe_status_string(-2)


A = 0x100000  # a 256-byte aligned fake address: never dereferenced, every call fails before use


def test_dequant_argument_checks(lib):
    f = lib.mxfp4_dequantize
    assert f(A, A, A, 10, 33, None) == -2
    assert f(A, A, A, -1, 32, None) == -2
    assert f(A, A, A, 10, 0, None) == -2
    assert f(None, A, A, 10, 32, None) == -1
    assert f(A, None, A, 10, 32, None) == -1
    assert f(A, A, None, 10, 32, None) == -1
    assert f(A + 1, A, A, 10, 32, None) == -4
    assert f(A, A, A + 8, 10, 32, None) == -4
    assert f(None, None, None, 0, 32, None) == 0  # empty: no-op


def test_dequant_from_host_argument_checks(lib):
    f = lib.mxfp4_dequantize_from_host
    n = ctypes.c_size_t(0)
    assert f(None, None, None, 737280, 2880, None, ctypes.byref(n), None) == 0  # size query
    assert 2 * 15 * 2**20 <= n.value <= 2 * 17 * 2**20  # two slots of about 16 MiB of packed rows
    assert f(None, None, None, 3, 64, None, ctypes.byref(n), None) == 0 and n.value >= 2 * 3 * (32 + 2)
    big = ctypes.c_size_t(1 << 40)
    assert f(A, A, A, 10, 48, A, ctypes.byref(big), None) == -2   # K not a multiple of 32
    assert f(A, A, A, -1, 32, A, ctypes.byref(big), None) == -2
    assert f(A, A, A, 10, 32, A, None, None) == -1                # no size argument
    assert f(None, A, A, 10, 32, A, ctypes.byref(big), None) == -1
    assert f(A, A, None, 10, 32, A, ctypes.byref(big), None) == -1
    small = ctypes.c_size_t(16)
    assert f(A, A, A, 10, 32, A, ctypes.byref(small), None) == -3
    assert f(A, A, A, 10, 32, A + 16, ctypes.byref(big), None) == -4   # staging not 256-byte aligned
    assert f(A, A, A + 8, 10, 32, A, ctypes.byref(big), None) == -4    # output not 16-byte aligned
    assert f(None, None, None, 0, 32, A, ctypes.byref(big), None) == 0  # empty: no-op


def _fwd(lib, T=4, H=64, I=64, E=4, k=2, ws=A, ws_bytes=1 << 30, x=A, lg=A, b13=A, b2=A, y=A,
         wb=A, s13=A, s2=A):
    n = ctypes.c_size_t(ws_bytes)
    return lib.moe_mxfp4_forward(x, lg, wb, s13, b13, wb, s2, b2, y, T, H, I, E, k, ws,
                                 ctypes.byref(n), None), n.value


def test_forward_workspace_query(lib):
    st, n = _fwd(lib, ws=None, ws_bytes=0)
    assert st == 0 and n > 0
    P, H, I = 8, 64, 64
    assert n >= P * I * 2 + P * H * 2  # activations and per-pair output rows in bf16
    st2, n2 = _fwd(lib, T=4096, H=2880, I=2880, E=128, k=4, ws=None, ws_bytes=0)
    assert st2 == 0 and n2 >= 16384 * 2880 * 4
    assert binding.workspace_bytes(4, 64, 64, 4, 2) == n


def test_forward_argument_checks(lib):
    assert _fwd(lib, T=-1)[0] == -2
    assert _fwd(lib, k=5)[0] == -2            # top_k > E
    assert _fwd(lib, k=0)[0] == -2
    assert _fwd(lib, E=513, k=2)[0] == -2     # more experts than supported
    assert _fwd(lib, E=64, k=33)[0] == -2     # top_k above the maximum
    assert _fwd(lib, H=48)[0] == -2           # not a multiple of 32
    assert _fwd(lib, I=40)[0] == -2
    assert _fwd(lib, H=4128)[0] == -2         # above the largest supported hidden size
    assert _fwd(lib, I=4128)[0] == -2
    assert _fwd(lib, H=4096, I=4096, ws=None, ws_bytes=0)[0] == 0  # size query accepted
    assert _fwd(lib, b13=None)[0] == -1       # biases are required
    assert _fwd(lib, b2=None)[0] == -1
    assert _fwd(lib, x=None)[0] == -1
    assert _fwd(lib, ws_bytes=16)[0] == -3
    assert _fwd(lib, ws=A + 16)[0] == -4
    assert _fwd(lib, x=A + 2)[0] == -4
    assert _fwd(lib, wb=A + 4)[0] == -4
    assert _fwd(lib, s13=A + 8)[0] == -4      # scale rows are staged with 16-byte loads
    assert _fwd(lib, s2=A + 4)[0] == -4
    assert _fwd(lib, b13=A + 4)[0] == -4      # biases are read four at a time
    assert _fwd(lib, b2=A + 2)[0] == -4
    n = ctypes.c_size_t(0)
    assert lib.moe_mxfp4_forward(A, A, A, A, A, A, A, A, A, 4, 64, 64, 4, 2, A, None, None) == -1
    assert _fwd(lib, T=0, x=None, lg=None, y=None)[0] == 0  # empty batch: nothing to do
    del n


def test_forward_ex_rejects_unknown_flags(lib):
    n = ctypes.c_size_t(0)
    f = lib.moe_mxfp4_forward_ex
    assert f(A, A, A, A, A, A, A, A, A, 4, 64, 64, 4, 2, 16, None, ctypes.byref(n), None) == -1
    assert f(A, A, A, A, A, A, A, A, A, 4, 64, 64, 4, 2, 8, None, ctypes.byref(n), None) == 0  # streaming tiles
    assert f(A, A, A, A, A, A, A, A, A, 4, 64, 64, 4, 2, 1, None, ctypes.byref(n), None) == 0 and n.value > 0
    base = n.value
    # the MXFP8 activation flags need room for the quantized activations
    for flags in (2, 4, 6, 7):
        assert f(None, None, None, None, None, None, None, None, None, 4096, 2880, 2880, 128, 4, flags, None,
                 ctypes.byref(n), None) == 0
        assert n.value >= binding.workspace_bytes(4096, 2880, 2880, 128, 4) + 4096 * 5760 + 16384 * 5760
    del base


def test_nvfp4_forward_argument_checks(lib):
    f = lib.moe_nvfp4_forward
    n = ctypes.c_size_t(0)
    assert f(None, None, None, None, None, None, None, None, None, None, None, 4, 64, 64, 4, 2, None,
             ctypes.byref(n), None) == 0 and n.value > 0  # size query
    big = ctypes.c_size_t(1 << 30)
    assert f(A, A, A, A, None, A, A, A, A, A, A, 4, 64, 64, 4, 2, A, ctypes.byref(big), None) == -1  # no scale2
    assert f(A, A, A, A, A, A, A, A, None, A, A, 4, 64, 64, 4, 2, A, ctypes.byref(big), None) == -1
    assert f(A, A, A, A, A, A, A, A, A, A, A, 4, 48, 64, 4, 2, A, ctypes.byref(big), None) == -2
    assert f(A, A, A, A, A + 2, A, A, A, A, A, A, 4, 64, 64, 4, 2, A, ctypes.byref(big), None) == -4  # scale2
    assert f(A, A, A, A + 8, A, A, A, A, A, A, A, 4, 64, 64, 4, 2, A, ctypes.byref(big), None) == -4  # scales


def test_route_argument_checks(lib):
    f = lib.moe_mxfp4_route
    assert f(A, 4, 0, 1, A, A, A, A, None) == -2
    assert f(A, 4, 8, 9, A, A, A, A, None) == -2
    assert f(A, 4, 8, 2, A, A, None, A, None) == -1
    assert f(None, 4, 8, 2, A, A, A, A, None) == -1


def test_router_argument_checks(lib):
    f = lib.moe_mxfp4_router
    assert f(A, A, A, 4, 64, 0, 1, A, A, A, None) == -2      # no experts
    assert f(A, A, A, 4, 64, 8, 9, A, A, A, None) == -2      # top_k > E
    assert f(A, A, A, 4, 48, 8, 2, A, A, A, None) == -2      # H not a multiple of 32
    assert f(A, A, None, 4, 64, 8, 2, A, A, A, None) == -1   # the router bias is required
    assert f(A, None, A, 4, 64, 8, 2, A, A, A, None) == -1
    assert f(A, A, A, 4, 64, 8, 2, None, A, A, None) == -1   # logits out
    assert f(A + 2, A, A, 4, 64, 8, 2, A, A, A, None) == -4
    assert f(A, A + 4, A, 4, 64, 8, 2, A, A, A, None) == -4
    assert f(None, None, None, 0, 64, 8, 2, None, None, None, None) == 0  # empty batch


def test_forward_router_argument_checks(lib):
    f = lib.moe_mxfp4_forward_router
    n = ctypes.c_size_t(0)
    assert f(*([None] * 10), 4, 64, 64, 4, 2, 0, None, ctypes.byref(n), None) == 0
    assert n.value == binding.workspace_bytes(4, 64, 64, 4, 2)  # same workspace as the logits entry
    big = ctypes.c_size_t(1 << 30)
    w = [A] * 6
    assert f(A, None, A, *w, A, 4, 64, 64, 4, 2, 0, A, ctypes.byref(big), None) == -1  # no router weights
    assert f(A, A, None, *w, A, 4, 64, 64, 4, 2, 0, A, ctypes.byref(big), None) == -1  # no router bias
    assert f(A, A, A, *w, A, 4, 64, 64, 4, 2, 16, A, ctypes.byref(big), None) == -1    # unknown flag
    assert f(A, A + 2, A, *w, A, 4, 64, 64, 4, 2, 0, A, ctypes.byref(big), None) == -4  # misaligned router
    assert f(A, A, A, *w, A, 4, 48, 64, 4, 2, 0, A, ctypes.byref(big), None) == -2


def test_mxfp8_quantize_argument_checks(lib):
    f = lib.moe_mxfp8_quantize
    assert f(A, 4, 48, 1, A, A, None) == -2      # K not a multiple of 32
    assert f(A, -1, 64, 1, A, A, None) == -2
    assert f(None, 4, 64, 1, A, A, None) == -1
    assert f(A, 4, 64, 1, None, A, None) == -1
    assert f(A + 2, 4, 64, 1, A, A, None) == -4
    assert f(A, 4, 64, 1, A, A + 2, None) == -4  # scale rows are read as 4-byte words
    assert f(None, 0, 64, 1, None, None, None) == 0
    assert f(A, 1 << 31, 64, 1, A, A, None) == -2  # more rows than the kernel counts


def test_forward_noalloc_argument_checks(lib):
    # Every host check runs before the scratch address is looked up (no GPU here).
    f = lib.moe_mxfp4_forward_noalloc
    assert f(A, A, A, A, A, A, A, A, A, 4, 48, 64, 4, 2, None) == -2       # H not a multiple of 32
    assert f(A, A, A, A, A, A, A, A, A, 4, 64, 64, 4, 5, None) == -2       # top_k > E
    assert f(A, A, A, A, None, A, A, A, A, 4, 64, 64, 4, 2, None) == -1    # biases are required
    assert f(A, A, A, A, A, A, A, None, A, 4, 64, 64, 4, 2, None) == -1
    assert f(A + 2, A, A, A, A, A, A, A, A, 4, 64, 64, 4, 2, None) == -4   # x misaligned
    assert f(A, A, A, A + 8, A, A, A, A, A, 4, 64, 64, 4, 2, None) == -4   # scales misaligned
    assert f(None, None, A, A, A, A, A, A, None, 0, 64, 64, 4, 2, None) == 0  # empty batch: nothing to do
    # more than the fixed scratch: 4096 tokens of the 120b layer need ~190 MB
    assert f(A, A, A, A, A, A, A, A, A, 4096, 2880, 2880, 128, 4, None) == -6
    n = ctypes.c_size_t(0)
    assert lib.moe_mxfp4_forward(None, None, None, None, None, None, None, None, None, 256, 2880, 2880, 32, 4,
                                 None, ctypes.byref(n), None) == 0
    assert n.value <= binding.NOALLOC_SCRATCH_BYTES  # the 20b prefill layer fits
    assert b"scratch" in lib.mxfp4moe_status_string(-6)
