"""Pins of the CPU oracle against facts fixed outside it (CPU only).

Each test ties an oracle function to something other than its own formula:
the OCP MX element tables, hand-derived bit patterns, torch's bf16 rounding,
brute force on tiny inputs, closed-form special cases and algebraic
identities.  Planted-mistake variants of the oracle show that the parity bar
(normwise 1e-2) would catch each defect class the pages warn about.
"""

import math
import os

import numpy as np
import pytest
import torch
from scipy.special import expit, softmax

from oracle import mxfp4_moe as O
from mxfp4_quantized_expert_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- encodings

def test_e2m1_matches_ocp_table():
    # OCP Microscaling Formats v1.0, FP4 (E2M1) element: the eight magnitudes.
    spec = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert list(O.E2M1_VALUES[:8]) == spec
    assert list(O.E2M1_VALUES[8:]) == [-v for v in spec]
    assert math.copysign(1.0, O.E2M1_VALUES[8]) == -1.0  # code 0x8 is -0


def test_e8m0_values():
    assert O.e8m0_value(127) == 1.0
    assert O.e8m0_value(128) == 2.0
    assert O.e8m0_value(0) == math.ldexp(1.0, -127)
    assert O.e8m0_value(254) == math.ldexp(1.0, 127)
    assert np.isnan(O.e8m0_value(255))


def test_bf16_encoder_matches_torch_on_float32_values():
    rng = np.random.default_rng(7)
    # random bit patterns cover normals, subnormals, ties and near-overflow
    bits = rng.integers(0, 2 ** 32, size=200000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    extra = np.array([0.0, -0.0, 1.0, 2.0 ** -133, 2.0 ** -134, 3 * 2.0 ** -134,
                      (2 - 2 ** -8) * 2.0 ** 127, 3.3e38, 1 + 2 ** -8, 1 + 3 * 2 ** -8],
                     dtype=np.float32)
    f = np.concatenate([f, extra, -extra])
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = O.bf16_encode_rne(f.astype(np.float64))
    assert np.array_equal(got, ref)


def test_bf16_encoder_special_bits():
    enc = lambda v: int(O.bf16_encode_rne(np.array([v]))[0])  # noqa: E731
    assert enc(1.0) == 0x3F80
    assert enc(-0.0) == 0x8000
    assert enc(2.0 ** -133) == 0x0001
    assert enc(2.0 ** -134) == 0x0000  # tie to even (zero)
    assert enc(3 * 2.0 ** -134) == 0x0002  # 1.5 quanta: tie to even (2)
    assert enc(float("inf")) == 0x7F80
    assert enc(float("nan")) == 0x7FC0
    assert enc(2.0 ** 128) == 0x7F80
    assert enc((2 - 2 ** -7) * 2.0 ** 127) == 0x7F7F


def _golden_cases():
    rows = []
    with open(os.path.join(GOLDEN, "dequant_cases.txt")) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if line:
                c, s, b = line.split()
                rows.append((int(c, 16), int(s), int(b, 16)))
    return rows


def test_dequant_golden_cases():
    for code, s, bits in _golden_cases():
        # one 32-element group whose element 0 carries the code (low nibble of byte 0)
        blocks = np.zeros((1, 16), np.uint8)
        blocks[0, 0] = code
        out = O.mxfp4_dequantize(blocks, np.array([[s]], np.uint8))
        assert out[0, 0] == bits, (hex(code), s, hex(out[0, 0]), hex(bits))
        assert O.bf16_encode_rne(O.dequantize_f64(blocks, np.array([[s]], np.uint8)))[0, 0] == bits


def test_dequant_exhaustive_against_spec_table_and_torch():
    # All 16 codes x 256 scale bytes.  Values from the OCP table literal times
    # 2^(s-127) computed by math.ldexp, rounded by torch (float32 -> bf16 RNE).
    spec = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    codes = np.arange(16, dtype=np.uint8)
    blocks = np.zeros((256, 16), np.uint8)
    blocks[:, :8] = (codes[0::2] | (codes[1::2] << 4))[None, :]
    scales = np.arange(256, dtype=np.uint8)[:, None]
    out = O.mxfp4_dequantize(blocks, scales)
    for s in range(256):
        for c in range(16):
            got = int(out[s, c])
            if s == 255:
                assert got == 0x7FC0
                continue
            v = math.ldexp(spec[c & 7], s - 127)
            v = -v if c & 8 else v
            with np.errstate(over="ignore"):
                f32 = np.array([v], dtype=np.float32)
            ref = int(torch.from_numpy(f32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)[0])
            assert got == ref, (c, s, hex(got), hex(ref))


def test_nibble_order_and_group_axis():
    # Reading: element 2i is the low nibble of byte i; element k uses scale k // 32.
    blocks = np.zeros((1, 32), np.uint8)
    blocks[0, 0] = 0x21   # k=0 -> code 1 (0.5), k=1 -> code 2 (1.0)
    blocks[0, 16] = 0x73  # k=32 -> code 3 (1.5), k=33 -> code 7 (6.0)
    scales = np.array([[127, 128]], np.uint8)
    v = O.dequantize_f64(blocks, scales)
    assert v[0, 0] == 0.5 and v[0, 1] == 1.0
    assert v[0, 32] == 3.0 and v[0, 33] == 12.0
    assert np.all(v[0, 2:32] == 0) and np.all(v[0, 34:] == 0)


# ---------------------------------------------------------------- routing

def test_route_against_python_brute_force():
    rng = np.random.default_rng(3)
    for T, E, k in [(16, 4, 2), (9, 32, 4), (5, 128, 4), (3, 7, 7), (4, 5, 1)]:
        logits = rng.standard_normal((T, E)).astype(np.float32)
        logits[0, :] = np.round(logits[0, :])  # plenty of ties
        ids, w = O.route(logits, k)
        for t in range(T):
            order = sorted(range(E), key=lambda e: (-float(logits[t, e]), e))[:k]
            assert list(ids[t]) == order
            sel = [float(logits[t, e]) for e in order]
            ex = [math.exp(v - sel[0]) for v in sel]
            assert np.allclose(w[t], [v / sum(ex) for v in ex], rtol=0, atol=1e-15)
        assert np.all(np.abs(w.sum(1) - 1.0) <= 1e-12)


def test_route_softmax_over_selected_equals_renormalised_full_softmax():
    rng = np.random.default_rng(4)
    logits = (rng.standard_normal((64, 32)) * 2).astype(np.float32)
    ids, w = O.route(logits, 4)
    full = softmax(logits.astype(np.float64), axis=1)
    sel = np.take_along_axis(full, ids, axis=1)
    assert np.allclose(w, sel / sel.sum(1, keepdims=True), rtol=1e-12, atol=0)


def test_route_tie_rule():
    ids, w = O.route(np.array([[1.0, 3.0, 3.0, 0.0]], np.float32), 2)
    assert list(ids[0]) == [1, 2]
    assert np.allclose(w[0], [0.5, 0.5])


def test_group_against_brute_force():
    rng = np.random.default_rng(5)
    for T, E, k in [(16, 4, 2), (33, 32, 4), (50, 128, 4)]:
        ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
        counts, offsets, perm = O.group_by_expert(ids, E)
        flat = ids.ravel()
        bf = [p for e in range(E) for p in range(T * k) if flat[p] == e]
        assert list(perm) == bf
        assert list(counts) == [int((flat == e).sum()) for e in range(E)]
        assert offsets[0] == 0 and offsets[-1] == T * k


# ---------------------------------------------------------------- SwiGLU

def test_swiglu_special_cases():
    g = np.linspace(-30, 30, 241)
    a = O.swiglu_clamped(g, -np.ones_like(g))
    assert np.all(a == 0)  # up = -1 kills the unit, saturated gate or not
    u = np.linspace(-30, 30, 241)
    assert np.all(O.swiglu_clamped(np.zeros_like(u), u) == 0)
    # gate clamp from above only, up clamp on both sides
    for gv in [7.0, 7.5, 100.0, 1e6]:
        assert O.swiglu_clamped(gv, 0.3) == O.swiglu_clamped(7.0, 0.3)
    for uv in [7.0, 8.0, 1e5]:
        assert O.swiglu_clamped(0.9, uv) == O.swiglu_clamped(0.9, 7.0)
    for uv in [-7.0, -8.0, -1e5]:
        assert O.swiglu_clamped(0.9, uv) == O.swiglu_clamped(0.9, -7.0)
    assert abs(O.swiglu_clamped(-60.0, 3.0)) < 1e-40
    assert math.isclose(O.swiglu_clamped(7.0, 7.0), 7.0 * 8.0 * expit(1.702 * 7.0), rel_tol=1e-15)


def test_swiglu_odd_even_identities():
    # g*s(ag) - (-g)*s(-ag) = g and g*s(ag) + (-g)*s(-ag) = g*tanh(a*g/2)
    g = np.linspace(-6.9, 6.9, 139)
    for uv in [-0.5, 0.0, 2.0]:
        u = np.full_like(g, uv)
        d = O.swiglu_clamped(g, u) - O.swiglu_clamped(-g, u)
        assert np.allclose(d, g * (uv + 1), rtol=1e-12, atol=1e-12)
    s = O.swiglu_clamped(g, np.zeros_like(g)) + O.swiglu_clamped(-g, np.zeros_like(g))
    assert np.allclose(s, g * np.tanh(1.702 * g / 2), rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- whole layer

def _tiny(seed, **kw):
    spec = W.LAYERS["tiny"].with_(**kw) if kw else W.LAYERS["tiny"]
    return W.make_layer(spec, seed=seed), spec


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_grouped_equals_dense_brute_force(seed):
    L, spec = _tiny(seed)
    y = O.moe_forward(L, spec.top_k)
    yd = O.moe_forward_dense(L, spec.top_k)
    rel, mx = O.parity_errors(y, yd)
    assert rel <= 1e-12 and mx <= 1e-12


def test_dense_matches_float64_loops_on_one_token():
    # Scalar loops over one token, against the oracle's vectorised path.
    L, spec = _tiny(0, T=3, H=32, I=32, E=3)
    y = O.moe_forward(L, spec.top_k)
    x = O.bf16_decode(L["x"])
    ids, w = O.route(L["router_logits"], spec.top_k)
    t = 1
    acc = np.zeros(spec.H)
    for j in range(spec.top_k):
        e = ids[t, j]
        W13 = O.dequantize_f64(L["w13_blocks"][e], L["w13_scales"][e])
        b13 = O.bf16_decode(L["w13_bias"][e])
        W2 = O.dequantize_f64(L["w2_blocks"][e], L["w2_scales"][e])
        b2 = O.bf16_decode(L["w2_bias"][e])
        a = np.zeros(spec.I)
        for i in range(spec.I):
            hg = sum(W13[2 * i, c] * x[t, c] for c in range(spec.H)) + b13[2 * i]
            hu = sum(W13[2 * i + 1, c] * x[t, c] for c in range(spec.H)) + b13[2 * i + 1]
            a[i] = O.swiglu_clamped(hg, hu)
        for n in range(spec.H):
            acc[n] += w[t, j] * (sum(W2[n, i] * a[i] for i in range(spec.I)) + b2[n])
    assert np.allclose(acc, y[t], rtol=1e-12, atol=1e-9)


def test_zero_down_weights_give_weighted_down_bias():
    # All w2 codes zero: z = b2 exactly, so y_t = sum_j w_tj * b2[e_tj]; a
    # down bias added after the routing weight would give sum_j b2 instead.
    L, spec = _tiny(0)
    L["w2_blocks"][:] = 0
    y = O.moe_forward(L, spec.top_k)
    ids, w = O.route(L["router_logits"], spec.top_k)
    b2 = O.bf16_decode(L["w2_bias"])
    ref = (w[:, :, None] * b2[ids]).sum(1)
    assert np.allclose(y, ref, rtol=1e-14, atol=0)


def test_one_hot_weights_closed_form():
    # W13 row n holds code 0x2 (1.0) at column pi(n), W2 row m at column sig(m):
    # the GEMMs become gathers, which fixes orientation, interleave and biases.
    rng = np.random.default_rng(11)
    L, spec = _tiny(0, T=5, H=64, I=32, E=3)
    E, H, I = spec.E, spec.H, spec.I
    pi = rng.integers(0, H, size=(E, 2 * I))
    sg = rng.integers(0, I, size=(E, H))
    L["w13_blocks"][:] = 0
    L["w2_blocks"][:] = 0
    for e in range(E):
        for n in range(2 * I):
            c = pi[e, n]
            L["w13_blocks"][e, n, c // 2] |= np.uint8(0x2 << (4 * (c % 2)))
        for m in range(H):
            c = sg[e, m]
            L["w2_blocks"][e, m, c // 2] |= np.uint8(0x2 << (4 * (c % 2)))
    y = O.moe_forward(L, spec.top_k)
    x = O.bf16_decode(L["x"])
    ids, w = O.route(L["router_logits"], spec.top_k)
    ref = np.zeros((spec.T, H))
    for t in range(spec.T):
        for j in range(spec.top_k):
            e = ids[t, j]
            s13 = 2.0 ** (L["w13_scales"][e].astype(np.int64) - 127)  # [2I, H/32]
            h = np.array([x[t, pi[e, n]] * s13[n, pi[e, n] // 32] for n in range(2 * I)])
            h = h + O.bf16_decode(L["w13_bias"][e])
            a = O.swiglu_clamped(h[0::2], h[1::2])  # even rows gate, odd rows up
            s2 = 2.0 ** (L["w2_scales"][e].astype(np.int64) - 127)
            z = np.array([a[sg[e, m]] * s2[m, sg[e, m] // 32] for m in range(H)])
            ref[t] += w[t, j] * (z + O.bf16_decode(L["w2_bias"][e]))
    assert np.allclose(y, ref, rtol=1e-13, atol=1e-13)


def test_bias_after_scale_identity():
    # All w2 scale bytes = c: z(c) = 2^(c-127) * z(127, b2=0) + b2 exactly
    # (power-of-two scaling commutes with rounding when nothing over- or underflows).
    L, spec = _tiny(0, I=64, H=64, scale_lo=112, scale_hi=120, bias_std=1.0)
    c = 120
    Lc = {k: v.copy() for k, v in L.items()}
    Lc["w2_scales"][:] = c
    L0 = {k: v.copy() for k, v in L.items()}
    L0["w2_scales"][:] = 127
    L0["w2_bias"][:] = 0
    yc = O.moe_forward(Lc, spec.top_k)
    ids, w = O.route(L["router_logits"], spec.top_k)
    x = O.bf16_decode(L["x"])
    ref = np.zeros_like(yc)
    for t in range(spec.T):
        for j in range(spec.top_k):
            e = ids[t, j]
            z0 = O.expert_ffn(x[t:t + 1], L0["w13_blocks"][e], L0["w13_scales"][e], L0["w13_bias"][e],
                              L0["w2_blocks"][e], L0["w2_scales"][e], L0["w2_bias"][e])[0]
            ref[t] += w[t, j] * (2.0 ** (c - 127) * z0 + O.bf16_decode(L["w2_bias"][e]))
    assert np.array_equal(yc, ref) or O.parity_errors(yc, ref)[0] <= 1e-15
    # the scaled-bias variant sum w*s*(z0 + b) must miss the 1e-2 bar by >= 10x
    bad = np.zeros_like(yc)
    for t in range(spec.T):
        for j in range(spec.top_k):
            e = ids[t, j]
            z0 = O.expert_ffn(x[t:t + 1], L0["w13_blocks"][e], L0["w13_scales"][e], L0["w13_bias"][e],
                              L0["w2_blocks"][e], L0["w2_scales"][e], L0["w2_bias"][e])[0]
            bad[t] += w[t, j] * 2.0 ** (c - 127) * (z0 + O.bf16_decode(L["w2_bias"][e]))
    assert O.parity_errors(bad, yc)[0] >= 0.1


# ------------------------------------------------------- non-vacuity controls

def _variant_forward(L, k, defect):
    """The oracle with one planted defect (CPU only), for the non-vacuity checks."""
    x = O.bf16_decode(L["x"])
    lg = L["router_logits"].astype(np.float64)
    ids, w = O.route(L["router_logits"], k)
    if defect == "no_softmax":
        w = np.take_along_axis(lg, ids, axis=1)
    T, H = x.shape
    y = np.zeros((T, H))

    def deq(b, s):
        if defect == "high_nibble_first":
            b = ((b & 0x0F) << 4) | (b >> 4)
        if defect == "e8m0_bias_128":
            return O.dequantize_f64(b, s) / 2.0
        return O.dequantize_f64(b, s)

    for t in range(T):
        for j in range(k):
            e = ids[t, j]
            xin = x[t] * (w[t, j] if defect == "weight_on_input" else 1.0)
            W13 = deq(L["w13_blocks"][e], L["w13_scales"][e])
            h = W13 @ xin + O.bf16_decode(L["w13_bias"][e])
            gate, up = h[0::2], h[1::2]
            if defect == "gate_up_swap":
                gate, up = up, gate
            if defect == "no_clamp":
                a = gate * expit(1.702 * gate) * (up + 1)
            else:
                a = O.swiglu_clamped(gate, up)
            W2 = deq(L["w2_blocks"][e], L["w2_scales"][e])
            b2 = O.bf16_decode(L["w2_bias"][e])
            z = W2 @ a
            if defect != "no_bias":
                z = z + b2
            y[t] += z if defect == "weight_on_input" else w[t, j] * z
    return y


@pytest.mark.parametrize("defect,case", [
    ("high_nibble_first", "live"), ("e8m0_bias_128", "live"), ("gate_up_swap", "live"),
    ("no_clamp", "saturated"), ("no_softmax", "live"), ("weight_on_input", "live"),
    ("no_bias", "live")])
def test_planted_defects_fail_parity(defect, case):
    # "live": small scales keep the SwiGLU unsaturated and the biases significant;
    # "saturated": the gpt-oss-shaped scale range [118,132], where the clamps bite.
    base = W.LAYERS["20b_live"] if case == "live" else W.LAYERS["20b_decode"]
    spec = base.with_(H=256, I=256, E=8, T=6)
    L = W.make_layer(spec)
    ref = O.moe_forward(L, spec.top_k)
    assert O.parity_errors(_variant_forward(L, spec.top_k, "none"), ref)[0] <= 1e-12
    rel, _ = O.parity_errors(_variant_forward(L, spec.top_k, defect), ref)
    assert rel > 1e-2, (defect, rel)


# ---------------------------------------------------------------- NVFP4 variant

def test_e4m3_matches_torch_float8():
    # FP8 E4M3 (OCP, finite-only): an independent decoder is torch's float8_e4m3fn.
    import torch

    b = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(b).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    got = O.e4m3_value(b)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert O.e4m3_value(0x7E) == 448.0 and O.e4m3_value(0x38) == 1.0 and O.e4m3_value(0x01) == 2.0 ** -9


def test_nvfp4_block_axis_and_nibble_order():
    # one row of 64 elements: codes 2 (1.0) everywhere except element 17 (high
    # nibble of byte 8) = code 7 (6.0); four 16-element blocks with scales 1, 2, 4, 0.5
    blocks = np.full((1, 32), 0x22, np.uint8)
    blocks[0, 8] = 0x72
    scales = np.array([[0x38, 0x40, 0x48, 0x30]], np.uint8)
    got = O.nvfp4_dequantize_f64(blocks, scales)[0]
    want = np.repeat([1.0, 2.0, 4.0, 0.5], 16)
    want[17] = 6.0 * 2.0
    assert np.array_equal(got, want)


def _nvfp4_small_layer(T=5, H=64, I=32, E=3, k=2, seed=3, bias_std=0.5, scale_lo=0x30, scale_hi=0x48):
    spec = W.LAYERS["20b_live"].with_(T=T, H=H, I=I, E=E, top_k=k, bias_std=bias_std)
    return W.make_nvfp4_layer(spec, seed=seed, scale_lo=scale_lo, scale_hi=scale_hi), k


def test_nvfp4_expert_against_scalar_loops():
    L, k = _nvfp4_small_layer()
    e, t = 1, 2
    x = O.bf16_decode(L["x"][t])
    codes13 = O.unpack_codes(L["w13_blocks"][e])
    codes2 = O.unpack_codes(L["w2_blocks"][e])
    H = x.shape[0]
    I = codes2.shape[1]
    s13 = float(L["w13_scale2"][e])
    s2 = float(L["w2_scale2"][e])
    h = []
    for r in range(2 * I):
        acc = 0.0
        for kk in range(H):
            acc += x[kk] * O.E2M1_VALUES[codes13[r, kk]] * float(O.e4m3_value(L["w13_scales"][e][r, kk // 16]))
        h.append(s13 * acc + float(O.bf16_decode(L["w13_bias"][e][r])))
    a = [float(O.swiglu_clamped(h[2 * i], h[2 * i + 1])) for i in range(I)]
    z = []
    for n in range(H):
        acc = 0.0
        for i in range(I):
            acc += a[i] * O.E2M1_VALUES[codes2[n, i]] * float(O.e4m3_value(L["w2_scales"][e][n, i // 16]))
        z.append(s2 * acc + float(O.bf16_decode(L["w2_bias"][e][n])))
    got = O.expert_ffn_nvfp4(x[None, :], L["w13_blocks"][e], L["w13_scales"][e], L["w13_scale2"][e],
                             L["w13_bias"][e], L["w2_blocks"][e], L["w2_scales"][e], L["w2_scale2"][e],
                             L["w2_bias"][e])[0]
    assert np.allclose(got, z, rtol=1e-12, atol=1e-12)


def test_nvfp4_bias_after_second_level_scale():
    # z(s2 = c) = c * z(s2 = 1, b2 = 0) + b2 exactly for a power-of-two c; folding
    # the scale into the routing weight ahead of the bias (sum w*s*(y + b)) must
    # miss the parity bar by far.
    # small block scales and large biases: the bias is a large part of z
    L, k = _nvfp4_small_layer(T=8, H=128, I=64, E=4, k=2, seed=9, bias_std=2.0, scale_lo=0x18, scale_hi=0x20)
    c = 0.125
    L["w2_scale2"][:] = c
    ref = O.moe_forward_nvfp4(L, k)
    L1 = dict(L, w2_scale2=np.ones_like(L["w2_scale2"]), w2_bias=np.zeros_like(L["w2_bias"]))
    y1 = O.moe_forward_nvfp4(L1, k)
    ids, w = O.route(L["router_logits"], k)
    b2 = O.bf16_decode(L["w2_bias"])
    ident = c * y1 + sum(w[:, j:j + 1] * b2[ids[:, j]] for j in range(k))
    assert np.allclose(ident, ref, rtol=1e-13, atol=1e-13)
    folded = c * (y1 + sum(w[:, j:j + 1] * b2[ids[:, j]] for j in range(k)))  # sum w*s*(y + b)
    assert O.parity_errors(folded, ref)[0] > 10 * 1e-2


# ---------------------------------------------------------------- router projection

def _router_case(T, H, E, seed):
    rng = np.random.default_rng(seed)
    x = W.to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
    w = W.to_bf16_bits(rng.standard_normal((E, H), dtype=np.float32) / np.float32(np.sqrt(H)))
    b = W.to_bf16_bits(rng.standard_normal(E, dtype=np.float32))
    return x, w, b


def test_router_logits_against_torch_linear():
    # A linear layer with a bias: torch.nn.functional.linear in float64.
    x, w, b = _router_case(37, 96, 12, 1)
    ref = torch.nn.functional.linear(torch.from_numpy(O.bf16_decode(x)), torch.from_numpy(O.bf16_decode(w)),
                                     torch.from_numpy(O.bf16_decode(b))).numpy()
    np.testing.assert_allclose(O.router_logits(x, w, b), ref, rtol=1e-12, atol=1e-12)


def test_router_logits_one_hot_rows_pick_weight_columns():
    # Square case (E == H) so that a transposed W_r would pass a shape check:
    # x = e_h gives logits = W_r[:, h] + b_r.
    H = E = 16
    _, w, b = _router_case(1, H, E, 2)
    one = W.to_bf16_bits(np.eye(H, dtype=np.float32))
    got = O.router_logits(one, w, b)
    wd, bd = O.bf16_decode(w), O.bf16_decode(b)
    for h in range(H):
        assert np.array_equal(got[h], wd[:, h] + bd)


def test_router_logits_zero_weights_give_bias_on_every_token():
    x, w, b = _router_case(5, 64, 7, 3)
    w0 = np.zeros_like(w)
    got = O.router_logits(x, w0, b)
    assert np.array_equal(got, np.broadcast_to(O.bf16_decode(b), (5, 7)))


def test_moe_forward_router_dominant_bias_is_one_expert():
    # A router bias of +64 on expert 2 sends every token there first; with
    # top_k = 1 the layer is that expert's FFN with weight 1 (closed form).
    spec = W.LAYERS["tiny"].with_(T=8, E=4, top_k=1)
    L = dict(W.make_layer(spec), **W.make_router(spec))
    bias = O.bf16_decode(L["router_b"]).astype(np.float32)
    bias[2] = 64.0
    L["router_b"] = W.to_bf16_bits(bias)
    y = O.moe_forward_router(L, 1)
    z = O.expert_ffn(O.bf16_decode(L["x"]), L["w13_blocks"][2], L["w13_scales"][2], L["w13_bias"][2],
                     L["w2_blocks"][2], L["w2_scales"][2], L["w2_bias"][2])
    np.testing.assert_allclose(y, z, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- MXFP8 activations (FP4 scaled-MFMA path)

def test_e4m3_encode_round_trips_every_code():
    codes = np.arange(256, dtype=np.uint8)
    codes = codes[(codes & 0x7F) != 0x7F]  # not NaN
    assert np.array_equal(O.e4m3_encode_rne(O.e4m3_value(codes)), codes)


def test_e4m3_encode_matches_torch_incl_ties():
    rng = np.random.default_rng(3)
    v = np.concatenate([rng.uniform(-448, 448, 20000), rng.uniform(-2 ** -5, 2 ** -5, 20000)])
    # every midpoint between adjacent positive codes: ties go to the even code
    pos = O.e4m3_value(np.arange(0, 0x7E, dtype=np.uint8))
    mids = (pos[:-1] + pos[1:]) / 2
    v = np.concatenate([v, mids, -mids])
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.e4m3_encode_rne(v), ref)
    got = O.e4m3_encode_rne(mids)
    assert np.all(got % 2 == 0)  # even mantissa at every tie


def test_mxfp8_scale_rule():
    # max|block| = 1 -> shared exponent -7 (byte 120); 3 -> -6 (121); zeros -> 127
    v = np.zeros((3, 32))
    v[0, 5] = 1.0
    v[1, :] = np.linspace(-3.0, 3.0, 32)
    codes, scales = O.mxfp8_quantize(v)
    assert list(scales) == [120, 121, 127]
    assert np.all(codes[2] == 0)
    scaled = O.e4m3_value(codes[:2])
    assert np.abs(scaled).max(axis=1).tolist() == [128.0, 192.0]  # 1 * 2^7, 3 * 2^6


def test_mxfp8_split_error_bound_and_exact_cases():
    rng = np.random.default_rng(4)
    v = O.bf16_decode(W.to_bf16_bits(rng.standard_normal((64, 256)).astype(np.float32)))
    q = O.mxfp8_activations(v, "split")
    amax = np.repeat(np.abs(v.reshape(64, 8, 32)).max(axis=-1), 32, axis=-1)
    assert np.all(np.abs(v - q) <= 2.0 ** -8 * amax)
    # values with at most four significant bits inside a block's range need no residual
    codes = rng.integers(0x30, 0x50, size=(4, 64)).astype(np.uint8)
    w = O.e4m3_value(codes) * 2.0 ** -3
    assert np.array_equal(O.mxfp8_activations(w, "split"), w)
    assert np.array_equal(O.mxfp8_activations(w, "single"), w)
    # a single MXFP8 tensor is coarser than the split
    e1 = np.abs(v - O.mxfp8_activations(v, "single")).max()
    assert e1 > 4 * np.abs(v - q).max()


def _mxfp8_blocks_scalar(v, mode):
    """Plain loops over blocks of 32: shared scale 2^(floor(log2 max|v|) - 7) (the
    implementation's rule: the block maximum lands in [128, 256), E4M3's top
    binade but one; the OCP rule would subtract emax = 8), elements rounded to
    E4M3 by torch's float8_e4m3fn; "split" adds the same quantization of the
    residual."""
    def one(vals):
        amax = max(abs(u) for u in vals)
        if amax == 0.0:
            return [0.0] * len(vals)
        s = 2.0 ** (math.floor(math.log2(amax)) - 7)
        enc = torch.tensor([u / s for u in vals], dtype=torch.float32).to(torch.float8_e4m3fn)
        return [float(c) * s for c in enc.to(torch.float64)]

    out = []
    for b0 in range(0, len(v), 32):
        blk = [float(u) for u in v[b0:b0 + 32]]
        hi = one(blk)
        if mode == "split":
            hi = [h + r for h, r in zip(hi, one([u - h for u, h in zip(blk, hi)]))]
        out += hi
    return out


@pytest.mark.parametrize("mode", ["split", "single"])
def test_fp8act_forward_matches_scalar_loops_on_one_token(mode):
    # The FP4 scaled-MFMA path's oracle (moe_forward_fp8act) against scalar
    # loops with their own quantizer, on a layer where one of the three experts
    # keeps exact activations: x quantized per 32-block before the gate_up
    # GEMM, the SwiGLU output rounded to bf16 (torch) and quantized before the
    # down GEMM, exact experts untouched.
    L, spec = _tiny(5, T=3, H=64, I=32, E=3)
    quantized = np.array([True, False, True])
    y = O.moe_forward_fp8act(L, spec.top_k, quantized, mode)
    x = O.bf16_decode(L["x"])
    ids, w = O.route(L["router_logits"], spec.top_k)
    t = 1
    acc = np.zeros(spec.H)
    for j in range(spec.top_k):
        e = ids[t, j]
        W13 = O.dequantize_f64(L["w13_blocks"][e], L["w13_scales"][e])
        b13 = O.bf16_decode(L["w13_bias"][e])
        W2 = O.dequantize_f64(L["w2_blocks"][e], L["w2_scales"][e])
        b2 = O.bf16_decode(L["w2_bias"][e])
        xq = _mxfp8_blocks_scalar(x[t], mode) if quantized[e] else list(x[t])
        a = []
        for i in range(spec.I):
            hg = sum(W13[2 * i, c] * xq[c] for c in range(spec.H)) + b13[2 * i]
            hu = sum(W13[2 * i + 1, c] * xq[c] for c in range(spec.H)) + b13[2 * i + 1]
            a.append(float(O.swiglu_clamped(hg, hu)))
        if quantized[e]:
            a = torch.tensor(a, dtype=torch.float32).to(torch.bfloat16).to(torch.float64).tolist()
            a = _mxfp8_blocks_scalar(a, mode)
        for n in range(spec.H):
            acc[n] += w[t, j] * (sum(W2[n, i] * a[i] for i in range(spec.I)) + b2[n])
    assert np.allclose(acc, y[t], rtol=1e-12, atol=1e-9)
    # the quantized experts really differ from the exact layer here
    assert not np.allclose(y[t], O.moe_forward(L, spec.top_k)[t], rtol=1e-6, atol=0)


# ---------------------------------------------------------------- the acceptance measure

def test_parity_errors_hand_computed():
    # ||y - y_ref||_2 / ||y_ref||_2 and max|y - y_ref| / max|y_ref|, worked by hand.
    rel, mx = O.parity_errors(np.array([3.0, 4.5]), np.array([3.0, 4.0]))
    assert rel == pytest.approx(0.5 / 5.0, abs=1e-15)        # ||(0, .5)|| / ||(3, 4)||
    assert mx == pytest.approx(0.5 / 4.0, abs=1e-15)
    # the max-element error is relative to max|y_ref| (2), not max|y| (5)
    rel, mx = O.parity_errors(np.array([1.0, -5.0]), np.array([1.0, -2.0]))
    assert rel == pytest.approx(3.0 / math.sqrt(5.0), abs=1e-15)
    assert mx == pytest.approx(1.5, abs=1e-15)
    # the norms run over every element of a 2-D output, not a row or a column
    rel, mx = O.parity_errors(np.array([[1.0, 0.0], [0.0, 2.0]]), np.array([[1.0, 0.0], [0.0, 1.0]]))
    assert rel == pytest.approx(1.0 / math.sqrt(2.0), abs=1e-15)
    assert mx == pytest.approx(1.0, abs=1e-15)
    rel, mx = O.parity_errors(np.array([[2.0, 0.0], [0.0, 0.0]]), np.array([[1.0, 0.0], [0.0, 3.0]]))
    assert rel == pytest.approx(math.sqrt(10.0) / math.sqrt(10.0), abs=1e-15)  # ||(1, -3)|| / ||(1, 3)||
    assert mx == pytest.approx(3.0 / 3.0, abs=1e-15)
    # a sign flip is off by 2 in both measures; equal inputs by 0
    rel, mx = O.parity_errors(-np.array([0.25, -8.0, 1.0]), np.array([0.25, -8.0, 1.0]))
    assert (rel, mx) == (pytest.approx(2.0, abs=1e-15), pytest.approx(2.0, abs=1e-15))
    assert O.parity_errors(np.arange(6.0), np.arange(6.0)) == (0.0, 0.0)
    # differences below float32 resolution still count (float64 arithmetic)
    rel, _ = O.parity_errors(np.array([1.0 + 2.0 ** -40]), np.array([1.0]))
    assert rel == 2.0 ** -40


# ---------------------------------------------------------------- E8M0 0xFF inside the layer

def test_nan_scale_byte_poisons_exactly_the_rows_it_reaches():
    # A 0xFF scale byte makes its 32 weights NaN (OCP MX).  In gate_up row r of
    # expert e every h[:, r] of e's tokens is NaN, so their whole activation,
    # down output and routed output rows are NaN; in down row n only column n
    # of the outputs of that expert's tokens.  Every other element stays finite.
    L, spec = _tiny(7, T=12, H=64, I=64, E=4)
    k = spec.top_k
    ids, _ = O.route(L["router_logits"], k)
    e_up, e_down, n_bad = 1, 2, 37
    L["w13_scales"] = L["w13_scales"].copy()
    L["w2_scales"] = L["w2_scales"].copy()
    L["w13_scales"][e_up, 5, 1] = 255
    L["w2_scales"][e_down, n_bad, 0] = 255
    y = O.moe_forward(L, k)
    hit_up = (ids == e_up).any(axis=1)
    hit_down = (ids == e_down).any(axis=1)
    assert hit_up.any() and (~hit_up).any() and (hit_down & ~hit_up).any()
    expect = np.zeros(y.shape, dtype=bool)
    expect[hit_up, :] = True
    expect[hit_down, n_bad] = True
    assert np.array_equal(np.isnan(y), expect)
    # every element the bad bytes cannot reach is the clean layer's, bit for bit
    clean = O.moe_forward(_tiny(7, T=12, H=64, I=64, E=4)[0], k)
    assert np.array_equal(y[~expect], clean[~expect])


# ---------------------------------------------------------------- MXFP8 codes worked by hand

def test_mxfp8_quantize_hand_derived_codes():
    # This implementation's rule (not the OCP emax rule): shared exponent
    # floor(log2 max|v|) - 7.  Block max 3.0 -> exponent 1 - 7 = -6, byte 121.
    #   3.0 / 2^-6 = 192 = 1.5 * 2^7     -> E4M3 exponent field 14, mantissa 4: 0x74
    #   0.1 / 2^-6 = 6.4 = 1.6 * 2^2     -> mantissa 4.8 rounds to 5: 0x4D (value 6.5)
    #  -0.5 / 2^-6 = -32 = -1.0 * 2^5    -> 0x80 | (12 << 3): 0xE0
    #   2^-16 / 2^-6 = 2^-10 < 2^-9 / 2  -> rounds to zero: 0x00
    #   0.0703125 / 2^-6 = 4.5 = 1.125*4 -> mantissa 1: 0x49
    #   0.0546875 / 2^-6 = 3.5 = 1.75*2  -> mantissa 6: 0x46
    v = np.zeros((1, 32))
    v[0, :6] = [3.0, 0.1, -0.5, 2.0 ** -16, 0.0703125, 0.0546875]
    codes, scales = O.mxfp8_quantize(v)
    assert scales.tolist() == [[121]]
    assert codes[0, :6].tolist() == [0x74, 0x4D, 0xE0, 0x00, 0x49, 0x46]
    assert np.all(codes[0, 6:] == 0)
    # a tie: 0.06640625 / 2^-6 = 4.25, halfway between 4 (mantissa 0) and 4.5
    # (mantissa 1): ties to even -> 0x48; 4.75 halfway between 4.5 and 5 -> 5 (0x4A)
    v[0, 1:3] = [0.06640625, 0.07421875]
    codes, _ = O.mxfp8_quantize(v)
    assert codes[0, 1:3].tolist() == [0x48, 0x4A]
