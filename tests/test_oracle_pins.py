"""Pins of the CPU oracle against what the pages and the mathematics fix.

Nothing here compares the oracle with itself: every expected value comes from
a closed form, a hand-worked fixture under tests/golden/, an independent
library routine (numpy float64 / int64 matmul, torch's BF16 rounding), brute
force in float64, or an invariant the method guarantees.
"""
import math

import numpy as np
import pytest

from conftest import read_golden
from swiglu_mlp_amd import workloads as W

f32 = np.float32


def sylvester_kron(g):
    """Unnormalised Sylvester matrix built by the Kronecker recursion
    H_{2n} = [[H_n, H_n], [H_n, -H_n]] (a construction independent of the
    popcount closed form the oracle uses)."""
    h = np.array([[1]], dtype=np.int64)
    h2 = np.array([[1, 1], [1, -1]], dtype=np.int64)
    while h.shape[0] < g:
        h = np.kron(h2, h)
    return h


def ulp32(x):
    return np.spacing(np.abs(np.asarray(x, dtype=np.float32))).astype(np.float64)


# ---------------------------------------------------------------------------
# Rotation: H and the FWHT
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("g", [1, 2, 4, 8, 16, 32, 64, 128, 256])
def test_hadamard_closed_form(orc, g):
    h = orc.hadamard(g)
    np.testing.assert_array_equal(h, h.T)                         # symmetric
    np.testing.assert_allclose(h @ h.T, np.eye(g), atol=1e-12)    # orthogonal
    np.testing.assert_allclose(np.abs(h), 1 / math.sqrt(g), rtol=1e-15)
    np.testing.assert_allclose(h * math.sqrt(g), sylvester_kron(g), rtol=1e-15)
    if g == 2:
        np.testing.assert_allclose(h, np.array([[1, 1], [1, -1]]) / math.sqrt(2))


def test_hadamard_rejects_non_power_of_two(orc):
    with pytest.raises(ValueError):
        orc.hadamard(96)


@pytest.mark.parametrize("g", [1, 2, 4, 8, 16, 32, 64, 128, 256])
def test_norm_const_is_rounded_inverse_sqrt(orc, g):
    from fractions import Fraction
    c = orc.norm_const(g)
    # |c - 1/sqrt(g)| <= half an ulp, checked with exact rationals (c^2 g vs 1)
    lo = Fraction(float(c) - float(ulp32(c)) / 2)
    hi = Fraction(float(c) + float(ulp32(c)) / 2)
    assert lo * lo * g <= 1 <= hi * hi * g


@pytest.mark.parametrize("g", [2, 8, 64, 128, 256])
def test_fwht_matches_dense_float64(orc, g):
    rng = np.random.default_rng(1)
    x = rng.standard_normal((7, 3 * g)).astype(np.float32)
    u = orc.fwht(x, g)
    hk = sylvester_kron(g).astype(np.float64)
    ref = np.concatenate([x[:, j * g:(j + 1) * g].astype(np.float64) @ hk
                          for j in range(3)], axis=1)
    err = np.linalg.norm(u - ref, axis=1) / np.linalg.norm(ref, axis=1)
    assert err.max() < 1e-6


@pytest.mark.parametrize("g", [4, 32, 128, 256])
def test_fwht_exact_on_small_integers(orc, g):
    """With small integer inputs every FP32 sum is exact, so the transform must
    equal the integer matrix product bit for bit (catches a wrong sign, a
    dropped stage or a mis-indexed butterfly)."""
    rng = np.random.default_rng(2)
    x = rng.integers(-8, 9, size=(5, 2 * g))
    u = orc.fwht(x.astype(np.float32), g)
    hk = sylvester_kron(g)
    ref = np.concatenate([x[:, j * g:(j + 1) * g] @ hk for j in range(2)], axis=1)
    np.testing.assert_array_equal(u, ref.astype(np.float32))


def test_fwht_stage_order_golden(orc):
    rows = read_golden("fwht_order_g4.txt")
    g = int(rows[0][0])
    x = np.array([float.fromhex(t) for t in rows[1]], dtype=np.float32)
    want = np.array([float.fromhex(t) for t in rows[2]], dtype=np.float32)
    np.testing.assert_array_equal(orc.fwht(x, g), want)


def test_single_outlier_closed_form(orc):
    rows = read_golden("single_outlier_g128.txt")
    g, j, a = int(rows[0][0]), int(rows[1][0]), float(rows[2][0])
    s_want = float.fromhex(rows[3][0])
    codes_want = np.array([int(t) for t in rows[4]], dtype=np.int8)
    x = np.zeros((1, 3 * g), dtype=np.float32)
    x[0, g + j] = a                       # outlier in the middle group
    xb = W.to_bf16_bits(x)
    q, s = orc.act_quant(xb, 0, g)
    np.testing.assert_array_equal(q[0, g:2 * g], codes_want)
    assert not q[0, :g].any() and not q[0, 2 * g:].any()
    assert float(s[0]) == s_want
    assert abs(float(s[0]) - a / (math.sqrt(g) * 127)) <= float(ulp32(s[0]))


# ---------------------------------------------------------------------------
# Pinned elementary functions (exhaustive where the domain is small)
# ---------------------------------------------------------------------------
def all_bf16_finite():
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    f = (b.astype(np.uint32) << 16).view(np.float32)
    keep = np.isfinite(f)
    return b[keep], f[keep]


def test_exp_neg_within_2ulp_on_all_bf16_arguments(orc):
    _, f = all_bf16_finite()
    t = f[(f >= -80) & (f <= 80)]
    y = orc.exp_neg(t)
    ref = np.exp(-t.astype(np.float64))
    assert (np.abs(y - ref) / ulp32(ref)).max() <= 2.0


def test_rcp_exhaustive_on_one_binade(orc):
    """All 2^23 values of [1, 2): error <= 1 ulp against 1/d in float64."""
    d = (np.arange(1 << 23, dtype=np.uint32) | np.uint32(127 << 23)).view(np.float32)
    y = orc.rcp(d)
    ref = 1.0 / d.astype(np.float64)
    assert (np.abs(y - ref) / ulp32(ref)).max() <= 1.0


def test_rcp_scales_exactly_across_binades(orc):
    """The seed and Newton steps commute with powers of two, so checking one
    binade covers [1, 2^116]; confirm on samples of other binades."""
    rng = np.random.default_rng(3)
    d = (rng.integers(0, 1 << 23, 4096).astype(np.uint32) | np.uint32(127 << 23)).view(np.float32)
    y = orc.rcp(d)
    for e in (1, 7, 40, 80, 116):
        np.testing.assert_array_equal(orc.rcp(np.ldexp(d, e)), np.ldexp(y, -e))


def test_silu_exhaustive_over_bf16(orc):
    b, f = all_bf16_finite()
    y = orc.silu_bf16(b)
    g = f.astype(np.float64)
    inside = np.abs(g) < 80
    ref = g[inside] / (1 + np.exp(-g[inside]))
    err = np.abs(y[inside] - ref) / np.maximum(ulp32(ref), np.spacing(np.float32(0)))
    assert err.max() <= 4.0
    # for g >= 17, e^{-g} < 2^-24 so 1 + e^{-g} rounds to 1 and silu(g) = g exactly
    big = g >= 17
    np.testing.assert_array_equal(y[big], f[big])
    neg = g <= -80
    s80 = orc.silu_bf16(np.array([0xC2A0], dtype=np.uint16))[0]     # silu(-80)
    assert -2e-33 < s80 < 0 and np.all(y[neg] == s80)
    assert orc.silu_bf16(np.array([0, 0x8000], dtype=np.uint16)).tolist() == [0.0, 0.0]


# ---------------------------------------------------------------------------
# Quantizer
# ---------------------------------------------------------------------------
def test_quant_ties_golden(orc):
    rows = read_golden("quant_ties_g1.txt")
    g = int(rows[0][0])
    x = np.array([float.fromhex(t) for t in rows[1]], dtype=np.float32)
    want = np.array([int(t) for t in rows[2]], dtype=np.int8)
    s_want = float.fromhex(rows[3][0])
    q, s = orc.act_quant(W.to_bf16_bits(x[None, :]), 0, g)
    np.testing.assert_array_equal(q[0], want)
    assert float(s[0]) == s_want


@pytest.mark.parametrize("g", [1, 64, 128, 256])
def test_quant_invariants(orc, g):
    rng = np.random.default_rng(4)
    x = rng.standard_normal((64, 4 * 256)).astype(np.float32)
    x[:, [5, 300, 901]] *= 20
    xb = W.to_bf16_bits(x)
    q, s = orc.act_quant(xb, 0, g)
    u = orc.act_rotate(xb, 0, g).astype(np.float64)
    amax = np.abs(u).max(axis=1)
    assert np.all(np.abs(q).max(axis=1) == 127)
    assert q.min() >= -127
    # codes round 127 u / amax to the nearest integer (exact maths, within the
    # rounding of r = 127/amax: |u r - 127 u/amax| < 127 * 2^-23)
    z = 127 * u / amax[:, None]
    assert np.abs(z - q).max() <= 0.5 + 127 * 2.0 ** -23
    # scale = amax(x_rot) / 127 with x_rot = u / sqrt(g)
    s_ref = amax / math.sqrt(g) / 127
    assert np.all(np.abs(s - s_ref) <= 1.5 * ulp32(s_ref))


def test_quant_all_zero_row(orc):
    x = np.zeros((3, 256), dtype=np.uint16)
    x[1, 7] = 0x3F80          # 1.0 in one row only
    q, s = orc.act_quant(x, 0, 128)
    assert s[0] == 0 and s[2] == 0 and not q[0].any() and not q[2].any()
    assert s[1] > 0 and np.abs(q[1]).max() == 127


def test_group_one_is_textbook_w8a8(orc):
    """g = 1: no rotation, so the quantizer is textbook per-token symmetric
    INT8: round(x / (amax/127)).  Codes agree except where 127 x / amax lies
    within 1e-5 of a half-integer (the one rounding of r)."""
    rng = np.random.default_rng(5)
    x = W.to_bf16_bits(rng.standard_normal((32, 512)).astype(np.float32))
    xf = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    q, s = orc.act_quant(x, 0, 1)
    amax = np.abs(xf).max(axis=1, keepdims=True)
    z = xf / (amax / 127)
    ref = np.rint(z)
    near_tie = np.abs(np.abs(z - np.floor(z)) - 0.5) < 1e-5
    assert np.all((q == ref) | near_tie)
    assert near_tie.mean() < 1e-2      # BF16 inputs make exact ties fairly common


def test_divisibility_contract(orc):
    """sglang PR #35994 report: input size must be divisible by the group."""
    with pytest.raises(ValueError):
        orc.weight_prep(np.zeros((4, 192), np.float32), 128)


# ---------------------------------------------------------------------------
# GEMM and epilogue
# ---------------------------------------------------------------------------
def test_gemm_i32_matches_int64_matmul(orc):
    rng = np.random.default_rng(6)
    xq = rng.integers(-127, 128, size=(37, 384), dtype=np.int8)
    wq = rng.integers(-127, 128, size=(53, 384), dtype=np.int8)
    ref = xq.astype(np.int64) @ wq.astype(np.int64).T
    np.testing.assert_array_equal(orc.gemm_i32(xq, wq), ref)


def test_gemm_i32_extremes(orc):
    k = 4096
    xq = np.full((2, k), -127, np.int8)
    wq = np.stack([np.full(k, -127, np.int8), np.full(k, 127, np.int8)])
    np.testing.assert_array_equal(orc.gemm_i32(xq, wq),
                                  [[127 * 127 * k, -127 * 127 * k]] * 2)


def test_bf16_rounding_matches_torch(orc):
    import torch
    rng = np.random.default_rng(7)
    f = np.concatenate([
        rng.standard_normal(100000).astype(np.float32) * 1e3,
        # exact ties between two BF16 values, even and odd low bit
        ((np.arange(256, dtype=np.uint32) << 16) | 0x8000 | (0x3F80 << 16)).view(np.float32),
    ])
    want = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(orc.f32_to_bf16(f), want)


def test_dequant_matches_numpy_float32(orc):
    import torch
    rng = np.random.default_rng(8)
    acc = rng.integers(-(1 << 28), 1 << 28, size=(33, 65), dtype=np.int32)
    sx = (rng.random(33) * 1e-2).astype(np.float32)
    sw = (rng.random(65) * 1e-3).astype(np.float32)
    y32 = (acc.astype(np.float32) * sx[:, None]) * sw[None, :]
    want = torch.from_numpy(y32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(orc.dequant(acc, sx, sw), want)


# ---------------------------------------------------------------------------
# Method-level pins
# ---------------------------------------------------------------------------
def test_rotation_identity_before_quantization(orc):
    """comfy-kitchen PR #277, "The key observation": x W^T = x_rot W_rot^T."""
    rng = np.random.default_rng(9)
    g = 128
    x = rng.standard_normal((16, 512)).astype(np.float32)
    w = (0.02 * rng.standard_normal((48, 512))).astype(np.float32)
    c = orc.norm_const(g)
    xr = orc.fwht(x, g) * c
    wr = orc.fwht(w, g) * c
    y = x.astype(np.float64) @ w.astype(np.float64).T
    y_rot = xr.astype(np.float64) @ wr.astype(np.float64).T
    assert np.linalg.norm(y - y_rot) / np.linalg.norm(y) < 1e-5


def test_row_norm_invariance(orc):
    """sglang PR #35994 report, review notes: the rotation keeps each weight
    row's norm, which the pages use to match rows across checkpoints."""
    rng = np.random.default_rng(10)
    g = 128
    w = (0.02 * rng.standard_normal((64, 1024))).astype(np.float32)
    wr = orc.fwht(w, g).astype(np.float64) * float(orc.norm_const(g))
    n0 = np.linalg.norm(w.astype(np.float64), axis=1)
    assert (np.abs(np.linalg.norm(wr, axis=1) - n0) / n0).max() < 1e-6
    q, s = orc.weight_prep(w, g)
    deq = q.astype(np.float64) * s.astype(np.float64)[:, None]
    assert (np.abs(np.linalg.norm(deq, axis=1) - n0) / n0).max() < 5e-3


def test_brute_force_tiny(orc):
    """Tiny case in float64 with the dense H: codes agree except at near-ties,
    and the BF16 output agrees to BF16 rounding."""
    rng = np.random.default_rng(11)
    g, m, k, n = 8, 6, 32, 10
    x32 = rng.standard_normal((m, k)).astype(np.float32)
    x32[:, 3] *= 20
    xb = W.to_bf16_bits(x32)
    xf = (xb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    w = (0.02 * rng.standard_normal((n, k))).astype(np.float32)
    hd = np.kron(np.eye(k // g), sylvester_kron(g) / math.sqrt(g))

    def quant64(v):
        amax = np.abs(v).max(axis=1, keepdims=True)
        z = 127 * v / amax
        return np.rint(z), (amax / 127)[:, 0], z

    qx_ref, sx_ref, zx = quant64(xf @ hd)
    qw_ref, sw_ref, zw = quant64(w.astype(np.float64) @ hd.T)
    qx, sx = orc.act_quant(xb, 0, g)
    qw, sw = orc.weight_prep(w, g)

    def tie(z):
        return np.abs(np.abs(z - np.floor(z)) - 0.5) < 1e-4
    assert np.all((qx == qx_ref) | tie(zx)) and np.all((qw == qw_ref) | tie(zw))
    np.testing.assert_allclose(sx, sx_ref, rtol=3e-7)
    np.testing.assert_allclose(sw, sw_ref, rtol=3e-7)
    y = orc.int8_linear(xb, 0, qw, sw, g)
    y_ref = (qx.astype(np.float64) @ qw.astype(np.float64).T) * sx_ref[:, None] * sw_ref[None, :]
    yf = (y.astype(np.uint32) << 16).view(np.float32)
    np.testing.assert_allclose(yf, y_ref, rtol=2 ** -8, atol=1e-30)


def test_packed_gate_up_equals_separate_projections(orc):
    """sglang PR #44196, "Accuracy Tests": the stacked [gate | up] GEMM does
    the same per-column arithmetic as the two separate projections."""
    rng = np.random.default_rng(12)
    g = 128
    xb = W.to_bf16_bits(rng.standard_normal((20, 256)).astype(np.float32))
    wg = (0.02 * rng.standard_normal((64, 256))).astype(np.float32)
    wu = (0.02 * rng.standard_normal((64, 256))).astype(np.float32)
    qg, sg = orc.weight_prep(wg, g)
    qu, su = orc.weight_prep(wu, g)
    qgu, sgu = orc.weight_prep(np.concatenate([wg, wu]), g)
    y = orc.int8_linear(xb, 0, qgu, sgu, g)
    np.testing.assert_array_equal(y[:, :64], orc.int8_linear(xb, 0, qg, sg, g))
    np.testing.assert_array_equal(y[:, 64:], orc.int8_linear(xb, 0, qu, su, g))


def test_accuracy_class_tiny_workload(orc):
    """Relative L2 against the unrotated, unquantized float64 product sits in
    the ~1% class the pages report (0.885% to 1.46%)."""
    w = W.WORKLOADS["c1"]
    d = W.linear_inputs(w)
    qw, sw = orc.weight_prep(d["w"], w.group)
    y = orc.int8_linear(d["x"], 0, qw, sw, w.group)
    e = orc.rel_l2(y, orc.reference_linear_f64(d["x"], 0, d["w"]))
    assert 0.003 < e < 0.03, e


def test_eager_swiglu_golden(orc):
    """sglang PR #44196, "Motivation": the eager path rounds silu(gate) to BF16,
    multiplies by up and rounds the product to BF16 (round-half-even).  The
    golden's values are worked out by hand from the exact silu; cases 1-3 and
    5-6 change if the silu rounding is dropped, case 2 and 5 if the final
    rounding truncates, cases 4-6 if ties do not go to even."""
    rows = read_golden("eager_swiglu_bf16.txt")
    gate = np.array([int(r[0], 16) for r in rows], dtype=np.uint16)
    up = np.array([int(r[1], 16) for r in rows], dtype=np.uint16)
    eager = np.array([int(r[2], 16) for r in rows], dtype=np.uint16)
    once = np.array([int(r[3], 16) for r in rows], dtype=np.uint16)
    # one row [gate | up] per case, k = 1
    x = np.stack([gate, up], axis=1)
    got = orc.eager_swiglu_bf16(x)[:, 0]
    np.testing.assert_array_equal(got, eager)
    # the same cases with silu kept in FP32 (rounded once, after the product)
    fused = orc.f32_to_bf16(orc.silu_bf16(gate) * orc.bf16_to_f32(up))
    np.testing.assert_array_equal(fused, once)
    assert np.count_nonzero(eager != once) == 5


def test_fused_swiglu_not_worse_than_eager(orc):
    """sglang PR #44196, "Accuracy Tests": keeping silu(gate)*up in FP32 is no
    worse against the FP32 reference than rounding it to BF16 first."""
    w = W.WORKLOADS["c2"]
    d = W.linear_inputs(w, m=128)
    qw, sw = orc.weight_prep(d["w"], w.group)
    ref = orc.reference_linear_f64(d["x"], 1, d["w"])
    fused = orc.int8_linear(d["x"], 1, qw, sw, w.group)
    eager_a = orc.eager_swiglu_bf16(d["x"])
    eager = orc.int8_linear(eager_a, 0, qw, sw, w.group)
    e_f, e_e = orc.rel_l2(fused, ref), orc.rel_l2(eager, ref)
    assert 0.003 < e_f < 0.03
    assert e_f <= e_e * 1.02, (e_f, e_e)


# ---------------------------------------------------------------------------
# Epilogue with bias and residual (comfy-kitchen PR #277 "Changes"; PR #248
# commit list).  Reading: one FP32 sum, one BF16 rounding.
# ---------------------------------------------------------------------------
def _bf16_bits_of_exact(v):
    """BF16 bits of float32 values that are exactly representable in BF16."""
    b = np.asarray(v, dtype=np.float32).view(np.uint32)
    assert np.all((b & 0xFFFF) == 0)
    return (b >> 16).astype(np.uint16)


def test_epilogue_closed_form_zero_accumulator(orc):
    # acc = 0: y = bf16(fl(0 + b) + r); integers below 256 are exact in BF16,
    # so the result is the exact integer sum
    rng = np.random.default_rng(5)
    m, n = 7, 32
    acc = np.zeros((m, n), dtype=np.int32)
    b = rng.integers(-100, 100, n).astype(np.float32)
    r = rng.integers(-100, 100, (m, n)).astype(np.float32)
    y = orc.epilogue(acc, np.ones(m, np.float32), np.ones(n, np.float32), b,
                     _bf16_bits_of_exact(r))
    np.testing.assert_array_equal(y, _bf16_bits_of_exact(r + b[None, :]))
    # residual alone passes through bit for bit
    y = orc.epilogue(acc, np.ones(m, np.float32), np.ones(n, np.float32), None,
                     _bf16_bits_of_exact(r))
    np.testing.assert_array_equal(y, _bf16_bits_of_exact(r))


def test_epilogue_without_extras_is_the_dequant(orc):
    rng = np.random.default_rng(6)
    acc = rng.integers(-2**24, 2**24, (9, 48)).astype(np.int32)
    sx = rng.random(9).astype(np.float32)
    sw = rng.random(48).astype(np.float32)
    np.testing.assert_array_equal(orc.epilogue(acc, sx, sw), orc.dequant(acc, sx, sw))


def test_epilogue_error_bound_vs_float64(orc):
    rng = np.random.default_rng(7)
    m, n = 33, 64
    acc = rng.integers(-2**20, 2**20, (m, n)).astype(np.int32)
    sx = (rng.random(m) * 1e-3).astype(np.float32)
    sw = (rng.random(n) * 1e-3).astype(np.float32)
    b = rng.standard_normal(n).astype(np.float32)
    r = orc.f32_to_bf16(rng.standard_normal((m, n)).astype(np.float32))
    y = orc.bf16_to_f32(orc.epilogue(acc, sx, sw, b, r)).astype(np.float64)
    t1 = acc.astype(np.float64) * sx[:, None] * sw[None, :]
    ref = t1 + b[None, :] + orc.bf16_to_f32(r).astype(np.float64)
    # four FP32 roundings (each <= 2^-24 of its operand magnitudes) then one
    # BF16 rounding (half a BF16 ulp: <= 2^-8 of the result)
    bound = 2.0 ** -8 * np.abs(ref) + 4 * 2.0 ** -24 * (np.abs(t1) + np.abs(b)[None, :] +
                                                       np.abs(ref)) + 1e-30
    assert np.all(np.abs(y - ref) <= bound)


# ---------------------------------------------------------------------------
# W8A16 (comfy-kitchen PR #277, "Notes for the reviewer": the rotated
# activation kept in 16-bit floating point, the INT8 weight widened on the fly)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("g", [64, 128, 256])
def test_rotate_bf16_of_a_hadamard_row(orc, g):
    """x = row j of the unnormalised Sylvester matrix (entries +-1, exact in
    BF16) rotates to sqrt(g) e_j: u = g e_j exactly, then fl(g * fl(1/sqrt g))."""
    h = sylvester_kron(g)
    k = 2 * g
    x = np.zeros((3, k), dtype=np.float32)
    js = [0, g // 2 + 1, g - 1]
    for r, j in enumerate(js):
        x[r, g:] = h[j]                      # second group only
    xb = orc.f32_to_bf16(x)
    got = orc.bf16_to_f32(orc.act_rotate_bf16(xb, 0, g))
    want = np.zeros((3, k), dtype=np.float32)
    peak = f32(f32(g) * f32(1.0 / math.sqrt(g)))
    for r, j in enumerate(js):
        want[r, g + j] = orc.bf16_to_f32(orc.f32_to_bf16(np.array([peak], np.float32)))[0]
    np.testing.assert_array_equal(got, want)
    assert abs(float(want[0, g]) - math.sqrt(g)) <= 2 ** -8 * math.sqrt(g)


def test_rotate_bf16_matches_float64_rotation(orc):
    """Against an independent dense rotation: x @ blockdiag(H_g) / sqrt(g) in
    float64 (Kronecker-built H), then within half a BF16 ulp plus the FP32
    transform's rounding."""
    g, m, k = 128, 16, 512
    rng = np.random.default_rng(11)
    xb = orc.f32_to_bf16(rng.standard_normal((m, k)).astype(np.float32))
    x = orc.bf16_to_f32(xb).astype(np.float64)
    hd = sylvester_kron(g).astype(np.float64) / math.sqrt(g)
    ref = (x.reshape(m, k // g, g) @ hd).reshape(m, k)
    got = orc.bf16_to_f32(orc.act_rotate_bf16(xb, 0, g)).astype(np.float64)
    rownorm = np.linalg.norm(x, axis=1, keepdims=True)
    bound = 2.0 ** -8 * np.abs(ref) + 16 * 2.0 ** -24 * rownorm
    assert np.all(np.abs(got - ref) <= bound)


def test_rotated_zeros_are_positive(orc):
    """Reading: x H is defined over the reals, so an exact zero of the rotated
    row is written as +0.  Rows whose every input is -0 (x = -0; SwiGLU with a
    negative gate and up = +0, silu(gate) * up = -0) sum to -0 in the first
    output of each group under IEEE addition; the rotation writes +0 there,
    and leaves a nonzero row's values as they are."""
    g, k = 4, 8
    neg0 = np.full((1, k), 0x8000, dtype=np.uint16)
    gate = orc.f32_to_bf16(np.full((1, k), -1.0, dtype=np.float32))
    up0 = np.zeros((1, k), dtype=np.uint16)
    for xb, act in ((neg0, 0), (np.concatenate([gate, up0], axis=1), 1)):
        u = orc.act_rotate(xb, act, g, k=k)
        np.testing.assert_array_equal(u.view(np.uint32), np.zeros((1, k), np.uint32))
        np.testing.assert_array_equal(orc.act_rotate_bf16(xb, act, g, k=k), np.zeros((1, k), np.uint16))
    # a nonzero row: u = x (sqrt(g) H) exactly for small integers, with +0 where
    # the sums cancel
    x = np.array([[1, 1, 1, 1, 3, -1, 2, 0]], dtype=np.float32)
    u = orc.act_rotate(orc.f32_to_bf16(x), 0, g, k=k)
    want = (x.reshape(2, 4) @ sylvester_kron(4)).reshape(1, k).astype(np.float32)
    np.testing.assert_array_equal(u, want)
    assert not np.signbit(u[0, 1:4]).any() and u[0, 1] == 0


def test_w8a16_acc_matches_int64_matmul(orc):
    """Small integer activations (exact in BF16): the accumulator is the
    integer product, computed by numpy int64 matmul."""
    rng = np.random.default_rng(12)
    xi = rng.integers(-64, 65, (7, 192))
    q = rng.integers(-127, 128, (40, 192)).astype(np.int8)
    xb = orc.f32_to_bf16(xi.astype(np.float32))
    np.testing.assert_array_equal(orc.w8a16_acc(xb, q), (xi @ q.astype(np.int64).T).astype(np.float64))


def test_w8a16_linear_closed_form_on_hadamard_rows(orc):
    """x = Sylvester row j of one group, g = 256: x_rot = 16 e_j exactly, so
    y[n] = bf16(f32(16 q[n, j] s_w[n])): checks the rotation index, the
    orientation of the product and the per-row scale."""
    g, k, n = 256, 512, 48
    rng = np.random.default_rng(13)
    w = (0.02 * rng.standard_normal((n, k))).astype(np.float32)
    q, sw = orc.weight_prep(w, g)
    h = sylvester_kron(g)
    j = 37
    x = np.zeros((1, k), dtype=np.float32)
    x[0, :g] = h[j]
    y = orc.w8a16_linear(orc.f32_to_bf16(x), 0, q, sw, g)
    want = orc.f32_to_bf16((16.0 * q[:, j].astype(np.float64) * sw.astype(np.float64)).astype(np.float32))
    np.testing.assert_array_equal(y[0], want)


def test_w8a16_more_accurate_than_int8(orc):
    """Keeping the activation in 16 bits leaves only the weight's INT8 error
    (~0.75% relative for Gaussian rows: step absmax/127 ~ 3.3 sigma / 127,
    rms step/sqrt(12)) plus BF16 rounding, below the INT8 path's combined
    activation and weight error."""
    w = W.WORKLOADS["c1"]
    d = W.linear_inputs(w)
    qw, sw = orc.weight_prep(d["w"], w.group)
    ref = orc.reference_linear_f64(d["x"], 0, d["w"])
    e16 = orc.rel_l2(orc.w8a16_linear(d["x"], 0, qw, sw, w.group), ref)
    e8 = orc.rel_l2(orc.int8_linear(d["x"], 0, qw, sw, w.group), ref)
    assert 0.002 < e16 < 0.012, e16
    assert e16 < e8, (e16, e8)


def test_w8a16_epilogue_order(orc):
    """bias then residual in FP32, one BF16 rounding; integers stay exact."""
    acc = np.array([[3.0, -5.0, 0.0, 200.0]])
    sw = np.array([2.0, 0.5, 1.0, 0.25], np.float32)
    b = np.array([1.0, 0.5, -3.0, 0.0], np.float32)
    r = orc.f32_to_bf16(np.array([[10.0, -1.0, 4.0, -50.0]], np.float32))
    y = orc.bf16_to_f32(orc.w8a16_epilogue(acc, sw, b, r))
    np.testing.assert_array_equal(y, np.array([[17.0, -3.0, 1.0, 0.0]], np.float32))


def test_w8a16_swiglu_input_and_mlp_accuracy(orc):
    """The fused SwiGLU input of the W8A16 linear and the W8A16 MLP block sit
    closer to the float64 product than their INT8 counterparts."""
    w = W.WORKLOADS["c2"]
    d = W.linear_inputs(w, m=64)
    qw, sw = orc.weight_prep(d["w"], w.group)
    ref = orc.reference_linear_f64(d["x"], 1, d["w"])
    e16 = orc.rel_l2(orc.w8a16_linear(d["x"], 1, qw, sw, w.group), ref)
    e8 = orc.rel_l2(orc.int8_linear(d["x"], 1, qw, sw, w.group), ref)
    assert 0.002 < e16 < 0.012 and e16 < e8, (e16, e8)
    rng = np.random.default_rng(14)
    m, h, i, g = 32, 256, 512, 128
    xb = W.to_bf16_bits(rng.standard_normal((m, h)).astype(np.float32))
    w_gu = (0.05 * rng.standard_normal((2 * i, h))).astype(np.float32)
    w_dn = (0.05 * rng.standard_normal((h, i))).astype(np.float32)
    (gq, gs), (dq, ds) = orc.weight_prep(w_gu, g), orc.weight_prep(w_dn, g)
    y64 = orc.reference_mlp_f64(xb, w_gu, w_dn)
    e16 = orc.rel_l2(orc.swiglu_mlp_w8a16(xb, gq, gs, dq, ds, g), y64)
    e8 = orc.rel_l2(orc.swiglu_mlp(xb, gq, gs, dq, ds, g), y64)
    assert e16 < 0.02 and e16 < e8, (e16, e8)
