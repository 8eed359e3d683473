"""Pins of the oracle's fp64 W4A4 GEMM and epilogues.

Checked against exact integer / rational arithmetic, the closed form of the
fused-GEMM global-scale mismatch, and closed forms of the epilogue functions.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import epilogue as E
from oracle import formats as F
from oracle import gemm as G
from oracle import quantize as Q
from nvfp4_w4a4_gemm_quantize_amd import inputs


def test_p8_unit_scales_give_an_exact_small_integer_matmul():
    """P8: scale byte 0x38 (1.0) and g = 1 turn the GEMM into a matmul of code values.

    2*e2m1 is an integer in [-12, 12]; the product is checked in int64, with
    non-square, asymmetric operands so that a transposed operand fails.
    """
    rng = np.random.default_rng(8)
    M, N, K = 5, 7, 64
    ca = rng.integers(0, 16, size=(M, K)).astype(np.uint8)
    cw = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
    sa = np.full((M, K // 16), 0x38, dtype=np.uint8)
    sw = np.full((N, K // 16), 0x38, dtype=np.uint8)
    y, bound = G.gemm(Q.pack_nibbles(ca), sa, 1.0, Q.pack_nibbles(cw), sw, np.ones(N))
    ia = np.rint(2 * F.E2M1_TABLE[ca]).astype(np.int64)
    iw = np.rint(2 * F.E2M1_TABLE[cw]).astype(np.int64)
    np.testing.assert_array_equal(y * 4, (ia @ iw.T).astype(np.float64))
    np.testing.assert_array_equal(bound * 4, (np.abs(ia) @ np.abs(iw).T).astype(np.float64))


def test_dequant_applies_each_scale_to_its_own_block():
    codes = np.full((1, 32), 2, dtype=np.uint8)          # value 1.0 everywhere
    scales = np.array([[0x38, 0x40]], dtype=np.uint8)    # 1.0 and 2.0
    v = G.dequant(Q.pack_nibbles(codes), scales)
    assert np.all(v[0, :16] == 1.0) and np.all(v[0, 16:] == 2.0)
    # nibble order: low nibble is the even element
    v = G.dequant(np.array([[0x72] + [0] * 7], dtype=np.uint8), np.array([[0x38]], dtype=np.uint8))
    assert v[0, 0] == 1.0 and v[0, 1] == 6.0


def test_p9_tiny_gemm_equals_exact_rational_triple_loop():
    """P9: the 16x64x128 workload, fp64 oracle vs a Fractions triple loop."""
    d = inputs.tiny()
    ca, sa, ga = Q.quantize(d["A"])
    cw, sw, gw = Q.quantize(d["W"])
    y, bound = G.gemm(ca, sa, ga, cw, sw, np.full(64, gw))
    na, nw = Q.unpack_nibbles(ca), Q.unpack_nibbles(cw)
    va = [[Fraction(F.E2M1_TABLE[na[m, k]]) * Fraction(F.E4M3_TABLE[sa[m, k // 16]]) for k in range(128)]
          for m in range(16)]
    vw = [[Fraction(F.E2M1_TABLE[nw[n, k]]) * Fraction(F.E4M3_TABLE[sw[n, k // 16]]) for k in range(128)]
          for n in range(64)]
    denom = Fraction(float(ga)) * Fraction(float(gw))
    for m in range(16):
        for n in range(64):
            exact = sum(a * b for a, b in zip(va[m], vw[n])) / denom
            babs = sum(abs(a * b) for a, b in zip(va[m], vw[n])) / denom
            assert abs(Fraction(y[m, n]) - exact) <= Fraction(1, 10 ** 12) * babs
            assert abs(Fraction(bound[m, n]) - babs) <= Fraction(1, 10 ** 12) * babs
    # the outlier channel really is there, and A's global scale reflects it
    assert ga < np.float32(2688.0 / 50)


def test_p10_single_global_scale_misscales_by_the_ratio():
    """P10: one alpha for a fused weight is off, per segment s, by exactly g_w[s] / g_w[0].

    This is the global-scale mismatch of fused kernels on per-module-calibrated
    checkpoints (bayesiansapien page, "Two practical repairs"; aimodeling page,
    "What engineers should actually take away").
    """
    rng = np.random.default_rng(10)
    K = 64
    widths, f = [8, 8, 16, 4], [1.0, 8.0, 2.0, 5.0]
    w = np.concatenate([rng.standard_normal((n, K)) * fs for n, fs in zip(widths, f)]).astype(np.float32)
    off = np.cumsum([0] + widths)
    cw, sw, gs = Q.quantize_segments(inputs.f32_to_bf16_bits(w), off)
    ca, sa, ga = Q.quantize(inputs.f32_to_bf16_bits(rng.standard_normal((6, K)).astype(np.float32)))
    y_ok, _ = G.gemm(ca, sa, ga, cw, sw, G.column_global(off[-1], off, gs))
    y_one, _ = G.gemm(ca, sa, ga, cw, sw, np.full(off[-1], np.float64(gs[0])))
    for s in range(len(widths)):
        cols = slice(off[s], off[s + 1])
        ratio = y_one[:, cols] / y_ok[:, cols]
        np.testing.assert_allclose(ratio, np.float64(gs[s]) / np.float64(gs[0]), rtol=1e-14)
    assert not np.allclose(gs, gs[0])     # the scales really differ


def test_p11_epilogue_closed_forms():
    """P11: special values and identities of the epilogue functions."""
    assert E.sigmoid(0.0) == 0.5
    assert E.silu(0.0) == 0.0
    assert abs(E.softplus(0.0) - np.log(2.0)) < 1e-16
    x = np.linspace(-40, 40, 801)
    np.testing.assert_allclose(E.softplus(x) - E.softplus(-x), x, atol=1e-12)   # softplus(x)-softplus(-x)=x
    np.testing.assert_allclose(E.sigmoid(x) + E.sigmoid(-x), 1.0, atol=1e-15)
    np.testing.assert_allclose(E.silu(x), x * E.sigmoid(x), rtol=1e-15)
    assert E.softplus(800.0) == 800.0 and E.softplus(-800.0) == 0.0
    assert E.sigmoid(-800.0) == 0.0 and E.sigmoid(800.0) == 1.0
    # decay: -exp(A) * softplus(a + d); at a = -d it is -exp(A) ln 2
    A = np.array([0.0, 1.0, -0.5])
    d = np.array([0.3, -0.2, 1.0])
    np.testing.assert_allclose(E.gdn_decay((-d)[None, :], A, d)[0], -np.exp(A) * np.log(2), rtol=1e-15)
    assert np.all(E.gdn_decay(np.array([[5.0, -5.0, 0.0]]), A, d) < 0)
    np.testing.assert_allclose(E.silu_mul(np.array([1.0]), np.array([2.0])), 2.0 / (1 + np.exp(-1.0)))


def test_epilogue_tolerances_contain_the_true_perturbation():
    """The Lipschitz allowances bound the change of each epilogue under a GEMM-sized error."""
    rng = np.random.default_rng(12)
    z = rng.uniform(-12, 12, 5000)
    t = np.abs(z) * 1e-3 + 1e-3
    dz = t * rng.choice([-1, 1], 5000)
    up = rng.standard_normal(5000)
    assert np.all(np.abs(E.sigmoid(z + dz) - E.sigmoid(z)) <= E.sigmoid_tolerance(z, t, False))
    assert np.all(np.abs(E.silu_mul(z + dz, up + t) - E.silu_mul(z, up)) <= E.silu_mul_tolerance(z, up, t, t, False))
    A = rng.standard_normal(5000) * 0.5
    d = rng.standard_normal(5000) * 0.5
    got = np.abs(E.gdn_decay((z + dz)[None, :], A, d) - E.gdn_decay(z[None, :], A, d))
    assert np.all(got <= E.gdn_decay_tolerance(z[None, :], A, d, t[None, :], False))


def test_bf16_round_is_nearest_even():
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7 -> 1 ; 1 + 3*2^-8 -> 1 + 2^-6
    v = G.bf16_round(np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8 + 2.0 ** -30), 0.0]))
    np.testing.assert_array_equal(v, [1.0, 1 + 2.0 ** -6, -(1 + 2.0 ** -7), 0.0])
    x = np.random.default_rng(0).standard_normal(10000)
    got = G.f64_to_bf16_bits(x)
    back = (got.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.all(np.abs(back - x) <= 2.0 ** -8 * np.abs(x))
