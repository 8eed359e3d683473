"""Pins of the oracle's NVFP4 quantizer.

Checked against hand-worked blocks (tests/golden), invariants of the format
(on-grid round trip, outlier locality, idempotence), brute force over all
codes x scales, and a second, exact-rational implementation (oracle.scalar).
"""
import os

import numpy as np
import pytest

from oracle import formats as F
from oracle import quantize as Q
from oracle import scalar as S
from nvfp4_w4a4_gemm_quantize_amd.inputs import f32_to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "quantize_blocks.txt")


def load_golden():
    cases = []
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        name, g, xs, sb, codes, gexp = [f.strip() for f in line.split("|")]
        x = np.array([float(v) for v in xs.split()], dtype=np.float32)
        assert np.all(f32_to_bf16_bits(x).astype(np.uint32) << 16 == x.view(np.uint32))
        cases.append(dict(name=name, g=None if g == "dyn" else np.float32(float(g)),
                          bits=f32_to_bf16_bits(x)[None, :], scales=[int(b, 16) for b in sb.split()],
                          codes=[int(c, 16) for c in codes.split()], g_expected=np.float32(float(gexp))))
    return cases


@pytest.mark.parametrize("case", load_golden(), ids=lambda c: c["name"])
def test_golden_blocks(case):
    codes, scales, g = Q.quantize(case["bits"], case["g"])
    assert list(scales[0]) == case["scales"]
    assert list(Q.unpack_nibbles(codes)[0]) == case["codes"]
    assert g == case["g_expected"]
    # the exact-rational implementation agrees on the hand-worked blocks too
    sc, ss, sg = S.quantize_rows(case["bits"].tolist(), None if case["g"] is None else float(case["g"]))
    assert ss[0] == case["scales"] and sc[0] == case["codes"] and sg == case["g_expected"]


def _bits(x):
    x = np.asarray(x, dtype=np.float32)
    b = f32_to_bf16_bits(x)
    assert np.array_equal(Q.bf16_bits_to_f32(b), x), "value not exact in bf16"
    return b


def test_p3_on_grid_round_trip():
    """P3: x = code * s / g with g a power of two quantizes back to exactly (codes, S)."""
    rng = np.random.default_rng(3)
    for g in (np.float32(1.0), np.float32(2.0 ** -5), np.float32(2.0 ** 7)):
        for S_byte in range(1, 0x7F):
            s = F.E4M3_POSITIVE[S_byte]
            codes = rng.integers(0, 16, size=(2, 16)).astype(np.uint8)
            codes[:, 3] = rng.choice([7, 15], size=2)            # a +-6 anchor per block
            vals = F.E2M1_TABLE[codes] * s / np.float64(g)
            c, sc, _ = Q.quantize(_bits(vals.astype(np.float32)), g)
            nib = Q.unpack_nibbles(c)
            assert np.all(sc == S_byte), (g, S_byte)
            # code 8 (-0) and 0 both decode to 0: compare values, and the sign bits of non-zeros
            np.testing.assert_array_equal(F.E2M1_TABLE[nib], F.E2M1_TABLE[codes])
            nz = (codes & 7) != 0
            np.testing.assert_array_equal(nib[nz], codes[nz])


def test_p4_outlier_locality():
    """P4: with g fixed, an outlier changes only its own 16-element block.

    Statement of the bayesiansapien page (mechanism study, first item): one
    scale covers 16 elements, so an outlier contaminates only its block.
    """
    rng = np.random.default_rng(4)
    x = rng.standard_normal((8, 256)).astype(np.float32)
    base_bits = f32_to_bf16_bits(x)
    g = np.float32(2688.0 / 50.0)
    c0, s0, _ = Q.quantize(base_bits, g)
    for (r, k, v) in [(0, 0, 40.0), (3, 77, -35.0), (7, 255, 48.0), (5, 128, 1e-3)]:
        bits = base_bits.copy()
        bits[r, k] = f32_to_bf16_bits(np.array([v], dtype=np.float32))[0]
        c1, s1, _ = Q.quantize(bits, g)
        blk = k // 16
        mask_s = np.ones_like(s0, dtype=bool)
        mask_s[r, blk] = False
        np.testing.assert_array_equal(s1[mask_s], s0[mask_s])
        n0, n1 = Q.unpack_nibbles(c0), Q.unpack_nibbles(c1)
        mask_c = np.ones_like(n0, dtype=bool)
        mask_c[r, blk * 16:(blk + 1) * 16] = False
        np.testing.assert_array_equal(n1[mask_c], n0[mask_c])
        if abs(v) > 10:   # a real outlier does move its own block's scale
            assert s1[r, blk] != s0[r, blk]
    # with a dynamic global scale the outlier raises amax and reaches other blocks:
    bits = base_bits.copy()
    bits[0, 0] = f32_to_bf16_bits(np.array([1000.0], dtype=np.float32))[0]
    _, s_dyn, _ = Q.quantize(bits)
    _, s_ref, _ = Q.quantize(base_bits)
    assert np.count_nonzero(s_dyn != s_ref) > 16


def test_p5_all_codes_times_all_scales():
    """P5: every code (16) at every non-zero scale (126), next to a +-6*s anchor, round-trips."""
    g = np.float32(1.0)
    for S_byte in range(1, 0x7F):
        s = F.E4M3_POSITIVE[S_byte]
        vals = np.zeros((16, 16), dtype=np.float64)
        vals[:, 0] = F.E2M1_TABLE[np.arange(16)] * s       # the code under test
        vals[:, 1] = np.where(np.arange(16) % 2, -6.0, 6.0) * s   # anchor
        x = vals.astype(np.float32)
        x[8, 0] = -0.0
        c, sc, _ = Q.quantize(_bits(x), g)
        nib = Q.unpack_nibbles(c)
        assert np.all(sc == S_byte)
        np.testing.assert_array_equal(nib[:, 0], np.arange(16))
        np.testing.assert_array_equal(nib[:, 1], np.where(np.arange(16) % 2, 15, 7))


def test_p6_idempotence():
    """P6: quantize(dequant(quantize(x))) == quantize(x) for power-of-two g, normal scales."""
    rng = np.random.default_rng(6)
    x = (rng.standard_t(4, size=(32, 512)) * np.exp(rng.uniform(-3, 3, size=(32, 1)))).astype(np.float32)
    bits = f32_to_bf16_bits(x)
    g = np.float32(2.0 ** 4)
    c, s, _ = Q.quantize(bits, g)
    assert np.all(s >= 0x08), "test input must keep every scale normal"
    deq = F.E2M1_TABLE[Q.unpack_nibbles(c)].reshape(32, 32, 16) * F.E4M3_POSITIVE[s][:, :, None] / np.float64(g)
    c2, s2, _ = Q.quantize(_bits(deq.reshape(32, 512).astype(np.float32)), g)
    np.testing.assert_array_equal(s2, s)
    n1, n2 = Q.unpack_nibbles(c), Q.unpack_nibbles(c2)
    np.testing.assert_array_equal(F.E2M1_TABLE[n2], F.E2M1_TABLE[n1])


def _edge_bits(rng, rows, cols):
    """Random finite bf16 bit patterns over the whole exponent range, plus edge values."""
    b = rng.integers(0, 1 << 16, size=(rows, cols), dtype=np.uint32).astype(np.uint16)
    finite = ((b >> 7) & 0xFF) != 0xFF
    b = np.where(finite, b, b & 0x807F)             # NaN/Inf -> subnormal
    return b.astype(np.uint16)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_p7_scalar_equals_vectorised(seed):
    """P7: exact-rational scalar oracle == numpy float32 oracle, bit for bit."""
    rng = np.random.default_rng(70 + seed)
    cases = []
    # ordinary data with outliers, dynamic scale
    x = rng.standard_t(4, size=(6, 64)).astype(np.float32)
    x[:, 5] *= 50
    cases.append((f32_to_bf16_bits(x), None))
    # random bit patterns spanning every exponent (subnormals, huge values), dynamic
    cases.append((_edge_bits(rng, 4, 64), None))
    # same, with a static calibrated scale that saturates some blocks
    xs = rng.standard_normal((4, 64)).astype(np.float32)
    cases.append((f32_to_bf16_bits(xs), np.float32(2688.0 / 0.5)))
    # ties everywhere: multiples of 1/64 in a narrow range
    xt = (rng.integers(-384, 385, size=(4, 64)) / 64.0).astype(np.float32)
    cases.append((f32_to_bf16_bits(xt), np.float32(1.0)))
    # zeros, negative zeros and tiny blocks
    xz = np.zeros((2, 64), dtype=np.float32)
    xz[0, 16:32] = -0.0
    xz[1, 32:48] = 1e-30
    xz[1, 0] = 3.0
    cases.append((f32_to_bf16_bits(xz), None))
    for bits, g in cases:
        c, s, gv = Q.quantize(bits, g)
        sc, ss, sg = S.quantize_rows(bits.tolist(), None if g is None else float(g))
        assert float(gv) == sg
        np.testing.assert_array_equal(s, np.array(ss, dtype=np.uint8))
        np.testing.assert_array_equal(Q.unpack_nibbles(c), np.array(sc, dtype=np.uint8))


def test_scalar_binary32_rounding_matches_ieee_hardware():
    """The scalar oracle's binary32 rounding agrees with numpy's float32 casts."""
    from fractions import Fraction
    rng = np.random.default_rng(9)
    xs = rng.standard_normal(2000) * np.exp2(rng.integers(-140, 120, 2000))
    xs = np.concatenate([xs, [2.0 ** -149 * 1.5, 2.0 ** -149 * 2.5, 1 + 2.0 ** -24, 1 + 3 * 2.0 ** -24]])
    for v in xs:
        assert S.round_binary32(Fraction(float(v))) == Fraction(float(np.float32(v)))


def test_zero_tensor_and_sign_of_zero():
    c, s, g = Q.quantize(np.zeros((2, 32), dtype=np.uint16))
    assert g == 1.0 and not s.any() and not c.any()
    bits = f32_to_bf16_bits(np.array([[-0.1, 6.0] + [0.0] * 14], dtype=np.float32))
    c, s, _ = Q.quantize(bits, np.float32(1.0))
    assert Q.unpack_nibbles(c)[0, 0] == 0x8     # -0.1 -> -0 keeps the sign


def test_segmented_weights_use_their_own_global_scale():
    rng = np.random.default_rng(11)
    w = np.concatenate([rng.standard_normal((32, 64)) * f for f in (1.0, 8.0, 2.5)]).astype(np.float32)
    bits = f32_to_bf16_bits(w)
    off = [0, 32, 64, 96]
    c, s, gs = Q.quantize_segments(bits, off)
    for i in range(3):
        amax = np.max(np.abs(Q.bf16_bits_to_f32(bits[off[i]:off[i + 1]])))
        assert gs[i] == np.float32(np.float32(2688.0) / amax)
        ci, si, _ = Q.quantize(bits[off[i]:off[i + 1]], gs[i])
        np.testing.assert_array_equal(c[off[i]:off[i + 1]], ci)
        np.testing.assert_array_equal(s[off[i]:off[i + 1]], si)
    assert gs.max() / gs.min() > 4
    with pytest.raises(ValueError):
        Q.quantize_segments(bits, [0, 64, 32, 96])


def test_rejects_non_finite():
    bits = np.array([[0x7F80] + [0] * 15], dtype=np.uint16)    # +inf
    with pytest.raises(ValueError):
        Q.quantize(bits)
