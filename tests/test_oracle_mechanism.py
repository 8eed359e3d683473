"""Pins of ``oracle/mechanism.py``, the coarser-scaled reference formats of
the outlier-locality comparison (bayesiansapien page, "The four-part
mechanism study", first item).  No GPU."""
import numpy as np

from nvfp4_w4a4_gemm_quantize_amd import inputs
from oracle import formats as F
from oracle import mechanism as MX
from oracle import quantize as OQ


def test_block_16_is_the_nvfp4_quantizer():
    rng = np.random.default_rng(11)
    x = np.concatenate([rng.standard_normal((20, 64)), rng.standard_t(3, (20, 64)) * 30,
                        np.zeros((2, 64)), rng.standard_normal((4, 64)) * 1e-6]).astype(np.float32)
    x = inputs.bf16_bits_to_f32(inputs.f32_to_bf16_bits(x))
    for g in (np.float32(1.0), np.float32(37.25), OQ.dynamic_global_scale(inputs.f32_to_bf16_bits(x))):
        c1, s1 = MX.block_quantize(x, g, 16)
        c2, s2 = OQ.quantize_f32(x, g)
        np.testing.assert_array_equal(c1, c2)
        np.testing.assert_array_equal(s1, s2)


def test_block_dequantize_closed_form():
    # one block of 32: the largest magnitude 6 * 2^k with g = 1 gives scale 2^k exactly (E4M3 normal),
    # so every on-grid value e2m1 * 2^k comes back unchanged
    grid = np.array([F.e2m1_value(c) for c in range(16)], dtype=np.float32)
    for k in (-3, 0, 4):
        row = np.resize(grid, 32).astype(np.float32) * np.float32(2.0 ** k)
        codes, S = MX.block_quantize(row[None, :], 1.0, 32)
        assert F.e4m3_value(int(S[0, 0])) == 2.0 ** k
        np.testing.assert_array_equal(MX.block_dequantize(codes, S, 1.0)[0], row.astype(np.float64))


def test_per_tensor_round_trip_on_grid():
    # amax = 6 * 2^k: r = 2^-k exactly, so values e2m1 * 2^k are reproduced, other values round to the grid
    grid = np.array([F.e2m1_value(c) for c in range(16)], dtype=np.float32)
    x = (np.resize(grid, (4, 48)) * np.float32(8.0)).astype(np.float32)
    codes, r = MX.per_tensor_quantize(x)
    assert r == np.float32(1.0 / 8.0)
    np.testing.assert_array_equal(MX.per_tensor_dequantize(codes, r), x.astype(np.float64))
    np.testing.assert_array_equal(codes & 7, np.resize(np.arange(16, dtype=np.uint8), (4, 48)) & 7)


def test_an_outlier_crushes_exactly_its_own_block():
    """One element 1000x the rest: with g fixed, every other element of its block (B = 16 or 32)
    falls below a quarter of the smallest E2M1 step and becomes 0; blocks elsewhere keep nonzero codes.
    Per-tensor, the whole tensor collapses to 0 except the outlier."""
    rng = np.random.default_rng(3)
    x = (np.abs(rng.standard_normal((3, 128))) + 0.5).astype(np.float32)
    x[:, 40] = 1000.0
    g = np.float32(2.0)
    for B in (16, 32):
        codes, S = MX.block_quantize(x, g, B)
        flat = codes.reshape(3, 128)
        b0 = (40 // B) * B
        own = np.zeros(128, dtype=bool)
        own[b0:b0 + B] = True
        own[40] = False
        assert np.all(flat[:, own] == 0)
        assert np.all(flat[:, ~own & (np.arange(128) != 40)] != 0)
        # changing the outlier changes no code outside its block
        y = x.copy()
        y[:, 40] = 500.0
        codes_y, _ = MX.block_quantize(y, g, B)
        outside = np.ones(128, dtype=bool)
        outside[b0:b0 + B] = False
        np.testing.assert_array_equal(codes_y.reshape(3, 128)[:, outside], flat[:, outside])
    codes, r = MX.per_tensor_quantize(x)
    assert np.all(codes[:, np.arange(128) != 40] == 0) and np.all(codes[:, 40] == 7)


def test_contaminated_mask():
    m = MX.contaminated_mask((2, 64), [3, 40], 16)
    want = np.zeros(64, dtype=bool)
    want[0:16] = True
    want[32:48] = True
    want[[3, 40]] = False
    np.testing.assert_array_equal(m[1], want)
    assert MX.contaminated_mask((1, 8), [2], None)[0].sum() == 7


def test_rel_l2():
    assert MX.rel_l2([1.0, 2.0], [1.0, 2.0]) == 0.0
    assert abs(MX.rel_l2([0.0, 4.0], [3.0, 4.0]) - 3.0 / 5.0) < 1e-15
