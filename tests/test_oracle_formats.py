"""Pins of the oracle's format layer (E2M1 / E4M3 tables and rounding).

Each test checks the oracle against something other than itself: brute
force over the representable values, a library cast, or facts of the
formats' definitions.
"""
import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import quantize as Q

CHUNK = 1 << 24


def _f32_range(lo_bits, hi_bits):
    for start in range(lo_bits, hi_bits, CHUNK):
        stop = min(start + CHUNK, hi_bits)
        yield np.arange(start, stop, dtype=np.uint32).view(np.float32)


def _f32_bits(x):
    return int(np.array(x, dtype=np.float32).view(np.uint32))


def test_e2m1_table_from_definition():
    assert list(F.E2M1_MAGNITUDES) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert F.E2M1_TABLE[8] == 0 and np.signbit(F.E2M1_TABLE[8])
    assert list(F.E2M1_TABLE[8:]) == [-v for v in F.E2M1_MAGNITUDES]


def test_e4m3_table_from_definition():
    # known points of E4M3FN: 0x38 = 1, 0x01 = 2^-9, 0x08 = 2^-6 (smallest normal),
    # 0x7e = 448 (largest), 0x7f NaN, no infinity
    assert F.E4M3_TABLE[0x38] == 1.0
    assert F.E4M3_TABLE[0x01] == 2.0 ** -9
    assert F.E4M3_TABLE[0x07] == 7 * 2.0 ** -9
    assert F.E4M3_TABLE[0x08] == 2.0 ** -6
    assert F.E4M3_TABLE[0x7E] == 448.0
    assert np.isnan(F.E4M3_TABLE[0x7F]) and np.isnan(F.E4M3_TABLE[0xFF])
    assert np.all(np.isfinite(np.delete(F.E4M3_TABLE, [0x7F, 0xFF])))
    # torch's float8_e4m3fn decodes every byte to the same value
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    same = (t == F.E4M3_TABLE) | (np.isnan(t) & np.isnan(F.E4M3_TABLE))
    assert np.all(same)


def _e2m1_brute(a):
    """Nearest magnitude by scanning all 8 values; tie -> even code."""
    a = a.astype(np.float64)
    best = np.zeros(a.shape, dtype=np.uint8)
    bestd = np.abs(a - F.E2M1_MAGNITUDES[0])
    for c in range(1, 8):
        d = np.abs(a - F.E2M1_MAGNITUDES[c])
        take = (d < bestd) | ((d == bestd) & (c % 2 == 0))
        best = np.where(take, np.uint8(c), best)
        bestd = np.where(take, d, bestd)
    return best


@pytest.mark.slow
def test_p1_e2m1_closed_form_exhaustive():
    """P1: the closed form equals brute-force nearest-even for every finite fp32 magnitude."""
    lo = _f32_bits(2.0 ** -4)
    hi = _f32_bits(8.0)
    maxf = 0x7F7FFFFF + 1
    # [0, 2^-4): nearest is 0 for every value (0.25 is the first midpoint)
    for a in _f32_range(0, lo):
        assert not np.any(F.e2m1_rne_sat(a))
    # [2^-4, 8): brute force over the 8 magnitudes
    for a in _f32_range(lo, hi):
        np.testing.assert_array_equal(F.e2m1_rne_sat(a), _e2m1_brute(a))
    # [8, max]: saturates at 6 (code 7) -- 6 is the nearest value for all of them
    for a in _f32_range(hi, maxf):
        assert np.all(F.e2m1_rne_sat(a) == 7)


def _e4m3_brute(u):
    """Nearest of the 127 non-negative finite E4M3 values, scanning all; tie -> even byte."""
    u = u.astype(np.float64)
    best = np.zeros(u.shape, dtype=np.uint8)
    bestd = np.abs(u)
    for b in range(1, 0x7F):
        d = np.abs(u - F.E4M3_POSITIVE[b])
        take = (d < bestd) | ((d == bestd) & (b % 2 == 0))
        best = np.where(take, np.uint8(b), best)
        bestd = np.where(take, d, bestd)
    return best


@pytest.mark.slow
def test_p2_e4m3_rne_matches_torch_cast_dense():
    """P2a: every fp32 in [2^-12, 448] rounds like torch's float32 -> float8_e4m3fn cast."""
    lo, hi = _f32_bits(2.0 ** -12), _f32_bits(448.0) + 1
    for u in _f32_range(lo, hi):
        mine = F.e4m3_rne(u)
        ref = torch.from_numpy(u).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        np.testing.assert_array_equal(mine, ref)
    # below 2^-12 everything is closer to 0 than to 2^-9 (every 97th value checked)
    for u in _f32_range(0, lo):
        assert not np.any(F.e4m3_rne(u[::97]))


def test_p2_e4m3_rne_brute_force_at_midpoints():
    """P2b: brute force over all 127 values at grid points, midpoints and 1 ulp beside them."""
    v = F.E4M3_POSITIVE
    mids = (v[:-1] + v[1:]) / 2
    pts = np.concatenate([v, mids]).astype(np.float32)
    assert np.all(pts.astype(np.float64) == np.concatenate([v, mids]))  # all exact in fp32
    up = np.nextafter(pts, np.float32(np.inf))
    dn = np.nextafter(pts, np.float32(0))
    rnd = np.random.default_rng(1).uniform(0, 448, 200000).astype(np.float32)
    u = np.concatenate([pts, up, dn, rnd])
    u = u[(u >= 0) & (u <= 448)]
    np.testing.assert_array_equal(F.e4m3_rne(u), _e4m3_brute(u))
    # ties really go to the even byte: 1.0625 -> 1.0 (0x38), 1.1875 -> 1.25 (0x3a)
    assert F.e4m3_rne(np.float32(1.0625)) == 0x38
    assert F.e4m3_rne(np.float32(1.1875)) == 0x3A
    # half of the smallest subnormal is a tie between 0 and 2^-9 -> 0
    assert F.e4m3_rne(np.float32(2.0 ** -10)) == 0
    assert F.e4m3_rne(np.nextafter(np.float32(2.0 ** -10), np.float32(1))) == 1


def test_p12_bf16_holds_every_dequantised_product():
    """P12: e2m1 * e4m3 is exact in bf16 (and f16) for all 16 x 127 pairs.

    This is what allows exact in-register dequantisation before a 16-bit
    matrix multiply: no element of an NVFP4 tensor is rounded on the way.
    """
    prods = (F.E2M1_TABLE[:, None] * F.E4M3_POSITIVE[None, :]).ravel()
    as_bf16 = torch.from_numpy(prods).to(torch.bfloat16).to(torch.float64).numpy()
    as_f16 = torch.from_numpy(prods).to(torch.float16).to(torch.float64).numpy()
    np.testing.assert_array_equal(as_bf16, prods)
    np.testing.assert_array_equal(as_f16, prods)


def test_p13_packed_sizes():
    """P13: NVFP4 storage is 1/2 byte of code plus 1/16 byte of scale per element (4.5 bits)."""
    for r, c in [(1, 16), (16, 128), (17408, 5120), (5120, 17408)]:
        assert Q.packed_bytes(r, c) * 8 == r * c * 4.5
    codes, scales, _ = Q.quantize(np.zeros((3, 48), dtype=np.uint16))
    assert codes.nbytes + scales.nbytes == Q.packed_bytes(3, 48)
    # the decode weight of the 17408 x 5120 projection
    assert Q.packed_bytes(17408, 5120) == 50135040
