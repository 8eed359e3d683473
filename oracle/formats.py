"""NVFP4 element and scale codes, from their bit-level definitions.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The pages name the format only as NVIDIA's FP4 format, NVFP4, with one scale
per 16 elements (aipulsen page, second paragraph; bayesiansapien page,
mechanism study, first item).  The element and scale codes used here are the
standard NVFP4 ones:

E2M1 element code (4 bits)
    bit 3 sign, bits 2..1 exponent, bit 0 mantissa, exponent bias 1.
    exponent 0 is subnormal: value = m * 2**-1.
    otherwise value = 2**(e-1) * (1 + m/2).
    Magnitudes of codes 0..7: 0, 0.5, 1, 1.5, 2, 3, 4, 6; code 8 is -0.

E4M3 ("FN") scale code (8 bits, only non-negative codes are produced)
    bit 7 sign, bits 6..3 exponent, bits 2..0 mantissa, exponent bias 7.
    exponent 0 is subnormal: value = m * 2**-9.
    otherwise value = 2**(e-7) * (1 + m/8); 0x7F / 0xFF are NaN, there is no
    infinity, the largest finite value is 448 (0x7E).

Rounding (reading of the pages' silence: round to nearest, ties to even)
    e4m3_rne  -- nearest of the 127 non-negative finite values, a tie goes to
                 the code whose mantissa LSB is 0.
    e2m1_rne_sat -- nearest of the 8 magnitudes, ties to the even code, any
                 magnitude above 6 gives 6 (code 7).
"""
import numpy as np

E2M1_MAX = 6.0
E4M3_MAX = 448.0


def e2m1_magnitude(code):
    """Magnitude of a 3-bit E2M1 magnitude code (0..7) from the bit fields."""
    e = (code >> 1) & 3
    m = code & 1
    if e == 0:
        return 0.5 * m
    return 2.0 ** (e - 1) * (1.0 + m / 2.0)


def e2m1_value(code):
    """Signed value of a 4-bit E2M1 code (0..15)."""
    mag = e2m1_magnitude(code & 7)
    return -mag if code & 8 else mag


def e4m3_value(byte):
    """Value of an E4M3FN byte; NaN for 0x7F/0xFF."""
    s = -1.0 if byte & 0x80 else 1.0
    e = (byte >> 3) & 0xF
    m = byte & 7
    if e == 0xF and m == 7:
        return float("nan")
    if e == 0:
        return s * m * 2.0 ** -9
    return s * 2.0 ** (e - 7) * (1.0 + m / 8.0)


# Tables built from the definitions above (exact in float64).
E2M1_TABLE = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
E2M1_MAGNITUDES = np.array([e2m1_magnitude(c) for c in range(8)], dtype=np.float64)
E4M3_TABLE = np.array([e4m3_value(b) for b in range(256)], dtype=np.float64)
# Non-negative finite scale values in code order; they increase with the code.
E4M3_POSITIVE = E4M3_TABLE[:0x7F].copy()
assert np.all(np.diff(E4M3_POSITIVE) > 0)
assert E4M3_POSITIVE[-1] == E4M3_MAX


def e4m3_rne(u):
    """Round non-negative float32 magnitudes in [0, 448] to E4M3 bytes.

    Nearest representable value; on an exact tie the code with an even
    mantissa (byte LSB 0) wins.  Differences are taken in float64, which is
    exact wherever a tie can occur (both operands are multiples of 2**-34
    and below 2**9 there).
    """
    u = np.asarray(u, dtype=np.float32).astype(np.float64)
    if np.any(~np.isfinite(u)) or np.any(u < 0) or np.any(u > E4M3_MAX):
        raise ValueError("e4m3_rne expects magnitudes in [0, 448]")
    hi = np.searchsorted(E4M3_POSITIVE, u, side="left")      # first value >= u
    hi = np.minimum(hi, len(E4M3_POSITIVE) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = u - E4M3_POSITIVE[lo]
    d_hi = E4M3_POSITIVE[hi] - u
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((hi & 1) == 0))
    # u exactly on a grid value: hi is that value and d_hi == 0.
    code = np.where(pick_hi, hi, lo)
    return code.astype(np.uint8)


def e2m1_rne_sat(a):
    """Round non-negative float32 magnitudes to 3-bit E2M1 magnitude codes.

    Closed form of "nearest of {0,.5,1,1.5,2,3,4,6}, ties to the even code,
    saturate above 6": the midpoints are .25 .75 1.25 1.75 2.5 3.5 5 and a
    midpoint belongs to the neighbour with the even code.
    """
    a = np.asarray(a, dtype=np.float32)
    code = np.zeros(a.shape, dtype=np.uint8)
    code += (a > np.float32(0.25))
    code += (a >= np.float32(0.75))
    code += (a > np.float32(1.25))
    code += (a >= np.float32(1.75))
    code += (a > np.float32(2.5))
    code += (a >= np.float32(3.5))
    code += (a > np.float32(5.0))
    return code
