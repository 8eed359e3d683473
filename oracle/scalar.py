"""Definitional scalar NVFP4 quantizer in exact rationals -- TEST INFRASTRUCTURE ONLY.

A second, independent implementation of the quantizer in ``oracle.quantize``:
every real-valued quantity is a ``fractions.Fraction`` and every place where
the method rounds to binary32 calls ``round_binary32``, which is written from
the IEEE 754 definition (24-bit significand, subnormals below 2**-126,
round-to-nearest with ties to the even significand).  Scale and element
codes are chosen by scanning all representable values for the nearest one.
No numpy floating point is involved, so agreement with the vectorised numpy
quantizer pins both.

Steps and readings are those listed in ``oracle.quantize`` (block of 16
consecutive elements, g = 2688/amax, t = m/6, u = t*g clamped to 448,
S = nearest E4M3, r = g/s, q = x*r, nearest E2M1 with saturation at 6).
Pure-Python loops: small inputs only.
"""
from fractions import Fraction

from .formats import e2m1_magnitude, e4m3_value

_EMIN = -126           # binary32 smallest normal exponent
_P = 24                # binary32 significand bits
_MAXF = (2 - Fraction(1, 2 ** 23)) * Fraction(2) ** 127


def _floor_log2(r):
    """floor(log2(r)) for a positive Fraction, exactly."""
    e = r.numerator.bit_length() - r.denominator.bit_length()
    # now 2**(e-1) < r < 2**(e+1); adjust to 2**e <= r < 2**(e+1)
    if Fraction(2) ** e > r:
        e -= 1
    return e


def round_binary32(r):
    """Round a Fraction to the nearest binary32 value (ties to even), exactly."""
    if r == 0:
        return Fraction(0)
    sign = -1 if r < 0 else 1
    a = abs(r)
    e = max(_floor_log2(a), _EMIN)
    ulp = Fraction(2) ** (e - (_P - 1))
    n = a / ulp
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    v = fl * ulp
    if v > _MAXF:
        raise OverflowError("binary32 overflow")
    return sign * v


def bf16_to_fraction(bits):
    """Exact value of a finite bf16 bit pattern and its sign bit."""
    sign = (bits >> 15) & 1
    e = (bits >> 7) & 0xFF
    m = bits & 0x7F
    if e == 0xFF:
        raise ValueError("NVFP4 quantizer inputs must be finite")
    if e == 0:
        v = Fraction(m, 128) * Fraction(2) ** -126
    else:
        v = (1 + Fraction(m, 128)) * Fraction(2) ** (e - 127)
    return (-v if sign else v), sign


_E4M3 = [(b, Fraction(e4m3_value(b))) for b in range(0x7F)]   # exact (dyadic)
_E2M1 = [(c, Fraction(e2m1_magnitude(c))) for c in range(8)]


def _nearest(table, v):
    """Nearest table entry to v; a tie goes to the even code."""
    best = None
    for code, val in table:
        d = abs(v - val)
        if best is None or d < best[0] or (d == best[0] and code % 2 == 0 and best[1] % 2 == 1):
            best = (d, code)
    return best[1]


def global_scale(bits_rows):
    """g = round32(2688 / amax) over all elements; 1 for an all-zero tensor."""
    amax = Fraction(0)
    for row in bits_rows:
        for b in row:
            v, _ = bf16_to_fraction(b)
            amax = max(amax, abs(v))
    if amax == 0:
        return Fraction(1)
    return round_binary32(Fraction(2688) / amax)


def quantize_block(bits16, g):
    """Quantize 16 bf16 bit patterns with global scale g (a binary32 Fraction).

    Returns (list of 16 codes, scale byte).
    """
    xs = [bf16_to_fraction(b) for b in bits16]
    m = max(abs(v) for v, _ in xs)
    t = round_binary32(m / 6)
    u = round_binary32(t * g)
    u = min(u, Fraction(448))
    S = _nearest(_E4M3, u)
    if S == 0:
        return [0] * 16, 0
    s = Fraction(e4m3_value(S))
    r = round_binary32(g / s)
    codes = []
    for v, sign in xs:
        q = round_binary32(v * r)
        codes.append((sign << 3) | _nearest(_E2M1, abs(q)))
    return codes, S


def quantize_rows(bits_rows, g=None):
    """Quantize rows of bf16 bit patterns.  Returns (codes rows, scale rows, g)."""
    if g is None:
        g = global_scale(bits_rows)
    else:
        g = Fraction(g)
    all_codes, all_scales = [], []
    for row in bits_rows:
        if len(row) % 16:
            raise ValueError("row length must be a multiple of 16")
        rc, rs = [], []
        for j in range(0, len(row), 16):
            c, s = quantize_block(row[j:j + 16], g)
            rc.extend(c)
            rs.append(s)
        all_codes.append(rc)
        all_scales.append(rs)
    return all_codes, all_scales, g
