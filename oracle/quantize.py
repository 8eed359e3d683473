"""Vectorised NVFP4 quantizer in numpy float32 -- TEST INFRASTRUCTURE ONLY.

Follows the steps of NVFP4 16-element block scaling (bayesiansapien page,
"The four-part mechanism study", first item: one scale per 16 elements) with
a per-tensor FP32 global scale (the per-module global scales of the same
page's "Two practical repairs").  Every floating-point step below is one
IEEE binary32 operation with round-to-nearest-even, done by numpy on float32
arrays, in the order written:

1. x = float32(bf16)                                  (exact)
2. g: given, or dynamic  g = 2688 / max|x|  (2688 = 6 * 448; g = 1 if the
   tensor is all zero)
3. per block of 16 consecutive elements along a row:  m = max|x_i|
4. t = m / 6;  u = t * g;  u = min(u, 448);  S = E4M3_RNE(u)
5. S == 0:  the 16 codes are 0x0
6. else s = value(S);  r = g / s;  q_i = x_i * r;
   code_i = (sign bit of x_i) << 3 | E2M1_RNE_SAT(|q_i|)
7. pack: byte j of a row = code[2j] | code[2j+1] << 4

Readings taken where the pages are silent: blocks run along the contraction
(column) axis; the global scale is stored in encode form; the E4M3 scale is
computed as (m/6)*g in that order; u is clamped to 448 before rounding;
r = g/s is formed once per block; a zero scale byte forces zero codes; the
sign of zero codes is kept (-0.1 -> 0x8); inputs must be finite.
"""
import numpy as np

from .formats import E4M3_POSITIVE, e2m1_rne_sat, e4m3_rne

GLOBAL_NUMERATOR = np.float32(6.0 * 448.0)  # E2M1 max times E4M3 max


def bf16_bits_to_f32(bits):
    """bf16 bit patterns (uint16) -> float32 values (exact)."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def global_scale_from_amax(amax):
    """Encode-form global scale g = 2688 / amax as one float32 division."""
    amax = np.float32(amax)
    if amax == 0:
        return np.float32(1.0)
    return np.float32(GLOBAL_NUMERATOR / amax)


def dynamic_global_scale(x_bits):
    """Global scale of a whole bf16 tensor (per-tensor amax)."""
    x = bf16_bits_to_f32(x_bits)
    if not np.all(np.isfinite(x)):
        raise ValueError("NVFP4 quantizer inputs must be finite")
    return global_scale_from_amax(np.max(np.abs(x)) if x.size else 0.0)


def quantize_f32(x, g):
    """Quantize float32 rows [R, C] (C % 16 == 0) with global scale g.

    Returns (codes uint8 [R, C/16, 16] unpacked nibbles, scales uint8 [R, C/16]).
    """
    x = np.asarray(x, dtype=np.float32)
    if x.ndim != 2 or x.shape[1] % 16:
        raise ValueError("expected [rows, cols] with cols % 16 == 0")
    if not np.all(np.isfinite(x)):
        raise ValueError("NVFP4 quantizer inputs must be finite")
    g = np.float32(g)
    rows, cols = x.shape
    blocks = x.reshape(rows, cols // 16, 16)
    m = np.max(np.abs(blocks), axis=2)                      # step 3
    t = (m / np.float32(6.0)).astype(np.float32)             # step 4
    u = (t * g).astype(np.float32)
    u = np.minimum(u, np.float32(448.0))
    S = e4m3_rne(u)
    s = E4M3_POSITIVE[S].astype(np.float32)                  # exact
    nz = S != 0
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(nz, g / np.where(nz, s, np.float32(1.0)), np.float32(0.0))
    r = r.astype(np.float32)                                 # step 6
    q = (blocks * r[:, :, None]).astype(np.float32)
    mag = e2m1_rne_sat(np.abs(q))
    sign = np.signbit(blocks).astype(np.uint8) << 3
    codes = (sign | mag).astype(np.uint8)
    codes[~nz] = 0                                           # step 5
    return codes, S


def pack_nibbles(codes):
    """[R, C/16, 16] or [R, C] nibbles -> [R, C/2] bytes, low nibble = even index."""
    c = np.asarray(codes, dtype=np.uint8)
    c = c.reshape(c.shape[0], -1)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed):
    """[R, C/2] bytes -> [R, C] nibbles."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty((p.shape[0], p.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = p & 0xF
    out[:, 1::2] = p >> 4
    return out


def quantize(x_bits, g=None):
    """bf16 bits [R, C] -> (codes [R, C/2] uint8, scales [R, C/16] uint8, g).

    ``g`` None means dynamic (per-tensor amax); otherwise the given float32
    global scale is used (a calibrated, static scale).
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    if g is None:
        g = dynamic_global_scale(x_bits)
    codes, scales = quantize_f32(bf16_bits_to_f32(x_bits), g)
    return pack_nibbles(codes), scales, np.float32(g)


def quantize_segments(w_bits, seg_offsets, seg_global=None):
    """Quantize a fused weight [N, K] whose row ranges are separate modules.

    Row segment s = rows [seg_offsets[s], seg_offsets[s+1]) has its own global
    scale (the per-module-calibrated global scales of the bayesiansapien
    page, "Two practical repairs").  ``seg_global`` None means each segment's
    scale is computed from that segment's own amax.
    Returns (codes [N, K/2], scales [N, K/16], g float32 [S]).
    """
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    off = [int(o) for o in seg_offsets]
    nseg = len(off) - 1
    if off[0] != 0 or off[-1] != w_bits.shape[0] or any(
            off[i] >= off[i + 1] for i in range(nseg)):
        raise ValueError("segment offsets must rise strictly from 0 to N")
    if seg_global is None:
        gs = np.array([dynamic_global_scale(w_bits[off[s]:off[s + 1]])
                       for s in range(nseg)], dtype=np.float32)
    else:
        gs = np.asarray(seg_global, dtype=np.float32).reshape(nseg)
    codes = np.empty((w_bits.shape[0], w_bits.shape[1] // 2), dtype=np.uint8)
    scales = np.empty((w_bits.shape[0], w_bits.shape[1] // 16), dtype=np.uint8)
    for s in range(nseg):
        c, sc, _ = quantize(w_bits[off[s]:off[s + 1]], gs[s])
        codes[off[s]:off[s + 1]] = c
        scales[off[s]:off[s + 1]] = sc
    return codes, scales, gs


def packed_bytes(rows, cols):
    """Storage of an NVFP4 tensor: 1/2 byte of code + 1/16 byte of scale per element."""
    return rows * cols // 2 + rows * cols // 16
