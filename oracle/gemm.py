"""fp64 NVFP4 dequantisation and W4A4 GEMM -- TEST INFRASTRUCTURE ONLY.

The W4A4 linear layer of the pages (bayesiansapien page, TL;DR: 4-bit
weights and 4-bit activations) computes y = A W^T with both operands held as
NVFP4.  Dequantised element value = e2m1(code) * e4m3(scale byte); the global
scales are not folded into the elements but divided out of the product:

    y[m, n] = sum_k vA[m, k] * vW[n, k] / (g_A * g_W[seg(n)])

where seg(n) is the weight module (row segment of the fused weight) that
output column n belongs to.  Keeping one g_W per segment is the repair of the
global-scale mismatch of fused kernels (bayesiansapien page, "Two practical
repairs"; aimodeling page, "What engineers should actually take away").

Acceptance bound used by the tests, per output element:
    B[m, n] = sum_k |vA[m, k] * vW[n, k]| / (g_A * g_W[seg(n)])
    |y_gpu - y| <= 1e-5 * B           (FP32 outputs)
A numpy float64 matmul serves as the summation step; it is exact up to
float64 rounding, far below the bound.
"""
import numpy as np

from .formats import E2M1_TABLE, E4M3_TABLE
from .quantize import unpack_nibbles

GEMM_REL_TOL = 1e-5
BF16_UNIT_ROUNDOFF = 2.0 ** -8


def dequant(codes, scales):
    """codes [R, C/2] bytes + scales [R, C/16] bytes -> float64 [R, C] (no global)."""
    nib = unpack_nibbles(codes)
    rows, cols = nib.shape
    vals = E2M1_TABLE[nib].reshape(rows, cols // 16, 16)
    sc = E4M3_TABLE[np.asarray(scales, dtype=np.uint8)]
    if np.any(np.isnan(sc)):
        raise ValueError("scale byte 0x7F / 0xFF (NaN) in an NVFP4 tensor")
    return (vals * sc[:, :, None]).reshape(rows, cols)


def column_global(n, seg_offsets, seg_global):
    """Per-output-column weight global scale from a segment table."""
    g = np.empty(n, dtype=np.float64)
    off = [int(o) for o in seg_offsets]
    for s in range(len(off) - 1):
        g[off[s]:off[s + 1]] = np.float64(np.float32(seg_global[s]))
    return g


def gemm(a_codes, a_scales, g_a, w_codes, w_scales, g_w_col):
    """fp64 W4A4 GEMM.  g_w_col: per-output-column weight global scale [N].

    Returns (y [M, N] float64, bound [M, N] float64).
    """
    va = dequant(a_codes, a_scales)
    vw = dequant(w_codes, w_scales)
    denom = np.float64(np.float32(g_a)) * np.asarray(g_w_col, dtype=np.float64)[None, :]
    y = (va @ vw.T) / denom
    bound = (np.abs(va) @ np.abs(vw).T) / denom
    return y, bound


def bf16_round(y):
    """Round float64 values to the nearest bf16 (ties to even), returned as float64.

    bf16 keeps 8 significant bits: with y = m * 2**e, 0.5 <= |m| < 1, the
    result is rint(m * 2**8) * 2**(e - 8) (numpy's rint rounds half to even).
    Normal range only (|y| >= 2**-126), which is all the oracle needs.
    """
    y = np.asarray(y, dtype=np.float64)
    m, e = np.frexp(y)
    return np.ldexp(np.rint(m * 256.0), e - 8)


def f64_to_bf16_bits(y):
    """bf16 bit patterns (uint16) of bf16_round(y)."""
    r = bf16_round(y).astype(np.float32)          # exact: 8-bit significand
    return (r.view(np.uint32) >> 16).astype(np.uint16)


def tolerance(bound, y_ref, out_is_bf16):
    """Per-element acceptance: 1e-5*B, plus bf16 output rounding when stored as bf16."""
    tol = GEMM_REL_TOL * bound
    if out_is_bf16:
        tol = tol + BF16_UNIT_ROUNDOFF * (np.abs(y_ref) + tol)
    return tol
