"""Reference number formats and error measures for the mechanism study --
TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Part one of the pages' mechanism study credits NVFP4's 16-element block
scaling with keeping an activation outlier inside its own block, so that
activation error comes out alike across layer roles (bayesiansapien page,
"The four-part mechanism study", first item; nefut page, first bullet).  To
measure that, the E2M1 element grid is given coarser scales:

  block(B)    one E4M3 scale per B consecutive elements of a row and the FP32
              global scale, exactly the NVFP4 recipe of ``oracle/quantize.py``
              with 16 replaced by B (B = 16 is NVFP4 itself);
  per_tensor  no block scale: one FP32 scale for the whole tensor,
              r = 6 / amax (one division), code = sign | E2M1_RNE_SAT(|x * r|).

Part two says the gate parameterisations absorb GEMM error (same page,
second item; about 11% GEMM error becomes about 2% after the gate): the
error measures below are the relative L2 error used for that comparison.

Each float step is one float32 operation with round-to-nearest-even, in the
order written; dequantised values and errors are fp64.
"""
import numpy as np

from .formats import E2M1_TABLE, E4M3_POSITIVE, E4M3_TABLE, e2m1_rne_sat, e4m3_rne


def block_quantize(x, g, block):
    """float32 rows [R, C] (C % block == 0), global scale g -> (codes [R, C/block, block], scales [R, C/block]).

    Per block: m = max|x|; t = m / 6; u = min(t * g, 448); S = E4M3_RNE(u);
    S == 0 -> zero codes; else r = g / value(S), code = sign | E2M1_RNE_SAT(|x * r|).
    """
    x = np.asarray(x, dtype=np.float32)
    if x.ndim != 2 or x.shape[1] % block:
        raise ValueError("expected [rows, cols] with cols % block == 0")
    g = np.float32(g)
    rows, cols = x.shape
    blocks = x.reshape(rows, cols // block, block)
    m = np.max(np.abs(blocks), axis=2)
    t = (m / np.float32(6.0)).astype(np.float32)
    u = np.minimum((t * g).astype(np.float32), np.float32(448.0))
    S = e4m3_rne(u)
    nz = S != 0
    s = E4M3_POSITIVE[S].astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(nz, g / np.where(nz, s, np.float32(1.0)), np.float32(0.0)).astype(np.float32)
    q = (blocks * r[:, :, None]).astype(np.float32)
    codes = ((np.signbit(blocks).astype(np.uint8) << 3) | e2m1_rne_sat(np.abs(q))).astype(np.uint8)
    codes[~nz] = 0
    return codes, S


def block_dequantize(codes, scales, g):
    """fp64 values e2m1(code) * e4m3(S) / g, [R, C] (codes [R, C/B, B] or [R, C] with B inferred)."""
    codes = np.asarray(codes)
    S = np.asarray(scales)
    if codes.ndim == 2:
        codes = codes.reshape(S.shape[0], S.shape[1], -1)
    v = E2M1_TABLE[codes] * E4M3_TABLE[S][:, :, None] / np.float64(g)
    return v.reshape(v.shape[0], -1)


def per_tensor_quantize(x):
    """float32 tensor -> (codes uint8 same shape, r float32): one scale r = 6 / amax for everything."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.float32(np.max(np.abs(x)))
    r = np.float32(1.0) if amax == 0 else np.float32(np.float32(6.0) / amax)
    q = (x * r).astype(np.float32)
    return ((np.signbit(x).astype(np.uint8) << 3) | e2m1_rne_sat(np.abs(q))).astype(np.uint8), r


def per_tensor_dequantize(codes, r):
    return E2M1_TABLE[np.asarray(codes)] / np.float64(r)


def rel_l2(approx, exact, mask=None):
    """||approx - exact|| / ||exact|| in fp64, over `mask` if given."""
    a = np.asarray(approx, dtype=np.float64)
    e = np.asarray(exact, dtype=np.float64)
    if mask is not None:
        a, e = a[mask], e[mask]
    den = np.linalg.norm(e)
    return float(np.linalg.norm(a - e) / den) if den > 0 else 0.0


def contaminated_mask(shape, outlier_cols, block):
    """Elements that share a block (of `block` columns; None = the whole tensor) with an outlier
    column, the outlier columns themselves excluded."""
    rows, cols = shape
    hit = np.zeros(cols, dtype=bool)
    if block is None:
        hit[:] = len(outlier_cols) > 0
    else:
        for c in outlier_cols:
            b0 = (int(c) // block) * block
            hit[b0:b0 + block] = True
    hit[np.asarray(outlier_cols, dtype=np.int64)] = False
    return np.broadcast_to(hit, (rows, cols))
