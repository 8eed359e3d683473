"""Helpers shared by the GPU parity tests: device transfer, the oracle side of
each comparison, and the acceptance checks (bit-exact codes/scales; GEMM
outputs within 1e-5 * sum|a*w| * alpha, plus bf16 output rounding)."""
import numpy as np
import torch

from oracle import epilogue as OE
from oracle import gemm as OG
from oracle import quantize as OQ


def dev_bf16(bits):
    """numpy bf16 bit patterns -> contiguous torch.bfloat16 on cuda:0."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return torch.from_numpy(b.view(np.int16)).to("cuda").view(torch.bfloat16)


def host(t):
    return t.detach().cpu().numpy()


def f32(x):
    return torch.tensor(np.asarray(x, dtype=np.float32).reshape(-1), device="cuda")


def oracle_quantize_rows(bits, g, chunk=4096):
    """Oracle quantisation of a large tensor with a known global scale, in row chunks."""
    codes, scales = [], []
    for r0 in range(0, bits.shape[0], chunk):
        c, s, _ = OQ.quantize(bits[r0:r0 + chunk], g)
        codes.append(c)
        scales.append(s)
    return np.concatenate(codes), np.concatenate(scales)


def assert_bytes_equal(got, want, what):
    got, want = np.asarray(got), np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    bad = np.argwhere(got != want)
    assert bad.size == 0, "%s: %d mismatching bytes, first at %s (got %s want %s)" % (
        what, len(bad), tuple(bad[0]), got[tuple(bad[0])], want[tuple(bad[0])])


def oracle_gemm_rows(a_codes, a_scales, g_a, w_codes, w_scales, g_w_col, col_chunk=4096):
    """fp64 y and bound for the given A rows against every W row, in column chunks."""
    ys, bs = [], []
    for c0 in range(0, w_codes.shape[0], col_chunk):
        y, b = OG.gemm(a_codes, a_scales, g_a, w_codes[c0:c0 + col_chunk], w_scales[c0:c0 + col_chunk],
                       g_w_col[c0:c0 + col_chunk])
        ys.append(y)
        bs.append(b)
    return np.concatenate(ys, axis=1), np.concatenate(bs, axis=1)


def gpu_out_f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def assert_within(got, ref, tol, what):
    err = np.abs(got - ref)
    bad = np.argwhere(~(err <= tol))
    if bad.size:
        i = tuple(bad[0])
        raise AssertionError("%s: %d of %d outside tolerance; first %s got %r want %r tol %r (worst err/tol %.3g)" % (
            what, len(bad), err.size, i, got[i], ref[i], tol[i], float(np.max(err / np.maximum(tol, 1e-300)))))


def check_gemm(got, y, bound, out_is_bf16, what):
    assert_within(got, y, OG.tolerance(bound, y, out_is_bf16), what)


__all__ = ["dev_bf16", "host", "f32", "oracle_quantize_rows", "assert_bytes_equal", "oracle_gemm_rows",
           "gpu_out_f64", "assert_within", "check_gemm", "OE", "OG", "OQ"]
