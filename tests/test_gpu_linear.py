"""GPU parity of nvfp4_linear, the W4A4 layer on a bf16 activation (the
on-the-fly "A4" quantizer feeding the GEMM; bayesiansapien page, TL;DR).

For every shape: the quantised activation it writes is bit-exact against the
oracle quantizer (codes, scale bytes, global scale), its output is
bit-identical to nvfp4_quantize + gemm_w4a4 on the same input, and within
1e-5 * sum|a*w| * alpha (+ bf16 rounding) of the fp64 oracle.  Decode shapes
(m <= 2, K <= 6144) run the one-kernel path that quantises inside the GEMM;
the others run the two calls."""
import functools

import numpy as np
import pytest
import torch

from nvfp4_w4a4_gemm_quantize_amd import inputs
from tests.parity import (OG, OQ, assert_bytes_equal, check_gemm, dev_bf16, f32, gpu_out_f64, host,
                          oracle_gemm_rows, oracle_quantize_rows)

pytestmark = pytest.mark.gpu


@functools.lru_cache(maxsize=4)
def packed_weight(N, K, seed):
    """bf16 weight bits, its oracle codes/scales and g (dynamic, one module)."""
    if (N, K, seed) == (17408, 5120, 0):
        w_bits = inputs.decode(1)["W"]
    else:
        rng = np.random.default_rng(seed)
        w_bits = inputs.f32_to_bf16_bits((rng.standard_normal((N, K)) / np.sqrt(K)).astype(np.float32))
    g = np.float32(OQ.dynamic_global_scale(w_bits))
    cw, sw = oracle_quantize_rows(w_bits, g)
    return w_bits, cw, sw, g


def activation(M, K, seed):
    rng = np.random.default_rng(seed)
    a = rng.standard_t(4, size=(M, K)).astype(np.float32)
    a[:, rng.choice(K, max(1, K // 1000), replace=False)] *= 50
    return inputs.f32_to_bf16_bits(a)


def run_case(lib, M, N, K, seed, out_dtype=torch.bfloat16, static_g=None, ld_x=None):
    w_bits, cw, sw, gw = packed_weight(N, K, 0 if N == 17408 else seed)
    packed, wg = lib.nvfp4_pack_weights(dev_bf16(w_bits))
    a_bits = activation(M, K, seed)
    x = dev_bf16(a_bits)
    if ld_x is not None:
        wide = torch.zeros((M, ld_x), dtype=torch.bfloat16, device="cuda")
        wide[:, :K] = x
        x = wide[:, :K]
    ag = None if static_g is None else f32([static_g])
    y, ac, asc, agout = lib.nvfp4_linear(x, packed, wg, N, out_dtype=out_dtype, a_global=ag,
                                         dynamic=static_g is None)
    # the two-call path on the same input
    ac2, asc2, ag2 = lib.nvfp4_quantize(x, None if static_g is None else f32([static_g]), dynamic=static_g is None)
    y2 = lib.gemm_w4a4(ac2, asc2, ag2, packed, wg, N, K, out_dtype=out_dtype)
    torch.cuda.synchronize()
    oc, os_, og = OQ.quantize(a_bits, None if static_g is None else np.float32(static_g))
    assert np.float32(host(agout)[0]) == og
    assert_bytes_equal(host(asc), os_, "linear M=%d scales" % M)
    assert_bytes_equal(host(ac), oc, "linear M=%d codes" % M)
    assert torch.equal(y, y2), "nvfp4_linear differs from nvfp4_quantize + gemm_w4a4 (M=%d)" % M
    yr, br = oracle_gemm_rows(oc, os_, og, cw, sw, OG.column_global(N, [0, N], np.array([gw], np.float32)))
    check_gemm(gpu_out_f64(y), yr, br, out_dtype == torch.bfloat16, "linear %dx%dx%d" % (M, N, K))


@pytest.mark.parametrize("M,N,K,out", [
    (1, 17408, 5120, "bf16"), (2, 17408, 5120, "bf16"), (3, 17408, 5120, "f32"), (4, 17408, 5120, "bf16"),
    (1, 1000, 5120, "f32"), (2, 200, 6144, "f32"),       # one kernel: ragged N; the longest fused K at m <= 2
    (1, 96, 48, "f32"), (4, 160, 5136, "bf16"),          # K = 16 (mod 32); m = 4 (two calls)
    (1, 5120, 17408, "bf16"),                             # K beyond the fused staging: two calls
    (8, 17408, 5120, "bf16"), (37, 640, 5120, "f32"),    # f16 decode kernel
    (300, 520, 320, "bf16"),                              # tiled kernel
])
def test_linear_matches_two_calls_and_oracle(gpu_lib, M, N, K, out):
    run_case(gpu_lib, M, N, K, seed=M * 131 + N + K, out_dtype=torch.float32 if out == "f32" else torch.bfloat16)


def test_linear_static_global_scale(gpu_lib):
    """A calibrated activation scale (read, not written), small enough that blocks saturate."""
    run_case(gpu_lib, 1, 17408, 5120, seed=5, static_g=3.0)
    run_case(gpu_lib, 2, 1000, 5120, seed=6, static_g=300.0)


def test_linear_strided_activation(gpu_lib):
    run_case(gpu_lib, 2, 17408, 5120, seed=7, ld_x=5200)


def test_linear_zero_activation(gpu_lib):
    """amax = 0: g = 1, every scale and code 0, output 0."""
    packed, wg = gpu_lib.nvfp4_pack_weights(dev_bf16(packed_weight(17408, 5120, 0)[0]))
    x = torch.zeros((1, 5120), dtype=torch.bfloat16, device="cuda")
    y, ac, asc, ag = gpu_lib.nvfp4_linear(x, packed, wg, 17408, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert float(ag.item()) == 1.0 and not host(ac).any() and not host(asc).any()
    assert not host(y).any()


def test_linear_back_to_back_and_in_a_graph(gpu_lib):
    """Two calls in a row on one stream (the second with fewer rows) and the
    same calls replayed from a HIP graph give the eager results bit for bit."""
    w_bits = packed_weight(17408, 5120, 0)[0]
    packed, wg = gpu_lib.nvfp4_pack_weights(dev_bf16(w_bits))
    xs = [dev_bf16(activation(m, 5120, 40 + m)) for m in (3, 1)]
    eager = [gpu_lib.nvfp4_linear(x, packed, wg, 17408)[0].clone() for x in xs]
    outs = [torch.empty_like(e) for e in eager]

    def calls():
        for x, o in zip(xs, outs):
            gpu_lib.nvfp4_linear(x, packed, wg, 17408, out=o)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    for _ in range(3):
        for o in outs:
            o.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o, e)
