"""GPU parity of the quantising SiLU*mul epilogue (gemm_w4a4_silu_mul_quantize).

The MLP's activation h = silu(gate) * up leaves the gate/up GEMM as NVFP4
codes and scales, quantised with a static (calibrated) global scale.  Checked
stage by stage, as the unfused chain is:
  (i)   the bf16 h the epilogue quantised (returned on request) is within the
        SiLU*mul tolerance of the fp64 oracle;
  (ii)  its codes and scale bytes equal the oracle quantiser's on those same
        h bits with the same static scale, bit for bit;
  (iii) the call without the h output writes the same bytes, and h equals the
        unfused tiled kernel's bf16 h;
  (iv)  at the full MLP size, on sampled rows, the same, and the down
        projection run on the fused codes is within the GEMM tolerance.
A static scale above 2688/amax(h) makes blocks saturate (scale clamped to
448, codes to 6); the oracle's quantiser applies the same clamps.
"""
import numpy as np
import pytest
import torch

from nvfp4_w4a4_gemm_quantize_amd import inputs
from tests.parity import (OE, OG, OQ, assert_bytes_equal, assert_within, check_gemm, dev_bf16, f32, gpu_out_f64,
                          host, oracle_gemm_rows)
from tests.test_gpu_gemm import gpu_prepare, oracle_prepare, sample_rows

pytestmark = pytest.mark.gpu


def bf16_bits(t):
    return host(t.view(torch.int16)).view(np.uint16)


def fused(lib, ac, asc, ag, packed, wg, n, k, gh, return_h):
    return lib.gemm_w4a4_silu_mul_quantize(ac, asc, ag, packed, wg, n, k, f32([gh]), return_h=return_h)


@pytest.mark.parametrize("M,K,N", [
    (1, 192, 256),       # three K steps: the register-staged tiled kernel; one row
    (40, 256, 256),      # four K steps: the DMA kernel; rows past m
    (130, 320, 512),     # ragged m over two row tiles
    (300, 96, 128),      # k % 64 != 0: register-staged kernel, ragged K tile
    (512, 256, 38400),   # 300 tiles: the last 44 run as half-height tiles
])
@pytest.mark.parametrize("g_factor", [1.0, 4.0])
def test_fused_quantize_small(gpu_lib, M, K, N, g_factor):
    rng = np.random.default_rng(700 + M)
    a = rng.standard_t(4, size=(M, K)).astype(np.float32)
    w = (rng.standard_normal((N, K)) / 8).astype(np.float32)
    a_bits, w_bits = inputs.f32_to_bf16_bits(a), inputs.f32_to_bf16_bits(w)
    ac, asc, ag, packed, wg = gpu_prepare(gpu_lib, a_bits, w_bits)
    # a calibrated scale for h: from the unfused kernel's h, optionally too
    # large so that blocks saturate
    h_unfused = gpu_lib.gemm_w4a4(ac, asc, ag, packed, wg, N, K, out_dtype=torch.bfloat16, epilogue="silu_mul")
    gh = np.float32(OQ.dynamic_global_scale(bf16_bits(h_unfused)) * g_factor)

    hc, hs, h = fused(gpu_lib, ac, asc, ag, packed, wg, N, K, gh, True)
    h_bits = bf16_bits(h)
    # (i) h against the fp64 oracle
    ca, sa, ga, cw, sw, gs, gcol = oracle_prepare(a_bits, w_bits)
    yr, br = OG.gemm(ca, sa, ga, cw, sw, gcol)
    g_, u_ = yr[:, :N // 2], yr[:, N // 2:]
    tol = OE.silu_mul_tolerance(g_, u_, OG.GEMM_REL_TOL * br[:, :N // 2], OG.GEMM_REL_TOL * br[:, N // 2:], True)
    assert_within(inputs.bf16_bits_to_f32(h_bits).astype(np.float64), OE.silu_mul(g_, u_), tol,
                  "fused h M=%d" % M)
    # (ii) codes and scales against the oracle quantiser on the same h bits
    oc, os_, _ = OQ.quantize(h_bits, gh)
    assert_bytes_equal(host(hc), oc, "fused h codes M=%d" % M)
    assert_bytes_equal(host(hs), os_, "fused h scales M=%d" % M)
    if g_factor > 1.0:
        assert (os_ == 0x7E).any(), "the oversized scale should saturate some blocks"
    # (iii) the same bytes without the h output; h equals the unfused tiled kernel's
    hc2, hs2 = fused(gpu_lib, ac, asc, ag, packed, wg, N, K, gh, False)
    assert_bytes_equal(host(hc2), host(hc), "codes without h output")
    assert_bytes_equal(host(hs2), host(hs), "scales without h output")
    if M > 64:   # both calls run the tiled kernel (smaller m streams weights in gemm_w4a4)
        assert_bytes_equal(h_bits, bf16_bits(h_unfused), "fused h vs unfused h")


def test_fused_quantize_rejects_bad_arguments(gpu_lib):
    rng = np.random.default_rng(5)
    a_bits = inputs.f32_to_bf16_bits(rng.standard_normal((8, 128)).astype(np.float32))
    w_bits = inputs.f32_to_bf16_bits(rng.standard_normal((96, 128)).astype(np.float32))
    ac, asc, ag, packed, wg = gpu_prepare(gpu_lib, a_bits, w_bits)
    with pytest.raises(gpu_lib.NVFP4Error):   # n % 64 != 0
        fused(gpu_lib, ac, asc, ag, packed, wg, 96, 128, 1.0, False)


def test_fused_quantize_mlp_config(gpu_lib):
    """Full MLP size (M 4096, gate_up N 34816, K 5120; down K 17408) on sampled rows."""
    d = inputs.mlp()
    M, K, N2, KD = 4096, 5120, 34816, 17408
    ac, asc, ag, packed, wg = gpu_prepare(gpu_lib, d["A"], d["W_gate_up"])
    # static scale of h calibrated on another batch (seed 1) through the unfused path
    cal = inputs.mlp(seed=1, M=512, weights=False)["A"]
    cac, casc, cag = gpu_lib.nvfp4_quantize(dev_bf16(cal))
    h_cal = gpu_lib.gemm_w4a4(cac, casc, cag, packed, wg, N2, K, out_dtype=torch.bfloat16, epilogue="silu_mul")
    _, _, gh_t = gpu_lib.nvfp4_quantize(h_cal)
    gh = np.float32(host(gh_t)[0])

    hc, hs, h = fused(gpu_lib, ac, asc, ag, packed, wg, N2, K, gh, True)
    hc2, hs2 = fused(gpu_lib, ac, asc, ag, packed, wg, N2, K, gh, False)
    assert_bytes_equal(host(hc2), host(hc), "codes without h output")
    assert_bytes_equal(host(hs2), host(hs), "scales without h output")
    rows = sample_rows(M, 12)
    sel = torch.as_tensor(rows, device="cuda")
    h_bits = bf16_bits(h[sel])
    ca, sa, ga, cw, sw, gs, gcol = oracle_prepare(d["A"], d["W_gate_up"], rows=rows)
    yr, br = oracle_gemm_rows(ca, sa, ga, cw, sw, gcol)
    g_, u_ = yr[:, :KD], yr[:, KD:]
    tol = OE.silu_mul_tolerance(g_, u_, OG.GEMM_REL_TOL * br[:, :KD], OG.GEMM_REL_TOL * br[:, KD:], True)
    assert_within(inputs.bf16_bits_to_f32(h_bits).astype(np.float64), OE.silu_mul(g_, u_), tol, "fused h rows")
    oc, os_, _ = OQ.quantize(h_bits, gh)
    assert_bytes_equal(host(hc[sel]), oc, "fused h codes rows")
    assert_bytes_equal(host(hs[sel]), os_, "fused h scales rows")
    # the down projection consumes the fused codes directly
    packed2, wg2 = gpu_lib.nvfp4_pack_weights(dev_bf16(d["W_down"]))
    y = gpu_lib.gemm_w4a4(hc, hs, f32([gh]), packed2, wg2, 5120, KD, out_dtype=torch.bfloat16)
    _, _, _, cw2, sw2, gs2, gcol2 = oracle_prepare(h_bits[:1], d["W_down"])
    yr2, br2 = oracle_gemm_rows(oc, os_, gh, cw2, sw2, gcol2)
    check_gemm(gpu_out_f64(y[sel]), yr2, br2, True, "down on fused codes")
