"""The two repairs of the fused-module global-scale mismatch, side by side on
the fused GDN in-projection (bayesiansapien page, mechanism study, "Two
practical repairs"; aimodeling page, "What engineers should actually take
away").  Six modules whose weights differ up to 8x in magnitude, so their
calibrated global scales differ:
  per-segment alpha  each module keeps its own global scale; the epilogue
                     applies alpha_s = 1 / (g_a g_w[s]) per column segment;
  pre-harmonised     the fused weight is quantised with one shared global
                     scale (2688 / amax over all modules), so one alpha
                     serves every column and a plain GEMM is correct.
Parity: each GPU result is within the GEMM tolerance of the oracle run on
the same quantisation; the single-alpha GEMM and the segmented entry point
given six equal scales write the same bits.
Measurement: per module, the relative L2 error of each repair against the
exact product of the unquantised bf16 operands (fp64), with the mismatched
single alpha (each module's own scale, alpha of module 0) as the negative
control.  An 8x magnitude spread keeps every shared-scale block scale in
E4M3's normal range, so the two repairs come out within a few percent of
each other, while the mismatch is off by the scale ratio.
"""
import numpy as np
import pytest
import torch

from nvfp4_w4a4_gemm_quantize_amd import inputs
from tests.parity import OG, assert_bytes_equal, check_gemm, dev_bf16, gpu_out_f64, host
from tests.test_gpu_gemm import gpu_prepare, oracle_prepare

pytestmark = pytest.mark.gpu


def rel_l2(y, ref):
    return float(np.linalg.norm(y - ref) / np.linalg.norm(ref))


def test_repairs_parity_and_error(gpu_lib):
    d = inputs.gdn_inproj(M=128)
    K = 5120
    offs = [int(v) for v in d["seg_offsets"]]
    N = offs[-1]
    names = d["seg_names"]
    # per-module scales + per-segment alpha
    ac, asc, ag, packed_m, wg_m = gpu_prepare(gpu_lib, d["A"], d["W"], offs)
    y_seg = gpu_lib.gemm_w4a4_fused_segments(ac, asc, ag, packed_m, N, K, offs, wg_m, None,
                                             out_dtype=torch.float32)
    # one shared scale for the fused weight + one alpha
    packed_h, wg_h = gpu_lib.nvfp4_pack_weights(dev_bf16(d["W"]))
    y_harm = gpu_lib.gemm_w4a4(ac, asc, ag, packed_h, wg_h, N, K, out_dtype=torch.float32)
    y_harm_seg = gpu_lib.gemm_w4a4_fused_segments(ac, asc, ag, packed_h, N, K, offs, wg_h.repeat(len(offs) - 1),
                                                  None, out_dtype=torch.float32)
    assert_bytes_equal(host(y_harm_seg).view(np.uint32), host(y_harm).view(np.uint32),
                       "single alpha vs six equal segment scales")
    # negative control: per-module scales, one alpha
    y_mis = gpu_lib.gemm_w4a4(ac, asc, ag, packed_m, wg_m[:1], N, K, out_dtype=torch.float32)

    ca, sa, ga, cw, sw, gs, gcol = oracle_prepare(d["A"], d["W"], offs)
    yr, br = OG.gemm(ca, sa, ga, cw, sw, gcol)
    check_gemm(gpu_out_f64(y_seg), yr, br, False, "per-segment alpha")
    ca2, sa2, ga2, cw2, sw2, gs2, gcol2 = oracle_prepare(d["A"], d["W"])
    assert float(gs2[0]) == float(host(wg_h)[0]) == float(gs.min())   # the shared scale is the smallest
    yr2, br2 = OG.gemm(ca2, sa2, ga2, cw2, sw2, gcol2)
    check_gemm(gpu_out_f64(y_harm), yr2, br2, False, "pre-harmonised single alpha")

    a64 = inputs.bf16_bits_to_f32(d["A"]).astype(np.float64)
    w64 = inputs.bf16_bits_to_f32(d["W"]).astype(np.float64)
    y_exact = a64 @ w64.T
    ys, yh, ym = gpu_out_f64(y_seg), gpu_out_f64(y_harm), gpu_out_f64(y_mis)
    report = []
    for s in range(len(offs) - 1):
        c = slice(offs[s], offs[s + 1])
        e_s, e_h, e_m = rel_l2(ys[:, c], y_exact[:, c]), rel_l2(yh[:, c], y_exact[:, c]), rel_l2(ym[:, c], y_exact[:, c])
        report.append("%s: per-segment %.4f  harmonised %.4f  mismatch %.4f  (g_w ratio to module 0: %.3f)" % (
            names[s], e_s, e_h, e_m, gs[s] / gs[0]))
        assert 0.02 < e_s < 0.2 and 0.02 < e_h < 0.2, report[-1]
        assert abs(e_h - e_s) <= 0.1 * e_s, report[-1]
        if abs(gs[s] / gs[0] - 1.0) > 0.2:
            assert e_m > 1.4 * e_s, report[-1]
    print("\n".join(report))

