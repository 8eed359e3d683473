"""Mechanism harness on the oracle and the GPU path (bayesiansapien page,
"The four-part mechanism study", first two items).

1. Outlier locality of 16-element block scaling.  Activations of four
   synthetic "roles" (Student-t(4) and normal, each with and without five
   outlier channels x50) are quantised by the GPU quantizer (NVFP4: E4M3
   scale per 16 elements), whose codes must equal the oracle's bit for bit,
   and by the oracle's coarser references (E4M3 scale per 32 and 64
   elements; one per-tensor scale).  Measured per format: the relative L2
   error overall, on the non-outlier elements, and the share of elements
   that sit in an outlier's block.  Checked: that share is 5 * 15 of the
   K - 5 non-outlier elements at 16 and grows with the block; the
   non-outlier error grows with the block and is worst per tensor; the
   16-element format's error varies little across roles while the
   per-tensor one varies several-fold.
2. Gate error.  On the fused GDN in-projection, the GPU's pre-gate GEMM
   output of the b and a columns against the exact product of the
   unquantised bf16 operands, and the post-gate error of sigmoid(b) and
   -exp(A_log) * softplus(a + dt_bias).  Checked: the fused gate epilogue
   equals the gate applied to the GPU's own pre-gate values (to fp32
   evaluation error), and the gates' Lipschitz bounds (1/4 for the sigmoid,
   exp(A_log) for the decay) hold element by element.  Measured: relative
   errors before and after each gate, with the gate input scaled by powers
   of two (NVFP4 with a dynamic global scale quantises a weight scaled by
   2^j to exactly 2^j times the same result, so one GEMM serves the sweep).
"""
import numpy as np
import pytest
import torch

from nvfp4_w4a4_gemm_quantize_amd import inputs
from oracle import mechanism as MX
from tests.parity import OE, OQ, assert_bytes_equal, dev_bf16, f32, gpu_out_f64, host
from tests.test_gpu_gemm import gpu_prepare

pytestmark = pytest.mark.gpu

M_ROWS, K = 256, 5120


def roles():
    return {
        "t4 + outliers": (inputs.student_t_activations(M_ROWS, K, "mech/t4o"), "mech/t4o/outliers"),
        "t4": (inputs.student_t_activations(M_ROWS, K, "mech/t4", outlier_gain=1.0), None),
        "normal + outliers": (inputs.normal_activations(M_ROWS, K, "mech/no"), "mech/no/outliers"),
        "normal": (inputs.normal_activations(M_ROWS, K, "mech/n", n_outliers=0), None),
    }


def test_block_scaling_localises_outliers(gpu_lib):
    table, overall = [], {16: [], 32: [], 64: [], "tensor": []}
    for name, (bits, oc_name) in roles().items():
        x = inputs.bf16_bits_to_f32(bits)
        codes, scales, g = gpu_lib.nvfp4_quantize(dev_bf16(bits))
        oc, os_, og = OQ.quantize(bits)
        assert float(host(g)[0]) == float(og)
        assert_bytes_equal(host(codes), oc, name + " codes")
        assert_bytes_equal(host(scales), os_, name + " scales")
        gq = np.float32(host(g)[0])
        deq = {16: MX.block_dequantize(OQ.unpack_nibbles(host(codes)), host(scales), gq)}
        for B in (32, 64):
            c, S = MX.block_quantize(x, gq, B)
            deq[B] = MX.block_dequantize(c, S, gq)
        c, r = MX.per_tensor_quantize(x)
        deq["tensor"] = MX.per_tensor_dequantize(c, r)
        ocols = [] if oc_name is None else list(inputs.outlier_channels(K, 5, oc_name))
        non = np.ones(K, dtype=bool)
        non[ocols] = False
        non = np.broadcast_to(non, x.shape)
        errs = {}
        for fmt, v in deq.items():
            cm = MX.contaminated_mask(x.shape, ocols, None if fmt == "tensor" else fmt)
            errs[fmt] = (MX.rel_l2(v, x), MX.rel_l2(v, x, non), cm[0].sum() / non[0].sum())
            overall[fmt].append(errs[fmt][0])
            table.append("%-18s %-6s overall %.4f  non-outlier %.4f  in an outlier's block %.4f" % (
                name, fmt, *errs[fmt]))
        if ocols:
            assert errs[16][2] == pytest.approx(5 * 15 / (K - 5))
            assert errs[16][2] < errs[32][2] < errs[64][2] < errs["tensor"][2] == 1.0
            assert errs[16][1] < errs[32][1] < errs[64][1] < errs["tensor"][1]
    spread = {f: max(v) / min(v) for f, v in overall.items()}
    table.append("spread of the overall error across roles (max/min): " +
                 "  ".join("%s %.2f" % (f, s) for f, s in spread.items()))
    print("\n" + "\n".join(table))
    assert spread[16] < 1.5 and spread["tensor"] > 3.0


def test_gate_error_through_sigmoid_and_decay(gpu_lib):
    d = inputs.gdn_inproj(M=M_ROWS)
    offs = [int(v) for v in d["seg_offsets"]]
    N = offs[-1]
    ac, asc, ag, packed, wg = gpu_prepare(gpu_lib, d["A"], d["W"], offs)
    a_log, dt = d["A_log"], d["dt_bias"]
    y_pre = gpu_lib.gemm_w4a4_fused_segments(ac, asc, ag, packed, N, K, offs, wg, None, out_dtype=torch.float32)
    y_post = gpu_lib.gemm_w4a4_fused_segments(ac, asc, ag, packed, N, K, offs, wg,
                                              ["none"] * 4 + ["sigmoid", "gdn_decay"], f32(a_log), f32(dt),
                                              out_dtype=torch.float32)
    b = slice(offs[4], offs[5])
    a = slice(offs[5], offs[6])
    pre, post = gpu_out_f64(y_pre), gpu_out_f64(y_post)
    a64 = inputs.bf16_bits_to_f32(d["A"]).astype(np.float64)
    w64 = inputs.bf16_bits_to_f32(d["W"][offs[4]:offs[6]]).astype(np.float64)
    ex = a64 @ w64.T
    ex_b, ex_a = ex[:, :offs[5] - offs[4]], ex[:, offs[5] - offs[4]:]
    # the fused epilogue is the gate of the GEMM's own fp32 result
    np.testing.assert_allclose(post[:, b], OE.sigmoid(pre[:, b]), rtol=0, atol=2e-6)
    np.testing.assert_allclose(post[:, a], OE.gdn_decay(pre[:, a], a_log, dt), rtol=2e-5, atol=1e-6)
    # Lipschitz bounds of the gates, element by element
    lip_a = np.exp(a_log.astype(np.float64))[None, :]
    assert np.all(np.abs(post[:, b] - OE.sigmoid(ex_b)) <= 0.25 * np.abs(pre[:, b] - ex_b) + 2e-6)
    assert np.all(np.abs(post[:, a] - OE.gdn_decay(ex_a, a_log, dt)) <=
                  lip_a * np.abs(pre[:, a] - ex_a) * (1 + 1e-6) + 2e-5 * np.abs(post[:, a]) + 1e-6)
    # measured: relative L2 error before and after each gate, gate input scaled by 2^j
    lines = ["gate input scale   b: GEMM -> sigmoid     a: GEMM -> decay"]
    for j in range(-4, 3):
        c = 2.0 ** j
        lines.append("2^%-3d              %.4f -> %.4f        %.4f -> %.4f" % (
            j, MX.rel_l2(c * pre[:, b], c * ex_b), MX.rel_l2(OE.sigmoid(c * pre[:, b]), OE.sigmoid(c * ex_b)),
            MX.rel_l2(c * pre[:, a], c * ex_a),
            MX.rel_l2(OE.gdn_decay(c * pre[:, a], a_log, dt), OE.gdn_decay(c * ex_a, a_log, dt))))
    lines.append("median |gate input| at scale 1: b %.2f, a %.2f" % (np.median(np.abs(ex_b)), np.median(np.abs(ex_a))))
    print("\n" + "\n".join(lines))
