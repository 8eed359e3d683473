"""GPU parity of the W4A4 GEMMs against the fp64 oracle.

Inputs come from the seeded generators and are quantised by the oracle for
the expected side; the GPU side runs the whole HIP path (quantizer, packer,
GEMM).  Acceptance per element: |y_gpu - y| <= 1e-5 * sum_k |a_k w_k| * alpha
(+ bf16 output rounding), bit-exact where the GEMM is an exact small-integer
product, and Lipschitz-propagated bounds through the epilogues.
"""
import functools

import numpy as np
import pytest
import torch

from nvfp4_w4a4_gemm_quantize_amd import inputs
from oracle import formats as F
from tests.parity import (OE, OG, OQ, check_gemm, dev_bf16, f32, gpu_out_f64, host, assert_within,
                          oracle_gemm_rows, oracle_quantize_rows)

pytestmark = pytest.mark.gpu


def gpu_prepare(lib, a_bits, w_bits, offs=None, a_g=None, w_g=None):
    """Quantise A and pack W on the GPU (dynamic scales unless given)."""
    a = dev_bf16(a_bits)
    ac, asc, ag = lib.nvfp4_quantize(a, None if a_g is None else f32([a_g]), dynamic=a_g is None)
    packed, wg = lib.nvfp4_pack_weights(dev_bf16(w_bits), offs, None if w_g is None else f32(w_g),
                                        dynamic=w_g is None)
    return ac, asc, ag, packed, wg


def oracle_prepare(a_bits, w_bits, offs=None, a_g=None, w_g=None, rows=None):
    ca, sa, ga = OQ.quantize(a_bits, a_g)
    n = w_bits.shape[0]
    offs = [0, n] if offs is None else list(offs)
    if w_g is None:
        gs = np.array([OQ.dynamic_global_scale(w_bits[offs[i]:offs[i + 1]]) for i in range(len(offs) - 1)],
                      dtype=np.float32)
    else:
        gs = np.asarray(w_g, dtype=np.float32)
    cw = np.empty((n, w_bits.shape[1] // 2), np.uint8)
    sw = np.empty((n, w_bits.shape[1] // 16), np.uint8)
    for i in range(len(offs) - 1):
        cw[offs[i]:offs[i + 1]], sw[offs[i]:offs[i + 1]] = oracle_quantize_rows(w_bits[offs[i]:offs[i + 1]], gs[i])
    if rows is not None:
        ca, sa = ca[rows], sa[rows]
    return ca, sa, ga, cw, sw, gs, OG.column_global(n, offs, gs)


# ------------------------------------------------------------ exactness ----
def test_unit_scales_give_the_exact_integer_product(gpu_lib):
    """Oracle pin P8 on the GPU: scale 1.0, g = 1, K = 128 -> exact fp32 result."""
    rng = np.random.default_rng(80)
    for (M, N) in [(16, 64), (100, 96), (1, 64)]:
        K = 128
        ca = rng.integers(0, 16, size=(M, K)).astype(np.uint8)
        cw = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
        cw[:, ::16] = 7                                       # a +6 per block -> scale exactly 1.0
        ca[:, ::16] = 15                                      # a -6 per block
        a_bits = inputs.f32_to_bf16_bits(F.E2M1_TABLE[ca].astype(np.float32))
        w_bits = inputs.f32_to_bf16_bits(F.E2M1_TABLE[cw].astype(np.float32))
        ac, asc, ag, packed, wg = gpu_prepare(gpu_lib, a_bits, w_bits, a_g=1.0, w_g=[1.0])
        assert np.all(host(asc) == 0x38)
        y = gpu_lib.gemm_w4a4(ac, asc, ag, packed, wg, N, K, out_dtype=torch.float32)
        ia = np.rint(2 * F.E2M1_TABLE[ca]).astype(np.int64)
        iw = np.rint(2 * F.E2M1_TABLE[cw]).astype(np.int64)
        np.testing.assert_array_equal(host(y).astype(np.float64) * 4, (ia @ iw.T).astype(np.float64))


# ------------------------------------------------------ full comparison ----
@pytest.mark.parametrize("M,N,K,out", [
    (16, 64, 128, "f32"),        # the tiny workload's shape
    (300, 520, 320, "bf16"),     # several tiles, ragged M and N tails, 5 K tiles
    (129, 100, 96, "f32"),       # N not a multiple of 32, K % 64 == 32
    (65, 160, 64, "bf16"),       # just above the decode limit, a single K tile
    (37, 96, 5120, "f32"),       # decode kernel, long K
    (1, 33, 32, "f32"),          # smallest K
    (7, 1000, 5120, "bf16"),     # f16 decode kernel just above the FP4 path's rows, ragged N
    (5, 64, 320, "f32"),         # f16 decode kernel, a K of 1.25 weight super-tiles
    # decode with A fetched in 4-tile groups (k % 256 == 0); wave ranges are whole
    # groups, so some waves get none:
    (20, 96, 768, "f32"),        # 3 groups over 4 waves
    (45, 64, 256, "bf16"),       # 1 group over 2 waves, two row fragments
    (32, 200, 1280, "bf16"),     # exactly one row fragment, ragged N
    (512, 256, 1024, "bf16"),
    # last-round cuts on 256 CUs (tiles of 256x256, two row blocks at M=512):
    (512, 33184, 256, "bf16"),   # 260 tiles: the last 4 run as 16 pieces of 64x64 each; ragged N
    (512, 35712, 256, "f32"),    # 280 tiles: the last 24 as 8 pieces of 64x128
    (512, 38336, 256, "bf16"),   # 300 tiles: the last 44 as quarters (128x128)
    (512, 46040, 256, "f32"),    # 360 tiles: the last 104 as half-height tiles; ragged N
    # the same cuts with K in whole weight super-tiles, at least one per wave:
    # split-K pieces, four waves each over its own quarter of K
    (512, 33184, 1024, "bf16"),  # 260 tiles: 16 pieces of 2x2 fragments; ragged N
    (512, 35712, 1280, "f32"),   # 280 tiles: 2x4-fragment pieces, K quarters of 1, 1, 1 and 2 super-tiles
    (512, 38336, 1024, "bf16"),  # 300 tiles: 4x4-fragment pieces
    (500, 38336, 1024, "f32"),   # the same with ragged M: the last row band's pieces clamp rows past M
    # 128x320 tiles (five column fragments per wave), chosen when they need fewer rounds:
    (384, 65617, 256, "bf16"),   # 618 tiles: two rounds, the last 106 as 212 half-height pieces; ragged N
    (2048, 5120, 320, "f32"),    # exactly one round of 256 tiles
])
def test_gemm_matches_oracle_everywhere(gpu_lib, M, N, K, out):
    rng = np.random.default_rng(M * 1000003 + N * 101 + K)
    a = rng.standard_t(4, size=(M, K)).astype(np.float32)
    a[:, rng.choice(K, max(1, K // 1000), replace=False)] *= 50
    w = (rng.standard_normal((N, K)) / np.sqrt(K)).astype(np.float32)
    a_bits, w_bits = inputs.f32_to_bf16_bits(a), inputs.f32_to_bf16_bits(w)
    ac, asc, ag, packed, wg = gpu_prepare(gpu_lib, a_bits, w_bits)
    y = gpu_lib.gemm_w4a4(ac, asc, ag, packed, wg, N, K,
                          out_dtype=torch.float32 if out == "f32" else torch.bfloat16)
    ca, sa, ga, cw, sw, gs, gcol = oracle_prepare(a_bits, w_bits)
    yr, br = OG.gemm(ca, sa, ga, cw, sw, gcol)
    check_gemm(gpu_out_f64(y), yr, br, out == "bf16", "gemm %dx%dx%d" % (M, N, K))


@functools.lru_cache(maxsize=1)
def decode_weight_prepared():
    """The decode weight [17408, 5120], its oracle codes/scales/global scale."""
    w_bits = inputs.decode(1)["W"]
    g = OQ.dynamic_global_scale(w_bits)
    cw, sw = oracle_quantize_rows(w_bits, g)
    return w_bits, cw, sw, np.float32(g)


# The FP4-MFMA decode kernel (m <= 8) and the branches around it: two, four and
# eight rows per MFMA (m = 2: the second row of the two-row kernel is stored;
# m = 3, 4: the four-row kernel; m = 5..8: the eight-row kernel, whose A scales
# are read late), compile-time super-tile counts (K = 5120, 4096) and the
# run-time count (K = 3072), the general A staging loop (more A records than
# the unrolled staging covers: m <= 2 at K >= 8192), and the f16 decode kernel
# that takes over when the A records exceed the LDS budget.
@pytest.mark.parametrize("M,N,K,out", [
    (2, 17408, 5120, "bf16"), (3, 17408, 5120, "bf16"), (4, 17408, 5120, "bf16"),   # the decode config's W
    (2, 1000, 5120, "f32"), (3, 1000, 5120, "f32"), (4, 1000, 5120, "f32"),         # ragged N
    (1, 5120, 17408, "f32"), (2, 5120, 17408, "bf16"),     # K = 17408: general staging loop, 2-row kernel
    (1, 96, 8192, "f32"), (2, 200, 9216, "f32"),
    (3, 640, 17408, "f32"), (4, 640, 17408, "bf16"),       # 4-row records exceed LDS: f16 decode kernel
    (5, 17408, 5120, "bf16"), (8, 17408, 5120, "bf16"), (7, 1000, 5120, "f32"),      # eight-row kernel
    (6, 640, 4096, "f32"), (8, 200, 3072, "bf16"),
    (8, 96, 6144, "f32"), (5, 5120, 17408, "bf16"),       # 8-row records exceed LDS: f16 decode kernel
])
def test_small_m_decode_paths(gpu_lib, M, N, K, out):
    rng = np.random.default_rng(M * 7919 + N + K)
    a = rng.standard_normal((M, K)).astype(np.float32)
    a[:, rng.choice(K, 5, replace=False)] *= 50
    a_bits = inputs.f32_to_bf16_bits(a)
    if (N, K) == (17408, 5120):
        w_bits, cw, sw, gw = decode_weight_prepared()
        gs = np.array([gw], np.float32)
    else:
        w_bits = inputs.f32_to_bf16_bits((rng.standard_normal((N, K)) / np.sqrt(K)).astype(np.float32))
        gw = OQ.dynamic_global_scale(w_bits)
        cw, sw = oracle_quantize_rows(w_bits, gw)
        gs = np.array([gw], np.float32)
    ac, asc, ag, packed, wg = gpu_prepare(gpu_lib, a_bits, w_bits)
    assert np.float32(host(wg)[0]) == gs[0]
    y = gpu_lib.gemm_w4a4(ac, asc, ag, packed, wg, N, K,
                          out_dtype=torch.float32 if out == "f32" else torch.bfloat16)
    ca, sa, ga = OQ.quantize(a_bits)
    yr, br = oracle_gemm_rows(ca, sa, ga, cw, sw, OG.column_global(N, [0, N], gs))
    check_gemm(gpu_out_f64(y), yr, br, out == "bf16", "decode %dx%dx%d" % (M, N, K))


@pytest.mark.parametrize("M", [2, 3, 4, 6, 8])
def test_fused_segments_small_m_long_k(gpu_lib, M):
    """Fused segments with sigmoid and decay gates through the FP4-MFMA decode
    kernel at m = 2..8 and K = 5120, over a ragged N with six modules."""
    rng = np.random.default_rng(500 + M)
    K = 5120
    widths = [256, 256, 384, 96, 48, 48]
    offs = list(np.cumsum([0] + widths))
    N = offs[-1]
    f = [1.0, 8.0, 2.0, 4.0, 1.5, 3.0]
    w = np.concatenate([rng.standard_normal((n, K)) * fs / np.sqrt(K) for n, fs in zip(widths, f)]).astype(np.float32)
    a = rng.standard_t(4, size=(M, K)).astype(np.float32)
    a[:, rng.choice(K, 5, replace=False)] *= 50
    a_bits, w_bits = inputs.f32_to_bf16_bits(a), inputs.f32_to_bf16_bits(w)
    a_log = (rng.standard_normal(48) * 0.5).astype(np.float32)
    dt = (rng.standard_normal(48) * 0.5).astype(np.float32)
    ac, asc, ag, packed, wg = gpu_prepare(gpu_lib, a_bits, w_bits, offs)
    epis = ["none", "none", "none", "none", "sigmoid", "gdn_decay"]
    y = gpu_lib.gemm_w4a4_fused_segments(ac, asc, ag, packed, N, K, offs, wg, epis, f32(a_log), f32(dt),
                                         out_dtype=torch.bfloat16)
    ca, sa, ga, cw, sw, gs, gcol = oracle_prepare(a_bits, w_bits, offs)
    yr, br = OG.gemm(ca, sa, ga, cw, sw, gcol)
    ref, tol = gdn_reference(yr, br, offs, a_log, dt)
    assert_within(gpu_out_f64(y), ref, tol, "fused segments M=%d K=%d" % (M, K))



# The f16 decode kernel (8 < m <= 64) over many slabs: 257 to 768 32-column
# slabs (ragged N at 257 and 376), one, two and five K groups of 256 per wave
# range, one and two row fragments, rows 9..64.  K % 256 != 0 (the last rows)
# takes its per-tile A fetch instead of the grouped one, at one and two row
# fragments.
@pytest.mark.parametrize("M,N,K,out", [
    (9, 8200, 256, "f32"), (33, 10240, 1024, "bf16"), (48, 12010, 768, "f32"),
    (17, 17408, 5120, "bf16"), (64, 17408, 5120, "f32"), (40, 24576, 512, "bf16"),
    (64, 9000, 1280, "f32"), (31, 9000, 1280, "bf16"),
    (31, 1500, 2080, "bf16"), (20, 3000, 1312, "f32"), (48, 1200, 800, "bf16"), (64, 2000, 4128, "f32"),
])
def test_f16_decode_many_slabs(gpu_lib, M, N, K, out):
    rng = np.random.default_rng(M * 31 + N * 7 + K)
    a = rng.standard_t(4, size=(M, K)).astype(np.float32)
    a[:, rng.choice(K, 3, replace=False)] *= 50
    a_bits = inputs.f32_to_bf16_bits(a)
    if (N, K) == (17408, 5120):
        w_bits, cw, sw, gw = decode_weight_prepared()
    else:
        w_bits = inputs.f32_to_bf16_bits((rng.standard_normal((N, K)) / np.sqrt(K)).astype(np.float32))
        gw = OQ.dynamic_global_scale(w_bits)
        cw, sw = oracle_quantize_rows(w_bits, gw)
    gs = np.array([gw], np.float32)
    ac, asc, ag, packed, wg = gpu_prepare(gpu_lib, a_bits, w_bits)
    assert np.float32(host(wg)[0]) == gs[0]
    y = gpu_lib.gemm_w4a4(ac, asc, ag, packed, wg, N, K,
                          out_dtype=torch.float32 if out == "f32" else torch.bfloat16)
    ca, sa, ga = OQ.quantize(a_bits)
    yr, br = oracle_gemm_rows(ca, sa, ga, cw, sw, OG.column_global(N, [0, N], gs))
    check_gemm(gpu_out_f64(y), yr, br, out == "bf16", "f16 decode %dx%dx%d" % (M, N, K))


@pytest.mark.parametrize("M", [16, 40, 64])
def test_fused_segments_f16_decode(gpu_lib, M):
    """Fused segments with sigmoid and decay gates through the f16 decode
    kernel: six modules over 262 slabs, ragged N."""
    rng = np.random.default_rng(900 + M)
    K = 512
    widths = [4096, 2048, 2016, 96, 48, 44]
    offs = list(np.cumsum([0] + widths))
    N = offs[-1]
    f = [1.0, 8.0, 2.0, 4.0, 1.5, 3.0]
    w = np.concatenate([rng.standard_normal((n, K)) * fs / np.sqrt(K) for n, fs in zip(widths, f)]).astype(np.float32)
    a = rng.standard_t(4, size=(M, K)).astype(np.float32)
    a[:, rng.choice(K, 3, replace=False)] *= 50
    a_bits, w_bits = inputs.f32_to_bf16_bits(a), inputs.f32_to_bf16_bits(w)
    a_log = (rng.standard_normal(44) * 0.5).astype(np.float32)
    dt = (rng.standard_normal(44) * 0.5).astype(np.float32)
    ac, asc, ag, packed, wg = gpu_prepare(gpu_lib, a_bits, w_bits, offs)
    epis = ["none", "none", "none", "none", "sigmoid", "gdn_decay"]
    y = gpu_lib.gemm_w4a4_fused_segments(ac, asc, ag, packed, N, K, offs, wg, epis, f32(a_log), f32(dt),
                                         out_dtype=torch.bfloat16)
    ca, sa, ga, cw, sw, gs, gcol = oracle_prepare(a_bits, w_bits, offs)
    yr, br = OG.gemm(ca, sa, ga, cw, sw, gcol)
    ref, tol = gdn_reference(yr, br, offs, a_log, dt)
    assert_within(gpu_out_f64(y), ref, tol, "fused segments f16 decode M=%d" % M)

# K = 16 (mod 32): a valid NVFP4 K whose last 32-element half holds one block.
@pytest.mark.parametrize("M,N,K", [(1, 96, 48), (3, 64, 80), (8, 100, 48), (20, 256, 5136), (100, 96, 80),
                                   (300, 160, 5136), (2, 512, 5136)])
def test_k_odd_multiple_of_16(gpu_lib, M, N, K):
    rng = np.random.default_rng(M * 31 + K)
    a = rng.standard_t(4, size=(M, K)).astype(np.float32)
    w = (rng.standard_normal((N, K)) / np.sqrt(K)).astype(np.float32)
    a_bits, w_bits = inputs.f32_to_bf16_bits(a), inputs.f32_to_bf16_bits(w)
    ac, asc, ag, packed, wg = gpu_prepare(gpu_lib, a_bits, w_bits)
    ca, sa, ga, cw, sw, gs, gcol = oracle_prepare(a_bits, w_bits)
    yr, br = OG.gemm(ca, sa, ga, cw, sw, gcol)
    y = gpu_lib.gemm_w4a4(ac, asc, ag, packed, wg, N, K, out_dtype=torch.float32)
    check_gemm(gpu_out_f64(y), yr, br, False, "gemm %dx%dx%d" % (M, N, K))
    # the fused-segment entry point with a gate, and SiLU*mul (n % 64 == 0), at the same K
    offs = [0, N // 2, N]
    y2 = gpu_lib.gemm_w4a4_fused_segments(ac, asc, ag, packed, N, K, offs, wg.repeat(2), ["none", "sigmoid"],
                                          out_dtype=torch.float32)
    ref, tol = yr.copy(), OG.tolerance(br, yr, False)
    c = slice(N // 2, N)
    ref[:, c], tol[:, c] = OE.sigmoid(yr[:, c]), OE.sigmoid_tolerance(yr[:, c], OG.GEMM_REL_TOL * br[:, c], False)
    assert_within(gpu_out_f64(y2), ref, tol, "fused segments %dx%dx%d" % (M, N, K))
    if N % 64 == 0:
        h = gpu_lib.gemm_w4a4(ac, asc, ag, packed, wg, N, K, out_dtype=torch.float32, epilogue="silu_mul")
        g_, u_ = yr[:, :N // 2], yr[:, N // 2:]
        tol_h = OE.silu_mul_tolerance(g_, u_, OG.GEMM_REL_TOL * br[:, :N // 2], OG.GEMM_REL_TOL * br[:, N // 2:],
                                      False)
        assert_within(gpu_out_f64(h), OE.silu_mul(g_, u_), tol_h, "silu_mul %dx%dx%d" % (M, N, K))


def test_tiny_workload(gpu_lib):
    d = inputs.tiny()
    ac, asc, ag, packed, wg = gpu_prepare(gpu_lib, d["A"], d["W"])
    y = gpu_lib.gemm_w4a4(ac, asc, ag, packed, wg, 64, 128, out_dtype=torch.float32)
    ca, sa, ga, cw, sw, gs, gcol = oracle_prepare(d["A"], d["W"])
    yr, br = OG.gemm(ca, sa, ga, cw, sw, gcol)
    check_gemm(gpu_out_f64(y), yr, br, False, "tiny")


# ---------------------------------------------------- full-size configs ----
def sample_rows(M, count=24, seed=0):
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 31, 32, M // 2, M - 1]
    return np.unique(np.concatenate([fixed, rng.choice(M, count, replace=False)]))


def test_linear_prefill_config(gpu_lib):
    d = inputs.linear()
    M, N, K = 2048, 5120, 5120
    ac, asc, ag, packed, wg = gpu_prepare(gpu_lib, d["A"], d["W"])
    y = gpu_lib.gemm_w4a4(ac, asc, ag, packed, wg, N, K, out_dtype=torch.bfloat16)
    rows = sample_rows(M)
    got = gpu_out_f64(y[torch.as_tensor(rows, device="cuda")])
    ca, sa, ga, cw, sw, gs, gcol = oracle_prepare(d["A"], d["W"], rows=rows)
    yr, br = oracle_gemm_rows(ca, sa, ga, cw, sw, gcol)
    check_gemm(got, yr, br, True, "linear prefill")


@pytest.mark.parametrize("M", inputs.DECODE_M)
def test_decode_config(gpu_lib, M):
    d = inputs.decode(M)
    N, K = 17408, 5120
    ac, asc, ag, packed, wg = gpu_prepare(gpu_lib, d["A"], d["W"])
    y = gpu_lib.gemm_w4a4(ac, asc, ag, packed, wg, N, K, out_dtype=torch.bfloat16)
    ca, sa, ga, cw, sw, gs, gcol = oracle_prepare(d["A"], d["W"])
    yr, br = oracle_gemm_rows(ca, sa, ga, cw, sw, gcol)
    check_gemm(gpu_out_f64(y), yr, br, True, "decode M=%d" % M)


def test_mlp_config_stages(gpu_lib):
    """MLP block: (i) gate_up + SiLU*mul, (iii) down-projection on the oracle's
    quantised h; and the whole GPU chain run end to end (reported by finiteness)."""
    d = inputs.mlp()
    M, K, N2, KD = 4096, 5120, 34816, 17408
    ac, asc, ag, packed, wg = gpu_prepare(gpu_lib, d["A"], d["W_gate_up"])
    h = gpu_lib.gemm_w4a4(ac, asc, ag, packed, wg, N2, K, out_dtype=torch.bfloat16, epilogue="silu_mul")
    rows = sample_rows(M, 16)
    got = gpu_out_f64(h[torch.as_tensor(rows, device="cuda")])
    ca, sa, ga, cw, sw, gs, gcol = oracle_prepare(d["A"], d["W_gate_up"], rows=rows)
    yr, br = oracle_gemm_rows(ca, sa, ga, cw, sw, gcol)
    g_, u_ = yr[:, :KD], yr[:, KD:]
    tg, tu = OG.GEMM_REL_TOL * br[:, :KD], OG.GEMM_REL_TOL * br[:, KD:]
    assert_within(got, OE.silu_mul(g_, u_), OE.silu_mul_tolerance(g_, u_, tg, tu, True), "gate_up silu*mul")
    # (iii) down-projection on the oracle's own h (bf16) for 96 rows (prefill path)
    h_or = OG.f64_to_bf16_bits(OE.silu_mul(g_, u_))
    h_rows = np.concatenate([h_or] * 6)[:96]
    ac2, asc2, ag2, packed2, wg2 = gpu_prepare(gpu_lib, h_rows, d["W_down"])
    y2 = gpu_lib.gemm_w4a4(ac2, asc2, ag2, packed2, wg2, 5120, KD, out_dtype=torch.bfloat16)
    ca2, sa2, ga2, cw2, sw2, gs2, gcol2 = oracle_prepare(h_rows, d["W_down"])
    yr2, br2 = oracle_gemm_rows(ca2, sa2, ga2, cw2, sw2, gcol2)
    check_gemm(gpu_out_f64(y2), yr2, br2, True, "down K=17408")
    # the GPU chain end to end
    hq, hs, hg = gpu_lib.nvfp4_quantize(h)
    y3 = gpu_lib.gemm_w4a4(hq, hs, hg, packed2, wg2, 5120, KD, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.isfinite(y3.float()).all()


def gdn_reference(yr, br, offs, a_log, dt_bias):
    """Oracle output of the fused in-projection and its per-element tolerance."""
    ref = yr.copy()
    tol = OG.tolerance(br, yr, True)
    b0, b1, a0, a1 = offs[4], offs[5], offs[5], offs[6]
    ref[:, b0:b1] = OE.sigmoid(yr[:, b0:b1])
    tol[:, b0:b1] = OE.sigmoid_tolerance(yr[:, b0:b1], OG.GEMM_REL_TOL * br[:, b0:b1], True)
    ref[:, a0:a1] = OE.gdn_decay(yr[:, a0:a1], a_log, dt_bias)
    tol[:, a0:a1] = OE.gdn_decay_tolerance(yr[:, a0:a1], a_log, dt_bias, OG.GEMM_REL_TOL * br[:, a0:a1], True)
    return ref, tol


def test_gdn_inproj_config_with_per_module_scales(gpu_lib):
    d = inputs.gdn_inproj()
    M, K = 4096, 5120
    offs = [int(v) for v in d["seg_offsets"]]
    N = offs[-1]
    ac, asc, ag, packed, wg = gpu_prepare(gpu_lib, d["A"], d["W"], offs)
    epis = ["none", "none", "none", "none", "sigmoid", "gdn_decay"]
    y = gpu_lib.gemm_w4a4_fused_segments(ac, asc, ag, packed, N, K, offs, wg, epis,
                                         f32(d["A_log"]), f32(d["dt_bias"]), out_dtype=torch.bfloat16)
    rows = sample_rows(M, 16)
    got = gpu_out_f64(y[torch.as_tensor(rows, device="cuda")])
    ca, sa, ga, cw, sw, gs, gcol = oracle_prepare(d["A"], d["W"], offs, rows=rows)
    assert gs.max() / gs.min() > 2.0          # the modules really are calibrated differently
    yr, br = oracle_gemm_rows(ca, sa, ga, cw, sw, gcol)
    ref, tol = gdn_reference(yr, br, offs, d["A_log"], d["dt_bias"])
    assert_within(got, ref, tol, "gdn in-proj")


def test_single_alpha_negative_control(gpu_lib):
    """One alpha for the fused weight (the mis-scaling fused kernels do) is off per
    segment by g_w[s] / g_w[0]; the per-segment entry point matches the oracle."""
    d = inputs.gdn_inproj(M=256)
    K = 5120
    offs = [int(v) for v in d["seg_offsets"]]
    N = offs[-1]
    ac, asc, ag, packed, wg = gpu_prepare(gpu_lib, d["A"], d["W"], offs)
    y_seg = gpu_lib.gemm_w4a4_fused_segments(ac, asc, ag, packed, N, K, offs, wg, None, out_dtype=torch.float32)
    y_one = gpu_lib.gemm_w4a4(ac, asc, ag, packed, wg[:1], N, K, out_dtype=torch.float32)
    gs = host(wg).astype(np.float64)
    ys, yo = gpu_out_f64(y_seg), gpu_out_f64(y_one)
    ca, sa, ga, cw, sw, ogs, gcol = oracle_prepare(d["A"], d["W"], offs)
    yr, br = OG.gemm(ca, sa, ga, cw, sw, gcol)
    check_gemm(ys, yr, br, False, "per-segment alpha")
    big = np.abs(yr) > 1e-3 * np.abs(yr).max()
    for s in range(len(offs) - 1):
        c = slice(offs[s], offs[s + 1])
        ratio = yo[:, c][big[:, c]] / ys[:, c][big[:, c]]
        np.testing.assert_allclose(ratio, gs[s] / gs[0], rtol=1e-5)
        if abs(gs[s] / gs[0] - 1) > 0.01:
            assert not np.all(np.abs(yo[:, c] - yr[:, c]) <= OG.tolerance(br[:, c], yr[:, c], False))


@pytest.mark.parametrize("M", [1, 2, 3, 4, 48, 200])
def test_fused_segments_small(gpu_lib, M):
    """Fused segments on small shapes, whole output compared, both kernels."""
    rng = np.random.default_rng(M)
    K = 256
    widths = [64, 32, 48, 8, 40]
    offs = list(np.cumsum([0] + widths))
    N = offs[-1]
    f = [1.0, 8.0, 0.5, 3.0, 2.0]
    w = np.concatenate([rng.standard_normal((n, K)) * fs / 16 for n, fs in zip(widths, f)]).astype(np.float32)
    a = rng.standard_t(4, size=(M, K)).astype(np.float32)
    a_bits, w_bits = inputs.f32_to_bf16_bits(a), inputs.f32_to_bf16_bits(w)
    a_log = (rng.standard_normal(40) * 0.5).astype(np.float32)
    dt = (rng.standard_normal(40) * 0.5).astype(np.float32)
    ac, asc, ag, packed, wg = gpu_prepare(gpu_lib, a_bits, w_bits, offs)
    epis = ["none", "sigmoid", "none", "sigmoid", "gdn_decay"]
    y = gpu_lib.gemm_w4a4_fused_segments(ac, asc, ag, packed, N, K, offs, wg, epis, f32(a_log), f32(dt),
                                         out_dtype=torch.bfloat16)
    ca, sa, ga, cw, sw, gs, gcol = oracle_prepare(a_bits, w_bits, offs)
    yr, br = OG.gemm(ca, sa, ga, cw, sw, gcol)
    ref = yr.copy()
    tol = OG.tolerance(br, yr, True)
    for s, e in enumerate(epis):
        c = slice(offs[s], offs[s + 1])
        t = OG.GEMM_REL_TOL * br[:, c]
        if e == "sigmoid":
            ref[:, c], tol[:, c] = OE.sigmoid(yr[:, c]), OE.sigmoid_tolerance(yr[:, c], t, True)
        elif e == "gdn_decay":
            ref[:, c] = OE.gdn_decay(yr[:, c], a_log, dt)
            tol[:, c] = OE.gdn_decay_tolerance(yr[:, c], a_log, dt, t, True)
    assert_within(gpu_out_f64(y), ref, tol, "fused segments M=%d" % M)


@pytest.mark.parametrize("M,K,N", [(1, 192, 256), (40, 192, 256), (130, 192, 256),
                                   (20, 768, 256), (50, 512, 192),   # decode with grouped A fetch
                                   (512, 256, 38400),    # 300 gate/up tiles: the last 44 as 4 row bands each
                                   (512, 256, 43520)])   # 340 tiles: the last 84 as half-height tiles
def test_silu_mul_small(gpu_lib, M, K, N):
    rng = np.random.default_rng(100 + M)
    a = rng.standard_t(4, size=(M, K)).astype(np.float32)
    w = (rng.standard_normal((N, K)) / 8).astype(np.float32)
    a_bits, w_bits = inputs.f32_to_bf16_bits(a), inputs.f32_to_bf16_bits(w)
    ac, asc, ag, packed, wg = gpu_prepare(gpu_lib, a_bits, w_bits)
    h = gpu_lib.gemm_w4a4(ac, asc, ag, packed, wg, N, K, out_dtype=torch.float32, epilogue="silu_mul")
    ca, sa, ga, cw, sw, gs, gcol = oracle_prepare(a_bits, w_bits)
    yr, br = OG.gemm(ca, sa, ga, cw, sw, gcol)
    g_, u_ = yr[:, :N // 2], yr[:, N // 2:]
    tol = OE.silu_mul_tolerance(g_, u_, OG.GEMM_REL_TOL * br[:, :N // 2], OG.GEMM_REL_TOL * br[:, N // 2:], False)
    assert_within(gpu_out_f64(h), OE.silu_mul(g_, u_), tol, "silu_mul M=%d" % M)


# ------------------------------------------------- canaries, determinism ----
@pytest.mark.parametrize("M", [7, 150])
def test_output_canaries_and_run_to_run_identity(gpu_lib, M):
    rng = np.random.default_rng(M)
    K, N = 320, 200
    a_bits = inputs.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    w_bits = inputs.f32_to_bf16_bits(rng.standard_normal((N, K)).astype(np.float32))
    ac, asc, ag, packed, wg = gpu_prepare(gpu_lib, a_bits, w_bits)
    big = torch.full((M + 5, 264), -7.0, dtype=torch.float32, device="cuda")
    view = big[:M, :N]
    gpu_lib.gemm_w4a4(ac, asc, ag, packed, wg, N, K, out_dtype=torch.float32, out=view)
    first = host(big).copy()
    assert np.all(first[:, N:] == -7.0) and np.all(first[M:, :] == -7.0)
    gpu_lib.gemm_w4a4(ac, asc, ag, packed, wg, N, K, out_dtype=torch.float32, out=view)
    np.testing.assert_array_equal(host(big), first)
    ca, sa, ga, cw, sw, gs, gcol = oracle_prepare(a_bits, w_bits)
    yr, br = OG.gemm(ca, sa, ga, cw, sw, gcol)
    check_gemm(first[:M, :N].astype(np.float64), yr, br, False, "strided out")


def test_empty_m_is_a_no_op(gpu_lib):
    rng = np.random.default_rng(3)
    w_bits = inputs.f32_to_bf16_bits(rng.standard_normal((64, 128)).astype(np.float32))
    packed, wg = gpu_lib.nvfp4_pack_weights(dev_bf16(w_bits))
    ac = torch.empty((0, 64), dtype=torch.uint8, device="cuda")
    asc = torch.empty((0, 8), dtype=torch.uint8, device="cuda")
    y = gpu_lib.gemm_w4a4(ac, asc, f32([1.0]), packed, wg, 64, 128, out_dtype=torch.float32)
    assert y.shape == (0, 64)


# Every output element of the full-size launches is written, exactly once in
# effect: the output starts as NaN, must come back finite, and a second run
# must reproduce it bit for bit.  This covers the launch splitting (full rounds
# plus cut tail pieces) and the XCD-aware tile order at the bench's shapes,
# where the oracle comparisons above sample rows.
FULL_SHAPES = {
    "gdn_inproj": (4096, 16480, 5120, "gdn"),
    "gate_up": (4096, 34816, 5120, "silu_mul"),
    "down": (4096, 5120, 17408, "none"),
    "linear": (2048, 5120, 5120, "none"),
    "decode_m64": (64, 17408, 5120, "none"),
    "decode_m8_gate_up": (8, 34816, 5120, "silu_mul"),
}


@pytest.mark.parametrize("name", list(FULL_SHAPES))
def test_full_size_every_output_written(gpu_lib, name):
    M, N, K, epi = FULL_SHAPES[name]
    gen = torch.Generator(device="cuda").manual_seed(1000 + list(FULL_SHAPES).index(name))
    a = torch.randn(M, K, device="cuda", generator=gen).to(torch.bfloat16)
    w = (torch.randn(N, K, device="cuda", generator=gen) * 0.02).to(torch.bfloat16)
    ac, asc, ag = gpu_lib.nvfp4_quantize(a)
    offs = [0, 2048, 4096, 10240, 16384, 16432, 16480] if epi == "gdn" else None
    packed, wg = gpu_lib.nvfp4_pack_weights(w, offs)
    del w
    n_out = N // 2 if epi == "silu_mul" else N
    outs = []
    for _ in range(2):
        y = torch.full((M, n_out), float("nan"), dtype=torch.bfloat16, device="cuda")
        if epi == "gdn":
            zeros = torch.zeros(48, dtype=torch.float32, device="cuda")
            gpu_lib.gemm_w4a4_fused_segments(ac, asc, ag, packed, N, K, offs, wg,
                                             ["none"] * 4 + ["sigmoid", "gdn_decay"], zeros, zeros, out=y)
        else:
            gpu_lib.gemm_w4a4(ac, asc, ag, packed, wg, N, K, out=y, epilogue=epi)
        outs.append(y)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(outs[0].float()).all()), "%s: output elements left unwritten" % name
    assert torch.equal(outs[0], outs[1]), "%s: runs differ" % name
