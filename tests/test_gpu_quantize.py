"""GPU parity of the NVFP4 activation quantizer and the weight packer against
the CPU oracle: codes and scale bytes must be bit-identical, global scales
equal."""
import numpy as np
import pytest
import torch

from nvfp4_w4a4_gemm_quantize_amd import inputs
from tests.parity import OQ, assert_bytes_equal, dev_bf16, f32, host, oracle_quantize_rows
from tests.test_oracle_quantize import load_golden

pytestmark = pytest.mark.gpu


def gpu_quantize(lib, bits, g=None, ld=None):
    x = dev_bf16(bits)
    if ld is not None:                      # strided rows: embed in a wider buffer
        wide = torch.zeros((bits.shape[0], ld), dtype=torch.bfloat16, device="cuda")
        wide[:, :bits.shape[1]] = x
        x = wide[:, :bits.shape[1]]
    gs = None if g is None else f32([g])
    codes, scales, gout = lib.nvfp4_quantize(x, gs, dynamic=g is None)
    torch.cuda.synchronize()
    return host(codes), host(scales), np.float32(host(gout)[0])


def check_quantize(lib, bits, g=None, what="", ld=None):
    c, s, gg = gpu_quantize(lib, bits, g, ld)
    oc, os_, og = OQ.quantize(bits, g)
    assert gg == og, "%s: global scale %r vs oracle %r" % (what, gg, og)
    assert_bytes_equal(s, os_, what + " scales")
    assert_bytes_equal(c, oc, what + " codes")


@pytest.mark.parametrize("case", load_golden(), ids=lambda c: c["name"])
def test_golden_blocks(gpu_lib, case):
    """Hand-worked blocks (tests/golden/quantize_blocks.txt) on the GPU."""
    c, s, g = gpu_quantize(gpu_lib, case["bits"], case["g"])
    assert list(s[0]) == case["scales"]
    assert list(OQ.unpack_nibbles(c)[0]) == case["codes"]
    assert g == case["g_expected"]


# The seven E2M1 decision points (midpoints between neighbouring magnitudes).
E2M1_MIDPOINTS = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)


def _fp32_neighbourhood(x, span):
    """Every fp32 value within `span` ulps of the positive value x."""
    b = int(np.float32(x).view(np.uint32))
    return np.arange(b - span, b + span + 1, dtype=np.int64).astype(np.uint32).view(np.float32)


def test_e2m1_encoder_around_every_decision_point(gpu_lib):
    """The device E2M1 encoder (the hardware conversion the quantizer applies
    to x * g / s, run in both operand slots and all four byte positions)
    against the oracle's closed form (pinned exhaustively on the CPU): every fp32
    within 2^16 ulps of each decision point, within 2^12 ulps of each grid value
    and of 8, a strided sweep over all finite non-negative fp32 patterns
    (subnormals to the largest finite), each with both signs (-0 included)."""
    from oracle import formats as F
    parts = [_fp32_neighbourhood(p, 1 << 16) for p in E2M1_MIDPOINTS]
    parts += [_fp32_neighbourhood(p, 1 << 12) for p in (0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, 8.0)]
    parts.append(np.arange(0, 0x7F800000, 4099, dtype=np.uint32).view(np.float32))
    parts.append(np.array([0, 1, 2, 0x007FFFFF, 0x00800000, 0x3E7FFFFF, 0x7F7FFFFF], np.uint32).view(np.float32))
    mag = np.concatenate(parts)
    q = np.concatenate([mag, -mag])
    got = host(gpu_lib.nvfp4_e2m1_encode(torch.from_numpy(q).cuda()))
    want = F.e2m1_rne_sat(np.abs(q)) | (np.signbit(q).astype(np.uint8) << 3)
    assert_bytes_equal(got, want, "E2M1 encoder (%d values)" % q.size)



@pytest.mark.parametrize("n", [1, 2, 3, 5, 7, 9, 4097])
def test_e2m1_encode_odd_lengths_leave_the_tail_alone(gpu_lib, n):
    """Lengths that end on a half-filled conversion pair and in each byte
    position: codes[0..n) match the closed form, the bytes past n keep their canary."""
    from oracle import formats as F
    rng = np.random.default_rng(n)
    q = (rng.standard_normal(n) * 4).astype(np.float32)
    q[::3] = -q[::3]
    buf = torch.full((n + 16,), 0xA5, dtype=torch.uint8, device="cuda")
    gpu_lib.nvfp4_e2m1_encode(torch.from_numpy(q).cuda(), buf)
    got = host(buf)
    want = F.e2m1_rne_sat(np.abs(q)) | (np.signbit(q).astype(np.uint8) << 3)
    assert_bytes_equal(got[:n], want, "E2M1 encoder, n=%d" % n)
    assert np.all(got[n:] == 0xA5), "bytes past n were written"

ACTIVATIONS = {
    "tiny": lambda: inputs.tiny()["A"],
    "linear": lambda: inputs.linear()["A"],
    "mlp": lambda: inputs.mlp(weights=False)["A"],
    "gdn_inproj": lambda: inputs.gdn_inproj(weights=False)["A"],
}
for _m in inputs.DECODE_M:
    ACTIVATIONS["decode_m%d" % _m] = (lambda m: lambda: inputs.decode(m, weights=False)["A"])(_m)


@pytest.mark.parametrize("name", list(ACTIVATIONS))
def test_config_activations_bit_exact(gpu_lib, name):
    check_quantize(gpu_lib, ACTIVATIONS[name](), None, name)


def _edge_bits(rng, rows, cols):
    b = rng.integers(0, 1 << 16, size=(rows, cols), dtype=np.uint32).astype(np.uint16)
    finite = ((b >> 7) & 0xFF) != 0xFF
    return np.where(finite, b, b & 0x807F).astype(np.uint16)


@pytest.mark.parametrize("rows,cols", [(1, 16), (7, 48), (33, 5120), (4096, 16), (100, 656), (13, 5056)])
def test_edge_shapes_and_bit_patterns(gpu_lib, rows, cols):
    rng = np.random.default_rng(rows * 7919 + cols)
    bits = _edge_bits(rng, rows, cols)               # every exponent, subnormals, -0
    check_quantize(gpu_lib, bits, None, "random bits %dx%d" % (rows, cols))
    x = rng.standard_t(4, size=(rows, cols)).astype(np.float32)
    check_quantize(gpu_lib, inputs.f32_to_bf16_bits(x), None, "t4 %dx%d" % (rows, cols))


def test_dynamic_paths_across_the_small_tensor_threshold(gpu_lib):
    rng = np.random.default_rng(5)
    for rows, cols in [(12, 5120), (13, 5120), (4, 16384), (5, 16384), (64, 1024), (65, 1024)]:
        x = (rng.standard_normal((rows, cols)) * np.exp(rng.uniform(-4, 4, (rows, 1)))).astype(np.float32)
        check_quantize(gpu_lib, inputs.f32_to_bf16_bits(x), None, "%dx%d" % (rows, cols))


def test_static_global_scale_and_saturation(gpu_lib):
    rng = np.random.default_rng(6)
    x = rng.standard_normal((64, 512)).astype(np.float32)
    bits = inputs.f32_to_bf16_bits(x)
    for g in (2688.0 / 0.25, 2688.0 / 4.0, 1.0, 3.0e-3):   # the first saturates many blocks at 448
        check_quantize(gpu_lib, bits, np.float32(g), "static g=%g" % g)


def test_ties_zeros_and_signs(gpu_lib):
    rng = np.random.default_rng(8)
    xt = (rng.integers(-384, 385, size=(64, 256)) / 64.0).astype(np.float32)
    check_quantize(gpu_lib, inputs.f32_to_bf16_bits(xt), np.float32(1.0), "grid ties")
    xz = np.zeros((4, 64), dtype=np.float32)
    xz[0, 16:32] = -0.0
    xz[1, :] = -1e-30
    xz[2, 0] = 5.0
    check_quantize(gpu_lib, inputs.f32_to_bf16_bits(xz), None, "zeros")
    check_quantize(gpu_lib, np.zeros((3, 32), dtype=np.uint16), None, "all zero")


def test_all_scale_bytes_and_codes(gpu_lib):
    """Every code at every non-zero scale byte, with a +-6 anchor (oracle pin P5) on the GPU."""
    from oracle import formats as F
    rows = []
    for S_byte in range(1, 0x7F):
        s = F.E4M3_POSITIVE[S_byte]
        v = np.zeros((16, 16))
        v[:, 0] = F.E2M1_TABLE[np.arange(16)] * s
        v[:, 1] = np.where(np.arange(16) % 2, -6.0, 6.0) * s
        rows.append(v)
    x = np.concatenate(rows).astype(np.float32)
    check_quantize(gpu_lib, inputs.f32_to_bf16_bits(x), np.float32(1.0), "codes x scales")


def test_strided_rows(gpu_lib):
    rng = np.random.default_rng(9)
    bits = inputs.f32_to_bf16_bits(rng.standard_normal((37, 320)).astype(np.float32))
    check_quantize(gpu_lib, bits, None, "ld=328", ld=328)
    check_quantize(gpu_lib, bits, np.float32(100.0), "ld=512 static", ld=512)


def test_mlp_hidden_quantisation_stage(gpu_lib):
    """MLP chain stage (ii): the quantizer on the oracle's own SiLU*mul output h (bf16)."""
    from tests.parity import OE, oracle_gemm_rows
    from oracle import gemm as OG
    d = inputs.mlp()
    rows = np.arange(0, 4096, 128)[:32]
    ca, sa, ga = OQ.quantize(d["A"])
    gw = OQ.dynamic_global_scale(d["W_gate_up"])
    cw, sw = oracle_quantize_rows(d["W_gate_up"], gw)
    y, _ = oracle_gemm_rows(ca[rows], sa[rows], ga, cw, sw, np.full(cw.shape[0], np.float64(gw)))
    h = OE.silu_mul(y[:, :17408], y[:, 17408:])
    check_quantize(gpu_lib, OG.f64_to_bf16_bits(h), None, "mlp h")


def test_empty_input_is_a_no_op(gpu_lib):
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    g = f32([123.0])
    gpu_lib.nvfp4_quantize(x, g, dynamic=True)
    torch.cuda.synchronize()
    assert host(g)[0] == 123.0


# ----------------------------------------------------------------- packer ----
def gpu_pack_unpack(lib, bits, offs=None, seg_g=None):
    w = dev_bf16(bits)
    n, k = bits.shape
    sg = None if seg_g is None else f32(seg_g)
    packed, gs = lib.nvfp4_pack_weights(w, offs, sg, dynamic=seg_g is None)
    codes, scales = lib.nvfp4_unpack_weights_linear(packed, n, k)
    torch.cuda.synchronize()
    return host(packed), host(codes), host(scales), host(gs)


def check_pack(lib, bits, offs=None, seg_g=None, what=""):
    n = bits.shape[0]
    offs_l = [0, n] if offs is None else list(offs)
    _, c, s, gs = gpu_pack_unpack(lib, bits, offs, seg_g)
    if seg_g is None:
        og = np.array([OQ.dynamic_global_scale(bits[offs_l[i]:offs_l[i + 1]]) for i in range(len(offs_l) - 1)],
                      dtype=np.float32)
    else:
        og = np.asarray(seg_g, dtype=np.float32)
    np.testing.assert_array_equal(gs, og)
    for i in range(len(offs_l) - 1):
        oc, os_ = oracle_quantize_rows(bits[offs_l[i]:offs_l[i + 1]], og[i])
        assert_bytes_equal(c[offs_l[i]:offs_l[i + 1]], oc, "%s seg %d codes" % (what, i))
        assert_bytes_equal(s[offs_l[i]:offs_l[i + 1]], os_, "%s seg %d scales" % (what, i))


@pytest.mark.parametrize("name", ["tiny", "linear", "decode", "gdn_inproj", "mlp_gate_up", "mlp_down"])
def test_config_weights_bit_exact(gpu_lib, name):
    if name == "tiny":
        check_pack(gpu_lib, inputs.tiny()["W"], what=name)
    elif name == "linear":
        check_pack(gpu_lib, inputs.linear()["W"], what=name)
    elif name == "decode":
        check_pack(gpu_lib, inputs.decode(1)["W"], what=name)
    elif name == "gdn_inproj":
        d = inputs.gdn_inproj()
        check_pack(gpu_lib, d["W"], d["seg_offsets"], what=name)
    else:
        d = inputs.mlp()
        check_pack(gpu_lib, d["W_gate_up"] if name == "mlp_gate_up" else d["W_down"], what=name)


@pytest.mark.parametrize("n,k", [(1, 16), (100, 80), (33, 48), (64, 96), (257, 5120)])
def test_pack_ragged_and_padding(gpu_lib, n, k):
    rng = np.random.default_rng(n * 31 + k)
    bits = inputs.f32_to_bf16_bits(rng.standard_normal((n, k)).astype(np.float32))
    check_pack(gpu_lib, bits, what="%dx%d" % (n, k))
    # padding rows/columns of the tiles hold zero codes and zero scales
    packed, _, _, _ = gpu_pack_unpack(gpu_lib, bits)
    np_, kp = -(-n // 32) * 32, -(-k // 256) * 256
    kt = kp // 64
    sup = packed[:np_ * kp * 9 // 16].reshape(np_ // 32, kp // 256, 4608)   # [nt, super-tile, 4 x 1024 codes + 512]
    codes = sup[:, :, :4096].reshape(np_ // 32, kt, 2, 32, 16)             # [nt, kt, h, c, 16 bytes]
    scales = sup[:, :, 4096:].reshape(np_ // 32, kp // 256, 2, 32, 2, 4)   # [nt, s, g, c, tile 2g+i, block]
    scales = scales.transpose(0, 1, 2, 4, 3, 5).reshape(np_ // 32, kt, 32, 4)  # [nt, kt, c, block]
    rows = np.arange(np_).reshape(np_ // 32, 32)
    cols_block = np.arange(kp // 16).reshape(kt, 4)
    pad_row = rows >= n
    for nt in range(np_ // 32):
        for t in range(kt):
            for c in range(32):
                if pad_row[nt, c]:
                    assert not codes[nt, t, :, c].any() and not scales[nt, t, c].any()
                else:
                    for b in range(4):
                        if cols_block[t, b] * 16 >= k:
                            assert scales[nt, t, c, b] == 0
                            assert not codes[nt, t, b // 2, c, (b % 2) * 8:(b % 2) * 8 + 8].any()


def test_pack_static_segment_scales(gpu_lib):
    rng = np.random.default_rng(12)
    w = np.concatenate([rng.standard_normal((40, 128)) * f for f in (1.0, 6.0, 0.5)]).astype(np.float32)
    bits = inputs.f32_to_bf16_bits(w)
    check_pack(gpu_lib, bits, [0, 40, 80, 120], seg_g=[2688.0 / 3, 2688.0 / 30, 2688.0 / 5], what="static")
    check_pack(gpu_lib, bits, [0, 7, 80, 120], what="dynamic uneven")
