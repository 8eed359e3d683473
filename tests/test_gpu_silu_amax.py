"""GPU checks of the amax-reporting SiLU*mul GEMM (gemm_w4a4_silu_mul_amax)
and the quantizer that takes its partial maxima (nvfp4_quantize_amax_parts).

The pair replaces gemm_w4a4(SILU_MUL) followed by nvfp4_quantize(h,
dynamic_global=1).  The maximum of |h| does not depend on the order it is
taken in, so the replacement is exact: h, the global scale, the codes and the
scale bytes are compared bit for bit with the unfused chain (whose parity
with the fp64 oracle and the oracle quantiser the GEMM and quantizer tests
establish).  Every route is covered: the prefill kernels' full rounds and
cut last round (maxima from the epilogue), ragged rows, and the decode and
register-staged kernels (maxima from an amax pass over h).
"""
import numpy as np
import pytest
import torch

from nvfp4_w4a4_gemm_quantize_amd import inputs
from tests.parity import host
from tests.test_gpu_gemm import gpu_prepare

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M,N,K,route", [
    (4096, 34816, 5120, "prefill"),   # the MLP block's gate/up: eight full rounds and a cut last round
    (512, 34816, 1024, "prefill"),    # 272 tiles: the last 16 as 64-row pieces
    (300, 640, 512, "prefill"),       # one round, ragged rows (rows past m excluded from the maxima)
    (32, 2048, 512, "pass"),          # the decode kernel, then an amax pass
    (200, 256, 96, "pass"),           # k % 64 != 0: the register-staged kernel, then an amax pass
])
def test_matches_the_unfused_chain(gpu_lib, M, N, K, route):
    rng = np.random.default_rng(4400 + M)
    a = rng.standard_t(4, size=(M, K)).astype(np.float32)
    a[:, rng.choice(K, max(1, K // 1000), replace=False)] *= 50
    w = (rng.standard_normal((N, K)) / np.sqrt(K)).astype(np.float32)
    ac, asc, ag, packed, wg = gpu_prepare(gpu_lib, inputs.f32_to_bf16_bits(a), inputs.f32_to_bf16_bits(w))

    h_ref = gpu_lib.gemm_w4a4(ac, asc, ag, packed, wg, N, K, out_dtype=torch.bfloat16, epilogue="silu_mul")
    c_ref, s_ref, g_ref = gpu_lib.nvfp4_quantize(h_ref)

    # the partial maxima live in the codes buffer of the quantisation that follows
    need = gpu_lib.nvfp4_silu_amax_parts(M, N)
    codes = torch.empty((M, N // 4), dtype=torch.uint8, device="cuda")
    assert codes.numel() >= 4 * need
    parts = codes.view(-1)[:4 * need].view(torch.int32)
    h, _, n_parts = gpu_lib.gemm_w4a4_silu_mul_amax(ac, asc, ag, packed, wg, N, K, parts=parts)
    assert torch.equal(h.view(torch.int16), h_ref.view(torch.int16))
    if route == "prefill":
        assert n_parts > 1024 or M < 2048          # one maximum per wave of the prefill launches
    else:
        assert 1 <= n_parts <= 1024                # an amax pass's workgroups
    amax_bits = int(host(parts[:n_parts]).astype(np.uint32).max())
    ref_bits = int((host(h_ref.view(torch.int16)).astype(np.uint16) & 0x7FFF).max())
    assert amax_bits == ref_bits

    c, s, g = gpu_lib.nvfp4_quantize_amax_parts(h, parts, n_parts, codes=codes)
    assert host(g).view(np.uint32)[0] == host(g_ref).view(np.uint32)[0]
    assert torch.equal(c, c_ref) and torch.equal(s, s_ref)


def test_zero_h_gives_unit_scale(gpu_lib):
    """All-zero weights: h == 0 everywhere, amax 0, so g = 1 and every code and scale is 0 (the quantizer's
    amax == 0 convention)."""
    M, N, K = 300, 640, 512
    rng = np.random.default_rng(4500)
    a = rng.standard_normal((M, K)).astype(np.float32)
    ac, asc, ag, packed, wg = gpu_prepare(gpu_lib, inputs.f32_to_bf16_bits(a),
                                          inputs.f32_to_bf16_bits(np.zeros((N, K), np.float32)))
    h, parts, n_parts = gpu_lib.gemm_w4a4_silu_mul_amax(ac, asc, ag, packed, wg, N, K)
    c, s, g = gpu_lib.nvfp4_quantize_amax_parts(h, parts, n_parts)
    assert float(host(g)[0]) == 1.0
    assert int(host(c).max()) == 0 and int(host(s).max()) == 0
