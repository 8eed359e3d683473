"""The bounds-checked build of the library (libnvfp4_checked.so): every global
memory access of every kernel is tested against its buffer's extent, as the
call's shapes define it, and an access outside is dropped or redirected and
recorded.  Each entry point runs here over shapes that reach every kernel and
launch path -- quantizer (large, small, strided, static), packer and its
inverse, prefill tiles with tail pieces and narrow tiles, the register-staged
kernel (K % 64 != 0), SiLU*mul with and without the quantising epilogue,
fused segments, every decode kernel (FP4 MFMA at two, four and eight rows,
its general staging loop and its quantising variant; the f16 kernel with A in
LDS, per tile and in groups), the streaming-read reference and the
recurrence with a ragged chunk, an initial state and strided inputs.  No
access may fall outside its buffer, and every output must equal the normal
build's bit for bit (the checks only add tests; the arithmetic is the same)."""
import pytest

pytestmark = pytest.mark.gpu

# Skipped, and the checked build taken out of the library: the first GPU run
# of this test ended in a GPU memory fault, and the cause was not found by
# reading the code (the normal build's kernels were unchanged, instruction for
# instruction, and every instrumented access was traced to an in-bounds
# address).  Untested suspects: the host-side device-symbol copies
# (hipMemcpyFromSymbol / hipMemcpyToSymbol on a per-source static device
# flag) that read and cleared the record, and the two libraries, with the
# same kernel and symbol names, loaded into one process.  The test stays as
# the record of that run; it does not run until such a build exists again
# and the cause has been shown.
pytest.skip("the checked build's first GPU run faulted the GPU, cause not found; the build was removed",
            allow_module_level=True)

import contextlib  # noqa: E402

import numpy as np  # noqa: E402
import torch  # noqa: E402

from nvfp4_w4a4_gemm_quantize_amd import binding as B  # noqa: E402
from nvfp4_w4a4_gemm_quantize_amd import inputs  # noqa: E402


@contextlib.contextmanager
def library(path):
    saved = B._lib
    B._lib = None
    try:
        B.load(path)
        yield
    finally:
        B._lib = saved


def bf16(rng, shape, scale=1.0):
    x = (rng.standard_normal(shape) * scale).astype(np.float32)
    return torch.from_numpy(inputs.f32_to_bf16_bits(x).view(np.int16)).cuda().view(torch.bfloat16)


def calls(rng):
    """(name, fn) pairs; fn() returns a tuple of output tensors."""
    out = []
    a = bf16(rng, (300, 5120))
    a_small = bf16(rng, (8, 5120))
    a_wide = bf16(rng, (40, 1024))
    a_strided = a_wide[:, :512]                       # ld 1024, cols 512
    out.append(("quantize large", lambda: B.nvfp4_quantize(a)))
    out.append(("quantize small", lambda: B.nvfp4_quantize(a_small)))
    out.append(("quantize strided", lambda: B.nvfp4_quantize(a_strided)))
    g = torch.tensor([3.0], device="cuda")
    out.append(("quantize static", lambda: B.nvfp4_quantize(a_small, g, dynamic=False)))

    def gemm_case(m, n, k, epi="none", out_dtype=torch.bfloat16, segs=None, epis=None):
        x = bf16(rng, (m, k), 2.0)
        w = bf16(rng, (n, k), k ** -0.5)
        ac, asc, ag = B.nvfp4_quantize(x)
        offs = segs or [0, n]
        packed, wg = B.nvfp4_pack_weights(w, offs)
        if segs:
            return lambda: (B.gemm_w4a4_fused_segments(ac, asc, ag, packed, n, k, offs, wg, epis,
                                                       torch.zeros(offs[-1] - offs[-2], device="cuda"),
                                                       torch.zeros(offs[-1] - offs[-2], device="cuda"),
                                                       out_dtype=out_dtype),)
        return lambda: (B.gemm_w4a4(ac, asc, ag, packed, wg, n, k, out_dtype=out_dtype, epilogue=epi),)

    out.append(("pack + unpack", lambda: B.nvfp4_unpack_weights_linear(
        B.nvfp4_pack_weights(bf16(np.random.default_rng(3), (200, 640)), [0, 72, 200])[0], 200, 640)))
    out.append(("prefill tiles, ragged", gemm_case(300, 520, 320)))
    out.append(("prefill f32, K % 64 == 32", gemm_case(129, 100, 96, out_dtype=torch.float32)))
    out.append(("prefill K % 32 == 16", gemm_case(100, 96, 80)))
    out.append(("prefill tail pieces", gemm_case(512, 33184, 256)))
    out.append(("prefill narrow tiles", gemm_case(2048, 5120, 320, out_dtype=torch.float32)))
    out.append(("silu_mul prefill", gemm_case(512, 1024, 256, epi="silu_mul")))
    out.append(("silu_mul decode", gemm_case(20, 512, 768, epi="silu_mul")))
    out.append(("fused segments", gemm_case(200, 240, 256, segs=[0, 64, 96, 144, 152, 200, 240],
                                            epis=["none", "sigmoid", "none", "sigmoid", "none", "gdn_decay"])))
    for m in (1, 2, 3, 4, 7, 8):
        out.append(("decode fp4 m=%d" % m, gemm_case(m, 1000, 5120)))
    out.append(("decode fp4 general staging", gemm_case(2, 200, 9216)))
    for m in (16, 33, 64):
        out.append(("decode f16 m=%d" % m, gemm_case(m, 1000, 5120)))
    out.append(("decode f16, A in LDS", gemm_case(20, 256, 768)))
    out.append(("decode f16, A per tile", gemm_case(20, 256, 5152)))
    out.append(("decode f16 after the FP4 kernel's LDS limit", gemm_case(3, 640, 17408)))

    x1 = bf16(rng, (1, 5120))
    x5 = bf16(rng, (5, 5120))
    wl = bf16(rng, (1000, 5120), 5120 ** -0.5)
    pl, gl = B.nvfp4_pack_weights(wl)
    out.append(("linear m=1 (quantising decode kernel)", lambda: B.nvfp4_linear(x1, pl, gl, 1000)))
    out.append(("linear m=5 (quantize + GEMM)", lambda: B.nvfp4_linear(x5, pl, gl, 1000)))

    xg = bf16(rng, (256, 256), 2.0)
    wg2 = bf16(rng, (512, 256), 1 / 16)
    qc, qs, qg = B.nvfp4_quantize(xg)
    pq, gq = B.nvfp4_pack_weights(wg2)
    hg = torch.tensor([40.0], device="cuda")
    out.append(("silu_mul quantising epilogue", lambda: B.gemm_w4a4_silu_mul_quantize(
        qc, qs, qg, pq, gq, 512, 256, hg, return_h=True)))

    q = torch.from_numpy(np.random.default_rng(9).standard_normal(4099).astype(np.float32) * 4).cuda()
    out.append(("e2m1 encode", lambda: (B.nvfp4_e2m1_encode(q),)))
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    out.append(("stream read", lambda: (B.nvfp4_weight_stream_read(pl, 1000, 5120, sink), sink)))

    T, hk, hv = 77, 2, 6
    buf = bf16(rng, (T, 2 * hk * 128 + hv * 128 + 2 * hv + 12), 0.5)   # row stride a multiple of 8
    qv, kv = buf[:, :hk * 128], buf[:, hk * 128:2 * hk * 128]
    vv = buf[:, 2 * hk * 128:2 * hk * 128 + hv * 128]
    bv = buf[:, 2 * hk * 128 + hv * 128:2 * hk * 128 + hv * 128 + hv]
    gv = buf[:, 2 * hk * 128 + hv * 128 + hv:2 * hk * 128 + hv * 128 + 2 * hv]
    s0 = torch.from_numpy(np.random.default_rng(4).standard_normal((hv, 128, 128)).astype(np.float32) * 0.1).cuda()
    out.append(("recurrence", lambda: B.gdn_recurrence(qv, kv, vv, bv, gv, hk, hv, s_init=s0, return_state=True,
                                                        out_dtype=torch.bfloat16)))
    return out


def as_tuple(r):
    if isinstance(r, torch.Tensor):
        return (r,)
    return tuple(x for x in r if isinstance(x, torch.Tensor))


def test_checked_build_finds_no_access_outside_its_buffer(gpu_lib):
    assert B.CHECKED_LIB_PATH != B.LIB_PATH
    normal = {name: [t.clone() for t in as_tuple(fn())] for name, fn in calls(np.random.default_rng(1))}
    checked_flag, flags = B.nvfp4_bounds_status()
    assert not checked_flag and flags == 0, "the normal build records nothing"
    with library(B.CHECKED_LIB_PATH):
        is_checked, flags = B.nvfp4_bounds_status()          # clears any earlier record
        assert is_checked
        for name, fn in calls(np.random.default_rng(1)):
            got = as_tuple(fn())
            is_checked, flags = B.nvfp4_bounds_status()
            assert flags == 0, "%s: an access fell outside its buffer" % name
            ref = normal[name]
            assert len(got) == len(ref)
            for g_, r_ in zip(got, ref):
                assert torch.equal(g_, r_), "%s: the checked build's output differs from the normal build's" % name
