"""C ABI checks that need no GPU: the library loads, exports every function
include/nvfp4.h declares, and rejects invalid arguments with the documented
status codes before touching the device (no call here reaches a kernel)."""
import ctypes
import os
import re

import pytest

from nvfp4_w4a4_gemm_quantize_amd import binding

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "nvfp4.h")

OK, EINVAL, ESHAPE, EALIGN, EUNSUPPORTED, EHIP, ESIZE = 0, -1, -2, -3, -4, -5, -6
A16 = 0x10000          # a 16-byte-aligned fake device address (never dereferenced)
MIS = 0x10004          # a misaligned one


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int64_t|int|size_t|const char\*)\s+(\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    # These calls pass fake device addresses that validation must reject; they
    # are meant for a host without a GPU, where no launch could ever happen.
    import torch
    if torch.cuda.is_available():
        pytest.skip("validation tests with fake device pointers run on GPU-less hosts only")
    if not os.path.exists(binding.LIB_PATH):
        pytest.fail("libnvfp4.so is not built; run __graft_entry__.build() first")
    return binding.load()


def test_header_declares_the_four_entry_points_and_helpers():
    fns = declared_functions()
    for name in ("nvfp4_quantize", "nvfp4_e2m1_encode", "nvfp4_pack_weights", "gemm_w4a4", "gemm_w4a4_fused_segments",
                 "nvfp4_linear", "nvfp4_weight_stream_read",
                 "gemm_w4a4_silu_mul_quantize", "gemm_w4a4_silu_mul_amax", "nvfp4_quantize_amax_parts",
                 "nvfp4_silu_amax_parts", "gdn_recurrence", "nvfp4_packed_weight_bytes",
                 "nvfp4_unpack_weights_linear",
                 "nvfp4_status_string", "nvfp4_last_hip_error"):
        assert name in fns
    assert set(fns) == set(binding.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code in (OK, EINVAL, ESHAPE, EALIGN, EUNSUPPORTED, EHIP, ESIZE):
        assert lib.nvfp4_status_string(code)
    assert lib.nvfp4_status_string(123) == b"unknown status"
    assert lib.nvfp4_last_hip_error() == 0


def test_packed_weight_bytes(lib):
    f = lib.nvfp4_packed_weight_bytes
    assert f(17408, 5120) == 17408 * 5120 * 9 // 16          # 4.5 bits per weight, no padding
    assert f(16480, 5120) == 16480 * 5120 * 9 // 16
    assert f(100, 80) == 128 * 256 * 9 // 16                 # padded to 32-row slabs of 256-wide super-tiles
    assert f(0, 64) == 0 and f(64, 0) == 0 and f(64, 24) == 0 and f(-1, 64) == 0


def q(lib, x=A16, rows=4, cols=64, ld=64, g=A16, dyn=1, codes=A16, scales=A16):
    return lib.nvfp4_quantize(x, rows, cols, ld, g, dyn, codes, scales, None)


def test_quantize_validation(lib):
    assert q(lib, cols=24, ld=24) == ESHAPE          # cols % 16
    assert q(lib, cols=0, ld=0) == ESHAPE
    assert q(lib, rows=-1) == ESHAPE
    assert q(lib, ld=32) == ESHAPE                   # ld < cols
    assert q(lib, x=None) == EINVAL
    assert q(lib, g=None) == EINVAL
    assert q(lib, codes=None) == EINVAL
    assert q(lib, scales=None) == EINVAL
    assert q(lib, x=MIS) == EALIGN
    assert q(lib, ld=68) == EALIGN                   # rows not 16-byte aligned
    assert q(lib, codes=MIS) == EALIGN
    assert q(lib, rows=0, x=None, codes=None) == OK  # empty input: nothing to do


def pk(lib, w=A16, n=64, k=128, nseg=1, offs=(0, 64), g=A16, dyn=1, packed=A16, nbytes=None):
    arr = (ctypes.c_int64 * len(offs))(*offs)
    if nbytes is None:
        nbytes = lib.nvfp4_packed_weight_bytes(n, k)
    return lib.nvfp4_pack_weights(w, n, k, nseg, arr, g, dyn, packed, nbytes, None)


def test_pack_validation(lib):
    assert pk(lib, k=24) == ESHAPE
    assert pk(lib, n=0, offs=(0, 0)) == ESHAPE
    assert pk(lib, nseg=0) == EINVAL
    assert pk(lib, nseg=17, offs=tuple(range(0, 18))) == EINVAL
    assert pk(lib, nseg=2, offs=(0, 40, 40)) == ESHAPE           # last != n
    assert pk(lib, nseg=2, offs=(0, 70, 64)) == ESHAPE           # not rising
    assert pk(lib, nseg=2, offs=(1, 30, 64)) == ESHAPE           # first != 0
    assert pk(lib, w=None) == EINVAL
    assert pk(lib, packed=None) == EINVAL
    assert pk(lib, g=None) == EINVAL
    assert pk(lib, w=MIS) == EALIGN
    assert pk(lib, nbytes=100) == ESIZE
    assert lib.nvfp4_pack_weights(A16, 64, 128, 1, None, A16, 1, A16, 9000, None) == EINVAL


def test_e2m1_encode_validation(lib):
    f = lib.nvfp4_e2m1_encode
    assert f(A16, -1, A16, None) == ESHAPE
    assert f(None, 0, None, None) == OK              # nothing to do
    assert f(None, 8, A16, None) == EINVAL
    assert f(A16, 8, None, None) == EINVAL
    assert f(0x10002, 8, A16, None) == EALIGN        # fp32 input must be 4-byte aligned


def gm(lib, ac=A16, asc=A16, ag=A16, m=64, w=A16, wg=A16, n=128, k=128, out=A16, dt=1, ld=128, epi=0):
    return lib.gemm_w4a4(ac, asc, ag, m, w, wg, n, k, out, dt, ld, epi, None)


def test_gemm_validation(lib):
    assert gm(lib, k=48, ac=None) == EINVAL    # K = 48 (16 | K) passes the shape rule: the null pointer is caught
    assert gm(lib, k=16, out=None) == EINVAL   # so does the smallest K
    assert gm(lib, k=40) == ESHAPE
    assert gm(lib, n=0) == ESHAPE
    assert gm(lib, m=-3) == ESHAPE
    assert gm(lib, dt=7) == EINVAL
    assert gm(lib, epi=5) == EINVAL
    assert gm(lib, epi=1, n=96) == ESHAPE      # SiLU*mul needs n % 64
    assert gm(lib, ld=100) == ESHAPE           # ld_out < n
    assert gm(lib, epi=1, ld=60) == ESHAPE    # SiLU*mul output has n/2 = 64 columns
    assert gm(lib, out=0x10002, dt=0) == EALIGN   # fp32 output must be 4-byte aligned
    assert gm(lib, ac=None) == EINVAL
    assert gm(lib, wg=None) == EINVAL
    assert gm(lib, out=None) == EINVAL
    assert gm(lib, ac=MIS) == EALIGN
    assert gm(lib, w=MIS) == EALIGN
    assert gm(lib, m=0, ac=None, out=None) == OK


def fs(lib, m=64, n=128, k=128, nseg=2, offs=(0, 64, 128), epis=(0, 1), alog=A16, dtb=A16, sg=A16, ld=128):
    arr = (ctypes.c_int64 * len(offs))(*offs)
    ep = (ctypes.c_int * len(epis))(*epis)
    return lib.gemm_w4a4_fused_segments(A16, A16, A16, m, A16, n, k, nseg, arr, sg, ep, alog, dtb, A16, 1, ld, None)


def test_fused_segments_validation(lib):
    assert fs(lib, offs=(0, 64, 120)) == ESHAPE
    assert fs(lib, epis=(0, 9)) == EINVAL
    assert fs(lib, epis=(2, 2)) == EUNSUPPORTED          # at most one decay segment
    assert fs(lib, epis=(0, 2), alog=None) == EINVAL
    assert fs(lib, sg=None) == EINVAL
    assert fs(lib, nseg=0, offs=(0,), epis=(0,)) == EINVAL
    assert fs(lib, k=80, sg=None) == EINVAL     # K = 80 is a valid shape
    assert fs(lib, k=72) == ESHAPE
    assert fs(lib, m=0, sg=None) == OK


def sq(lib, m=64, n=128, k=128, ac=A16, wg=A16, hg=A16, hc=A16, hs=A16, ho=None):
    return lib.gemm_w4a4_silu_mul_quantize(ac, A16, A16, m, A16, wg, n, k, hg, hc, hs, ho, None)


def test_silu_mul_quantize_validation(lib):
    assert sq(lib, n=96) == ESHAPE              # gate/up halves of whole 32-column fragments: n % 64
    assert sq(lib, n=0) == ESHAPE
    assert sq(lib, m=-1) == ESHAPE
    assert sq(lib, k=48, hc=None) == EINVAL     # K = 48 is a valid shape
    assert sq(lib, k=40) == ESHAPE
    assert sq(lib, hg=None) == EINVAL           # the static scale of h is required
    assert sq(lib, hc=None) == EINVAL
    assert sq(lib, hs=None) == EINVAL
    assert sq(lib, wg=None) == EINVAL
    assert sq(lib, ac=MIS) == EALIGN
    assert sq(lib, hc=0x10008) == EALIGN         # codes rows move as 16-byte-aligned data
    assert sq(lib, ho=MIS) == EALIGN
    assert sq(lib, m=0, ac=None, hc=None) == OK


def sa(lib, m=300, n=128, k=128, ac=A16, wg=A16, h=A16, ldh=64, parts=A16, cap=None, wr=True):
    cap = lib.nvfp4_silu_amax_parts(m, n) if cap is None else cap
    written = ctypes.c_int64(-7)
    rc = lib.gemm_w4a4_silu_mul_amax(ac, A16, A16, m, A16, wg, n, k, h, ldh, parts, cap,
                                     ctypes.byref(written) if wr else None, None)
    return rc, written.value


def test_silu_mul_amax_validation(lib):
    assert lib.nvfp4_silu_amax_parts(0, 128) == 0
    assert lib.nvfp4_silu_amax_parts(300, 128) >= 1024              # at least an amax pass's grid
    assert lib.nvfp4_silu_amax_parts(4096, 34816) == 16 * 136 * 16 * 4   # 64 waves per tile at most
    assert sa(lib, n=96)[0] == ESHAPE             # gate/up halves: n % 64
    assert sa(lib, m=-1)[0] == ESHAPE
    assert sa(lib, k=40)[0] == ESHAPE
    assert sa(lib, wr=False)[0] == EINVAL          # the count of maxima goes back to the host
    assert sa(lib, wg=None)[0] == EINVAL
    assert sa(lib, parts=None)[0] == EINVAL
    assert sa(lib, h=None)[0] == EINVAL
    assert sa(lib, cap=1023)[0] == ESHAPE          # below the size query
    assert sa(lib, ldh=60)[0] == ESHAPE            # shorter than the n/2 columns
    assert sa(lib, ldh=68)[0] == EALIGN            # h rows are read with 16-byte loads
    assert sa(lib, h=0x10008)[0] == EALIGN
    assert sa(lib, parts=0x10002)[0] == EALIGN
    assert sa(lib, ac=MIS)[0] == EALIGN
    assert sa(lib, m=0, ac=None, parts=None, h=None) == (OK, 0)


def qp(lib, rows=16, cols=64, ld=64, x=A16, parts=A16, np_=4, g=A16, codes=A16, scales=A16):
    return lib.nvfp4_quantize_amax_parts(x, rows, cols, ld, parts, np_, g, codes, scales, None)


def test_quantize_amax_parts_validation(lib):
    assert qp(lib, cols=40) == ESHAPE
    assert qp(lib, ld=32) == ESHAPE
    assert qp(lib, np_=0) == ESHAPE               # a dynamic scale needs at least one maximum
    assert qp(lib, np_=2 ** 31) == ESHAPE
    assert qp(lib, parts=None) == EINVAL
    assert qp(lib, g=None) == EINVAL
    assert qp(lib, parts=0x10002) == EALIGN
    assert qp(lib, x=MIS) == EALIGN
    assert qp(lib, rows=0, x=None, parts=None) == OK


def rec(lib, q=A16, ldq=256, k=A16, ldk=256, v=A16, ldv=768, b=A16, ldb=6, g=A16, ldg=6, T=10, hk=2, hv=6, d=128,
        si=None, sf=None, out=A16, dt=0, ldo=768):
    return lib.gdn_recurrence(q, ldq, k, ldk, v, ldv, b, ldb, g, ldg, T, hk, hv, d, si, sf, out, dt, ldo, None)


def test_gdn_recurrence_validation(lib):
    assert rec(lib, hv=5) == ESHAPE            # value heads a multiple of key heads
    assert rec(lib, hk=0) == ESHAPE
    assert rec(lib, T=-1) == ESHAPE
    assert rec(lib, d=64) == EUNSUPPORTED      # head dimension 128 only
    assert rec(lib, d=0) == ESHAPE
    assert rec(lib, dt=3) == EINVAL
    assert rec(lib, ldq=200) == ESHAPE         # rows shorter than hk * 128
    assert rec(lib, ldv=700) == ESHAPE
    assert rec(lib, ldb=5) == ESHAPE
    assert rec(lib, ldo=512) == ESHAPE
    assert rec(lib, q=None) == EINVAL
    assert rec(lib, g=None) == EINVAL
    assert rec(lib, out=None) == EINVAL
    assert rec(lib, k=MIS) == EALIGN
    assert rec(lib, ldk=260) == EALIGN         # 16-byte row pieces need ld % 8 == 0
    assert rec(lib, b=0x10001) == EALIGN
    assert rec(lib, si=MIS) == EALIGN
    assert rec(lib, out=0x10002, dt=0) == EALIGN
    assert rec(lib, T=0, q=None, out=None) == OK


def test_abi_layer_under_address_and_ub_sanitizers(tmp_path):
    """abi.cpp and validate.cpp built for the host alone with ASan and UBSan,
    driven by tests/abi_host_check.cpp (launchers stubbed): every status code
    and the arguments that reach the launchers, with no sanitizer report."""
    import shutil
    import subprocess
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("no host C++ compiler")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    csrc = os.path.join(root, "nvfp4_w4a4_gemm_quantize_amd", "csrc")
    exe = str(tmp_path / "abi_host_check")
    cmd = [gxx, "-std=c++17", "-g", "-O1", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           os.path.join(root, "tests", "abi_host_check.cpp"), os.path.join(csrc, "abi.cpp"),
           os.path.join(csrc, "validate.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0 and "cases ok" in r.stdout, r.stdout + r.stderr[-4000:]
    assert "runtime error" not in r.stderr and "Sanitizer" not in r.stderr, r.stderr[-4000:]


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros((4, 32), dtype=torch.bfloat16)
    with pytest.raises(binding.NVFP4Error):
        binding.nvfp4_quantize(x)
