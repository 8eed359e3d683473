"""Thin Python binding of libnvfp4.so (ctypes).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/nvfp4.h.  PyTorch supplies the
device memory (output tensors are allocated here with torch.empty) and the
current HIP stream.  The functions carry the C names.  If the library is not
built, or there is no GPU, they raise -- there is no CPU fallback.
"""
import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libnvfp4.so")

OUT_F32, OUT_BF16 = 0, 1
EPI_NONE, EPI_SILU_MUL = 0, 1
SEG_NONE, SEG_SIGMOID, SEG_GDN_DECAY = 0, 1, 2
MAX_SEGMENTS = 16
_SEG_NAMES = {"none": SEG_NONE, "sigmoid": SEG_SIGMOID, "gdn_decay": SEG_GDN_DECAY}
_EPI_NAMES = {"none": EPI_NONE, "silu_mul": EPI_SILU_MUL}

_lib = None

_c_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_int = ctypes.c_int

_SIGNATURES = {
    "nvfp4_quantize": (_int, [_c_p, _i64, _i64, _i64, _c_p, _int, _c_p, _c_p, _c_p]),
    "nvfp4_e2m1_encode": (_int, [_c_p, _i64, _c_p, _c_p]),
    "nvfp4_packed_weight_bytes": (ctypes.c_size_t, [_i64, _i64]),
    "nvfp4_pack_weights": (_int, [_c_p, _i64, _i64, _int, _c_p, _c_p, _int, _c_p, ctypes.c_size_t, _c_p]),
    "nvfp4_unpack_weights_linear": (_int, [_c_p, _i64, _i64, _c_p, _c_p, _c_p]),
    "gemm_w4a4": (_int, [_c_p, _c_p, _c_p, _i64, _c_p, _c_p, _i64, _i64, _c_p, _int, _i64, _int, _c_p]),
    "nvfp4_linear": (_int, [_c_p, _i64, _i64, _i64, _c_p, _int, _c_p, _c_p, _c_p, _c_p, _i64, _c_p, _int, _i64,
                            _int, _c_p]),
    "gemm_w4a4_fused_segments": (_int, [_c_p, _c_p, _c_p, _i64, _c_p, _i64, _i64, _int, _c_p, _c_p, _c_p,
                                        _c_p, _c_p, _c_p, _int, _i64, _c_p]),
    "gemm_w4a4_silu_mul_quantize": (_int, [_c_p, _c_p, _c_p, _i64, _c_p, _c_p, _i64, _i64, _c_p, _c_p, _c_p,
                                           _c_p, _c_p]),
    "nvfp4_silu_amax_parts": (_i64, [_i64, _i64]),
    "gemm_w4a4_silu_mul_amax": (_int, [_c_p, _c_p, _c_p, _i64, _c_p, _c_p, _i64, _i64, _c_p, _i64, _c_p, _i64,
                                       _c_p, _c_p]),
    "nvfp4_quantize_amax_parts": (_int, [_c_p, _i64, _i64, _i64, _c_p, _i64, _c_p, _c_p, _c_p, _c_p]),
    "gdn_recurrence": (_int, [_c_p, _i64, _c_p, _i64, _c_p, _i64, _c_p, _i64, _c_p, _i64, _i64, _int, _int, _int,
                              _c_p, _c_p, _c_p, _int, _i64, _c_p]),
    "nvfp4_weight_stream_read": (_int, [_c_p, _i64, _i64, _c_p, _c_p]),
    "nvfp4_status_string": (ctypes.c_char_p, [_int]),
    "nvfp4_last_hip_error": (_int, []),
}
EXPORTED = tuple(_SIGNATURES)


class NVFP4Error(RuntimeError):
    pass


def load(path=LIB_PATH):
    """Load the shared library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise NVFP4Error("libnvfp4.so not found at %s; build it with "
                         "`python -m nvfp4_w4a4_gemm_quantize_amd.build`" % path)
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(rc, what):
    if rc != 0:
        lib = load()
        msg = lib.nvfp4_status_string(rc).decode()
        if rc == -5:
            msg += " (hipError %d)" % lib.nvfp4_last_hip_error()
        raise NVFP4Error("%s failed: %s [%d]" % (what, msg, rc))


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t, dtype, name):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise NVFP4Error("%s must be a GPU tensor" % name)
    if t.dtype != dtype:
        raise NVFP4Error("%s must be %s, got %s" % (name, dtype, t.dtype))
    return t


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _i64_array(vals):
    arr = (ctypes.c_int64 * len(vals))(*[int(v) for v in vals])
    return arr


def nvfp4_quantize(x, global_scale=None, dynamic=True, codes=None, scales=None):
    """bf16 [rows, cols] (row stride allowed) -> (codes u8 [rows, cols/2], scales u8 [rows, cols/16], g).

    dynamic=True writes g = 2688/amax into ``global_scale`` (allocated if None);
    dynamic=False reads a calibrated g from it.
    """
    lib = load()
    _dev(x, torch.bfloat16, "x")
    if x.dim() != 2 or x.stride(1) != 1:
        raise NVFP4Error("x must be 2-D with unit column stride")
    rows, cols = x.shape
    if global_scale is None:
        if not dynamic:
            raise NVFP4Error("a static quantisation needs global_scale")
        global_scale = torch.empty(1, dtype=torch.float32, device=x.device)
    _dev(global_scale, torch.float32, "global_scale")
    if codes is None:
        codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((rows, cols // 16), dtype=torch.uint8, device=x.device)
    _dev(codes, torch.uint8, "codes")
    _dev(scales, torch.uint8, "scales")
    if codes.numel() * 2 < rows * cols or scales.numel() * 16 < rows * cols or not codes.is_contiguous() \
            or not scales.is_contiguous():
        raise NVFP4Error("codes/scales must be contiguous [rows, cols/2] and [rows, cols/16]")
    ld = x.stride(0) if rows > 1 else cols          # a size-1 dimension's stride is arbitrary
    rc = lib.nvfp4_quantize(_ptr(x), rows, cols, ld, _ptr(global_scale), 1 if dynamic else 0,
                            _ptr(codes), _ptr(scales), _stream())
    _check(rc, "nvfp4_quantize")
    return codes, scales, global_scale


def nvfp4_e2m1_encode(q, codes=None):
    """fp32 [n] -> E2M1 codes u8 [n] (0..15), through the quantizer's device encoder."""
    lib = load()
    _dev(q, torch.float32, "q")
    if not q.is_contiguous():
        raise NVFP4Error("q must be contiguous")
    n = q.numel()
    if codes is None:
        codes = torch.empty(n, dtype=torch.uint8, device=q.device)
    _dev(codes, torch.uint8, "codes")
    if codes.numel() < n or not codes.is_contiguous():
        raise NVFP4Error("codes must be a contiguous uint8 buffer of at least n bytes")
    _check(lib.nvfp4_e2m1_encode(_ptr(q), n, _ptr(codes), _stream()), "nvfp4_e2m1_encode")
    return codes


def nvfp4_packed_weight_bytes(n, k):
    return int(load().nvfp4_packed_weight_bytes(int(n), int(k)))


def nvfp4_pack_weights(w, seg_offsets=None, seg_global=None, dynamic=True, packed=None):
    """bf16 [n, k] weight -> (opaque packed u8 buffer, per-segment global scales float32 [S])."""
    lib = load()
    _dev(w, torch.bfloat16, "w")
    if w.dim() != 2 or not w.is_contiguous():
        raise NVFP4Error("w must be a contiguous [n, k] tensor")
    n, k = w.shape
    offs = [0, n] if seg_offsets is None else [int(v) for v in seg_offsets]
    nseg = len(offs) - 1
    if seg_global is None:
        if not dynamic:
            raise NVFP4Error("a static pack needs seg_global")
        seg_global = torch.empty(max(nseg, 1), dtype=torch.float32, device=w.device)
    _dev(seg_global, torch.float32, "seg_global")
    nbytes = nvfp4_packed_weight_bytes(n, k)
    if packed is None:
        packed = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=w.device)
    _dev(packed, torch.uint8, "packed")
    rc = lib.nvfp4_pack_weights(_ptr(w), n, k, nseg, _i64_array(offs), _ptr(seg_global), 1 if dynamic else 0,
                                _ptr(packed), packed.numel(), _stream())
    _check(rc, "nvfp4_pack_weights")
    return packed, seg_global


def nvfp4_unpack_weights_linear(packed, n, k):
    lib = load()
    _dev(packed, torch.uint8, "packed")
    codes = torch.empty((n, k // 2), dtype=torch.uint8, device=packed.device)
    scales = torch.empty((n, k // 16), dtype=torch.uint8, device=packed.device)
    rc = lib.nvfp4_unpack_weights_linear(_ptr(packed), n, k, _ptr(codes), _ptr(scales), _stream())
    _check(rc, "nvfp4_unpack_weights_linear")
    return codes, scales


def _out(out, m, cols, out_dtype, device):
    dt = torch.bfloat16 if out_dtype in (OUT_BF16, torch.bfloat16) else torch.float32
    if out is None:
        out = torch.empty((m, cols), dtype=dt, device=device)
    _dev(out, dt, "out")
    if out.dim() != 2 or out.stride(1) != 1 or out.shape[0] != m or out.shape[1] != cols:
        raise NVFP4Error("out must be [%d, %d] with unit column stride" % (m, cols))
    return out, (OUT_BF16 if dt == torch.bfloat16 else OUT_F32)


def _ld(t):
    return t.stride(0) if t.shape[0] > 1 else t.shape[1]


def gemm_w4a4(a_codes, a_scales, a_global, w_packed, w_global, n, k, out_dtype=torch.bfloat16,
              epilogue="none", out=None):
    """y = A_q W_q^T / (g_a g_w), [m, n] (or [m, n/2] with epilogue='silu_mul')."""
    lib = load()
    _dev(a_codes, torch.uint8, "a_codes")
    _dev(a_scales, torch.uint8, "a_scales")
    _dev(a_global, torch.float32, "a_global")
    _dev(w_packed, torch.uint8, "w_packed")
    _dev(w_global, torch.float32, "w_global")
    epi = _EPI_NAMES[epilogue] if isinstance(epilogue, str) else int(epilogue)
    m = a_codes.shape[0]
    if a_codes.numel() != m * (k // 2) or a_scales.numel() != m * (k // 16):
        raise NVFP4Error("a_codes/a_scales do not match [m, k] with k=%d" % k)
    if w_packed.numel() < nvfp4_packed_weight_bytes(n, k):
        raise NVFP4Error("w_packed is smaller than the packed size of [%d, %d]" % (n, k))
    out, od = _out(out, m, n // 2 if epi == EPI_SILU_MUL else n, out_dtype, a_codes.device)
    rc = lib.gemm_w4a4(_ptr(a_codes), _ptr(a_scales), _ptr(a_global), m, _ptr(w_packed), _ptr(w_global), n, k,
                       _ptr(out), od, _ld(out), epi, _stream())
    _check(rc, "gemm_w4a4")
    return out


def nvfp4_linear(x, w_packed, w_global, n, out_dtype=torch.bfloat16, epilogue="none", out=None,
                 a_global=None, dynamic=True, a_codes=None, a_scales=None):
    """The W4A4 layer on a bf16 activation x [m, k]: quantise x (as nvfp4_quantize) and multiply.
    Returns (out, a_codes, a_scales, a_global)."""
    lib = load()
    _dev(x, torch.bfloat16, "x")
    if x.dim() != 2 or x.stride(1) != 1:
        raise NVFP4Error("x must be 2-D with unit column stride")
    m, k = x.shape
    _dev(w_packed, torch.uint8, "w_packed")
    _dev(w_global, torch.float32, "w_global")
    if a_global is None:
        if not dynamic:
            raise NVFP4Error("a static quantisation needs a_global")
        a_global = torch.empty(1, dtype=torch.float32, device=x.device)
    _dev(a_global, torch.float32, "a_global")
    if a_codes is None:
        a_codes = torch.empty((m, k // 2), dtype=torch.uint8, device=x.device)
    if a_scales is None:
        a_scales = torch.empty((m, k // 16), dtype=torch.uint8, device=x.device)
    _dev(a_codes, torch.uint8, "a_codes")
    _dev(a_scales, torch.uint8, "a_scales")
    if a_codes.numel() != m * (k // 2) or a_scales.numel() != m * (k // 16) or not a_codes.is_contiguous() \
            or not a_scales.is_contiguous():
        raise NVFP4Error("a_codes/a_scales must be contiguous [m, k/2] and [m, k/16]")
    if w_packed.numel() < nvfp4_packed_weight_bytes(n, k):
        raise NVFP4Error("w_packed is smaller than the packed size of [%d, %d]" % (n, k))
    epi = _EPI_NAMES[epilogue] if isinstance(epilogue, str) else int(epilogue)
    out, od = _out(out, m, n // 2 if epi == EPI_SILU_MUL else n, out_dtype, x.device)
    ld_x = x.stride(0) if m > 1 else k
    rc = lib.nvfp4_linear(_ptr(x), m, k, ld_x, _ptr(a_global), 1 if dynamic else 0, _ptr(a_codes), _ptr(a_scales),
                          _ptr(w_packed), _ptr(w_global), n, _ptr(out), od, _ld(out), epi, _stream())
    _check(rc, "nvfp4_linear")
    return out, a_codes, a_scales, a_global


def gemm_w4a4_fused_segments(a_codes, a_scales, a_global, w_packed, n, k, seg_offsets, seg_w_global,
                             seg_epilogue=None, a_log=None, dt_bias=None, out_dtype=torch.bfloat16, out=None):
    """One GEMM over a fused weight; column segment s gets alpha_s = 1/(g_a g_w[s]) and its epilogue."""
    lib = load()
    _dev(a_codes, torch.uint8, "a_codes")
    _dev(a_scales, torch.uint8, "a_scales")
    _dev(a_global, torch.float32, "a_global")
    _dev(w_packed, torch.uint8, "w_packed")
    _dev(seg_w_global, torch.float32, "seg_w_global")
    offs = [int(v) for v in seg_offsets]
    nseg = len(offs) - 1
    epis = [SEG_NONE] * nseg if seg_epilogue is None else \
        [_SEG_NAMES[e] if isinstance(e, str) else int(e) for e in seg_epilogue]
    if len(epis) != nseg:
        raise NVFP4Error("one epilogue per segment")
    if a_log is not None:
        _dev(a_log, torch.float32, "a_log")
    if dt_bias is not None:
        _dev(dt_bias, torch.float32, "dt_bias")
    m = a_codes.shape[0]
    if a_codes.numel() != m * (k // 2) or a_scales.numel() != m * (k // 16):
        raise NVFP4Error("a_codes/a_scales do not match [m, k] with k=%d" % k)
    if w_packed.numel() < nvfp4_packed_weight_bytes(n, k):
        raise NVFP4Error("w_packed is smaller than the packed size of [%d, %d]" % (n, k))
    out, od = _out(out, m, n, out_dtype, a_codes.device)
    ep = (ctypes.c_int * max(nseg, 1))(*epis)
    rc = lib.gemm_w4a4_fused_segments(_ptr(a_codes), _ptr(a_scales), _ptr(a_global), m, _ptr(w_packed), n, k,
                                      nseg, _i64_array(offs), _ptr(seg_w_global), ep, _ptr(a_log), _ptr(dt_bias),
                                      _ptr(out), od, _ld(out), _stream())
    _check(rc, "gemm_w4a4_fused_segments")
    return out


def nvfp4_silu_amax_parts(m, n):
    """Entries of the partial-maxima buffer gemm_w4a4_silu_mul_amax needs for an m x n gate/up projection."""
    return int(load().nvfp4_silu_amax_parts(int(m), int(n)))


def gemm_w4a4_silu_mul_amax(a_codes, a_scales, a_global, w_packed, w_global, n, k, h=None, parts=None):
    """Gate/up GEMM into bf16 h [m, n/2] (silu(gate) * up) that also leaves partial maxima of |h|.
    Returns (h, parts, n_parts); parts (uint32, allocated if None, at least nvfp4_silu_amax_parts(m, n)
    entries) may be a view of the codes buffer h is quantised into next (nvfp4_quantize_amax_parts)."""
    lib = load()
    _dev(a_codes, torch.uint8, "a_codes")
    _dev(a_scales, torch.uint8, "a_scales")
    _dev(a_global, torch.float32, "a_global")
    _dev(w_packed, torch.uint8, "w_packed")
    _dev(w_global, torch.float32, "w_global")
    m = a_codes.shape[0]
    if a_codes.numel() != m * (k // 2) or a_scales.numel() != m * (k // 16):
        raise NVFP4Error("a_codes/a_scales do not match [m, k] with k=%d" % k)
    if w_packed.numel() < nvfp4_packed_weight_bytes(n, k):
        raise NVFP4Error("w_packed is smaller than the packed size of [%d, %d]" % (n, k))
    h, _ = _out(h, m, n // 2, torch.bfloat16, a_codes.device)
    need = nvfp4_silu_amax_parts(m, n)
    if parts is None:
        parts = torch.empty(max(need, 1), dtype=torch.int32, device=a_codes.device)
    if not isinstance(parts, torch.Tensor) or not parts.is_cuda or parts.dtype not in (torch.int32, torch.uint32) \
            or not parts.is_contiguous():
        raise NVFP4Error("parts must be a contiguous 32-bit GPU tensor")
    written = ctypes.c_int64(0)
    rc = lib.gemm_w4a4_silu_mul_amax(_ptr(a_codes), _ptr(a_scales), _ptr(a_global), m, _ptr(w_packed),
                                     _ptr(w_global), n, k, _ptr(h), _ld(h), _ptr(parts), parts.numel(),
                                     ctypes.byref(written), _stream())
    _check(rc, "gemm_w4a4_silu_mul_amax")
    return h, parts, int(written.value)


def nvfp4_quantize_amax_parts(x, parts, n_parts, global_scale=None, codes=None, scales=None):
    """nvfp4_quantize with a dynamic global scale whose amax is the largest of n_parts partial maxima
    (from gemm_w4a4_silu_mul_amax over x).  Returns (codes, scales, g)."""
    lib = load()
    _dev(x, torch.bfloat16, "x")
    if x.dim() != 2 or x.stride(1) != 1:
        raise NVFP4Error("x must be 2-D with unit column stride")
    rows, cols = x.shape
    if global_scale is None:
        global_scale = torch.empty(1, dtype=torch.float32, device=x.device)
    _dev(global_scale, torch.float32, "global_scale")
    if codes is None:
        codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((rows, cols // 16), dtype=torch.uint8, device=x.device)
    _dev(codes, torch.uint8, "codes")
    _dev(scales, torch.uint8, "scales")
    if not isinstance(parts, torch.Tensor) or not parts.is_cuda or parts.numel() < n_parts:
        raise NVFP4Error("parts must be a GPU tensor of at least n_parts entries")
    ld = x.stride(0) if rows > 1 else cols
    rc = lib.nvfp4_quantize_amax_parts(_ptr(x), rows, cols, ld, _ptr(parts), int(n_parts), _ptr(global_scale),
                                       _ptr(codes), _ptr(scales), _stream())
    _check(rc, "nvfp4_quantize_amax_parts")
    return codes, scales, global_scale


def gemm_w4a4_silu_mul_quantize(a_codes, a_scales, a_global, w_packed, w_global, n, k, h_global,
                                h_codes=None, h_scales=None, return_h=False):
    """Gate/up GEMM with h = silu(gate)*up quantised to NVFP4 in the epilogue with the static scale h_global.

    Returns (h_codes u8 [m, n/4], h_scales u8 [m, n/32]) and, with return_h, also the bf16 h [m, n/2]
    that was quantised.
    """
    lib = load()
    _dev(a_codes, torch.uint8, "a_codes")
    _dev(a_scales, torch.uint8, "a_scales")
    _dev(a_global, torch.float32, "a_global")
    _dev(w_packed, torch.uint8, "w_packed")
    _dev(w_global, torch.float32, "w_global")
    _dev(h_global, torch.float32, "h_global")
    m = a_codes.shape[0]
    if a_codes.numel() != m * (k // 2) or a_scales.numel() != m * (k // 16):
        raise NVFP4Error("a_codes/a_scales do not match [m, k] with k=%d" % k)
    if w_packed.numel() < nvfp4_packed_weight_bytes(n, k):
        raise NVFP4Error("w_packed is smaller than the packed size of [%d, %d]" % (n, k))
    dev = a_codes.device
    if h_codes is None:
        h_codes = torch.empty((m, n // 4), dtype=torch.uint8, device=dev)
    if h_scales is None:
        h_scales = torch.empty((m, n // 32), dtype=torch.uint8, device=dev)
    _dev(h_codes, torch.uint8, "h_codes")
    _dev(h_scales, torch.uint8, "h_scales")
    if h_codes.numel() != m * (n // 4) or h_scales.numel() != m * (n // 32) or not h_codes.is_contiguous() \
            or not h_scales.is_contiguous():
        raise NVFP4Error("h_codes/h_scales must be contiguous [m, n/4] and [m, n/32]")
    h = torch.empty((m, n // 2), dtype=torch.bfloat16, device=dev) if return_h else None
    rc = lib.gemm_w4a4_silu_mul_quantize(_ptr(a_codes), _ptr(a_scales), _ptr(a_global), m, _ptr(w_packed),
                                         _ptr(w_global), n, k, _ptr(h_global), _ptr(h_codes), _ptr(h_scales),
                                         _ptr(h), _stream())
    _check(rc, "gemm_w4a4_silu_mul_quantize")
    return (h_codes, h_scales, h) if return_h else (h_codes, h_scales)


def nvfp4_weight_stream_read(w_packed, n, k, sink=None):
    """Read a packed weight exactly as the decode GEMM streams it, without arithmetic (roofline reference)."""
    lib = load()
    _dev(w_packed, torch.uint8, "w_packed")
    if w_packed.numel() < nvfp4_packed_weight_bytes(n, k):
        raise NVFP4Error("w_packed is smaller than the packed size of [%d, %d]" % (n, k))
    if sink is None:
        sink = torch.zeros(1, dtype=torch.int32, device=w_packed.device)
    _check(lib.nvfp4_weight_stream_read(_ptr(w_packed), n, k, _ptr(sink), _stream()), "nvfp4_weight_stream_read")
    return sink


def _ld2(t, name):
    """Row stride (elements) of a 2-D bf16 view with unit column stride."""
    _dev(t, torch.bfloat16, name)
    if t.dim() != 2 or t.stride(1) != 1:
        raise NVFP4Error("%s must be a 2-D view with unit column stride" % name)
    return t.stride(0) if t.shape[0] > 1 else t.shape[1]


def gdn_recurrence(q, k, v, beta, g, hk, hv, s_init=None, return_state=False, out_dtype=torch.float32, out=None):
    """Gated delta rule over T steps.  q, k [T, hk*128], v [T, hv*128], beta, g [T, hv]: bf16 2-D views
    (they may be column slices of the fused in-projection output).  Returns o [T, hv*128] (and the final
    fp32 state [hv, 128, 128] with return_state)."""
    lib = load()
    T = q.shape[0]
    lds = [_ld2(x, n) for x, n in ((q, "q"), (k, "k"), (v, "v"), (beta, "beta"), (g, "g"))]
    if any(x.shape[0] != T for x in (k, v, beta, g)):
        raise NVFP4Error("q, k, v, beta, g must have the same number of rows")
    if q.shape[1] != hk * 128 or k.shape[1] != hk * 128 or v.shape[1] != hv * 128 or beta.shape[1] != hv \
            or g.shape[1] != hv:
        raise NVFP4Error("shapes must be q, k [T, hk*128], v [T, hv*128], beta, g [T, hv]")
    if s_init is not None:
        _dev(s_init, torch.float32, "s_init")
        if s_init.shape != (hv, 128, 128) or not s_init.is_contiguous():
            raise NVFP4Error("s_init must be contiguous fp32 [hv, 128, 128]")
    s_final = torch.empty((hv, 128, 128), dtype=torch.float32, device=q.device) if return_state else None
    out, od = _out(out, T, hv * 128, out_dtype, q.device)
    rc = lib.gdn_recurrence(_ptr(q), lds[0], _ptr(k), lds[1], _ptr(v), lds[2], _ptr(beta), lds[3], _ptr(g), lds[4],
                            T, hk, hv, 128, _ptr(s_init), _ptr(s_final), _ptr(out), od, _ld(out), _stream())
    _check(rc, "gdn_recurrence")
    return (out, s_final) if return_state else out
