"""NVFP4 W4A4 linear layers for MI355X (gfx950): activation quantizer, weight
packer and block-scaled FP4 x FP4 GEMMs (plain, SiLU*mul, and fused modules
with per-segment global scales), as hand-written HIP kernels behind a C ABI
(include/nvfp4.h).

The C functions are available here under their C names once the library is
built (``python -m nvfp4_w4a4_gemm_quantize_amd.build``); they load it on
first use.  ``inputs`` holds the seeded synthetic workloads.
"""
_API = ("nvfp4_quantize", "nvfp4_packed_weight_bytes", "nvfp4_pack_weights", "nvfp4_unpack_weights_linear",
        "gemm_w4a4", "gemm_w4a4_fused_segments")


def __getattr__(name):
    if name in _API:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
