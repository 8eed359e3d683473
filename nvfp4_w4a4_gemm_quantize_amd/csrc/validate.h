// Host-side argument validation of the C ABI.  Pure C++ (no HIP headers), so
// it can be compiled and exercised on a machine without a GPU.
#pragma once
#include <stddef.h>
#include <stdint.h>

namespace nvfp4 {

int validate_quantize(const void* x, int64_t rows, int64_t cols, int64_t ld_x, const void* global_scale,
                      const void* codes, const void* scales);
int validate_e2m1_encode(const void* q, int64_t n, const void* codes);
size_t packed_weight_bytes(int64_t n, int64_t k);
int validate_segments(int num_segments, const int64_t* seg_offsets, int64_t extent);
int validate_pack(const void* w, int64_t n, int64_t k, int num_segments, const int64_t* seg_offsets,
                  const void* seg_global, const void* packed, size_t packed_bytes);
int validate_unpack(const void* packed, int64_t n, int64_t k, const void* codes, const void* scales);
int validate_gemm_common(const void* a_codes, const void* a_scales, const void* a_global, int64_t m,
                         const void* w_packed, int64_t n, int64_t k, const void* out, int out_dtype,
                         int64_t ld_out, int64_t out_cols);
int validate_gemm_silu_quantize(const void* a_codes, const void* a_scales, const void* a_global, int64_t m,
                                const void* w_packed, const void* w_global, int64_t n, int64_t k,
                                const void* h_global, const void* h_codes, const void* h_scales,
                                const void* h_out);
int validate_gemm_silu_amax(const void* a_codes, const void* a_scales, const void* a_global, int64_t m,
                            const void* w_packed, const void* w_global, int64_t n, int64_t k, const void* h,
                            int64_t ld_h, const void* amax_parts, int64_t parts_capacity, int64_t parts_needed,
                            const void* parts_written);
int validate_quantize_parts(const void* x, int64_t rows, int64_t cols, int64_t ld_x, const void* amax_parts,
                            int64_t num_parts, const void* global_scale, const void* codes, const void* scales);
int validate_gdn_recurrence(const void* q, int64_t ld_q, const void* k, int64_t ld_k, const void* v, int64_t ld_v,
                            const void* beta, int64_t ld_beta, const void* g, int64_t ld_g, int64_t T, int hk,
                            int hv, int head_dim, const void* s_init, const void* s_final, const void* out,
                            int out_dtype, int64_t ld_out);

}  // namespace nvfp4
