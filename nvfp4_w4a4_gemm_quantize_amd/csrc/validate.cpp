// Host-side argument validation of the C ABI (no HIP dependency).
#include "validate.h"

#include "../../include/nvfp4.h"

namespace nvfp4 {

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int validate_quantize(const void* x, int64_t rows, int64_t cols, int64_t ld_x, const void* global_scale,
                      const void* codes, const void* scales) {
  if (rows < 0 || cols <= 0) return NVFP4_ESHAPE;
  if (cols % 16 != 0 || ld_x < cols) return NVFP4_ESHAPE;
  if (rows == 0) return NVFP4_OK;
  if (!x || !global_scale || !codes || !scales) return NVFP4_EINVAL;
  if (ld_x % 8 != 0 || !aligned16(x) || !aligned16(codes) || (reinterpret_cast<uintptr_t>(global_scale) & 3u))
    return NVFP4_EALIGN;
  return NVFP4_OK;
}

int validate_e2m1_encode(const void* q, int64_t n, const void* codes) {
  if (n < 0) return NVFP4_ESHAPE;
  if (n == 0) return NVFP4_OK;
  if (!q || !codes) return NVFP4_EINVAL;
  if (reinterpret_cast<uintptr_t>(q) & 3u) return NVFP4_EALIGN;
  return NVFP4_OK;
}

size_t packed_weight_bytes(int64_t n, int64_t k) {
  if (n <= 0 || k <= 0 || k % 16 != 0) return 0;
  const int64_t np = (n + 31) / 32 * 32, kp = (k + 255) / 256 * 256;   // 32-row slabs, 256-wide super-tiles
  return (size_t)(np * kp / 2 + np * kp / 16);
}

int validate_segments(int num_segments, const int64_t* seg_offsets, int64_t extent) {
  if (num_segments < 1 || num_segments > NVFP4_MAX_SEGMENTS) return NVFP4_EINVAL;
  if (!seg_offsets) return NVFP4_EINVAL;
  if (seg_offsets[0] != 0 || seg_offsets[num_segments] != extent) return NVFP4_ESHAPE;
  for (int s = 0; s < num_segments; ++s)
    if (seg_offsets[s] >= seg_offsets[s + 1]) return NVFP4_ESHAPE;
  return NVFP4_OK;
}

int validate_pack(const void* w, int64_t n, int64_t k, int num_segments, const int64_t* seg_offsets,
                  const void* seg_global, const void* packed, size_t packed_bytes) {
  if (n <= 0 || k <= 0 || k % 16 != 0) return NVFP4_ESHAPE;
  int rc = validate_segments(num_segments, seg_offsets, n);
  if (rc) return rc;
  if (!w || !seg_global || !packed) return NVFP4_EINVAL;
  if (!aligned16(w) || !aligned16(packed) || (reinterpret_cast<uintptr_t>(seg_global) & 3u)) return NVFP4_EALIGN;
  if (packed_bytes < packed_weight_bytes(n, k)) return NVFP4_ESIZE;
  return NVFP4_OK;
}

int validate_unpack(const void* packed, int64_t n, int64_t k, const void* codes, const void* scales) {
  if (n <= 0 || k <= 0 || k % 16 != 0) return NVFP4_ESHAPE;
  if (!packed || !codes || !scales) return NVFP4_EINVAL;
  if (!aligned16(packed) || (reinterpret_cast<uintptr_t>(codes) & 7u)) return NVFP4_EALIGN;
  return NVFP4_OK;
}

int validate_gemm_common(const void* a_codes, const void* a_scales, const void* a_global, int64_t m,
                         const void* w_packed, int64_t n, int64_t k, const void* out, int out_dtype,
                         int64_t ld_out, int64_t out_cols) {
  if (m < 0 || n <= 0 || k <= 0 || k % 16 != 0) return NVFP4_ESHAPE;
  if (out_dtype != NVFP4_OUT_F32 && out_dtype != NVFP4_OUT_BF16) return NVFP4_EINVAL;
  if (ld_out < out_cols) return NVFP4_ESHAPE;
  if (m == 0) return NVFP4_OK;
  if (!a_codes || !a_scales || !a_global || !w_packed || !out) return NVFP4_EINVAL;
  const uintptr_t elem = out_dtype == NVFP4_OUT_F32 ? 4u : 2u;
  if (!aligned16(a_codes) || !aligned16(w_packed) || (reinterpret_cast<uintptr_t>(a_scales) & 3u) ||
      (reinterpret_cast<uintptr_t>(out) & (elem - 1)))
    return NVFP4_EALIGN;
  return NVFP4_OK;
}

int validate_gemm_silu_quantize(const void* a_codes, const void* a_scales, const void* a_global, int64_t m,
                                const void* w_packed, const void* w_global, int64_t n, int64_t k,
                                const void* h_global, const void* h_codes, const void* h_scales,
                                const void* h_out) {
  if (m < 0 || n <= 0 || k <= 0 || k % 16 != 0 || n % 64 != 0) return NVFP4_ESHAPE;
  if (m == 0) return NVFP4_OK;
  if (!a_codes || !a_scales || !a_global || !w_packed || !w_global || !h_global || !h_codes || !h_scales)
    return NVFP4_EINVAL;
  if (!aligned16(a_codes) || !aligned16(w_packed) || (reinterpret_cast<uintptr_t>(a_scales) & 3u) ||
      !aligned16(h_codes) || (h_out && !aligned16(h_out)))
    return NVFP4_EALIGN;
  return NVFP4_OK;
}

int validate_gemm_silu_amax(const void* a_codes, const void* a_scales, const void* a_global, int64_t m,
                            const void* w_packed, const void* w_global, int64_t n, int64_t k, const void* h,
                            int64_t ld_h, const void* amax_parts, int64_t parts_capacity, int64_t parts_needed,
                            const void* parts_written) {
  if (!parts_written) return NVFP4_EINVAL;
  if (n <= 0 || n % 64 != 0) return NVFP4_ESHAPE;
  int rc = validate_gemm_common(a_codes, a_scales, a_global, m, w_packed, n, k, h, NVFP4_OUT_BF16, ld_h, n / 2);
  if (rc || m == 0) return rc;
  if (!w_global || !amax_parts) return NVFP4_EINVAL;
  if (parts_capacity < parts_needed) return NVFP4_ESHAPE;
  // h is also read with 16-byte loads by the amax pass and the quantizer
  if (ld_h % 8 != 0 || !aligned16(h) || (reinterpret_cast<uintptr_t>(amax_parts) & 3u)) return NVFP4_EALIGN;
  return NVFP4_OK;
}

int validate_quantize_parts(const void* x, int64_t rows, int64_t cols, int64_t ld_x, const void* amax_parts,
                            int64_t num_parts, const void* global_scale, const void* codes, const void* scales) {
  int rc = validate_quantize(x, rows, cols, ld_x, global_scale, codes, scales);
  if (rc || rows == 0) return rc;
  if (!amax_parts) return NVFP4_EINVAL;
  if (num_parts < 1 || num_parts > INT32_MAX) return NVFP4_ESHAPE;
  if (reinterpret_cast<uintptr_t>(amax_parts) & 3u) return NVFP4_EALIGN;
  return NVFP4_OK;
}

int validate_gdn_recurrence(const void* q, int64_t ld_q, const void* k, int64_t ld_k, const void* v, int64_t ld_v,
                            const void* beta, int64_t ld_beta, const void* g, int64_t ld_g, int64_t T, int hk,
                            int hv, int head_dim, const void* s_init, const void* s_final, const void* out,
                            int out_dtype, int64_t ld_out) {
  if (T < 0 || hk <= 0 || hv <= 0 || hv % hk != 0) return NVFP4_ESHAPE;
  if (head_dim != 128) return head_dim > 0 ? NVFP4_EUNSUPPORTED : NVFP4_ESHAPE;
  if (out_dtype != NVFP4_OUT_F32 && out_dtype != NVFP4_OUT_BF16) return NVFP4_EINVAL;
  if (ld_q < (int64_t)hk * 128 || ld_k < (int64_t)hk * 128 || ld_v < (int64_t)hv * 128 || ld_beta < hv ||
      ld_g < hv || ld_out < (int64_t)hv * 128)
    return NVFP4_ESHAPE;
  if (T == 0) return NVFP4_OK;
  if (!q || !k || !v || !beta || !g || !out) return NVFP4_EINVAL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || (ld_q % 8) || (ld_k % 8) || (ld_v % 8) ||
      (reinterpret_cast<uintptr_t>(beta) & 1u) || (reinterpret_cast<uintptr_t>(g) & 1u) ||
      (s_init && !aligned16(s_init)) || (s_final && !aligned16(s_final)) ||
      (reinterpret_cast<uintptr_t>(out) & (out_dtype == NVFP4_OUT_F32 ? 3u : 1u)))
    return NVFP4_EALIGN;
  return NVFP4_OK;
}

}  // namespace nvfp4
