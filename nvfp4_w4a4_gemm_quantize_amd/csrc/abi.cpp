// C ABI entry points: validate, describe the epilogue, launch.  Declared and
// documented in include/nvfp4.h.
#include <hip/hip_runtime.h>

#include "../../include/nvfp4.h"
#include "kernels.h"
#include "validate.h"

using namespace nvfp4;

static thread_local int g_last_hip_error = 0;

static int hip_status(hipError_t e) {
  if (e == hipSuccess) return NVFP4_OK;
  g_last_hip_error = (int)e;
  return NVFP4_EHIP;
}

static SegmentTable make_table(int num, const int64_t* off) {
  SegmentTable t{};
  t.num = num;
  for (int s = 0; s <= num; ++s) t.off[s] = off[s];
  return t;
}

// Epilogue of a single-module GEMM (one segment, no gate), optionally SiLU*mul.
static EpilogueArgs plain_epilogue(const float* a_global, const float* w_global, int64_t n, bool silu, int out_dtype,
                                   int64_t ld_out) {
  EpilogueArgs epi{};
  epi.segs.num = 1;
  epi.segs.off[0] = 0;
  epi.segs.off[1] = n;
  epi.seg_epi[0] = NVFP4_SEG_NONE;
  epi.seg_w_global = w_global;
  epi.a_global = a_global;
  epi.silu_mul = silu ? 1 : 0;
  epi.out_bf16 = out_dtype == NVFP4_OUT_BF16;
  epi.ld_out = ld_out;
  return epi;
}

extern "C" {

int nvfp4_quantize(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, float* global_scale,
                   int dynamic_global, uint8_t* codes, uint8_t* scales, nvfp4_stream_t stream) {
  int rc = validate_quantize(x, rows, cols, ld_x, global_scale, codes, scales);
  if (rc || rows == 0) return rc;
  return hip_status(launch_quantize(x, rows, cols, ld_x, global_scale, dynamic_global != 0, codes, scales,
                                    (hipStream_t)stream));
}

int nvfp4_e2m1_encode(const float* q, int64_t n, uint8_t* codes, nvfp4_stream_t stream) {
  int rc = validate_e2m1_encode(q, n, codes);
  if (rc || n == 0) return rc;
  return hip_status(launch_e2m1_encode(q, n, codes, (hipStream_t)stream));
}

size_t nvfp4_packed_weight_bytes(int64_t n, int64_t k) { return packed_weight_bytes(n, k); }

int nvfp4_pack_weights(const uint16_t* w, int64_t n, int64_t k, int num_segments, const int64_t* seg_offsets,
                       float* seg_global, int dynamic_global, void* packed, size_t packed_bytes,
                       nvfp4_stream_t stream) {
  int rc = validate_pack(w, n, k, num_segments, seg_offsets, seg_global, packed, packed_bytes);
  if (rc) return rc;
  return hip_status(launch_pack(w, n, k, make_table(num_segments, seg_offsets), seg_global, dynamic_global != 0,
                                static_cast<uint8_t*>(packed), (hipStream_t)stream));
}

int nvfp4_unpack_weights_linear(const void* packed, int64_t n, int64_t k, uint8_t* codes, uint8_t* scales,
                                nvfp4_stream_t stream) {
  int rc = validate_unpack(packed, n, k, codes, scales);
  if (rc) return rc;
  return hip_status(launch_unpack(static_cast<const uint8_t*>(packed), n, k, codes, scales, (hipStream_t)stream));
}

int gemm_w4a4(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_global, int64_t m,
              const void* w_packed, const float* w_global, int64_t n, int64_t k, void* out, int out_dtype,
              int64_t ld_out, int epilogue, nvfp4_stream_t stream) {
  if (epilogue != NVFP4_EPI_NONE && epilogue != NVFP4_EPI_SILU_MUL) return NVFP4_EINVAL;
  const bool silu = epilogue == NVFP4_EPI_SILU_MUL;
  if (silu && (n <= 0 || n % 64 != 0)) return NVFP4_ESHAPE;
  int rc = validate_gemm_common(a_codes, a_scales, a_global, m, w_packed, n, k, out, out_dtype, ld_out,
                                silu ? n / 2 : n);
  if (rc) return rc;
  if (m == 0) return NVFP4_OK;
  if (!w_global) return NVFP4_EINVAL;
  EpilogueArgs epi = plain_epilogue(a_global, w_global, n, silu, out_dtype, ld_out);
  return hip_status(launch_gemm(a_codes, a_scales, m, static_cast<const uint8_t*>(w_packed), n, k, out, epi,
                                (hipStream_t)stream));
}

int nvfp4_linear(const uint16_t* x, int64_t m, int64_t k, int64_t ld_x, float* a_global, int dynamic_global,
                 uint8_t* a_codes, uint8_t* a_scales, const void* w_packed, const float* w_global, int64_t n,
                 void* out, int out_dtype, int64_t ld_out, int epilogue, nvfp4_stream_t stream) {
  if (epilogue != NVFP4_EPI_NONE && epilogue != NVFP4_EPI_SILU_MUL) return NVFP4_EINVAL;
  const bool silu = epilogue == NVFP4_EPI_SILU_MUL;
  if (silu && (n <= 0 || n % 64 != 0)) return NVFP4_ESHAPE;
  int rc = validate_quantize(x, m, k, ld_x, a_global, a_codes, a_scales);
  if (rc) return rc;
  rc = validate_gemm_common(a_codes, a_scales, a_global, m, w_packed, n, k, out, out_dtype, ld_out, silu ? n / 2 : n);
  if (rc) return rc;
  if (m == 0) return NVFP4_OK;
  if (!w_global) return NVFP4_EINVAL;
  EpilogueArgs epi = plain_epilogue(a_global, w_global, n, silu, out_dtype, ld_out);
  QuantSource qs{};
  qs.x = x;
  qs.ld_x = ld_x;
  qs.g = a_global;
  qs.dynamic = dynamic_global != 0;
  qs.codes = a_codes;
  qs.scales = a_scales;
  return hip_status(launch_linear(qs, m, static_cast<const uint8_t*>(w_packed), n, k, out, epi, (hipStream_t)stream));
}

int gemm_w4a4_fused_segments(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_global, int64_t m,
                             const void* w_packed, int64_t n, int64_t k, int num_segments,
                             const int64_t* seg_offsets, const float* seg_w_global, const int* seg_epilogue,
                             const float* a_log, const float* dt_bias, void* out, int out_dtype, int64_t ld_out,
                             nvfp4_stream_t stream) {
  int rc = validate_gemm_common(a_codes, a_scales, a_global, m, w_packed, n, k, out, out_dtype, ld_out, n);
  if (rc) return rc;
  rc = validate_segments(num_segments, seg_offsets, n);
  if (rc) return rc;
  if (!seg_epilogue) return NVFP4_EINVAL;
  int decay_segments = 0;
  for (int s = 0; s < num_segments; ++s) {
    const int e = seg_epilogue[s];
    if (e != NVFP4_SEG_NONE && e != NVFP4_SEG_SIGMOID && e != NVFP4_SEG_GDN_DECAY) return NVFP4_EINVAL;
    decay_segments += e == NVFP4_SEG_GDN_DECAY;
  }
  if (decay_segments > 1) return NVFP4_EUNSUPPORTED;
  if (decay_segments && (!a_log || !dt_bias)) return NVFP4_EINVAL;
  if (m == 0) return NVFP4_OK;
  if (!seg_w_global) return NVFP4_EINVAL;
  EpilogueArgs epi{};
  epi.segs = make_table(num_segments, seg_offsets);
  for (int s = 0; s < num_segments; ++s) epi.seg_epi[s] = seg_epilogue[s];
  epi.seg_w_global = seg_w_global;
  epi.a_global = a_global;
  epi.a_log = a_log;
  epi.dt_bias = dt_bias;
  epi.silu_mul = 0;
  epi.out_bf16 = out_dtype == NVFP4_OUT_BF16;
  epi.ld_out = ld_out;
  return hip_status(launch_gemm(a_codes, a_scales, m, static_cast<const uint8_t*>(w_packed), n, k, out, epi,
                                (hipStream_t)stream));
}

int gemm_w4a4_silu_mul_quantize(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_global, int64_t m,
                                const void* w_packed, const float* w_global, int64_t n, int64_t k,
                                const float* h_global, uint8_t* h_codes, uint8_t* h_scales, uint16_t* h_out,
                                nvfp4_stream_t stream) {
  int rc = validate_gemm_silu_quantize(a_codes, a_scales, a_global, m, w_packed, w_global, n, k, h_global, h_codes,
                                       h_scales, h_out);
  if (rc || m == 0) return rc;
  EpilogueArgs epi{};
  epi.segs.num = 1;
  epi.segs.off[0] = 0;
  epi.segs.off[1] = n;
  epi.seg_epi[0] = NVFP4_SEG_NONE;
  epi.seg_w_global = w_global;
  epi.a_global = a_global;
  epi.silu_mul = 1;
  epi.out_bf16 = 1;
  epi.ld_out = n / 2;
  epi.h_global = h_global;
  epi.h_codes = h_codes;
  epi.h_scales = h_scales;
  epi.h_out = h_out;
  return hip_status(launch_gemm_tiled(a_codes, a_scales, m, static_cast<const uint8_t*>(w_packed), n, k, nullptr,
                                      epi, (hipStream_t)stream));
}

int64_t nvfp4_silu_amax_parts(int64_t m, int64_t n) { return m > 0 && n > 0 ? silu_amax_parts_bound(m, n) : 0; }

int gemm_w4a4_silu_mul_amax(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_global, int64_t m,
                            const void* w_packed, const float* w_global, int64_t n, int64_t k, uint16_t* h,
                            int64_t ld_h, uint32_t* amax_parts, int64_t parts_capacity, int64_t* parts_written,
                            nvfp4_stream_t stream) {
  int rc = validate_gemm_silu_amax(a_codes, a_scales, a_global, m, w_packed, w_global, n, k, h, ld_h, amax_parts,
                                   parts_capacity, m > 0 ? silu_amax_parts_bound(m, n) : 0, parts_written);
  if (rc) return rc;
  *parts_written = 0;
  if (m == 0) return NVFP4_OK;
  EpilogueArgs epi = plain_epilogue(a_global, w_global, n, true, NVFP4_OUT_BF16, ld_h);
  return hip_status(launch_gemm_silu_amax(a_codes, a_scales, m, static_cast<const uint8_t*>(w_packed), n, k, h, epi,
                                          amax_parts, parts_capacity, parts_written, (hipStream_t)stream));
}

int nvfp4_quantize_amax_parts(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, const uint32_t* amax_parts,
                              int64_t num_parts, float* global_scale, uint8_t* codes, uint8_t* scales,
                              nvfp4_stream_t stream) {
  int rc = validate_quantize_parts(x, rows, cols, ld_x, amax_parts, num_parts, global_scale, codes, scales);
  if (rc || rows == 0) return rc;
  return hip_status(launch_quantize_from_parts(x, rows, cols, ld_x, amax_parts, num_parts, global_scale, codes, scales,
                                               (hipStream_t)stream));
}

int gdn_recurrence(const uint16_t* q, int64_t ld_q, const uint16_t* k, int64_t ld_k, const uint16_t* v, int64_t ld_v,
                   const uint16_t* beta, int64_t ld_beta, const uint16_t* g, int64_t ld_g, int64_t T, int hk, int hv,
                   int head_dim, const float* s_init, float* s_final, void* out, int out_dtype, int64_t ld_out,
                   nvfp4_stream_t stream) {
  int rc = validate_gdn_recurrence(q, ld_q, k, ld_k, v, ld_v, beta, ld_beta, g, ld_g, T, hk, hv, head_dim, s_init,
                                   s_final, out, out_dtype, ld_out);
  if (rc || T == 0) return rc;
  GdnArgs a{};
  a.q = q;
  a.ld_q = ld_q;
  a.k = k;
  a.ld_k = ld_k;
  a.v = v;
  a.ld_v = ld_v;
  a.beta = beta;
  a.ld_beta = ld_beta;
  a.g = g;
  a.ld_g = ld_g;
  a.T = T;
  a.hk = hk;
  a.hv = hv;
  a.s_init = s_init;
  a.s_final = s_final;
  a.o = out;
  a.o_bf16 = out_dtype == NVFP4_OUT_BF16;
  a.ld_o = ld_out;
  return hip_status(launch_gdn_recurrence(a, (hipStream_t)stream));
}

int nvfp4_weight_stream_read(const void* w_packed, int64_t n, int64_t k, uint32_t* sink, nvfp4_stream_t stream) {
  int rc = validate_unpack(w_packed, n, k, sink, sink);
  if (rc) return rc;
  return hip_status(launch_weight_stream_read(static_cast<const uint8_t*>(w_packed), n, k, sink, (hipStream_t)stream));
}

const char* nvfp4_status_string(int status) {
  switch (status) {
    case NVFP4_OK: return "ok";
    case NVFP4_EINVAL: return "invalid argument (null pointer, unknown enum value or count)";
    case NVFP4_ESHAPE: return "shape rule violated";
    case NVFP4_EALIGN: return "pointer or leading dimension misaligned";
    case NVFP4_EUNSUPPORTED: return "valid request not supported by this library";
    case NVFP4_EHIP: return "HIP launch failed";
    case NVFP4_ESIZE: return "caller buffer too small";
    default: return "unknown status";
  }
}

int nvfp4_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
