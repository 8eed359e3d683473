// Internal launcher interface between the C ABI layer and the HIP kernels.
// Launchers enqueue on the given stream and return the launch status; all
// argument validation happens before they are called.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

constexpr int kMaxSegments = 16;

// Row (packer) or column (GEMM) segments of a fused weight, passed by value
// as a kernel argument.
struct SegmentTable {
  int64_t off[kMaxSegments + 1];
  int num;
};

// Per-output-column epilogue description for the GEMM kernels.
struct EpilogueArgs {
  SegmentTable segs;            // column segments (num == 1 for a plain GEMM)
  int seg_epi[kMaxSegments];    // NVFP4_SEG_* per segment
  const float* seg_w_global;    // device [num] weight global scales
  const float* a_global;        // device scalar activation global scale
  const float* a_log;           // device, per column of the decay segment
  const float* dt_bias;         // device, per column of the decay segment
  int silu_mul;                 // 1: out[:, j] = silu(y[:, j]) * y[:, j + n/2]
  int out_bf16;                 // 1: bf16 output, 0: fp32
  int64_t ld_out;
  // SiLU*mul with NVFP4 output (h_codes != null): h is rounded to bf16 and
  // quantised with the static global scale *h_global into h_codes [m, n/4]
  // and h_scales [m, n/32]; h_out (optional) receives the bf16 h [m, n/2].
  const float* h_global;
  uint8_t* h_codes;
  uint8_t* h_scales;
  uint16_t* h_out;
  // SiLU*mul with bf16 h output (h_amax != null, prefill kernels): every wave
  // writes the largest |h| it stored, as a 15-bit bf16 magnitude pattern, to
  // h_amax[h_amax_base + block * waves + wave].
  uint32_t* h_amax;
  int64_t h_amax_base;
};

inline int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

hipError_t launch_quantize(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, float* g,
                           bool dynamic, uint8_t* codes, uint8_t* scales, hipStream_t st);
hipError_t launch_pack(const uint16_t* w, int64_t n, int64_t k, const SegmentTable& segs, float* seg_g,
                       bool dynamic, uint8_t* packed, hipStream_t st);
hipError_t launch_e2m1_encode(const float* q, int64_t n, uint8_t* codes, hipStream_t st);
hipError_t launch_unpack(const uint8_t* packed, int64_t n, int64_t k, uint8_t* codes, uint8_t* scales,
                         hipStream_t st);
hipError_t launch_gemm(const uint8_t* a_codes, const uint8_t* a_scales, int64_t m, const uint8_t* w_packed,
                       int64_t n, int64_t k, void* out, const EpilogueArgs& epi, hipStream_t st);
// SiLU*mul GEMM into bf16 h [m, n/2] (stride epi.ld_out) that also leaves
// partial maxima of |h| in parts[0 .. *written): from the prefill kernels'
// epilogue, or (other paths) from an amax pass over h.  cap >= the bound below.
hipError_t launch_gemm_silu_amax(const uint8_t* a_codes, const uint8_t* a_scales, int64_t m, const uint8_t* w_packed,
                                 int64_t n, int64_t k, uint16_t* h, const EpilogueArgs& epi, uint32_t* parts,
                                 int64_t cap, int64_t* written, hipStream_t st);
int64_t silu_amax_parts_bound(int64_t m, int64_t n);
// Partial maxima of |x| over a bf16 [rows, cols] (stride ld) into parts[0 .. nparts).
hipError_t launch_amax_partials(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, uint32_t* parts,
                                int nparts, hipStream_t st);
// Dynamic-scale quantisation whose amax is the maximum of nparts partial maxima
// (parts may alias codes: they are reduced before any code is written).
hipError_t launch_quantize_from_parts(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld,
                                      const uint32_t* parts, int64_t nparts, float* g, uint8_t* codes,
                                      uint8_t* scales, hipStream_t st);
// Gated delta-rule recurrence (head dimension 128): bf16 inputs with row
// strides in elements, fp32 state [hv, 128, 128], output [T, hv * 128].
struct GdnArgs {
  const uint16_t* q;
  int64_t ld_q;
  const uint16_t* k;
  int64_t ld_k;
  const uint16_t* v;
  int64_t ld_v;
  const uint16_t* beta;
  int64_t ld_beta;
  const uint16_t* g;
  int64_t ld_g;
  int64_t T;
  int hk;
  int hv;
  const float* s_init;
  float* s_final;
  void* o;
  int o_bf16;
  int64_t ld_o;
};
hipError_t launch_gdn_recurrence(const GdnArgs& a, hipStream_t st);

// Activation quantisation fused into a decode GEMM: the bf16 activation, its
// global scale (written when dynamic, else read) and where the quantised
// activation (codes [m, k/2], scales [m, k/16]) is written.
struct QuantSource {
  const uint16_t* x;
  int64_t ld_x;
  float* g;
  int dynamic;
  uint8_t* codes;
  uint8_t* scales;
};

// Weight-streaming decode kernels (small m); false: the shape is not theirs.
bool launch_gemm_decode(const uint8_t* a_codes, const uint8_t* a_scales, int64_t m, const uint8_t* w_packed,
                        int64_t n, int64_t k, void* out, const EpilogueArgs& epi, hipStream_t st);
// Quantise a small bf16 activation and multiply it in one decode kernel;
// false: not supported for this shape (quantise, then launch_gemm).
bool launch_gemm_decode_quantize(const QuantSource& qs, int64_t m, const uint8_t* w_packed, int64_t n, int64_t k,
                                 void* out, const EpilogueArgs& epi, hipStream_t st);

// Quantise the bf16 activation of qs and multiply: one kernel where
// launch_gemm_decode_quantize takes the shape, else launch_quantize and
// launch_gemm.  epi.a_global must be qs.g.
hipError_t launch_linear(const QuantSource& qs, int64_t m, const uint8_t* w_packed, int64_t n, int64_t k,
                         void* out, const EpilogueArgs& epi, hipStream_t st);

// The decode weight stream with no arithmetic (roofline reference).
hipError_t launch_weight_stream_read(const uint8_t* w_packed, int64_t n, int64_t k, uint32_t* sink, hipStream_t st);

// The tiled (prefill) kernels for any m; used for the quantising SiLU*mul epilogue.
hipError_t launch_gemm_tiled(const uint8_t* a_codes, const uint8_t* a_scales, int64_t m, const uint8_t* w_packed,
                             int64_t n, int64_t k, void* out, const EpilogueArgs& epi, hipStream_t st);

}  // namespace nvfp4
