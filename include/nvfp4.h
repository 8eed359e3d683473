/*
 * nvfp4.h -- C ABI of the MI355X (gfx950) NVFP4 W4A4 linear-layer library.
 *
 * What it computes (sources: the web pages about arXiv 2609.04098, "Why Gated
 * DeltaNet Survives 4-Bit Quantization: NVFP4 W4A4 for the Recurrent Half of
 * a Hybrid 27B LLM"):
 *   - linear layers with 4-bit weights and 4-bit activations, "W4A4"
 *     (bayesiansapien page, TL;DR), in NVIDIA's FP4 format NVFP4 (aipulsen
 *     page, second paragraph);
 *   - NVFP4 block scaling with one scale per 16 elements (bayesiansapien
 *     page, "The four-part mechanism study", first item; nefut page, first
 *     bullet);
 *   - per-module global scales that a kernel fusing several modules into one
 *     GEMM must apply module by module (bayesiansapien page, mechanism study,
 *     "Two practical repairs"; nefut page, last paragraph; aimodeling page,
 *     "What engineers should actually take away").
 *
 * Number format (standard NVFP4; the pages name only "NVFP4"):
 *   element  E2M1, 4 bits (sign, 2 exponent bits, 1 mantissa bit, bias 1):
 *            magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6; two per byte, the LOW
 *            nibble holds the even-indexed element.
 *   scale    E4M3 ("FN", bias 7, max 448), one byte per 16 consecutive
 *            elements along a row (the contraction axis of the GEMM).
 *   global   one FP32 per tensor (per module for fused weights), stored in
 *            encode form g = 2688 / amax (2688 = 6 * 448; g = 1 for amax 0).
 *
 * Quantisation of a 16-element block with maximum magnitude m (FP32, every
 * step one correctly rounded operation):
 *   u = min((m / 6) * g, 448); S = E4M3 round-to-nearest-even(u);
 *   S == 0 -> all 16 codes are 0; else r = g / value(S) and
 *   code_i = sign(x_i) << 3 | E2M1 round-to-nearest-even, saturating at 6, of |x_i * r|.
 * Dequantised element = e2m1(code) * e4m3(S); the GEMM divides the product
 * by g_a * g_w:  y[m][n] = sum_k a[m][k] w[n][k] / (g_a * g_w[segment of n]).
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless marked "host".  bf16 tensors are
 *     passed as uint16_t bit patterns.  All device buffers are owned and
 *     allocated by the caller; the library allocates no device memory and
 *     keeps no mutable global state (apart from a thread-local copy of the
 *     last HIP error).  Host arrays are only read during the call.
 *   - Work is enqueued on `stream` (0 = the null stream); no call
 *     synchronises.  Device-side failures surface at the caller's next
 *     synchronisation.
 *   - Return value 0 = success, a negative NVFP4_E* code otherwise.  On a
 *     validation error nothing is enqueued.
 *   - Inputs must be finite; NaN/Inf inputs give unspecified codes.
 *   - Device pointers must be 16-byte aligned; leading dimensions are in
 *     elements and must keep every row 16-byte aligned where noted.
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* nvfp4_stream_t; /* the same type as hipStream_t */

/* Status codes. */
#define NVFP4_OK 0
#define NVFP4_EINVAL (-1)       /* null pointer, unknown enum value, bad count */
#define NVFP4_ESHAPE (-2)       /* sizes that violate a stated shape rule */
#define NVFP4_EALIGN (-3)       /* pointer or leading dimension not aligned */
#define NVFP4_EUNSUPPORTED (-4) /* valid request outside what this library implements */
#define NVFP4_EHIP (-5)         /* a HIP launch failed (see nvfp4_last_hip_error) */
#define NVFP4_ESIZE (-6)        /* a caller buffer is smaller than required */

/* Output element types. */
#define NVFP4_OUT_F32 0
#define NVFP4_OUT_BF16 1

/* Epilogues of gemm_w4a4. */
#define NVFP4_EPI_NONE 0
#define NVFP4_EPI_SILU_MUL 1 /* out[:, j] = silu(y[:, j]) * y[:, j + n/2], j < n/2 */

/* Per-segment epilogues of gemm_w4a4_fused_segments. */
#define NVFP4_SEG_NONE 0
#define NVFP4_SEG_SIGMOID 1   /* write strength: 1 / (1 + exp(-y)) */
#define NVFP4_SEG_GDN_DECAY 2 /* decay: -exp(a_log[h]) * softplus(y + dt_bias[h]), h = column in segment */

#define NVFP4_MAX_SEGMENTS 16

/*
 * nvfp4_quantize -- on-the-fly activation quantizer (the "A4" of W4A4;
 * bayesiansapien page, TL;DR) with NVFP4 16-element block scaling
 * (bayesiansapien page, mechanism study, first item).
 *
 *   x        bf16 [rows, cols], row stride ld_x elements (ld_x >= cols,
 *            ld_x % 8 == 0 so rows are 16-byte aligned).
 *   rows     >= 0; rows == 0 enqueues nothing (and leaves *global_scale).
 *   cols     > 0, cols % 16 == 0.
 *   global_scale  one device float.  dynamic_global != 0: the call writes
 *            g = 2688 / max|x| (1 if x is all zero) there, on the device.
 *            dynamic_global == 0: the call reads a calibrated g from there.
 *   codes    out, uint8 [rows, cols/2], contiguous; low nibble = even column.
 *            With dynamic_global, codes is also used as scratch for the
 *            partial maxima before it is overwritten.
 *   scales   out, E4M3 bytes [rows, cols/16], contiguous.
 */
int nvfp4_quantize(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                   float* global_scale, int dynamic_global,
                   uint8_t* codes, uint8_t* scales, nvfp4_stream_t stream);

/*
 * nvfp4_e2m1_encode -- the element encoder of nvfp4_quantize on its own, for
 * verification: codes[i] = the 4-bit E2M1 code (0..15, one per byte) that the
 * quantizer gives the scaled value q[i] (q = x * g / value(S) in the
 * quantisation rule above): sign bit 3 = the sign bit of q[i] (-0 gives 8),
 * magnitude rounded to the nearest of 0, .5, 1, 1.5, 2, 3, 4, 6 with ties to
 * the even code, magnitudes above 6 giving 6 (code 7).  NVFP4's element type
 * (aipulsen page, second paragraph).  The kernels convert two values per
 * instruction into one of four byte positions; here values 2j and 2j+1 share
 * one conversion at position j % 4, so every slot the quantizer uses runs.
 *
 *   q      device float [n], 4-byte aligned; finite values (NaN unspecified).
 *   n      >= 0 (0 enqueues nothing).
 *   codes  device uint8 [n], out.
 */
int nvfp4_e2m1_encode(const float* q, int64_t n, uint8_t* codes, nvfp4_stream_t stream);

/*
 * nvfp4_packed_weight_bytes -- bytes of the opaque packed weight buffer for
 * an [n, k] weight (k % 16 == 0); 0 for invalid sizes.  It is the NVFP4
 * storage (k/2 + k/16 bytes per row, i.e. 4.5 bits per weight) of the weight
 * padded to 32-row x 256-column blocks (zero codes and scales in the padding).
 */
size_t nvfp4_packed_weight_bytes(int64_t n, int64_t k);

/*
 * nvfp4_pack_weights -- offline weight quantizer/packer (the "W4" of W4A4;
 * bayesiansapien page, TL;DR), with one global scale per module for fused
 * weights (bayesiansapien page, "Two practical repairs").
 *
 *   w            bf16 [n, k], nn.Linear layout (row = output feature),
 *                contiguous, k % 16 == 0, n >= 1.
 *   num_segments 1..NVFP4_MAX_SEGMENTS; segment s is rows
 *                [seg_offsets[s], seg_offsets[s+1]).
 *   seg_offsets  host, num_segments+1 int64, 0 = first < ... < last = n.
 *   seg_global   device float [num_segments]: written (2688/amax of the
 *                segment) when dynamic_global != 0, else read (calibrated).
 *   packed       out, opaque, nvfp4_packed_weight_bytes(n, k) bytes;
 *                padding rows/columns hold zero codes and zero scales.
 */
int nvfp4_pack_weights(const uint16_t* w, int64_t n, int64_t k,
                       int num_segments, const int64_t* seg_offsets,
                       float* seg_global, int dynamic_global,
                       void* packed, size_t packed_bytes, nvfp4_stream_t stream);

/*
 * nvfp4_unpack_weights_linear -- documented inverse of the packed layout:
 * writes linear codes [n, k/2] and scales [n, k/16] (the layout
 * nvfp4_quantize produces) so packed weights can be checked byte by byte.
 */
int nvfp4_unpack_weights_linear(const void* packed, int64_t n, int64_t k,
                                uint8_t* codes, uint8_t* scales, nvfp4_stream_t stream);

/*
 * gemm_w4a4 -- block-scaled FP4 x FP4 GEMM with FP32 accumulation, the W4A4
 * linear layer (bayesiansapien page, TL;DR; Figure node "Minima: NVFP4 W4A4
 * all 496 linear layers"):
 *     y[i][j] = alpha * sum_k a[i][k] * w[j][k],  alpha = 1 / (*a_global * *w_global)
 * with a, w the dequantised NVFP4 elements (global scale not folded in).
 *
 *   a_codes, a_scales  the activation as written by nvfp4_quantize for an
 *                      [m, k] tensor (contiguous).
 *   a_global, w_global device floats (encode-form global scales).
 *   m >= 0 (0 enqueues nothing), n >= 1, k >= 16, k % 16 == 0 (any K that
 *                      NVFP4 blocks divide).
 *   w_packed           from nvfp4_pack_weights with the same n, k.  A
 *                      weight packed with several segments is treated as one
 *                      module with scale *w_global (use the fused-segment
 *                      entry point to apply each module's own scale).
 *   out                [m, n] (epilogue NONE) or [m, n/2] (SILU_MUL), row
 *                      stride ld_out elements, element type out_dtype
 *                      (out aligned to its element size).
 *   epilogue           NONE, or SILU_MUL: requires n % 64 == 0 and computes
 *                      out[:, j] = silu(y[:, j]) * y[:, j + n/2].
 * m <= 64 runs a weight-streaming decode kernel (m <= 8 without an epilogue:
 * the block-scaled FP4 MFMA on the raw codes with the E4M3 scales applied in
 * FP32; otherwise exact dequantisation to f16 and the f16 MFMA), larger m the
 * tiled prefill kernel; all give results within 1e-5 * sum_k |a*w| * alpha.
 */
int gemm_w4a4(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_global, int64_t m,
              const void* w_packed, const float* w_global, int64_t n, int64_t k,
              void* out, int out_dtype, int64_t ld_out, int epilogue, nvfp4_stream_t stream);

/*
 * nvfp4_linear -- the whole W4A4 linear layer on a bf16 activation: the
 * on-the-fly quantisation of x ("A4"; bayesiansapien page, TL;DR), with the
 * same result bytes as nvfp4_quantize, which it also writes out, followed by
 * gemm_w4a4 on those codes.  Decode-sized calls (m <= 2, epilogue NONE,
 * k <= 6144) run as ONE kernel: every
 * workgroup computes the activation's amax and global scale and quantises
 * the (small) activation itself while its weight stream is in flight, and
 * workgroup 0 writes the codes, scales and global scale; the output is then
 * bit-identical to nvfp4_quantize + gemm_w4a4.  Other shapes enqueue those
 * two calls.
 *
 *   x, m, k, ld_x   the activation: bf16 [m, k] as nvfp4_quantize's x, rows,
 *                   cols, ld_x (k % 16 == 0, ld_x % 8 == 0).
 *   a_global, dynamic_global   as nvfp4_quantize's global_scale and
 *                   dynamic_global (written when dynamic, else read).
 *   a_codes, a_scales  out: the quantised activation, [m, k/2] and [m, k/16]
 *                   bytes, contiguous (codes 16-byte aligned).
 *   w_packed, w_global, n, out, out_dtype, ld_out, epilogue   as gemm_w4a4.
 */
int nvfp4_linear(const uint16_t* x, int64_t m, int64_t k, int64_t ld_x, float* a_global, int dynamic_global,
                 uint8_t* a_codes, uint8_t* a_scales, const void* w_packed, const float* w_global, int64_t n,
                 void* out, int out_dtype, int64_t ld_out, int epilogue, nvfp4_stream_t stream);

/*
 * gemm_w4a4_fused_segments -- one GEMM over a fused weight whose column
 * segments are separately calibrated modules: the global-scale-mismatch
 * repair of the bayesiansapien page ("Two practical repairs") and aimodeling
 * page ("What engineers should actually take away").  Output column j of
 * segment s gets alpha_s = 1 / (*a_global * seg_w_global[s]), then the
 * segment's epilogue (the Gated DeltaNet gate parameterisations of the
 * bayesiansapien page, mechanism study, second item).
 *
 *   A, m, k, w_packed, n, out, out_dtype, ld_out as for gemm_w4a4.
 *   num_segments  1..NVFP4_MAX_SEGMENTS; seg_offsets host int64
 *                 [num_segments+1], 0 = first < ... < last = n.
 *   seg_w_global  device float [num_segments].
 *   seg_epilogue  host int [num_segments]: NVFP4_SEG_NONE / SIGMOID / GDN_DECAY.
 *   a_log, dt_bias device float, one per column of the (at most one)
 *                 GDN_DECAY segment; may be null if no segment uses it.
 */
int gemm_w4a4_fused_segments(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_global,
                             int64_t m, const void* w_packed, int64_t n, int64_t k,
                             int num_segments, const int64_t* seg_offsets, const float* seg_w_global,
                             const int* seg_epilogue, const float* a_log, const float* dt_bias,
                             void* out, int out_dtype, int64_t ld_out, nvfp4_stream_t stream);

/*
 * gemm_w4a4_silu_mul_quantize -- the MLP gate/up projection whose activation
 * h = silu(gate) * up leaves the GEMM already quantised to NVFP4, as the A
 * operand of the down projection: the 4-bit activations of W4A4
 * (bayesiansapien page, TL;DR) produced in the epilogue, so h never goes
 * through HBM in bf16.  The global scale of h is static: a calibrated value
 * (h's amax is not known until the whole GEMM has finished).
 *
 * Each h[i][j] (j < n/2) is computed as by gemm_w4a4 with SILU_MUL from the
 * tiled kernel, rounded to bf16, and that bf16 row is quantised exactly as
 * nvfp4_quantize quantises a bf16 tensor with dynamic_global = 0 and global
 * scale *h_global (blocks that overflow the scale range saturate: u is
 * clamped to 448 and |x * r| to 6).
 *
 *   A, m, w_packed, w_global, n, k as for gemm_w4a4; n % 64 == 0 (gate
 *            columns [0, n/2), up columns [n/2, n)).  Every m runs the
 *            tiled kernel (no weight-streaming path).
 *   h_global device float, the encode-form global scale of h (read only).
 *   h_codes  [m, n/4] bytes, row-major contiguous, 16-byte aligned.
 *   h_scales [m, n/32] bytes, row-major contiguous.
 *   h_out    optional (may be null): receives the bf16 h [m, n/2] that was
 *            quantised, row-major contiguous, 16-byte aligned.
 */
int gemm_w4a4_silu_mul_quantize(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_global,
                                int64_t m, const void* w_packed, const float* w_global, int64_t n, int64_t k,
                                const float* h_global, uint8_t* h_codes, uint8_t* h_scales, uint16_t* h_out,
                                nvfp4_stream_t stream);

/*
 * nvfp4_silu_amax_parts -- size query: the number of uint32 partial maxima
 * gemm_w4a4_silu_mul_amax may write for an m x n gate/up projection (0 for
 * m <= 0 or n <= 0).
 *
 * gemm_w4a4_silu_mul_amax -- the MLP gate/up projection with bf16 h (as
 * gemm_w4a4 with SILU_MUL and bf16 output) that also leaves partial maxima
 * of |h| for the dynamic global scale of h's on-the-fly quantisation (the
 * 4-bit activations of W4A4 between the MLP's two GEMMs; bayesiansapien
 * page, TL;DR).  With nvfp4_quantize_amax_parts this replaces
 * nvfp4_quantize(h, dynamic_global = 1): the maximum is taken from the values
 * the GEMM stores, in its epilogue, instead of by a pass that reads h back,
 * and the codes, scales and global scale are bit-identical to that call's.
 *
 *   A, m, w_packed, w_global, n, k as for gemm_w4a4; n % 64 == 0.
 *   h            bf16 [m, n/2], row stride ld_h (a multiple of 8), 16-byte
 *                aligned: h = silu(gate) * up, identical to gemm_w4a4's.
 *   amax_parts   device uint32 [parts_capacity], 4-byte aligned: receives the
 *                partial maxima (15-bit bf16 magnitude patterns); the buffer
 *                may be h's codes buffer of the following
 *                nvfp4_quantize_amax_parts call.
 *   parts_capacity >= nvfp4_silu_amax_parts(m, n), else NVFP4_ESHAPE.
 *   parts_written  host int64: the number of partial maxima written (0 for
 *                m == 0).  Set when the call returns; no device sync.
 * The prefill kernels (m > 64, k % 64 == 0) write one maximum per wave from
 * the epilogue; other shapes run gemm_w4a4 and then an amax pass over h.
 *
 * nvfp4_quantize_amax_parts -- nvfp4_quantize with dynamic_global = 1 whose
 * amax is the largest of num_parts partial maxima (from
 * gemm_w4a4_silu_mul_amax over this x): writes *global_scale = 2688 / amax
 * (1 if amax == 0), then codes and scales as nvfp4_quantize.
 *   x, rows, cols, ld_x, global_scale, codes, scales as for nvfp4_quantize.
 *   amax_parts   device uint32 [num_parts] (4-byte aligned), 1 <= num_parts
 *                <= 2^31 - 1; may alias codes (the maxima are reduced before
 *                any code is written).
 */
int64_t nvfp4_silu_amax_parts(int64_t m, int64_t n);
int gemm_w4a4_silu_mul_amax(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_global, int64_t m,
                            const void* w_packed, const float* w_global, int64_t n, int64_t k, uint16_t* h,
                            int64_t ld_h, uint32_t* amax_parts, int64_t parts_capacity, int64_t* parts_written,
                            nvfp4_stream_t stream);
int nvfp4_quantize_amax_parts(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                              const uint32_t* amax_parts, int64_t num_parts, float* global_scale, uint8_t* codes,
                              uint8_t* scales, nvfp4_stream_t stream);

/*
 * gdn_recurrence -- the gated delta-rule recurrence of a Gated DeltaNet layer,
 * the recurrent half that the in-projection feeds.  The pages characterise
 * it by behaviour rather than by a formula: the delta rule replaces the
 * state's component along the key, so errors do not pile up and an old
 * disturbance fades (bayesiansapien page, "The four-part mechanism study",
 * third item).  The
 * rule computed (the standard gated delta rule), per value head h with key
 * head h / (hv / hk) and fp32 state S [head_dim, head_dim] (row = value
 * index, column = key index), for t = 0 .. T-1:
 *     k^ = k_t / sqrt(|k_t|^2 + 1e-6),  q^ = q_t / sqrt(|q_t|^2 + 1e-6),
 *     S <- exp(g_t) S (I - beta_t k^ k^T) + beta_t v_t k^T,   o_t = S q^.
 * beta and g are the outputs of the fused in-projection's SIGMOID and
 * GDN_DECAY segments; q, k, v its first three segments, so every input may
 * point into that one bf16 buffer with its row stride.
 *
 *   q, k      bf16 [T, hk * head_dim], row strides ld_q, ld_k (elements,
 *             multiples of 8); 16-byte aligned.
 *   v         bf16 [T, hv * head_dim], row stride ld_v (multiple of 8).
 *   beta, g   bf16 [T, hv], row strides ld_beta, ld_g.
 *   T >= 0 (0 enqueues nothing); hk >= 1; hv a multiple of hk;
 *   head_dim  128 (others: NVFP4_EUNSUPPORTED).
 *   s_init    optional fp32 [hv, head_dim, head_dim] initial state (null = 0).
 *   s_final   optional fp32 [hv, head_dim, head_dim], receives the last state.
 *   out       [T, hv * head_dim] fp32 or bf16 (out_dtype), row stride ld_out.
 * The state stays in fp32 registers for the whole sequence; results are
 * deterministic.
 */
int gdn_recurrence(const uint16_t* q, int64_t ld_q, const uint16_t* k, int64_t ld_k, const uint16_t* v,
                   int64_t ld_v, const uint16_t* beta, int64_t ld_beta, const uint16_t* g, int64_t ld_g,
                   int64_t T, int hk, int hv, int head_dim, const float* s_init, float* s_final, void* out,
                   int out_dtype, int64_t ld_out, nvfp4_stream_t stream);

/*
 * nvfp4_weight_stream_read -- measurement reference for the decode GEMMs,
 * which are bound by HBM bandwidth: reads every byte of a packed [n, k]
 * weight with the same loads, in the same order and launch shape as the
 * weight-streaming decode kernel (one workgroup per 32-column slab, four
 * waves splitting its K range), and does no arithmetic.  Its time is the
 * practical ceiling against which a decode GEMM's time is judged.
 *
 *   w_packed  from nvfp4_pack_weights with the same n, k (16-byte aligned).
 *   sink      device uint32, written only in the (practically impossible)
 *             case that the XOR of all words equals 0x9E3779B9.
 */
int nvfp4_weight_stream_read(const void* w_packed, int64_t n, int64_t k, uint32_t* sink, nvfp4_stream_t stream);

/* Human-readable text of a status code (static storage). */
const char* nvfp4_status_string(int status);

/* The HIP error code of the last NVFP4_EHIP returned on this thread (0 if none). */
int nvfp4_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H */
