// Device helpers shared by the gfx950 NVFP4 kernels: bf16 access, E4M3
// encode/decode, the 16-element block quantizer and the exact in-register
// NVFP4 -> f16 dequantiser that feeds the f16 MFMA.
//
// Format (NVFP4; one E4M3 scale per 16 elements -- bayesiansapien page, "The
// four-part mechanism study", first item): E2M1 codes, low nibble = even
// element; E4M3FN scale bytes; FP32 global scale in encode form.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace nvfp4 {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr float kGlobalNumerator = 2688.0f;  // E2M1 max (6) * E4M3 max (448)
constexpr float kE4M3Max = 448.0f;

// ---------------------------------------------------------------- bf16 ----
__device__ __forceinline__ float bf16_lo(uint32_t two) { return __uint_as_float(two << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t two) { return __uint_as_float(two & 0xFFFF0000u); }

// max over |bf16| of 8 packed values, as the 15-bit magnitude pattern (monotone in |x|).
__device__ __forceinline__ uint32_t absmax_bits8(uint4 v) {
  uint32_t a = v.x & 0x7FFF7FFFu, b = v.y & 0x7FFF7FFFu, c = v.z & 0x7FFF7FFFu, d = v.w & 0x7FFF7FFFu;
  uint32_t m0 = max(max(a & 0xFFFFu, a >> 16), max(b & 0xFFFFu, b >> 16));
  uint32_t m1 = max(max(c & 0xFFFFu, c >> 16), max(d & 0xFFFFu, d >> 16));
  return max(m0, m1);
}

// --------------------------------------------------------------- E4M3 ----
// Round a magnitude u in [0, 448] to the nearest E4M3FN byte, ties to the even
// mantissa.  Below 2^-6 the E4M3 grid is uniform with step 2^-9 (subnormals,
// continuing into 2^-6 = code 8), so rounding is rint(u * 2^9); above, the
// FP32 significand is rounded to 3 bits with the usual carry into the exponent.
__device__ __forceinline__ uint32_t e4m3_encode_rne(float u) {
  uint32_t b = __float_as_uint(u);
  if (b < 0x3C800000u) {                 // u < 2^-6
    return (uint32_t)__builtin_rintf(u * 512.0f);
  }
  uint32_t r = b + 0x7FFFFu + ((b >> 20) & 1u);
  return (r >> 20) - (120u << 3);        // rebias exponent 127 -> 7
}

// Exact value of an E4M3FN byte in [0, 0x7E].
__device__ __forceinline__ float e4m3_decode(uint32_t s) {
  uint32_t e = s >> 3, m = s & 7u;
  if (e == 0) return (float)m * 0x1p-9f;
  return __uint_as_float(((e + 120u) << 23) | (m << 20));
}

// --------------------------------------------------------------- E2M1 ----
// E2M1 codes of FP32 values by gfx950's FP32 -> FP4 conversion with a unit
// scale: two codes per instruction (a in the low nibble) into byte SEL of
// old.  Each code: sign bit 3 = the sign of the value (-0 gives 8), magnitude
// rounded to the nearest of 0, .5, 1, 1.5, 2, 3, 4, 6 with ties to the even
// code, magnitudes above 6 giving 6.  That this is the instruction's rounding
// is checked on the GPU through nvfp4_e2m1_encode (the same instruction in
// both operand slots and all four byte positions) against the closed form
// over every fp32 near each decision point and grid value, and a strided
// sweep of all finite values, both signs.
template <int SEL>
__device__ __forceinline__ uint32_t e2m1_pair(uint32_t old, float a, float b) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, SEL);
}

// ---------------------------------------------------- block quantizer ----
// Quantise 16 bf16 values (two uint4) with global scale g.  Writes 8 code
// bytes (low nibble = even element) and returns the E4M3 scale byte.
//   u = min((m/6)*g, 448); S = E4M3 RNE(u); S == 0 -> codes 0;
//   r = g / value(S); code_i = E2M1 RNE, saturating, of x_i * r, with the sign of x_i.
// Every step is one IEEE FP32 operation (correctly rounded division, a
// correctly rounded product q = x_i * r) followed by the E2M1 conversion.
__device__ __forceinline__ uint32_t pack_codes8(const uint32_t (&w)[4], float r) {
  uint32_t c = e2m1_pair<0>(0u, bf16_lo(w[0]) * r, bf16_hi(w[0]) * r);
  c = e2m1_pair<1>(c, bf16_lo(w[1]) * r, bf16_hi(w[1]) * r);
  c = e2m1_pair<2>(c, bf16_lo(w[2]) * r, bf16_hi(w[2]) * r);
  return e2m1_pair<3>(c, bf16_lo(w[3]) * r, bf16_hi(w[3]) * r);
}

// Scale of a block whose largest magnitude is the bf16 pattern mbits (15
// bits): returns the E4M3 byte S and sets r = g / value(S) (S != 0 only).
__device__ __forceinline__ uint32_t block_scale(uint32_t mbits, float g, float* r) {
  const float m = __uint_as_float(mbits << 16);
  const float t = m / 6.0f;
  const float u = fminf(t * g, kE4M3Max);
  const uint32_t S = e4m3_encode_rne(u);
  *r = S != 0 ? g / e4m3_decode(S) : 0.0f;
  return S;
}

__device__ __forceinline__ uint32_t quantize_block16(uint4 lo, uint4 hi, float g, uint2* codes_out) {
  float r;
  const uint32_t S = block_scale(max(absmax_bits8(lo), absmax_bits8(hi)), g, &r);
  uint2 c = make_uint2(0u, 0u);
  if (S != 0) {
    const uint32_t w[4] = {lo.x, lo.y, lo.z, lo.w};
    const uint32_t v[4] = {hi.x, hi.y, hi.z, hi.w};
    c = make_uint2(pack_codes8(w, r), pack_codes8(v, r));
  }
  *codes_out = c;
  return S;
}

// 4 E2M1 codes (16 bits, low nibble first) of two packed bf16 pairs times r.
__device__ __forceinline__ uint32_t pack_codes4(uint32_t p0, uint32_t p1, float r) {
  return e2m1_pair<1>(e2m1_pair<0>(0u, bf16_lo(p0) * r, bf16_hi(p0) * r), bf16_lo(p1) * r, bf16_hi(p1) * r);
}

// x of both lanes of the pair (l, l ^ 32) at each of them, with one VALU lane
// swap (gfx950's v_permlane32_swap) instead of an LDS permute: .x is the value
// from lanes 0-31, .y the value from lanes 32-63.
__device__ __forceinline__ uint2 lane_halves(uint32_t x) {
  const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return make_uint2(r[0], r[1]);
}

// Two floats to packed bf16 (round to nearest even; the low half holds a).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// --------------------------------------------------------- dequantiser ----
// E4M3 byte s as an f16 bit pattern: (s << 7) read as f16 is value(s) * 2^-8
// for every s (exponent and mantissa fields line up; E4M3 subnormals become
// f16 subnormals).  Two copies packed for v_pk_mul_f16.
__device__ __forceinline__ half2_t scale_pair_f16(uint32_t s) {
  uint32_t b = (s << 7) | (s << 23);
  return __builtin_bit_cast(half2_t, b);
}

// 8 E2M1 codes (one dword, low nibble first) times one E4M3 scale -> 8 exact
// f16 values.  The hardware FP4 -> f16 conversion applies only the exponent
// of its scale operand, so it is given 2^8 and the scale's 2^-8-shifted f16
// (mantissa included) is applied with v_pk_mul_f16; every product e2m1 * s
// has at most 6 significant bits and lies in [2^-10, 2688], so it is exact.
__device__ __forceinline__ half8_t dequant8(uint32_t codes, half2_t sc) {
  half2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 256.0f, 0) * sc;
  half2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 256.0f, 1) * sc;
  half2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 256.0f, 2) * sc;
  half2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 256.0f, 3) * sc;
  half8_t r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

__device__ __forceinline__ floatx16 mfma32x32x16(half8_t a, half8_t b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// The tiled GEMM's product of an activation fragment (32 rows of A) and a
// weight fragment (32 rows of W, i.e. 32 output columns), computed as W . A^T
// so that the result is row-major across lanes: lane l = r + 32h then holds
// output row r, columns 8q + 4h + e (q = 0..3, e = 0..3) in accumulator
// 4q + e -- four runs of four consecutive columns of one row.
__device__ __forceinline__ floatx16 mfma_rows(half8_t a_frag, half8_t w_frag, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(w_frag, a_frag, c, 0, 0, 0);
}

// ------------------------------------------------------------- outputs ----
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t b = __float_as_uint(f);
  return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}

// ---------------------------------------------------- wave reductions ----
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off, 64));
  return v;
}

// Compile-time loop: f(std::integral_constant<int, I>) for I in [B, E).  Used
// where indices into accumulator arrays must stay compile-time constants.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// --------------------------------------------------- packed weight layout ----
// Weights are stored in tiles of 32 rows (output features) x 64 columns (K),
// grouped four along K into super-tiles of 4608 bytes:
//   bytes [t*1024, t*1024+1024): tile t's codes in MFMA lane order -- lane
//     l = c + 32*h owns the 16 bytes of row c, columns 32h..32h+31;
//   bytes [4096, 4608): the scales of the four tiles -- at 4096 + (g*32 + c)*8
//     the eight bytes of row c for tiles 2g and 2g+1 (four block scales each).
// A 32-row slab is a run of K/256 super-tiles (K padded to 256 with zero
// codes and zero scales), so a wave streams it with coalesced 16-byte loads,
// and one 8-byte load per lane (plus a swap across the wave halves) brings a
// row's scales for four tiles.
constexpr int kTileN = 32;
constexpr int kTileK = 64;
constexpr int kTileCodeBytes = kTileN * kTileK / 2;   // 1024
constexpr int kTileScaleBytes = kTileN * kTileK / 16; // 128
constexpr int kSuperTiles = 4;                        // tiles per super-tile along K
constexpr int kSuperK = kSuperTiles * kTileK;         // 256
constexpr int kSuperBytes = kSuperTiles * (kTileCodeBytes + kTileScaleBytes);   // 4608
constexpr int kSuperScaleOff = kSuperTiles * kTileCodeBytes;                      // 4096

// Number of super-tiles along K for a K dimension of k elements.
__host__ __device__ inline int64_t super_count(int64_t k) { return (k + kSuperK - 1) / kSuperK; }
// Byte offset of tile (nt, kt)'s codes; ks = super_count(k).
__host__ __device__ inline int64_t tile_code_off(int64_t nt, int64_t kt, int64_t ks) {
  return (nt * ks + (kt >> 2)) * kSuperBytes + (kt & 3) * kTileCodeBytes;
}
// Byte offset of row c's four block scales of tile (nt, kt).
__host__ __device__ inline int64_t tile_scale_off(int64_t nt, int64_t kt, int64_t ks, int64_t c) {
  return (nt * ks + (kt >> 2)) * kSuperBytes + kSuperScaleOff + (((kt & 3) >> 1) * kTileN + c) * 8 + (kt & 1) * 4;
}

}  // namespace nvfp4
