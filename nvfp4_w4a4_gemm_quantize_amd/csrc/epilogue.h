// Device helpers shared by the GEMM kernels (tiled prefill and the
// weight-streaming decode kernels): the per-column epilogue -- alpha of the
// column's weight segment and the segment's gate (sigmoid write strength or
// the Gated DeltaNet decay), SiLU*mul -- output stores and guarded loads.
#pragma once
#include "kernels.h"
#include "nvfp4_device.h"

namespace nvfp4 {

// ----------------------------------------------------------- epilogue ----
struct ColumnEpilogue {
  float alpha;
  int type;
  float exp_alog;  // exp(A_log[h]) for the decay segment
  float dt_bias;
};

// The column's segment by a scan over the segment table.  The table and the
// segments' scales and gate types are read at wave-uniform addresses (scalar
// loads, no dependent chain); each lane only selects.  Columns of the decay
// segment also read their head's A_log and dt_bias.
__device__ __forceinline__ ColumnEpilogue column_epilogue(const EpilogueArgs& e, int64_t col, float ga) {
  float gw = e.seg_w_global[0];
  int type = e.seg_epi[0];
  int64_t first = 0;
  for (int s = 1; s < e.segs.num; ++s) {
    const int64_t o = e.segs.off[s];
    const float g = e.seg_w_global[s];
    const int t = e.seg_epi[s];
    if (col >= o) {
      gw = g;
      type = t;
      first = o;
    }
  }
  ColumnEpilogue c;
  c.alpha = 1.0f / (ga * gw);
  c.type = type;
  c.exp_alog = 0.0f;
  c.dt_bias = 0.0f;
  if (type == 2) {
    const int64_t h = col - first;
    c.exp_alog = expf(e.a_log[h]);
    c.dt_bias = e.dt_bias[h];
  }
  return c;
}

// Per-column epilogue parameters of a workgroup's BN output columns
// (col_base ...), written to LDS once per workgroup before its main loop so
// the epilogue reads one LDS entry per column instead of searching the
// segment table and dividing for every output.  Columns past n (never
// stored) get no gate, so a padded tile does no gate arithmetic for them.
template <int BN, int NT>
__device__ __forceinline__ void fill_column_table(ColumnEpilogue* tab, const EpilogueArgs& e, int64_t col_base,
                                                  int64_t n) {
  const float ga = *e.a_global;
  for (int c = (int)threadIdx.x; c < BN; c += NT) {
    const int64_t col = col_base + c;
    ColumnEpilogue ce = column_epilogue(e, col < n ? col : n - 1, ga);
    if (col >= n) ce.type = 0;
    tab[c] = ce;
  }
}

constexpr float kLog2e = 1.44269504088896341f;
constexpr float kLn2 = 0.693147180559945309f;

// 1 / (1 + e^-y) on the hardware exp2 and reciprocal.
__device__ __forceinline__ float sigmoid_f(float y) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-y * kLog2e));
}

// log(1 + e^x) = max(x, 0) + log1p(e^-|x|).  log1p(e) is taken as
// log(u) * e / (u - 1) with u = 1 + e rounded (u - 1 is exact), which keeps
// the relative accuracy of small e; u == 1 gives e itself.
__device__ __forceinline__ float softplus_f(float x) {
  const float e = __builtin_amdgcn_exp2f(-fabsf(x) * kLog2e);
  const float u = 1.0f + e;
  const float l = u == 1.0f ? e : __builtin_amdgcn_logf(u) * kLn2 * e * __builtin_amdgcn_rcpf(u - 1.0f);
  return fmaxf(x, 0.0f) + l;
}

__device__ __forceinline__ float apply_epilogue(const ColumnEpilogue& c, float acc) {
  float y = acc * c.alpha;
  if (c.type == 1) {
    y = sigmoid_f(y);
  } else if (c.type == 2) {
    y = -c.exp_alog * softplus_f(y + c.dt_bias);
  }
  return y;
}

// silu(g)*u = g*u / (1 + e^-g), with e^-g = 2^(-g*log2 e) on the hardware exp2
// and the division as the hardware reciprocal (each within about an ulp of
// fp32, far below the bf16 rounding of the result; e^-g = inf gives 0).
__device__ __forceinline__ float silu_mul(float g, float u) {
  const float e = __builtin_amdgcn_exp2f(-g * 1.44269504088896341f);
  return g * u * __builtin_amdgcn_rcpf(1.0f + e);
}

// The epilogue's LDS staging region belongs to one wave, and a wave's LDS
// instructions execute in issue order, so only the compiler has to keep the
// region's writes and reads in program order: no workgroup barrier.
__device__ __forceinline__ void wave_lds_order() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ void store_out(void* out, bool bf16, int64_t idx, float v) {
  if (bf16) reinterpret_cast<uint16_t*>(out)[idx] = f32_to_bf16_rne(v);
  else reinterpret_cast<float*>(out)[idx] = v;
}

// ------------------------------------------------------ shared helpers ----
// Load a 16-byte chunk if `ok`, zeros otherwise.
__device__ __forceinline__ uint4 ld16(const uint8_t* p, bool ok) {
  return ok ? *reinterpret_cast<const uint4*>(p) : make_uint4(0u, 0u, 0u, 0u);
}

// Scale pair (blocks 2h, 2h+1 of a 64-wide K tile) -> scale byte for sub-step s.
__device__ __forceinline__ uint32_t scale_byte(uint32_t pair, int s) { return (pair >> (8 * (s >> 1))) & 0xFFu; }

}  // namespace nvfp4
