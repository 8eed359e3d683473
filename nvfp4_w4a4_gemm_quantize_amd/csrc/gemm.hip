// W4A4 NVFP4 GEMM kernels for gfx950 (CDNA4): y = alpha * A_q . W_q^T with
// FP32 accumulation, for the 4-bit-weight / 4-bit-activation linear layers of
// the bayesiansapien page (TL;DR), including the fused-module case where each
// output-column segment has its own global scale (same page, "Two practical
// repairs").
//
// Arithmetic path: NVFP4 elements are dequantised exactly in registers to f16
// (e2m1 * e4m3 has at most 6 significant bits) and multiplied with
// v_mfma_f32_32x32x16_f16.  gfx950's block-scaled FP4 MFMA takes one E8M0
// (power-of-two) scale per 32 elements, which cannot represent NVFP4's E4M3
// scale per 16 elements, so the exact f16 path is used.
//
// Lane layout of one 32x32x16 MFMA: lane l = r + 32h supplies row r of A and
// column r of W at 8 K positions chosen by h.  Because a lane's 16 packed
// bytes hold 32 consecutive K values, sub-step s of a 64-wide K tile uses the
// lane's dword s: K positions 32h + 8s .. +7 -- the same set for A and W, so
// the contraction is over every K exactly once.  The 16 accumulators of lane
// l hold rows 8*(j/4) + 4h + (j%4) of column r.
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

// ------------------------------------------------------ tile epilogue ----
// Epilogue of a workgroup tile: each 32x32 accumulator fragment of a wave goes
// through a per-wave LDS staging tile (32 x 33 floats) so that every lane
// owns 4 rows x 4 consecutive columns; it applies alpha and the column's gate
// function and stores 4 contiguous outputs per row.  One runtime loop over
// the fragments keeps the epilogue code single; the fragment to stage is
// picked by compile-time cases, so the accumulators stay in registers.
// col_base: first output column of the workgroup; wave_n's fragment jj covers
// output columns col_base + (wave_n * NJ + jj) * 32 .. +31.
// ctab: the workgroup's per-column table (fill_column_table; unused for SiLU*mul).
template <int MF, int NF, int WM, int WN, bool SILU>
__device__ __forceinline__ void tile_epilogue(floatx16 (&acc)[MF][NF], uint8_t* lds, const ColumnEpilogue* ctab,
                                              int lane, int wave, int wave_m, int wave_n, int64_t m0,
                                              int64_t col_base, int64_t m, int64_t n, void* out,
                                              const EpilogueArgs& epi) {
  constexpr int EPI_STRIDE = 33;
  constexpr int NJ = SILU ? NF / 2 : NF;
  const int r = lane & 31, h = lane >> 5;
  float* ep = reinterpret_cast<float*>(lds) + wave * (32 * EPI_STRIDE);
  const int er = (lane >> 3) * 4, ec = (lane & 7) * 4;   // this lane: rows er..er+3, cols ec..ec+3
  const float ga = *epi.a_global;
  const bool bf16 = epi.out_bf16 != 0;
  const int64_t ld = epi.ld_out;
  const int64_t ncols = SILU ? n / 2 : n;

  auto stage_frag = [&](floatx16 f) __attribute__((always_inline)) {
#pragma unroll
    for (int e = 0; e < 16; ++e) ep[(8 * (e >> 2) + 4 * h + (e & 3)) * EPI_STRIDE + r] = f[e];
  };
  auto read_frag = [&](float (&v)[4][4]) __attribute__((always_inline)) {
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) v[a][b] = ep[(er + a) * EPI_STRIDE + ec + b];
  };
  auto store_row = [&](int64_t row, int64_t col0, const float (&v)[4]) __attribute__((always_inline)) {
    if (row >= m) return;
    const int64_t idx = row * ld + col0;
    if (col0 + 3 < ncols && (idx & 3) == 0) {
      if (bf16) {
        uint2 pk;
        pk.x = (uint32_t)f32_to_bf16_rne(v[0]) | ((uint32_t)f32_to_bf16_rne(v[1]) << 16);
        pk.y = (uint32_t)f32_to_bf16_rne(v[2]) | ((uint32_t)f32_to_bf16_rne(v[3]) << 16);
        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out) + idx) = pk;
      } else {
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + idx) = make_float4(v[0], v[1], v[2], v[3]);
      }
    } else {
#pragma unroll
      for (int b = 0; b < 4; ++b)
        if (col0 + b < ncols) store_out(out, bf16, idx + b, v[b]);
    }
  };

  const float alpha_silu = SILU ? 1.0f / (ga * epi.seg_w_global[0]) : 0.0f;
  // SiLU(gate) * up of a fragment pair, in the accumulator layout (the gate
  // and up fragments share it), so only the result goes through LDS.
  auto silu_frag = [&](const floatx16& g, const floatx16& u) __attribute__((always_inline)) -> floatx16 {
    floatx16 hv;
#pragma unroll
    for (int e = 0; e < 16; ++e) hv[e] = silu_mul(g[e] * alpha_silu, u[e] * alpha_silu);
    return hv;
  };
  // Quantising SiLU*mul: lane (r, h) takes row r, columns 16h..16h+15 of the
  // staged fragment -- one whole 16-element block of h.
  const bool quant = SILU && epi.h_codes != nullptr;
  const float hg = quant ? *epi.h_global : 0.0f;
  auto read_block = [&](float (&v)[16]) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < 16; ++c) v[c] = ep[r * EPI_STRIDE + 16 * h + c];
  };
  for (int f = 0; f < NJ * MF; ++f) {
    const int jj = f / MF, i = f % MF;
    const int c0 = (wave_n * NJ + jj) * 32 + ec;
    const int64_t col0 = col_base + c0;
    if constexpr (SILU) {
      if (quant) {
        float hq[16];
        wave_lds_order();
        static_for<0, NJ * MF>([&](auto c) __attribute__((always_inline)) {
          constexpr int F = decltype(c)::value;
          if (f == F) stage_frag(silu_frag(acc[F % MF][F / MF], acc[F % MF][F / MF + NF / 2]));
        });
        wave_lds_order();
        read_block(hq);
        // h rounded to bf16 first, then the quantiser's own block arithmetic:
        // the codes equal those of the bf16 h quantised on its own.
        uint32_t hb[8];
#pragma unroll
        for (int c = 0; c < 8; ++c)
          hb[c] = (uint32_t)f32_to_bf16_rne(hq[2 * c]) | ((uint32_t)f32_to_bf16_rne(hq[2 * c + 1]) << 16);
        const uint4 lo = make_uint4(hb[0], hb[1], hb[2], hb[3]), hi = make_uint4(hb[4], hb[5], hb[6], hb[7]);
        uint2 codes;
        const uint32_t S = quantize_block16(lo, hi, hg, &codes);
        const int64_t row = m0 + wave_m * MF * 32 + i * 32 + r;
        const int64_t hcol = col_base + (wave_n * NJ + jj) * 32 + 16 * h;
        // n/2 is a multiple of 32: a fragment's columns are all inside h or all past it
        if (row < m && hcol < n / 2) {
          *reinterpret_cast<uint2*>(epi.h_codes + row * (n / 4) + hcol / 2) = codes;
          epi.h_scales[row * (n / 32) + hcol / 16] = (uint8_t)S;
          if (epi.h_out) {
            uint4* dst = reinterpret_cast<uint4*>(epi.h_out + row * (n / 2) + hcol);
            dst[0] = lo;
            dst[1] = hi;
          }
        }
        continue;
      }
    }
    float v[4][4];
    wave_lds_order();
    static_for<0, NJ * MF>([&](auto c) __attribute__((always_inline)) {
      constexpr int F = decltype(c)::value;
      if constexpr (SILU) {
        if (f == F) stage_frag(silu_frag(acc[F % MF][F / MF], acc[F % MF][F / MF + NF / 2]));
      } else {
        if (f == F) stage_frag(acc[F % MF][F / MF]);
      }
    });
    wave_lds_order();
    read_frag(v);
    if constexpr (!SILU) {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const ColumnEpilogue ce = ctab[c0 + b];
#pragma unroll
        for (int a = 0; a < 4; ++a) v[a][b] = apply_epilogue(ce, v[a][b]);
      }
    }
    const int64_t row0 = m0 + wave_m * MF * 32 + i * 32 + er;
#pragma unroll
    for (int a = 0; a < 4; ++a) store_row(row0 + a, col0, v[a]);
  }
}

// The lane's two scale pairs (blocks 2h and 2h+1 of a 64-wide K tile) of each
// fragment as f16 pairs, computed once per K step: sub-steps 0, 1 use pair 0
// and sub-steps 2, 3 pair 1.
template <int MF, int NF>
__device__ __forceinline__ void scale_pairs(uint32_t hsh, const uint32_t (&asc)[MF], const uint32_t (&bsc)[NF],
                                            half2_t (&sa)[MF][2], half2_t (&sb)[NF][2]) {
#pragma unroll
  for (int i = 0; i < MF; ++i) {
    sa[i][0] = scale_pair_f16(__builtin_amdgcn_ubfe(asc[i], hsh, 8));
    sa[i][1] = scale_pair_f16(__builtin_amdgcn_ubfe(asc[i], hsh + 8u, 8));
  }
#pragma unroll
  for (int j = 0; j < NF; ++j) {
    sb[j][0] = scale_pair_f16(__builtin_amdgcn_ubfe(bsc[j], hsh, 8));
    sb[j][1] = scale_pair_f16(__builtin_amdgcn_ubfe(bsc[j], hsh + 8u, 8));
  }
}

template <int MF, int NF>
__device__ __forceinline__ void dequant_step_p(int s, const uint4 (&ac)[MF], const uint4 (&bc)[NF],
                                               const half2_t (&sa)[MF][2], const half2_t (&sb)[NF][2],
                                               half8_t (&av)[MF], half8_t (&bv)[NF]) {
#pragma unroll
  for (int i = 0; i < MF; ++i) {
    const uint32_t cw = s == 0 ? ac[i].x : s == 1 ? ac[i].y : s == 2 ? ac[i].z : ac[i].w;
    av[i] = dequant8(cw, sa[i][s >> 1]);
  }
#pragma unroll
  for (int j = 0; j < NF; ++j) {
    const uint32_t cw = s == 0 ? bc[j].x : s == 1 ? bc[j].y : s == 2 ? bc[j].z : bc[j].w;
    bv[j] = dequant8(cw, sb[j][s >> 1]);
  }
}

template <int MF, int NF>
__device__ __forceinline__ void mma_k64(floatx16 (&acc)[MF][NF], const uint4 (&ac)[MF], const uint32_t (&asc)[MF],
                                        const uint4 (&bc)[NF], const uint32_t (&bsc)[NF]) {
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    half8_t av[MF], bv[NF];
#pragma unroll
    for (int i = 0; i < MF; ++i) {
      const uint32_t cw = s == 0 ? ac[i].x : s == 1 ? ac[i].y : s == 2 ? ac[i].z : ac[i].w;
      av[i] = dequant8(cw, scale_pair_f16(scale_byte(asc[i], s)));
    }
#pragma unroll
    for (int j = 0; j < NF; ++j) {
      const uint32_t cw = s == 0 ? bc[j].x : s == 1 ? bc[j].y : s == 2 ? bc[j].z : bc[j].w;
      bv[j] = dequant8(cw, scale_pair_f16(scale_byte(bsc[j], s)));
    }
#pragma unroll
    for (int i = 0; i < MF; ++i)
#pragma unroll
      for (int j = 0; j < NF; ++j) acc[i][j] = mfma32x32x16(av[i], bv[j], acc[i][j]);
  }
}

// --------------------------------------------- prefill kernel, any K ----
// Register-staged variant for K % 64 == 32 (a half K tile at the end): every
// load is guarded and zero-filled.  Workgroup tile BM x BN over the whole K;
// per 64-wide K step the packed A rows and W tiles go global -> registers ->
// LDS (double buffered) and each wave multiplies its fragments.
// SILU: the workgroup covers BN/2 output columns o0.. and loads the matching
// gate tiles (columns o0..) and up tiles (columns n/2 + o0..); frag j < NF/2
// of a wave is a gate tile and frag j + NF/2 the up tile of the same columns.
template <int MF, int NF, int WM, int WN>
struct RegShape {
  static constexpr int NT = WM * WN * 64;
  static constexpr int BM = WM * MF * 32;
  static constexpr int BN = WN * NF * 32;
  static constexpr int NTILES = BN / 32;
  static constexpr int HSTRIDE = BM * 16 + 64;        // LDS bytes per K half of the A stage
  static constexpr int OFF_AS = 2 * HSTRIDE;
  static constexpr int OFF_BC = OFF_AS + BM * 4;
  static constexpr int OFF_BS = OFF_BC + NTILES * kTileCodeBytes;
  static constexpr int STAGE = OFF_BS + NTILES * 128;
  static constexpr int EPI_BYTES = WM * WN * 32 * 33 * 4;
  static constexpr int LDS = (2 * STAGE > EPI_BYTES) ? 2 * STAGE : EPI_BYTES;
};

template <int MF, int NF, int WM, int WN, bool SILU>
__global__ void __launch_bounds__(WM * WN * 64)
gemm_prefill_regs_kernel(const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales, int64_t m,
                         const uint8_t* __restrict__ w_packed, int64_t n, int64_t k, void* __restrict__ out,
                         EpilogueArgs epi) {
  using P = RegShape<MF, NF, WM, WN>;
  constexpr int NT = P::NT, BM = P::BM, BN = P::BN, NTILES = P::NTILES, HSTRIDE = P::HSTRIDE;
  constexpr int A_CHUNKS = 2 * BM;
  constexpr int B_CHUNKS = NTILES * 64;
  constexpr int A_PER_T = (A_CHUNKS + NT - 1) / NT;
  constexpr int B_PER_T = (B_CHUNKS + NT - 1) / NT;
  constexpr int AS_PER_T = (BM + NT - 1) / NT;
  constexpr int BS_PER_T = (BN + NT - 1) / NT;

  __shared__ __attribute__((aligned(16))) uint8_t lds[P::LDS];
  __shared__ ColumnEpilogue ctab[SILU ? 1 : P::BN];

  const int t = threadIdx.x;
  const int lane = t & 63, r = lane & 31, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6), wave_m = wave / WN, wave_n = wave % WN;
  const int64_t KT = (k + kTileK - 1) / kTileK;
  const int64_t KS = super_count(k);
  const int64_t ntiles_total = (n + kTileN - 1) / kTileN;
  const int64_t m0 = (int64_t)blockIdx.y * BM;
  const int64_t a_row_bytes = k / 2, a_row_scales = k / 16;
  const bool k_aligned64 = (k & 63) == 0;
  const int64_t o0 = SILU ? (int64_t)blockIdx.x * (BN / 2) : 0;
  if constexpr (!SILU) fill_column_table<BN, NT>(ctab, epi, (int64_t)blockIdx.x * BN, n);

  auto ntile_of = [&](int tl) -> int64_t {
    if (SILU) {
      const int half = NTILES / 2;
      return tl < half ? (o0 / 32 + tl) : ((n / 2 + o0) / 32 + (tl - half));
    }
    return (int64_t)blockIdx.x * NTILES + tl;
  };
  auto tile_ok = [&](int tl) -> bool {
    if (SILU) {
      const int half = NTILES / 2;
      return (o0 / 32 + (tl < half ? tl : tl - half)) < (n / 2) / 32;
    }
    return ntile_of(tl) < ntiles_total;
  };

  uint4 ra[A_PER_T], rb[B_PER_T];
  uint32_t ras[AS_PER_T], rbs[BS_PER_T];

  auto gload = [&](int64_t kt) {
#pragma unroll
    for (int i = 0; i < A_PER_T; ++i) {
      const int q = t + i * NT;
      const int row = q >> 1, hh = q & 1;
      const bool ok = q < A_CHUNKS && (m0 + row) < m && (kt * 64 + hh * 32) < k;
      ra[i] = ld16(a_codes + (m0 + row) * a_row_bytes + kt * 32 + hh * 16, ok);
    }
#pragma unroll
    for (int i = 0; i < AS_PER_T; ++i) {
      const int row = t + i * NT;
      uint32_t v = 0;
      if (row < BM && (m0 + row) < m) {
        const uint8_t* p = a_scales + (m0 + row) * a_row_scales + kt * 4;
        if (k_aligned64) {
          v = *reinterpret_cast<const uint32_t*>(p);
        } else {
          v = *reinterpret_cast<const uint16_t*>(p);
          if (kt * 64 + 32 < k) v |= (uint32_t)(*reinterpret_cast<const uint16_t*>(p + 2)) << 16;
        }
      }
      ras[i] = v;
    }
#pragma unroll
    for (int i = 0; i < B_PER_T; ++i) {
      const int q = t + i * NT;
      const int tl = q >> 6, ln = q & 63;
      const bool ok = q < B_CHUNKS && tile_ok(tl);
      rb[i] = ld16(w_packed + tile_code_off(ntile_of(tl), kt, KS) + ln * 16, ok);
    }
#pragma unroll
    for (int i = 0; i < BS_PER_T; ++i) {
      const int q = t + i * NT;
      const int tl = q >> 5, c = q & 31;
      uint32_t v = 0;
      if (q < BN && tile_ok(tl))
        v = *reinterpret_cast<const uint32_t*>(w_packed + tile_scale_off(ntile_of(tl), kt, KS, c));
      rbs[i] = v;
    }
  };
  auto sstore = [&](int stage) {
    uint8_t* base = lds + stage * P::STAGE;
#pragma unroll
    for (int i = 0; i < A_PER_T; ++i) {
      const int q = t + i * NT;
      if (q < A_CHUNKS) *reinterpret_cast<uint4*>(base + (q & 1) * HSTRIDE + (q >> 1) * 16) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < AS_PER_T; ++i) {
      const int row = t + i * NT;
      if (row < BM) reinterpret_cast<uint32_t*>(base + P::OFF_AS)[row] = ras[i];
    }
#pragma unroll
    for (int i = 0; i < B_PER_T; ++i) {
      const int q = t + i * NT;
      if (q < B_CHUNKS) *reinterpret_cast<uint4*>(base + P::OFF_BC + q * 16) = rb[i];
    }
#pragma unroll
    for (int i = 0; i < BS_PER_T; ++i) {
      const int q = t + i * NT;
      if (q < BN) reinterpret_cast<uint32_t*>(base + P::OFF_BS)[q] = rbs[i];
    }
  };

  floatx16 acc[MF][NF];
#pragma unroll
  for (int i = 0; i < MF; ++i)
#pragma unroll
    for (int j = 0; j < NF; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  auto lds_tile = [&](int j) -> int {
    if (SILU) return j < NF / 2 ? wave_n * (NF / 2) + j : NTILES / 2 + wave_n * (NF / 2) + (j - NF / 2);
    return wave_n * NF + j;
  };

  gload(0);
  sstore(0);
  __syncthreads();
  for (int64_t kt = 0; kt < KT; ++kt) {
    const int stage = (int)(kt & 1);
    const uint8_t* base = lds + stage * P::STAGE;
    if (kt + 1 < KT) gload(kt + 1);
    uint4 ac[MF], bc[NF];
    uint32_t asc[MF], bsc[NF];
#pragma unroll
    for (int i = 0; i < MF; ++i) {
      const int row = wave_m * MF * 32 + i * 32 + r;
      ac[i] = *reinterpret_cast<const uint4*>(base + h * HSTRIDE + row * 16);
      asc[i] = reinterpret_cast<const uint32_t*>(base + P::OFF_AS)[row] >> (16 * h);
    }
#pragma unroll
    for (int j = 0; j < NF; ++j) {
      const int tl = lds_tile(j);
      bc[j] = *reinterpret_cast<const uint4*>(base + P::OFF_BC + tl * kTileCodeBytes + lane * 16);
      bsc[j] = reinterpret_cast<const uint32_t*>(base + P::OFF_BS)[tl * 32 + r] >> (16 * h);
    }
    mma_k64<MF, NF>(acc, ac, asc, bc, bsc);
    if (kt + 1 < KT) sstore(stage ^ 1);
    __syncthreads();
  }

  tile_epilogue<MF, NF, WM, WN, SILU>(acc, lds, ctab, lane, wave, wave_m, wave_n, m0,
                                      SILU ? o0 : (int64_t)blockIdx.x * BN, m, n, out, epi);
}

// -------------------------------------- prefill kernel, K % 64 == 0 ----
// Global -> LDS DMA pipeline with NSTAGE stages.  Every wave issues a fixed
// set of global_load_lds (16-byte or 4-byte per lane) per stage straight into
// a fragment-ordered LDS layout (1 KB per 32-row x 64-K fragment, lane l's 16
// bytes at l*16 -- exactly where the MFMA operand read wants them), so no
// registers or VALU are spent on staging.  Rows past m and weight tiles past
// n are not masked: their addresses are clamped to the last valid row/tile,
// which keeps every wave's load count fixed (the vmcnt accounting below
// relies on it) and only feeds output rows/columns that are never stored.
// In step kt, right after the barrier that publishes stage kt+1, the loads
// for stage kt+NSTAGE go into buffer kt % NSTAGE, whose fragments every wave
// has read before that barrier.
// Tuning of the main loop's schedule: VALU ops issued after each MFMA, and
// MFMAs of the last sub-step issued before any VALU op that needs the next
// stage.
#ifndef NVFP4_XPIPE
#define NVFP4_XPIPE 5
#endif
#ifndef NVFP4_LATE
#define NVFP4_LATE 3
#endif

// Which output tile a workgroup of the prefill kernel computes (1-D grids).
// Tiles are numbered in groups of kGroupCols tile columns, row-major within a
// group (the grid is gx tiles wide and gy tall).  A workgroup takes tile
// `first + blockIdx.x / (ry * rx)` in that order, and piece
// blockIdx.x % (ry * rx) of it: the tile cut into ry row bands and rx column
// bands (ry = rx = 1: the whole tile; pieces serve the last, partly filled
// round of a launch).
// XCD-aware order (xcd_chunk > 0, whole tiles only): the hardware deals
// workgroups to the kXcds XCDs in turn, so XCD x runs blocks x, x + kXcds,
// ...; block b is given tile (b % kXcds) * xcd_chunk + b / kXcds, i.e. each
// XCD works through a contiguous run of the order.  The 32 tiles an XCD holds
// at once are then about 4 row bands x 8 columns: each weight slab is read by
// 4 of them and each A band by 8 through the same L2, where the row-major
// order spread a weight slab's tiles over several XCDs.
constexpr int kXcds = 8;
constexpr int kGroupCols = 8;
struct TileMap {
  int gx, gy;
  int first;
  int ry, rx;
  int xcd_chunk;
};

__device__ __forceinline__ void map_tile(const TileMap& tm, int& bx, int& by) {
  const int per = tm.ry * tm.rx;
  int b = (int)blockIdx.x / per;
  const int q = (int)blockIdx.x % per;
  if (tm.xcd_chunk > 0) b = (b % kXcds) * tm.xcd_chunk + b / kXcds;
  const int t = tm.first + b;
  const int per_group = kGroupCols * tm.gy;
  const int g = t / per_group, w = t - g * per_group;
  const int width = min(kGroupCols, tm.gx - g * kGroupCols);
  bx = (g * kGroupCols + w % width) * tm.rx + q % tm.rx;
  by = (w / width) * tm.ry + q / tm.rx;
}

template <int MF, int NF, int WM, int WN, int NSTAGE>
struct DmaShape {
  static constexpr int NWAVES = WM * WN;
  static constexpr int BM = WM * MF * 32;
  static constexpr int BN = WN * NF * 32;
  static constexpr int AFRAGS = BM / 32;
  static constexpr int NTILES = BN / 32;
  static constexpr int OFF_AS = AFRAGS * 1024;
  static constexpr int OFF_BC = OFF_AS + BM * 4;
  static constexpr int OFF_BS = OFF_BC + NTILES * 1024;
  static constexpr int STAGE = OFF_BS + NTILES * 128;
  // Load classes: A code fragments, A scale groups (64 rows), W tiles, W scale
  // pairs (two tiles).  Each wave issues the same number of DMA instructions
  // per class; where a class does not split evenly, the surplus issues repeat
  // an item (same source, same destination, same bytes), which keeps every
  // wave's vmcnt accounting identical.
  static constexpr int N_AC = AFRAGS, N_AS = BM / 64, N_BC = NTILES, N_BS = NTILES / 2;
  static constexpr int PC_AC = (N_AC + NWAVES - 1) / NWAVES, PC_AS = (N_AS + NWAVES - 1) / NWAVES;
  static constexpr int PC_BC = (N_BC + NWAVES - 1) / NWAVES, PC_BS = (N_BS + NWAVES - 1) / NWAVES;
  static constexpr int LPW = PC_AC + PC_AS + PC_BC + PC_BS;   // DMA instructions per wave per stage
  static constexpr int EPI_BYTES = NWAVES * 32 * 33 * 4;
  static_assert(BM % 64 == 0 && NTILES % 2 == 0, "A scales move in 64-row groups, W scales in tile pairs");
};

// Global -> LDS DMA of 16 (or 4) bytes per lane: lane l's bytes land at
// dst + l*16 (l*4), read from sbase + voff (a wave-uniform base in SGPRs and a
// 32-bit per-lane offset, so the per-stage address steps are scalar adds).
// Written as a single instruction in inline asm so the compiler does not add
// its own (conservative, pipeline-draining) vmcnt waits before later LDS
// reads; completion is tracked explicitly with wait_vmcnt and published to
// the other waves with the barrier.  The instruction has no register results
// (its data goes to LDS); the address registers are read at issue.  M0 holds
// the wave-uniform LDS destination; the leading s_nop covers the M0-write ->
// LDS-DMA hazard.
__device__ __forceinline__ uint32_t lds_offset(const uint8_t* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)p;
}
__device__ __forceinline__ void dma16s(const uint8_t* sbase, uint32_t voff, uint8_t* dst) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "{m0}"(lds_offset(dst)) : "memory");
}
__device__ __forceinline__ void dma4s(const uint8_t* sbase, uint32_t voff, uint8_t* dst) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase), "{m0}"(lds_offset(dst)) : "memory");
}
// Compiler-only fence: no memory access is moved across it.
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }
// s_waitcnt vmcnt(N) (gfx9 encoding; expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <int MF, int NF, int WM, int WN, int NSTAGE, bool SILU>
__global__ void __launch_bounds__(WM * WN * 64)
gemm_prefill_dma_kernel(const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales, int64_t m,
                        const uint8_t* __restrict__ w_packed, int64_t n, int64_t k, void* __restrict__ out,
                        EpilogueArgs epi, TileMap tmap) {
  using P = DmaShape<MF, NF, WM, WN, NSTAGE>;
  constexpr int NWAVES = P::NWAVES, BM = P::BM, BN = P::BN, NTILES = P::NTILES;
  static_assert(NSTAGE == 3 || NSTAGE == 4, "3 or 4 stages");
  // One LDS object per stage: the compiler can then tell that the DMA into the
  // stage being filled does not alias the reads of the stage being consumed
  // and does not wait for it before those reads.
  // (stage 0 starts 1 KB into its object: an LDS address of exactly 0 lets the
  // compiler fold the offsets into bit operations that lose the alias
  // information the DMA waits rely on)
  __shared__ __attribute__((aligned(1024))) uint8_t lds_s0[P::STAGE + 1024];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_s1[P::STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_s2[P::STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_s3[NSTAGE > 3 ? P::STAGE : 16];
  __shared__ __attribute__((aligned(16))) uint8_t lds_epi[P::EPI_BYTES];
  __shared__ ColumnEpilogue ctab[SILU ? 1 : BN];
  auto buf = [&](auto b) __attribute__((always_inline)) -> uint8_t* {
    constexpr int B = decltype(b)::value;
    if constexpr (B == 0) return lds_s0 + 1024;
    else if constexpr (B == 1) return lds_s1;
    else if constexpr (B == 2) return lds_s2;
    else return lds_s3;
  };

  const int lane = threadIdx.x & 63, r = lane & 31, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wave_m = wave / WN, wave_n = wave % WN;
  const int64_t KT = k / kTileK;
  const int64_t KS = super_count(k);
  const int64_t ntiles_total = (n + kTileN - 1) / kTileN;
  int bx, by;
  map_tile(tmap, bx, by);
  const int64_t m0 = (int64_t)by * BM;
  const uint32_t a_row_bytes = (uint32_t)(k / 2), a_row_scales = (uint32_t)(k / 16);
  const int64_t o0 = SILU ? (int64_t)bx * (BN / 2) : 0;
  if constexpr (!SILU) fill_column_table<BN, NWAVES * 64>(ctab, epi, (int64_t)bx * BN, n);

  auto ntile_of = [&](int tl) -> int64_t {
    int64_t nt;
    if (SILU) {
      const int half = NTILES / 2;
      nt = tl < half ? (o0 / 32 + tl) : ((n / 2 + o0) / 32 + (tl - half));
    } else {
      nt = (int64_t)bx * NTILES + tl;
    }
    return nt < ntiles_total ? nt : ntiles_total - 1;   // clamped: see the kernel comment
  };
  auto row_of = [&](int64_t row) -> int64_t { return row < m ? row : m - 1; };

  // Source addresses (K step 0: a wave-uniform base plus a per-lane offset)
  // and LDS offsets of this wave's loads.
  // Load classes in order: A code fragments, A scale groups (64 rows), W tiles,
  // W scale pairs; class sizes are multiples of the wave count, so load i of
  // every wave belongs to the same class (known at compile time).
  constexpr int I_AS = P::PC_AC, I_BC = I_AS + P::PC_AS, I_BS = I_BC + P::PC_BC;
  // Wave-uniform bases (SGPRs, advanced per stage) and per-lane offsets.
  const uint8_t* src[P::LPW];
  uint32_t voff[P::LPW];
  int dst[P::LPW];
#pragma unroll
  for (int i = 0; i < P::LPW; ++i) {
    if (i < I_AS) {
      const int f = (wave + i * NWAVES) % P::N_AC;
      src[i] = a_codes;
      voff[i] = (uint32_t)(row_of(m0 + 32 * f + r) * a_row_bytes) + h * 16;
      dst[i] = f * 1024;
    } else if (i < I_BC) {
      const int g = (wave + (i - I_AS) * NWAVES) % P::N_AS;
      src[i] = a_scales;
      voff[i] = (uint32_t)(row_of(m0 + 64 * g + lane) * a_row_scales);
      dst[i] = P::OFF_AS + g * 256;
    } else if (i < I_BS) {
      const int tl = (wave + (i - I_BC) * NWAVES) % P::N_BC;
      src[i] = w_packed + tile_code_off(ntile_of(tl), 0, KS);
      voff[i] = lane * 16;
      dst[i] = P::OFF_BC + tl * 1024;
    } else {
      const int p = (wave + (i - I_BS) * NWAVES) % P::N_BS;
      // the pair's two tiles (h = 0, 1) differ per lane half: the tile's base
      // offset goes in the lane part
      const int64_t o0 = tile_scale_off(ntile_of(2 * p), 0, KS, 0);
      const int64_t o1 = tile_scale_off(ntile_of(2 * p + 1), 0, KS, 0);
      src[i] = w_packed + o0;
      voff[i] = (uint32_t)(h ? o1 - o0 : 0) + r * 8;
      dst[i] = P::OFF_BS + p * 256;
    }
  }
  // Stages are issued strictly in order, so each load keeps a running
  // (wave-uniform) base that advances by its per-stage stride after every
  // issue; the per-lane offsets stay fixed.  With
  // four stages, the buffer of a stage is its tile's position T in the weight
  // super-tile, which fixes the weight strides at compile time.
  static_assert(NSTAGE == kSuperTiles, "one stage buffer per tile of a weight super-tile");
  auto issue = [&](uint8_t* base, auto tpos) __attribute__((always_inline)) {
    constexpr int T = decltype(tpos)::value;
    constexpr int W_CODE_STEP = T < kSuperTiles - 1 ? kTileCodeBytes : kSuperBytes - (kSuperTiles - 1) * kTileCodeBytes;
    constexpr int W_SCALE_STEP = T == 0 ? 4 : T == 1 ? kTileN * 8 - 4 : T == 2 ? 4 : kSuperBytes - kTileN * 8 - 4;
#pragma unroll
    for (int i = 0; i < P::LPW; ++i) {
      if (i < I_AS) { dma16s(src[i], voff[i], base + dst[i]); src[i] += 32; }
      else if (i < I_BC) { dma4s(src[i], voff[i], base + dst[i]); src[i] += 4; }
      else if (i < I_BS) { dma16s(src[i], voff[i], base + dst[i]); src[i] += W_CODE_STEP; }
      else { dma4s(src[i], voff[i], base + dst[i]); src[i] += W_SCALE_STEP; }
    }
  };

  floatx16 acc[MF][NF];
#pragma unroll
  for (int i = 0; i < MF; ++i)
#pragma unroll
    for (int j = 0; j < NF; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  auto lds_tile = [&](int j) -> int {
    if (SILU) return j < NF / 2 ? wave_n * (NF / 2) + j : NTILES / 2 + wave_n * (NF / 2) + (j - NF / 2);
    return wave_n * NF + j;
  };

  // Software pipeline across K steps.  Within step kt the four 16-wide
  // sub-steps multiply operands that were dequantised during the previous
  // sub-step, so the VALU work issues in the MFMA shadow.  Between sub-steps
  // 2 and 3 (the step's fragments are all dequantised by then) the wave waits
  // for stage kt+1, joins the barrier, reads its fragments of stage kt+1 and
  // refills buffer kt % NSTAGE (read before this barrier by every wave) with
  // stage kt + NSTAGE; sub-step 3 dequantises the first sub-step of kt+1.
  // Raw fragments of one stage: code bytes and the whole scale dword of the
  // lane's row (this lane's two blocks are its half h, picked at dequant time,
  // so no VALU op depends on the LDS reads before the next sub-step starts).
  struct Raw { uint4 ac[MF], bc[NF]; uint32_t asc[MF], bsc[NF]; };
  auto read_frags = [&](const uint8_t* base, Raw& R) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < MF; ++i) {
      const int f = wave_m * MF + i;
      R.ac[i] = *reinterpret_cast<const uint4*>(base + f * 1024 + lane * 16);
      R.asc[i] = reinterpret_cast<const uint32_t*>(base + P::OFF_AS)[f * 32 + r];
    }
#pragma unroll
    for (int j = 0; j < NF; ++j) {
      const int tl = lds_tile(j);
      R.bc[j] = *reinterpret_cast<const uint4*>(base + P::OFF_BC + tl * 1024 + lane * 16);
      R.bsc[j] = reinterpret_cast<const uint32_t*>(base + P::OFF_BS)[tl * 32 + r];
    }
  };
  const uint32_t hsh = 16u * h;   // bit offset of this lane's scale pair
  // Serpentine order: consecutive MFMAs always share one operand, also across
  // rows.  The chip runs this kernel power-limited, and fewer changing operand
  // bits let it clock a little higher.  Each accumulator still sees its
  // products in K order, so the results do not change.
  auto mma = [&](const half8_t (&av)[MF], const half8_t (&bv)[NF]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < MF; ++i)
#pragma unroll
      for (int jj = 0; jj < NF; ++jj) {
        const int j = (i & 1) ? NF - 1 - jj : jj;
        acc[i][j] = mfma32x32x16(av[i], bv[j], acc[i][j]);
      }
  };
  // One MFMA, then a few VALU ops, for every MFMA of a sub-step.
  auto interleave = [&]() __attribute__((always_inline)) {
    static_for<0, MF * NF>([&](auto) __attribute__((always_inline)) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, NVFP4_XPIPE, 0);
    });
  };
  auto sync_stage = [&](auto waitn) __attribute__((always_inline)) {
    wait_vmcnt<decltype(waitn)::value>();
    compiler_fence();
    __builtin_amdgcn_s_barrier();
    compiler_fence();
  };

  Raw R;
  half8_t oa0[MF], ob0[NF], oa1[MF], ob1[NF];
  half2_t spa[MF][2], spb[NF][2];
  // Prologue: all NSTAGE stages in flight (the launcher guarantees KT >= NSTAGE),
  // then stage 0 is read and its first sub-step dequantised.
  static_for<0, NSTAGE>([&](auto s) __attribute__((always_inline)) { issue(buf(s), s); });
  sync_stage(std::integral_constant<int, P::LPW * (NSTAGE - 1)>{});
  read_frags(buf(std::integral_constant<int, 0>{}), R);
  scale_pairs<MF, NF>(hsh, R.asc, R.bsc, spa, spb);
  dequant_step_p<MF, NF>(0, R.ac, R.bc, spa, spb, oa0, ob0);

  // Sub-step 3 follows the LDS reads of the next stage: its first MFMAs go out
  // before any VALU op that needs the new fragments.
  constexpr int LATE = NVFP4_LATE < MF * NF ? NVFP4_LATE : MF * NF;
  auto interleave_late = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_group_barrier(0x008, LATE, 0);
    static_for<0, MF * NF - LATE>([&](auto) __attribute__((always_inline)) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, NVFP4_XPIPE + 1, 0);
    });
  };

  // Each sub-step is its own scheduling region (sched_barrier), so the
  // compiler cannot drift the LDS reads or a dequantisation across sub-steps.
  auto fence_sched = [&]() __attribute__((always_inline)) { __builtin_amdgcn_sched_barrier(0); };
  auto kstep = [&](auto b, bool has_next, bool do_issue, auto waitn) __attribute__((always_inline)) {
    constexpr int B = decltype(b)::value;
    fence_sched();
    dequant_step_p<MF, NF>(1, R.ac, R.bc, spa, spb, oa1, ob1);
    mma(oa0, ob0);
    interleave();
    fence_sched();
    dequant_step_p<MF, NF>(2, R.ac, R.bc, spa, spb, oa0, ob0);
    mma(oa1, ob1);
    interleave();
    fence_sched();
    dequant_step_p<MF, NF>(3, R.ac, R.bc, spa, spb, oa1, ob1);
    mma(oa0, ob0);
    interleave();
    fence_sched();
    // The current fragments are dead here, so the next stage's can be read.
    if (has_next) {
      sync_stage(waitn);
      read_frags(buf(std::integral_constant<int, (B + 1) % NSTAGE>{}), R);
      if (do_issue) issue(buf(b), b);
      fence_sched();
      scale_pairs<MF, NF>(hsh, R.asc, R.bsc, spa, spb);
      dequant_step_p<MF, NF>(0, R.ac, R.bc, spa, spb, oa0, ob0);
    }
    mma(oa1, ob1);
    interleave_late();
  };
  // Steady state, NSTAGE steps per iteration (compile-time buffers); every step
  // issues a stage, so each waits with NSTAGE-2 stages still in flight.
  int64_t kt0 = 0;
  for (; kt0 + 2 * NSTAGE - 1 < KT; kt0 += NSTAGE) {
    static_for<0, NSTAGE>([&](auto b) __attribute__((always_inline)) {
      kstep(b, true, true, std::integral_constant<int, P::LPW * (NSTAGE - 2)>{});
    });
  }
  // Tail: the last steps wait for every load in flight.
  for (; kt0 < KT; kt0 += NSTAGE) {
    static_for<0, NSTAGE>([&](auto b) __attribute__((always_inline)) {
      const int64_t kt = kt0 + decltype(b)::value;
      if (kt < KT) kstep(b, kt + 1 < KT, kt + NSTAGE < KT, std::integral_constant<int, 0>{});
    });
  }

  tile_epilogue<MF, NF, WM, WN, SILU>(acc, lds_epi, ctab, lane, wave, wave_m, wave_n, m0,
                                      SILU ? o0 : (int64_t)bx * BN, m, n, out, epi);
}

// ------------------------------------------------------- decode kernel ----
// m <= 64: weight streaming.  One workgroup per 32-column weight slab (two
// slabs -- gate and up -- for SILU); its waves split K evenly, each
// streaming its part of the slab straight from HBM into registers with one
// 16-byte load per lane per 64-wide K tile (the packed layout is already in
// MFMA lane order).  Loads run up to eight tiles ahead of the MFMAs.
// ALDS (small m*k): the workgroup first dequantises A once into LDS as f16 in
// MFMA operand order (rows < m only; lanes of absent rows read a zero slot),
// so the loop spends VALU only on the weights.  Otherwise A is dequantised
// per tile in registers.  GA (k % 256 == 0, 16-byte aligned A scales): A is
// fetched four K tiles at a time, eight lanes per 128-byte row segment, and
// each wave re-orders its group through a private LDS area into MFMA lane
// order -- a per-tile fetch in lane order would touch one cache line per row
// per instruction, and at 32 or 64 rows those line lookups, not the bytes,
// limit the kernel.  The waves' partial accumulators are summed in LDS in a
// fixed order.
constexpr int kDecodeALdsBytes = 48 * 1024;
#ifndef NVFP4_DECODE_GROUP_A
#define NVFP4_DECODE_GROUP_A 6
#endif
// Tiles per load group with A staged in LDS (two groups are in flight; six is
// the most that fits three waves per SIMD without spilling).
constexpr int kDecodeGroupA = NVFP4_DECODE_GROUP_A;

// Sized so that three 4-wave workgroups fit on a CU (<= 168 VGPRs per wave,
// A staging in dynamic LDS of exactly (m+1)*k*2 bytes): the 544 workgroups of
// a 17408-column projection are then all resident at once instead of the
// last few running as a second round.
constexpr int kDecodeGroupRow = 144;          // LDS bytes per A row of a group (128 + 16: conflict-free reads)
constexpr int kDecodeGroupFrag = 32 * kDecodeGroupRow;

template <int MFD, bool SILU, bool ALDS, int DW, int WPE, int U, bool GA>
__global__ void __launch_bounds__(DW * 64) __attribute__((amdgpu_waves_per_eu(WPE)))
gemm_decode_kernel(const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales, int64_t m,
                   const uint8_t* __restrict__ w_packed, int64_t n, int64_t k, void* __restrict__ out,
                   EpilogueArgs epi) {
  constexpr int NS = SILU ? 2 : 1;                 // weight slabs per workgroup
  constexpr int NACC = MFD * NS;
  static_assert(!GA || (!ALDS && U == 4), "grouped A fetch: four tiles per load group");
  __shared__ float s_red[DW - 1][NACC][16][64];
  __shared__ __attribute__((aligned(16))) uint8_t s_ag[GA ? DW * MFD * kDecodeGroupFrag : 16];
  extern __shared__ __attribute__((aligned(16))) uint8_t s_a[];    // ALDS: (m+1)*k*2 bytes

  const int t = threadIdx.x;
  const int lane = t & 63, r = lane & 31, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int64_t KT = (k + kTileK - 1) / kTileK;
  const int64_t KS = super_count(k);
  const int64_t a_row_bytes = k / 2, a_row_scales = k / 16;
  int64_t slab[NS];
  slab[0] = blockIdx.x;
  if (SILU) slab[NS - 1] = blockIdx.x + (n / 2) / kTileN;
  // GA: wave ranges in whole groups of four tiles (KT % 4 == 0 there)
  const int64_t kt0 = GA ? (KT / 4) * wave / DW * 4 : KT * wave / DW;
  const int64_t kt1 = GA ? (KT / 4) * (wave + 1) / DW * 4 : KT * (wave + 1) / DW;

  // Independent accumulators per K sub-step break the MFMA dependency chain
  // (a single 32x32 output tile would otherwise serialise every MFMA).
  constexpr int NSUB = 2;
  floatx16 part[MFD][NS][NSUB];
#pragma unroll
  for (int i = 0; i < MFD; ++i)
#pragma unroll
    for (int j = 0; j < NS; ++j)
#pragma unroll
      for (int q = 0; q < NSUB; ++q)
#pragma unroll
        for (int e = 0; e < 16; ++e) part[i][j][q][e] = 0.0f;

  // Per-lane constant offsets; per-tile bases are wave-uniform (scalar).
  const uint32_t w_lane = lane * 16, ws_lane = r * 8 + 2 * h;
  // A in LDS (ALDS): 16-byte chunk (kt, s, hh, row) at ((kt*4 + s)*2 + hh)*(m+1) + row,
  // row m of every group is zero; lanes of rows >= m read it.
  const int64_t a_rows = m + 1;
  const uint32_t a_lane = (uint32_t)((h * a_rows + (r < m ? r : m)) * 16);

  constexpr bool ATILE = !ALDS && !GA;             // A fetched per tile in lane order
  struct Tile { uint4 a[ATILE ? MFD : 1]; uint32_t as[ATILE ? MFD : 1]; uint4 b[NS]; uint32_t bs[NS]; };
  // Loads are unconditional (no branches, so the compiler can count them and
  // wait only for the group about to be multiplied); tiles past the wave's
  // range are clamped to its last tile and never multiplied.
  auto load = [&](int64_t kt, Tile& T) __attribute__((always_inline)) {
    kt = kt < kt1 ? kt : kt1 - 1;
    if constexpr (ATILE) {
#pragma unroll
      for (int i = 0; i < MFD; ++i) {
        const int64_t row = i * 32 + r;
        const bool ok = row < m && (kt * 64 + h * 32) < k;
        T.a[i] = ld16(a_codes + row * a_row_bytes + kt * 32 + h * 16, ok);
        T.as[i] = ok ? *reinterpret_cast<const uint16_t*>(a_scales + row * a_row_scales + kt * 4 + 2 * h) : 0u;
      }
    }
#pragma unroll
    for (int j = 0; j < NS; ++j) {                                 // tile bases are wave-uniform
      T.b[j] = *reinterpret_cast<const uint4*>(w_packed + tile_code_off(slab[j], kt, KS) + w_lane);
      T.bs[j] = *reinterpret_cast<const uint16_t*>(w_packed + tile_scale_off(slab[j], kt, KS, 0) + ws_lane);
    }
  };
  // A of one tile for the non-ALDS paths: codes (16 bytes: K half h of row
  // i*32 + r) and the scale pair of those two blocks.
  struct ATileRegs { uint4 a[MFD]; uint32_t as[MFD]; };
  auto compute = [&](int64_t kt, const Tile& T, const ATileRegs& A) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      half8_t av[MFD], bv[NS];
      if constexpr (ALDS) {
        const uint32_t grp = (uint32_t)((kt * 4 + s) * 2 * a_rows * 16);   // wave-uniform
        av[0] = *reinterpret_cast<const half8_t*>(s_a + grp + a_lane);
      } else {
#pragma unroll
        for (int i = 0; i < MFD; ++i) {
          const uint32_t cw = s == 0 ? A.a[i].x : s == 1 ? A.a[i].y : s == 2 ? A.a[i].z : A.a[i].w;
          av[i] = dequant8(cw, scale_pair_f16(scale_byte(A.as[i], s)));
        }
      }
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        const uint32_t cw = s == 0 ? T.b[j].x : s == 1 ? T.b[j].y : s == 2 ? T.b[j].z : T.b[j].w;
        bv[j] = dequant8(cw, scale_pair_f16(scale_byte(T.bs[j], s)));
      }
#pragma unroll
      for (int i = 0; i < MFD; ++i)
#pragma unroll
        for (int j = 0; j < NS; ++j) part[i][j][s % NSUB] = mfma32x32x16(av[i], bv[j], part[i][j][s % NSUB]);
    }
  };
  // GA: one group's A -- codes of rows i*32 + 8j + lane/8, 16-byte segment
  // lane%8 of the group's 128 bytes per row, and each lane's row i*32 + r's
  // scales for the group's four tiles (16 bytes).
  struct AGroup { uint4 c[GA ? MFD : 1][GA ? 4 : 1]; uint4 s[GA ? MFD : 1]; };
  uint8_t* const ag_base = s_ag + (GA ? wave * MFD * kDecodeGroupFrag : 0);
  auto load_agroup = [&](int64_t g0, AGroup& G) __attribute__((always_inline)) {
    if constexpr (GA) {
      g0 = g0 < kt1 - 4 ? g0 : kt1 - 4;              // groups past the wave's range: never multiplied
#pragma unroll
      for (int i = 0; i < MFD; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int64_t row = i * 32 + 8 * j + (lane >> 3);
          G.c[i][j] = ld16(a_codes + row * a_row_bytes + g0 * 32 + (lane & 7) * 16, row < m);
        }
        const int64_t row = i * 32 + r;
        G.s[i] = ld16(a_scales + row * a_row_scales + g0 * 4, row < m);
      }
    }
  };
  auto load_group = [&](int64_t g0, Tile (&T)[U], AGroup& G) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < U; ++u) load(g0 + u, T[u]);
    load_agroup(g0, G);
  };
  auto compute_group = [&](int64_t g0, const Tile (&T)[U], const AGroup& G) __attribute__((always_inline)) {
    if constexpr (GA) {
      // this wave's group through its LDS area into lane order (the previous
      // group's reads were issued before these writes)
#pragma unroll
      for (int i = 0; i < MFD; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *reinterpret_cast<uint4*>(ag_base + i * kDecodeGroupFrag + (8 * j + (lane >> 3)) * kDecodeGroupRow +
                                    (lane & 7) * 16) = G.c[i][j];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (g0 + u < kt1) {
        ATileRegs A;
        if constexpr (GA) {
#pragma unroll
          for (int i = 0; i < MFD; ++i) {
            A.a[i] = *reinterpret_cast<const uint4*>(ag_base + i * kDecodeGroupFrag + r * kDecodeGroupRow +
                                                     (2 * u + h) * 16);
            const uint32_t w = u == 0 ? G.s[i].x : u == 1 ? G.s[i].y : u == 2 ? G.s[i].z : G.s[i].w;
            A.as[i] = (w >> (16 * h)) & 0xFFFFu;
          }
        } else if constexpr (ATILE) {
#pragma unroll
          for (int i = 0; i < MFD; ++i) {
            A.a[i] = T[u].a[i];
            A.as[i] = T[u].as[i];
          }
        }
        compute(g0 + u, T[u], A);
      }
    }
  };

  // The first weight group is requested before A is staged, so its latency
  // overlaps the staging.
  Tile g_a[U], g_b[U];
  AGroup ag_a, ag_b;
  if (kt0 < kt1) load_group(kt0, g_a, ag_a);
  // Stage A into LDS once per workgroup (ALDS): dequantised f16 chunks in MFMA
  // operand order plus one zero row per (kt, s, hh) group.
  if constexpr (ALDS) {
    const int64_t items = a_rows * KT * 2;         // (row, kt, hh): 32 values each
    for (int64_t it = t; it < items; it += DW * 64) {
      const int64_t row = it / (KT * 2), rem = it % (KT * 2), kt = rem >> 1, hh = rem & 1;
      uint4 c = make_uint4(0u, 0u, 0u, 0u);
      uint32_t sp = 0;
      if (row < m && kt * 64 + hh * 32 < k) {
        c = *reinterpret_cast<const uint4*>(a_codes + row * a_row_bytes + kt * 32 + hh * 16);
        sp = *reinterpret_cast<const uint16_t*>(a_scales + row * a_row_scales + kt * 4 + 2 * hh);
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint32_t cw = s == 0 ? c.x : s == 1 ? c.y : s == 2 ? c.z : c.w;
        *reinterpret_cast<half8_t*>(s_a + (((kt * 4 + s) * 2 + hh) * a_rows + row) * 16) =
            dequant8(cw, scale_pair_f16(scale_byte(sp, s)));
      }
    }
    __syncthreads();
  }

  if (kt0 < kt1) {
    for (int64_t g = kt0; g < kt1; g += 2 * U) {
      load_group(g + U, g_b, ag_b);
      compute_group(g, g_a, ag_a);
      load_group(g + 2 * U, g_a, ag_a);
      compute_group(g + U, g_b, ag_b);
    }
  }

  floatx16 acc[MFD][NS];
#pragma unroll
  for (int i = 0; i < MFD; ++i)
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      acc[i][j] = part[i][j][0];
#pragma unroll
      for (int q = 1; q < NSUB; ++q) acc[i][j] += part[i][j][q];
    }

  if (wave > 0) {
#pragma unroll
    for (int i = 0; i < MFD; ++i)
#pragma unroll
      for (int j = 0; j < NS; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) s_red[wave - 1][i * NS + j][e][lane] = acc[i][j][e];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 0; w < DW - 1; ++w)
#pragma unroll
    for (int i = 0; i < MFD; ++i)
#pragma unroll
      for (int j = 0; j < NS; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] += s_red[w][i * NS + j][e][lane];

  const float ga = *epi.a_global;
  const bool bf16 = epi.out_bf16 != 0;
  if (SILU) {
    const float alpha = 1.0f / (ga * epi.seg_w_global[0]);
    const int64_t col = slab[0] * 32 + r;
    if (col >= n / 2) return;
#pragma unroll
    for (int i = 0; i < MFD; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t row = i * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
        if (row < m) store_out(out, bf16, row * epi.ld_out + col,
                               silu_mul(acc[i][0][e] * alpha, acc[i][NS - 1][e] * alpha));
      }
  } else {
    const int64_t col = slab[0] * 32 + r;
    if (col >= n) return;
    const ColumnEpilogue ce = column_epilogue(epi, col, ga);
#pragma unroll
    for (int i = 0; i < MFD; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t row = i * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
        if (row < m) store_out(out, bf16, row * epi.ld_out + col, apply_epilogue(ce, acc[i][0][e]));
      }
  }
}

// ------------------------------------------------ decode kernel, FP4 MFMA ----
// m <= 4: weight streaming on gfx950's block-scaled FP4 MFMA, applied to the
// raw E2M1 codes (no dequantisation).  The packed weight tile is already the
// B operand of v_mfma_scale_f32_32x32x64_f8f6f4 (lane r + 32h: column r, K
// 32h..32h+31).  The A operand puts each 16-element block of each A row in a
// row of its own -- MFMA row 4*mm + q holds row mm's block q of the tile and
// zeros elsewhere -- so with unit E8M0 scales the 32x32 result holds the
// per-block partial sums sum_{k in block q} a[mm][k] * w[n][k], exactly (the
// products are multiples of 1/4 and a block sum stays far below 2^24).  Each
// lane then applies the NVFP4 block scales in FP32:
//   y[mm][n] += sum_q s_a[mm][q] * s_w[n][q] * C[4*mm + q][n].
// Lane (r, h) holds rows mm = h, 2+h, ... of column r, so no cross-lane
// reduction is needed; the K split across the workgroup's waves is summed in
// LDS in a fixed order.  A is staged once per workgroup into LDS: one 16-byte
// operand record per (tile, block, row) plus one zero record per tile (for
// lanes whose MFMA row is empty), and the A block scales as FP32.
typedef int v8i_t __attribute__((ext_vector_type(8)));

template <int MR>
struct Fp4DecodeLds {
  static constexpr int RECS = 4 * MR + 1;           // records per K tile (last: zeros)
  __host__ __device__ static int64_t rec_bytes(int64_t kt_count) { return kt_count * RECS * 16; }
  __host__ __device__ static int64_t scale_bytes(int64_t kt_count) { return (int64_t)MR * kt_count * 4 * 4; }
};

template <int MR, bool SILU, int DW, int SU>
__global__ void __launch_bounds__(DW * 64) __attribute__((amdgpu_waves_per_eu(3)))
gemm_decode_fp4_kernel(const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales, int64_t m,
                       const uint8_t* __restrict__ w_packed, int64_t n, int64_t k, void* __restrict__ out,
                       EpilogueArgs epi) {
  constexpr int NS = SILU ? 2 : 1;               // weight slabs per workgroup (gate, up)
  constexpr int MH = MR / 2;                     // A rows per lane: h, 2+h, ...
  using L = Fp4DecodeLds<MR>;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int t = threadIdx.x;
  const int lane = t & 63, r = lane & 31, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int64_t KS = super_count(k), KTP = KS * kSuperTiles;   // tiles incl. zero padding
  const int64_t a_row_bytes = k / 2, a_row_scales = k / 16;
  int64_t slab[NS];
  slab[0] = blockIdx.x;
  if (SILU) slab[NS - 1] = blockIdx.x + (n / 2) / kTileN;
  // The waves split the slab's super-tiles (padding tiles hold zeros).
  const int64_t ks0 = KS * wave / DW, ks1 = KS * (wave + 1) / DW;
  const int64_t rec_total = L::rec_bytes(KTP) / 16;
  float* s_sa = reinterpret_cast<float*>(smem + L::rec_bytes(KTP));

  // One super-tile of each slab: four tiles of codes and, per lane, row r's
  // scales for tiles 2h and 2h+1 (the other pair comes from lane r + 32(1-h)).
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
  struct Super { uint4 b[NS][kSuperTiles]; uint2 bs[NS]; };
  // Streaming loads (non-temporal: the weights are read once), unconditional
  // and clamped to the wave's range so the compiler can count them.
  auto load = [&](int64_t ks, Super& S) __attribute__((always_inline)) {
    ks = ks < ks1 ? ks : ks1 - 1;
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const uint8_t* sp = w_packed + (slab[j] * KS + ks) * kSuperBytes;   // wave-uniform
#pragma unroll
      for (int tt = 0; tt < kSuperTiles; ++tt) {
        const u32x4_t cv = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(sp + tt * kTileCodeBytes + lane * 16));
        S.b[j][tt] = make_uint4(cv[0], cv[1], cv[2], cv[3]);
      }
      const u32x2_t sv = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(sp + kSuperScaleOff + lane * 8));
      S.bs[j] = make_uint2(sv[0], sv[1]);
    }
  };
  Super g_a[SU], g_b[SU];
  auto load_group = [&](int64_t g0, Super (&G)[SU]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < SU; ++u) load(g0 + u, G[u]);
  };

  // Stage A: operand records (one per (tile, block, row), plus a zero record
  // per tile) and FP32 block scales.  When A is small (the usual decode case)
  // a fixed, unrolled set of unconditional staging loads (invalid items read
  // offset 0, which always exists, and are zeroed afterwards) is issued before
  // the weight loads, so waiting for it does not wait for the weight stream.
  constexpr int SPT = 4;
  const uint32_t kt4 = (uint32_t)KTP * 4u, k32 = (uint32_t)k, m32 = (uint32_t)m;
  const uint32_t nrec = (uint32_t)rec_total, nsc = (uint32_t)MR * kt4;
  const bool fast_stage = nrec <= (uint32_t)(SPT * DW * 64) && nsc <= (uint32_t)(SPT * DW * 64);
  auto rec_of = [&](uint32_t idx, bool& ok, bool& odd) __attribute__((always_inline)) -> uint32_t {
    const uint32_t kt = idx / L::RECS, rr = idx % L::RECS;
    const uint32_t q = rr / MR, mm = rr % MR;
    ok = idx < nrec && rr < 4 * MR && mm < m32 && kt * kTileK + q * 16 < k32;
    odd = (q & 1) != 0;
    return ok ? mm * (uint32_t)a_row_bytes + kt * 32 + q * 8 : 0u;
  };
  auto scale_of = [&](uint32_t idx, bool& ok) __attribute__((always_inline)) -> uint32_t {
    const uint32_t mm = idx / kt4, b = idx - mm * kt4;
    ok = idx < nsc && mm < m32 && b * 16 < k32;
    return ok ? mm * (uint32_t)a_row_scales + b : 0u;
  };
  auto record = [&](uint2 c, bool ok, bool odd) __attribute__((always_inline)) -> uint4 {
    if (!ok) c = make_uint2(0u, 0u);
    return odd ? make_uint4(0u, 0u, c.x, c.y) : make_uint4(c.x, c.y, 0u, 0u);
  };
  if (fast_stage) {
    uint2 rc[SPT];
    uint32_t sc[SPT];
    bool rok[SPT], sok[SPT], rodd[SPT];
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      const uint32_t idx = (uint32_t)t + (uint32_t)(i * DW * 64);
      rc[i] = *reinterpret_cast<const uint2*>(a_codes + rec_of(idx, rok[i], rodd[i]));
      sc[i] = a_scales[scale_of(idx, sok[i])];
    }
    __builtin_amdgcn_sched_barrier(0);
    if (ks0 < ks1) { load_group(ks0, g_a); load_group(ks0 + SU, g_b); }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      const uint32_t idx = (uint32_t)t + (uint32_t)(i * DW * 64);
      if (idx < nrec) *reinterpret_cast<uint4*>(smem + idx * 16) = record(rc[i], rok[i], rodd[i]);
      if (idx < nsc) s_sa[idx] = sok[i] ? e4m3_decode(sc[i]) : 0.0f;
    }
  } else {
    if (ks0 < ks1) { load_group(ks0, g_a); load_group(ks0 + SU, g_b); }
    for (uint32_t idx = t; idx < nrec; idx += DW * 64) {
      bool ok, odd;
      const uint32_t off = rec_of(idx, ok, odd);
      uint2 c = make_uint2(0u, 0u);
      if (ok) c = *reinterpret_cast<const uint2*>(a_codes + off);
      *reinterpret_cast<uint4*>(smem + idx * 16) = record(c, ok, odd);
    }
    for (uint32_t idx = t; idx < nsc; idx += DW * 64) {
      bool ok;
      const uint32_t off = scale_of(idx, ok);
      s_sa[idx] = ok ? e4m3_decode(a_scales[off]) : 0.0f;
    }
  }
  __syncthreads();

  // This lane's A operand record within a tile: MFMA row r = 4*amm + aq.
  const int amm = r >> 2, aq = r & 3;
  const bool a_on = amm < MR && h == (aq >> 1);
  const uint32_t a_lane = a_on ? (uint32_t)((aq * MR + amm) * 16) : (uint32_t)(4 * MR * 16);

  // Partial sums per (slab, row[, block slot]): with one row per lane the four
  // block slots get chains of their own, otherwise the rows are the chains.
  constexpr int QC = MH == 1 ? 4 : 1;
  float y4[NS][MH][QC];
#pragma unroll
  for (int j = 0; j < NS; ++j)
#pragma unroll
    for (int i = 0; i < MH; ++i)
#pragma unroll
      for (int q = 0; q < QC; ++q) y4[j][i][q] = 0.0f;

  // One tile: its MFMA results and the FP32 scale products s_a * s_w.
  struct Prod { floatx16 c[NS]; float p[NS][MH][4]; };
  auto tile_mfma = [&](int64_t kt, const uint4 (&wb)[NS], const uint32_t (&ws)[NS], Prod& P)
      __attribute__((always_inline)) {
    const uint4 a4 = *reinterpret_cast<const uint4*>(smem + kt * (L::RECS * 16) + a_lane);
    const v8i_t av = {(int)a4.x, (int)a4.y, (int)a4.z, (int)a4.w, 0, 0, 0, 0};
    float4 sa[MH];
#pragma unroll
    for (int i = 0; i < MH; ++i) sa[i] = *reinterpret_cast<const float4*>(s_sa + ((2 * i + h) * KTP + kt) * 4);
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const v8i_t bv = {(int)wb[j].x, (int)wb[j].y, (int)wb[j].z, (int)wb[j].w, 0, 0, 0, 0};
      const floatx16 zero = {};
      P.c[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, zero, 4, 4, 0, 127, 0, 127);
      const float sw0 = __builtin_amdgcn_cvt_f32_fp8((int)ws[j], 0);
      const float sw1 = __builtin_amdgcn_cvt_f32_fp8((int)ws[j], 1);
      const float sw2 = __builtin_amdgcn_cvt_f32_fp8((int)ws[j], 2);
      const float sw3 = __builtin_amdgcn_cvt_f32_fp8((int)ws[j], 3);
#pragma unroll
      for (int i = 0; i < MH; ++i) {
        P.p[j][i][0] = sa[i].x * sw0;
        P.p[j][i][1] = sa[i].y * sw1;
        P.p[j][i][2] = sa[i].z * sw2;
        P.p[j][i][3] = sa[i].w * sw3;
      }
    }
  };
  auto tile_accumulate = [&](const Prod& P) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < NS; ++j)
#pragma unroll
      for (int i = 0; i < MH; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) y4[j][i][q % QC] += P.p[j][i][q] * P.c[j][4 * i + q];
  };
  // One super-tile, branch-free: row r's scales for all four tiles (own pair
  // plus the other half's), then tile u+1's MFMA issued before tile u's
  // results are scaled and accumulated (with several rows or slabs per lane
  // two tiles' state does not fit the register budget; those run in order).
  auto compute_super = [&](int64_t ks, const Super& S) __attribute__((always_inline)) {
    uint32_t ws[kSuperTiles][NS];
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const uint32_t o0 = (uint32_t)__shfl_xor((int)S.bs[j].x, 32, 64);
      const uint32_t o1 = (uint32_t)__shfl_xor((int)S.bs[j].y, 32, 64);
      ws[0][j] = h == 0 ? S.bs[j].x : o0;
      ws[1][j] = h == 0 ? S.bs[j].y : o1;
      ws[2][j] = h == 0 ? o0 : S.bs[j].x;
      ws[3][j] = h == 0 ? o1 : S.bs[j].y;
    }
    auto wb = [&](int tt, uint4 (&o)[NS]) __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < NS; ++j) o[j] = S.b[j][tt];
    };
    const int64_t kt = ks * kSuperTiles;
    if constexpr (NS * MH <= 2) {
      Prod P[2];
      uint4 b0[NS];
      wb(0, b0);
      tile_mfma(kt, b0, ws[0], P[0]);
#pragma unroll
      for (int u = 1; u < kSuperTiles; ++u) {
        uint4 bu[NS];
        wb(u, bu);
        tile_mfma(kt + u, bu, ws[u], P[u & 1]);
        tile_accumulate(P[(u - 1) & 1]);
      }
      tile_accumulate(P[(kSuperTiles - 1) & 1]);
    } else {
#pragma unroll
      for (int u = 0; u < kSuperTiles; ++u) {
        uint4 bu[NS];
        wb(u, bu);
        Prod P1;
        tile_mfma(kt + u, bu, ws[u], P1);
        tile_accumulate(P1);
      }
    }
  };
  auto compute_group = [&](int64_t g0, const Super (&G)[SU]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < SU; ++u)
      if (g0 + u < ks1) compute_super(g0 + u, G[u]);
  };
  // Two groups of SU super-tiles in flight; each group is refilled after use.
  if (ks0 < ks1) {
    for (int64_t g = ks0; g < ks1; g += 2 * SU) {
      compute_group(g, g_a);
      if (g + 2 * SU < ks1) load_group(g + 2 * SU, g_a);
      if (g + SU < ks1) compute_group(g + SU, g_b);
      if (g + 3 * SU < ks1) load_group(g + 3 * SU, g_b);
    }
  }
  float y[NS][MH];
#pragma unroll
  for (int j = 0; j < NS; ++j)
#pragma unroll
    for (int i = 0; i < MH; ++i) {
      float v = y4[j][i][0];
#pragma unroll
      for (int q = 1; q < QC; ++q) v += y4[j][i][q];
      y[j][i] = v;
    }

  // Sum the waves' partial results in LDS (reusing the A staging area).
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);
  if (wave > 0) {
#pragma unroll
    for (int j = 0; j < NS; ++j)
#pragma unroll
      for (int i = 0; i < MH; ++i) red[(((wave - 1) * NS + j) * MH + i) * 64 + lane] = y[j][i];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 0; w < DW - 1; ++w)
#pragma unroll
    for (int j = 0; j < NS; ++j)
#pragma unroll
      for (int i = 0; i < MH; ++i) y[j][i] += red[((w * NS + j) * MH + i) * 64 + lane];

  const float ga = *epi.a_global;
  const bool bf16 = epi.out_bf16 != 0;
  const int64_t col = slab[0] * kTileN + r;
  if (SILU) {
    if (col >= n / 2) return;
    const float alpha = 1.0f / (ga * epi.seg_w_global[0]);
#pragma unroll
    for (int i = 0; i < MH; ++i) {
      const int64_t row = 2 * i + h;
      if (row < m) store_out(out, bf16, row * epi.ld_out + col, silu_mul(y[0][i] * alpha, y[NS - 1][i] * alpha));
    }
  } else {
    if (col >= n) return;
    const ColumnEpilogue ce = column_epilogue(epi, col, ga);
#pragma unroll
    for (int i = 0; i < MH; ++i) {
      const int64_t row = 2 * i + h;
      if (row < m) store_out(out, bf16, row * epi.ld_out + col, apply_epilogue(ce, y[0][i]));
    }
  }
}

// ------------------------------------------------------------ launcher ----
// Prefill tile: MF, NF (32x32 fragments per wave along M, N), WM, WN (waves), stages.
#ifndef NVFP4_PREFILL_TILE
#define NVFP4_PREFILL_TILE 4, 4, 2, 2
#endif
#ifndef NVFP4_PREFILL_STAGES
#define NVFP4_PREFILL_STAGES 4
#endif

// Compute units of the current device (cached per device).
static int cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    cached[dev] = v;
  }
  return cached[dev];
}

template <int MF, int NF, int WM, int WN>
static void launch_prefill(const uint8_t* ac, const uint8_t* as, int64_t m, const uint8_t* w, int64_t n,
                           int64_t k, void* out, const EpilogueArgs& epi, hipStream_t st) {
  constexpr int BM = WM * MF * 32, BN = WN * NF * 32;
  constexpr int NS = NVFP4_PREFILL_STAGES;
  const int64_t cols = epi.silu_mul ? n / 2 : n;
  const int64_t bn = epi.silu_mul ? BN / 2 : BN;
  dim3 grid((unsigned)((cols + bn - 1) / bn), (unsigned)((m + BM - 1) / BM));
  dim3 block(WM * WN * 64);
  // The DMA kernel addresses A through 32-bit per-lane offsets from a
  // wave-uniform base: A's codes must stay below 4 GiB (else the register-staged
  // kernel, with full 64-bit addresses, runs).
  const bool a_fits_32 = m * (k / 2) < ((int64_t)1 << 32) - 64;
  if ((k & 63) == 0 && k / kTileK >= NS && a_fits_32) {
    // One workgroup per CU at a time: when the last round would leave most
    // CUs idle, its tiles run as a second launch of smaller pieces -- each
    // tile cut into ry row bands and rx column bands, the finest cut whose
    // pieces still fit one round -- which fills the machine and finishes that
    // round sooner.  (SiLU*mul tiles are only cut into row bands: a column
    // cut would split gate from up.)
    const int64_t tiles = (int64_t)grid.x * grid.y, cus = cu_count(), rem = tiles % cus;
    int ry = 1, rx = 1;
    if (tiles > cus && rem > 0) {
      static const int cuts[4][2] = {{4, 4}, {4, 2}, {2, 2}, {2, 1}};
      static const int silu_cuts[2][2] = {{4, 1}, {2, 1}};
      const int (*c)[2] = epi.silu_mul ? silu_cuts : cuts;
      const int nc = epi.silu_mul ? 2 : 4;
      for (int i = 0; i < nc; ++i)
        if (rem * c[i][0] * c[i][1] <= cus) {
          ry = c[i][0];
          rx = c[i][1];
          break;
        }
    }
    const bool cut = ry * rx > 1;
    const int64_t nbig = cut ? tiles - rem : tiles;
    const int xcd_chunk = nbig % kXcds == 0 ? (int)(nbig / kXcds) : 0;
    const TileMap big{(int)grid.x, (int)grid.y, 0, 1, 1, xcd_chunk};
    const TileMap tail{(int)grid.x, (int)grid.y, (int)nbig, ry, rx, 0};
    const dim3 tail_grid((unsigned)(rem * ry * rx));
#define NVFP4_LAUNCH_PIECE(MFP, NFP, SL, GRID, MAP) \
  hipLaunchKernelGGL((gemm_prefill_dma_kernel<MFP, NFP, WM, WN, NS, SL>), GRID, block, 0, st, ac, as, m, w, n, \
                     k, out, epi, MAP)
    if (epi.silu_mul) {
      NVFP4_LAUNCH_PIECE(MF, NF, true, dim3((unsigned)nbig), big);
      if (ry == 2) NVFP4_LAUNCH_PIECE(MF / 2, NF, true, tail_grid, tail);
      if (ry == 4) NVFP4_LAUNCH_PIECE(MF / 4, NF, true, tail_grid, tail);
    } else {
      NVFP4_LAUNCH_PIECE(MF, NF, false, dim3((unsigned)nbig), big);
      if (ry == 2 && rx == 1) NVFP4_LAUNCH_PIECE(MF / 2, NF, false, tail_grid, tail);
      if (ry == 2 && rx == 2) NVFP4_LAUNCH_PIECE(MF / 2, NF / 2, false, tail_grid, tail);
      if (ry == 4 && rx == 2) NVFP4_LAUNCH_PIECE(MF / 4, NF / 2, false, tail_grid, tail);
      if (ry == 4 && rx == 4) NVFP4_LAUNCH_PIECE(MF / 4, NF / 4, false, tail_grid, tail);
    }
#undef NVFP4_LAUNCH_PIECE
  } else {
    if (epi.silu_mul)
      hipLaunchKernelGGL((gemm_prefill_regs_kernel<MF, NF, WM, WN, true>), grid, block, 0, st, ac, as, m, w, n, k, out, epi);
    else
      hipLaunchKernelGGL((gemm_prefill_regs_kernel<MF, NF, WM, WN, false>), grid, block, 0, st, ac, as, m, w, n, k, out, epi);
  }
}

// Decode launch shapes: every workgroup of a large projection must be resident
// at once (544 of them for N = 17408), so the number of waves per workgroup
// (the K split) and the register budget (waves per SIMD) are chosen together.
template <int MFD, bool SILU, bool ALDS, int DW, int WPE, int U>
static void launch_decode_kernel(const uint8_t* ac, const uint8_t* as, int64_t m, const uint8_t* w, int64_t n,
                                 int64_t k, void* out, const EpilogueArgs& epi, hipStream_t st) {
  const int64_t slabs = SILU ? (n / 2) / kTileN : (n + kTileN - 1) / kTileN;
  const unsigned lds = ALDS ? (unsigned)((m + 1) * ((k + kTileK - 1) / kTileK) * kTileK * 2) : 0u;
  // grouped A fetch: whole 4-tile groups per row (k % 256 == 0) and 16-byte scale loads
  const bool ga = !ALDS && U == 4 && k % 256 == 0 && (reinterpret_cast<uintptr_t>(as) & 15u) == 0;
  if constexpr (!ALDS && U == 4) {
    if (ga) {
      hipLaunchKernelGGL((gemm_decode_kernel<MFD, SILU, ALDS, DW, WPE, U, true>), dim3((unsigned)slabs),
                         dim3(DW * 64), lds, st, ac, as, m, w, n, k, out, epi);
      return;
    }
  }
  hipLaunchKernelGGL((gemm_decode_kernel<MFD, SILU, ALDS, DW, WPE, U, false>), dim3((unsigned)slabs), dim3(DW * 64),
                     lds, st, ac, as, m, w, n, k, out, epi);
}

template <int MFD, bool SILU>
static void launch_decode(const uint8_t* ac, const uint8_t* as, int64_t m, const uint8_t* w, int64_t n,
                          int64_t k, void* out, const EpilogueArgs& epi, hipStream_t st) {
  if constexpr (MFD == 1 && !SILU) {
    if ((m + 1) * k * 2 <= kDecodeALdsBytes)
      launch_decode_kernel<1, false, true, 4, 3, kDecodeGroupA>(ac, as, m, w, n, k, out, epi, st);
    else
      launch_decode_kernel<1, false, false, 4, 3, 4>(ac, as, m, w, n, k, out, epi, st);
  } else if constexpr (MFD == 2 && SILU) {
    launch_decode_kernel<2, true, false, 2, 1, 4>(ac, as, m, w, n, k, out, epi, st);
  } else {
    launch_decode_kernel<MFD, SILU, false, 2, 2, 4>(ac, as, m, w, n, k, out, epi, st);
  }
}

// FP4-MFMA decode: LDS for the A records and scales (reused for the K-split
// reduction); too large a K falls back to the f16 decode kernel.
#ifndef NVFP4_DECODE_FP4_SU
#define NVFP4_DECODE_FP4_SU 1
#endif
constexpr int kDecodeFp4Waves = 4;
constexpr int64_t kDecodeFp4MaxLds = 56 * 1024;

template <int MR, bool SILU>
static bool launch_decode_fp4(const uint8_t* ac, const uint8_t* as, int64_t m, const uint8_t* w, int64_t n,
                              int64_t k, void* out, const EpilogueArgs& epi, hipStream_t st) {
  using L = Fp4DecodeLds<MR>;
  constexpr int DW = kDecodeFp4Waves;
  const int64_t ktp = super_count(k) * kSuperTiles;
  const int64_t red = (int64_t)(DW - 1) * (SILU ? 2 : 1) * (MR / 2) * 64 * 4;
  int64_t lds = L::rec_bytes(ktp) + L::scale_bytes(ktp);
  if (lds < red) lds = red;
  if (lds > kDecodeFp4MaxLds) return false;
  const int64_t slabs = SILU ? (n / 2) / kTileN : (n + kTileN - 1) / kTileN;
  hipLaunchKernelGGL((gemm_decode_fp4_kernel<MR, SILU, DW, NVFP4_DECODE_FP4_SU>), dim3((unsigned)slabs),
                     dim3(DW * 64), (unsigned)lds, st, ac, as, m, w, n, k, out, epi);
  return true;
}

// The FP4 path covers plain (non-SILU) GEMMs with m <= 4: wider tiles of rows
// or a second (gate/up) slab exceed its register budget, and those shapes run
// no faster than the f16 decode kernel.
static bool try_decode_fp4(const uint8_t* ac, const uint8_t* as, int64_t m, const uint8_t* w, int64_t n,
                           int64_t k, void* out, const EpilogueArgs& epi, hipStream_t st) {
  if (epi.silu_mul) return false;
  if (m <= 2) return launch_decode_fp4<2, false>(ac, as, m, w, n, k, out, epi, st);
  if (m <= 4) return launch_decode_fp4<4, false>(ac, as, m, w, n, k, out, epi, st);
  return false;
}

hipError_t launch_gemm_tiled(const uint8_t* a_codes, const uint8_t* a_scales, int64_t m, const uint8_t* w_packed,
                             int64_t n, int64_t k, void* out, const EpilogueArgs& epi, hipStream_t st) {
  launch_prefill<NVFP4_PREFILL_TILE>(a_codes, a_scales, m, w_packed, n, k, out, epi, st);
  return hipGetLastError();
}

hipError_t launch_gemm(const uint8_t* a_codes, const uint8_t* a_scales, int64_t m, const uint8_t* w_packed,
                       int64_t n, int64_t k, void* out, const EpilogueArgs& epi, hipStream_t st) {
  if (m <= 4 && try_decode_fp4(a_codes, a_scales, m, w_packed, n, k, out, epi, st)) return hipGetLastError();
  if (m <= 64) {
    if (m <= 32) {
      if (epi.silu_mul) launch_decode<1, true>(a_codes, a_scales, m, w_packed, n, k, out, epi, st);
      else launch_decode<1, false>(a_codes, a_scales, m, w_packed, n, k, out, epi, st);
    } else {
      if (epi.silu_mul) launch_decode<2, true>(a_codes, a_scales, m, w_packed, n, k, out, epi, st);
      else launch_decode<2, false>(a_codes, a_scales, m, w_packed, n, k, out, epi, st);
    }
  } else {
    launch_prefill<NVFP4_PREFILL_TILE>(a_codes, a_scales, m, w_packed, n, k, out, epi, st);
  }
  return hipGetLastError();
}

}  // namespace nvfp4
