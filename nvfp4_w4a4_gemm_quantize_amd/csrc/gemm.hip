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

__device__ __forceinline__ ColumnEpilogue column_epilogue(const EpilogueArgs& e, int64_t col, float ga) {
  int s = 0;
  while (s + 1 < e.segs.num && col >= e.segs.off[s + 1]) ++s;
  ColumnEpilogue c;
  c.alpha = 1.0f / (ga * e.seg_w_global[s]);
  c.type = e.seg_epi[s];
  c.exp_alog = 0.0f;
  c.dt_bias = 0.0f;
  if (c.type == 2) {
    const int64_t h = col - e.segs.off[s];
    c.exp_alog = expf(e.a_log[h]);
    c.dt_bias = e.dt_bias[h];
  }
  return c;
}

__device__ __forceinline__ float apply_epilogue(const ColumnEpilogue& c, float acc) {
  float y = acc * c.alpha;
  if (c.type == 1) {
    y = 1.0f / (1.0f + expf(-y));
  } else if (c.type == 2) {
    const float x = y + c.dt_bias;
    const float sp = x > 20.0f ? x : log1pf(expf(x));
    y = -c.exp_alog * sp;
  }
  return y;
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

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

// ------------------------------------------------------ prefill kernel ----
// Workgroup tile BM x BN (BM = WM*MF*32, BN = WN*NF*32) over the whole K.
// Per 64-wide K step the packed A rows and the W tiles are staged through LDS
// (double buffered, 16-byte global loads held in registers while the current
// stage is multiplied); each wave reads its fragments from LDS, dequantises
// them in registers and issues MF*NF*4 MFMAs.
// SILU: the workgroup covers BN/2 output columns o0.. and loads the matching
// gate tiles (columns o0..) and up tiles (columns n/2 + o0..); frag j < NF/2
// of a wave is a gate tile and frag j + NF/2 the up tile of the same columns.
template <int MF, int NF, int WM, int WN, bool SILU>
__global__ void __launch_bounds__(WM * WN * 64)
gemm_prefill_kernel(const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales, int64_t m,
                    const uint8_t* __restrict__ w_packed, int64_t n, int64_t k, void* __restrict__ out,
                    EpilogueArgs epi) {
  constexpr int NT = WM * WN * 64;
  constexpr int BM = WM * MF * 32;
  constexpr int BN = WN * NF * 32;
  constexpr int NTILES = BN / 32;
  constexpr int HSTRIDE = BM * 16 + 64;             // LDS bytes per K half of the A stage
  constexpr int A_CHUNKS = 2 * BM;                  // 16-byte chunks of A codes per stage
  constexpr int B_CHUNKS = NTILES * 64;
  constexpr int A_PER_T = (A_CHUNKS + NT - 1) / NT;
  constexpr int B_PER_T = (B_CHUNKS + NT - 1) / NT;
  constexpr int AS_PER_T = (BM + NT - 1) / NT;
  constexpr int BS_PER_T = (BN + NT - 1) / NT;

  __shared__ __attribute__((aligned(16))) uint8_t s_ac[2][2 * HSTRIDE];
  __shared__ uint32_t s_as[2][BM];
  __shared__ __attribute__((aligned(16))) uint8_t s_bc[2][NTILES * kTileCodeBytes];
  __shared__ uint32_t s_bs[2][NTILES * 32];

  const int t = threadIdx.x;
  const int lane = t & 63, r = lane & 31, h = lane >> 5;
  const int wave = t >> 6, wave_m = wave / WN, wave_n = wave % WN;
  const int64_t KT = (k + kTileK - 1) / kTileK;
  const int64_t ntiles_total = (n + kTileN - 1) / kTileN;
  const int64_t m0 = (int64_t)blockIdx.y * BM;
  const int64_t a_row_bytes = k / 2, a_row_scales = k / 16;
  const uint8_t* w_scales = w_packed + ((n + kTileN - 1) / kTileN) * kTileN * (KT * kTileK) / 2;
  const bool k_aligned64 = (k & 63) == 0;

  int64_t o0 = 0;  // SILU: first output column of the workgroup
  auto ntile_of = [&](int tl) -> int64_t {
    if (SILU) {
      const int half = NTILES / 2;
      return tl < half ? (o0 / 32 + tl) : ((n / 2 + o0) / 32 + (tl - half));
    }
    return (int64_t)blockIdx.x * NTILES + tl;
  };
  bool tile_ok[NTILES];
  if (SILU) o0 = (int64_t)blockIdx.x * (BN / 2);
#pragma unroll
  for (int tl = 0; tl < NTILES; ++tl) {
    if (SILU) {
      const int half = NTILES / 2;
      tile_ok[tl] = (o0 / 32 + (tl < half ? tl : tl - half)) < (n / 2) / 32;
    } else {
      tile_ok[tl] = ntile_of(tl) < ntiles_total;
    }
  }

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
      const bool ok = q < B_CHUNKS && tile_ok[tl < NTILES ? tl : 0];
      rb[i] = ld16(w_packed + (ntile_of(tl) * KT + kt) * kTileCodeBytes + ln * 16, ok);
    }
#pragma unroll
    for (int i = 0; i < BS_PER_T; ++i) {
      const int q = t + i * NT;
      const int tl = q >> 5, c = q & 31;
      uint32_t v = 0;
      if (q < BN && tile_ok[tl < NTILES ? tl : 0])
        v = *reinterpret_cast<const uint32_t*>(w_scales + (ntile_of(tl) * KT + kt) * kTileScaleBytes + c * 4);
      rbs[i] = v;
    }
  };
  auto sstore = [&](int stage) {
#pragma unroll
    for (int i = 0; i < A_PER_T; ++i) {
      const int q = t + i * NT;
      if (q < A_CHUNKS) *reinterpret_cast<uint4*>(&s_ac[stage][(q & 1) * HSTRIDE + (q >> 1) * 16]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < AS_PER_T; ++i) {
      const int row = t + i * NT;
      if (row < BM) s_as[stage][row] = ras[i];
    }
#pragma unroll
    for (int i = 0; i < B_PER_T; ++i) {
      const int q = t + i * NT;
      if (q < B_CHUNKS) *reinterpret_cast<uint4*>(&s_bc[stage][q * 16]) = rb[i];
    }
#pragma unroll
    for (int i = 0; i < BS_PER_T; ++i) {
      const int q = t + i * NT;
      if (q < BN) s_bs[stage][q] = rbs[i];
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
    if (kt + 1 < KT) gload(kt + 1);
    uint4 ac[MF], bc[NF];
    uint32_t asc[MF], bsc[NF];
#pragma unroll
    for (int i = 0; i < MF; ++i) {
      const int row = wave_m * MF * 32 + i * 32 + r;
      ac[i] = *reinterpret_cast<const uint4*>(&s_ac[stage][h * HSTRIDE + row * 16]);
      asc[i] = s_as[stage][row] >> (16 * h);
    }
#pragma unroll
    for (int j = 0; j < NF; ++j) {
      const int tl = lds_tile(j);
      bc[j] = *reinterpret_cast<const uint4*>(&s_bc[stage][tl * kTileCodeBytes + lane * 16]);
      bsc[j] = s_bs[stage][tl * 32 + r] >> (16 * h);
    }
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
    if (kt + 1 < KT) sstore(stage ^ 1);
    __syncthreads();
  }

  // Epilogue: alpha (per column segment), gate functions, store.
  const float ga = *epi.a_global;
  const bool bf16 = epi.out_bf16 != 0;
  const int64_t row_base = m0 + wave_m * MF * 32 + 4 * h;
  if (SILU) {
    const float alpha = 1.0f / (ga * epi.seg_w_global[0]);
#pragma unroll
    for (int j = 0; j < NF / 2; ++j) {
      const int64_t col = o0 + (int64_t)(wave_n * (NF / 2) + j) * 32 + r;
      if (col >= n / 2) continue;
#pragma unroll
      for (int i = 0; i < MF; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int64_t row = row_base + i * 32 + 8 * (e >> 2) + (e & 3);
          if (row < m) store_out(out, bf16, row * epi.ld_out + col,
                                 silu_mul(acc[i][j][e] * alpha, acc[i][j + NF / 2][e] * alpha));
        }
    }
  } else {
#pragma unroll
    for (int j = 0; j < NF; ++j) {
      const int64_t col = ntile_of(wave_n * NF + j) * 32 + r;
      if (col >= n) continue;
      const ColumnEpilogue ce = column_epilogue(epi, col, ga);
#pragma unroll
      for (int i = 0; i < MF; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int64_t row = row_base + i * 32 + 8 * (e >> 2) + (e & 3);
          if (row < m) store_out(out, bf16, row * epi.ld_out + col, apply_epilogue(ce, acc[i][j][e]));
        }
    }
  }
}

// ------------------------------------------------------- decode kernel ----
// m <= 64: weight streaming.  One workgroup per 32-column weight slab (two
// slabs -- gate and up -- for SILU); its 4 waves split K four ways, each
// streaming its part of the slab straight from HBM into registers with one
// 16-byte load per lane per 64-wide K tile (the packed layout is already in
// MFMA lane order), with the next tile's loads issued before the current
// tile is multiplied.  The four partial accumulators are summed in LDS in a
// fixed order.
template <int MFD, bool SILU>
__global__ void __launch_bounds__(256)
gemm_decode_kernel(const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales, int64_t m,
                   const uint8_t* __restrict__ w_packed, int64_t n, int64_t k, void* __restrict__ out,
                   EpilogueArgs epi) {
  constexpr int NS = SILU ? 2 : 1;                 // weight slabs per workgroup
  constexpr int NACC = MFD * NS;
  __shared__ float s_red[3][NACC][16][64];

  const int t = threadIdx.x;
  const int lane = t & 63, r = lane & 31, h = lane >> 5, wave = t >> 6;
  const int64_t KT = (k + kTileK - 1) / kTileK;
  const int64_t np = (n + kTileN - 1) / kTileN * kTileN;
  const uint8_t* w_scales = w_packed + np * (KT * kTileK) / 2;
  const int64_t a_row_bytes = k / 2, a_row_scales = k / 16;
  int64_t slab[NS];
  slab[0] = blockIdx.x;
  if (SILU) slab[NS - 1] = blockIdx.x + (n / 2) / kTileN;
  const int64_t kt0 = KT * wave / 4, kt1 = KT * (wave + 1) / 4;

  floatx16 acc[MFD][NS];
#pragma unroll
  for (int i = 0; i < MFD; ++i)
#pragma unroll
    for (int j = 0; j < NS; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  struct Tile { uint4 a[MFD]; uint32_t as[MFD]; uint4 b[NS]; uint32_t bs[NS]; };
  auto load = [&](int64_t kt, Tile& T) {
#pragma unroll
    for (int i = 0; i < MFD; ++i) {
      const int64_t row = i * 32 + r;
      const bool ok = row < m && (kt * 64 + h * 32) < k;
      T.a[i] = ld16(a_codes + row * a_row_bytes + kt * 32 + h * 16, ok);
      T.as[i] = ok ? *reinterpret_cast<const uint16_t*>(a_scales + row * a_row_scales + kt * 4 + 2 * h) : 0u;
    }
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      T.b[j] = *reinterpret_cast<const uint4*>(w_packed + (slab[j] * KT + kt) * kTileCodeBytes + lane * 16);
      T.bs[j] = *reinterpret_cast<const uint16_t*>(w_scales + (slab[j] * KT + kt) * kTileScaleBytes + r * 4 + 2 * h);
    }
  };
  auto compute = [&](const Tile& T) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      half8_t av[MFD], bv[NS];
#pragma unroll
      for (int i = 0; i < MFD; ++i) {
        const uint32_t cw = s == 0 ? T.a[i].x : s == 1 ? T.a[i].y : s == 2 ? T.a[i].z : T.a[i].w;
        av[i] = dequant8(cw, scale_pair_f16(scale_byte(T.as[i], s)));
      }
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        const uint32_t cw = s == 0 ? T.b[j].x : s == 1 ? T.b[j].y : s == 2 ? T.b[j].z : T.b[j].w;
        bv[j] = dequant8(cw, scale_pair_f16(scale_byte(T.bs[j], s)));
      }
#pragma unroll
      for (int i = 0; i < MFD; ++i)
#pragma unroll
        for (int j = 0; j < NS; ++j) acc[i][j] = mfma32x32x16(av[i], bv[j], acc[i][j]);
    }
  };

  if (kt0 < kt1) {
    Tile cur, nxt;
    load(kt0, cur);
    for (int64_t kt = kt0; kt < kt1; ++kt) {
      if (kt + 1 < kt1) load(kt + 1, nxt);
      compute(cur);
      cur = nxt;
    }
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
  for (int w = 0; w < 3; ++w)
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

// ------------------------------------------------------------ launcher ----
template <int MF, int NF, int WM, int WN>
static void launch_prefill(const uint8_t* ac, const uint8_t* as, int64_t m, const uint8_t* w, int64_t n,
                           int64_t k, void* out, const EpilogueArgs& epi, hipStream_t st) {
  constexpr int BM = WM * MF * 32, BN = WN * NF * 32;
  const int64_t cols = epi.silu_mul ? n / 2 : n;
  const int64_t bn = epi.silu_mul ? BN / 2 : BN;
  dim3 grid((unsigned)((cols + bn - 1) / bn), (unsigned)((m + BM - 1) / BM));
  if (epi.silu_mul)
    hipLaunchKernelGGL((gemm_prefill_kernel<MF, NF, WM, WN, true>), grid, dim3(WM * WN * 64), 0, st,
                       ac, as, m, w, n, k, out, epi);
  else
    hipLaunchKernelGGL((gemm_prefill_kernel<MF, NF, WM, WN, false>), grid, dim3(WM * WN * 64), 0, st,
                       ac, as, m, w, n, k, out, epi);
}

hipError_t launch_gemm(const uint8_t* a_codes, const uint8_t* a_scales, int64_t m, const uint8_t* w_packed,
                       int64_t n, int64_t k, void* out, const EpilogueArgs& epi, hipStream_t st) {
  if (m <= 64) {
    const int64_t slabs = epi.silu_mul ? (n / 2) / kTileN : (n + kTileN - 1) / kTileN;
    dim3 grid((unsigned)slabs);
    if (m <= 32) {
      if (epi.silu_mul)
        hipLaunchKernelGGL((gemm_decode_kernel<1, true>), grid, dim3(256), 0, st, a_codes, a_scales, m, w_packed, n, k, out, epi);
      else
        hipLaunchKernelGGL((gemm_decode_kernel<1, false>), grid, dim3(256), 0, st, a_codes, a_scales, m, w_packed, n, k, out, epi);
    } else {
      if (epi.silu_mul)
        hipLaunchKernelGGL((gemm_decode_kernel<2, true>), grid, dim3(256), 0, st, a_codes, a_scales, m, w_packed, n, k, out, epi);
      else
        hipLaunchKernelGGL((gemm_decode_kernel<2, false>), grid, dim3(256), 0, st, a_codes, a_scales, m, w_packed, n, k, out, epi);
    }
  } else {
    launch_prefill<2, 2, 2, 2>(a_codes, a_scales, m, w_packed, n, k, out, epi, st);
  }
  return hipGetLastError();
}

}  // namespace nvfp4
