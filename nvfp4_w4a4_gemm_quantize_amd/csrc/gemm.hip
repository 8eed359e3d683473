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
// the contraction is over every K exactly once.  The product is taken as
// W . A^T (mfma_rows), so the 16 accumulators of lane l hold output row r,
// columns 8q + 4h + e (accumulator 4q + e): four runs of four consecutive
// columns, stored straight from registers.
#include "epilogue.h"
#include "kernels.h"
#include "nvfp4_device.h"

#include <cmath>

namespace nvfp4 {


// True when output columns [c0, c1] (clamped to n - 1) lie in one segment
// without a gate: one alpha then serves the whole tile.  Segments are
// contiguous, so the two end columns decide.
__device__ __forceinline__ bool columns_uniform(const EpilogueArgs& e, int64_t c0, int64_t c1, int64_t n) {
  c1 = c1 < n ? c1 : n - 1;
  int s0 = 0, s1 = 0;
  for (int s = 1; s < e.segs.num; ++s) {
    s0 += c0 >= e.segs.off[s];
    s1 += c1 >= e.segs.off[s];
  }
  return s0 == s1 && e.seg_epi[s0] == 0;
}

// ------------------------------------------------------ tile epilogue ----
#ifndef NVFP4_EPI_PAIRED
#define NVFP4_EPI_PAIRED 1   // 0: every bf16 run as its own 8-byte store
#endif

// Epilogue of a workgroup tile, straight from the accumulators (no LDS
// staging): lane (r, h) of fragment (i, j) holds output row
// m0 + wave_m*MF*32 + i*32 + r, columns c + 8q + 4h + e of the fragment's 32
// (accumulator 4q + e).  Each run of four columns gets alpha and its
// columns' gate functions and is stored as one 8-byte (bf16) or 16-byte
// (fp32) write.  A tile whose columns all share one ungated segment takes
// its alpha once (uniform); otherwise each run reads its four columns'
// entries of the per-column table ctab.
// col_base: first output column of the workgroup; wave_n's fragment jj covers
// output columns col_base + (wave_n * NJ + jj) * 32 .. +31.
// SILU: gate fragment jj and up fragment jj + NF/2 share the layout, so
// h = silu(gate) * up is formed in registers.  With h_codes set, h is rounded
// to bf16 and quantised: a 16-column block of h is split between lanes
// (r, 0) and (r, 1) (8 values each), which exchange their block maximum and
// their halves of the codes across the wave halves.
// Returns (SiLU*mul with epi.h_amax set) the largest |h| this lane stored,
// as a 15-bit bf16 magnitude pattern; 0 otherwise.
template <int MF, int NF, int WM, int WN, bool SILU>
__device__ __forceinline__ uint32_t tile_epilogue(floatx16 (&acc)[MF][NF], const ColumnEpilogue* ctab, bool uniform,
                                                  int lane, int wave_m, int wave_n, int64_t m0, int64_t col_base,
                                                  int64_t m, int64_t n, void* out, const EpilogueArgs& epi) {
  constexpr int NJ = SILU ? NF / 2 : NF;
  const int r = lane & 31, h = lane >> 5;
  const bool bf16 = epi.out_bf16 != 0;
  const int64_t ld = epi.ld_out;
  const int64_t ncols = SILU ? n / 2 : n;

  // four consecutive outputs of one row
  auto store4 = [&](int64_t row, int64_t col0, const float (&v)[4]) __attribute__((always_inline)) {
    const int64_t idx = row * ld + col0;
    if (col0 + 3 < ncols && (idx & 3) == 0) {
      if (bf16) {
        uint2 pk;
        pk.x = pack_bf16x2(v[0], v[1]);
        pk.y = pack_bf16x2(v[2], v[3]);
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

  // bf16, a whole fragment's 32 columns inside the output and 16-byte aligned
  // rows: the lane halves trade runs so that each lane stores 8 consecutive
  // columns at once -- lane (r, 0) columns 16p .. 16p+7, lane (r, 1) columns
  // 16p+8 .. 16p+15 of run pair p -- two 16-byte stores per fragment
  // instead of four 8-byte ones.
  const bool paired_ok = NVFP4_EPI_PAIRED && bf16 && (ld & 7) == 0 && (reinterpret_cast<uintptr_t>(out) & 15) == 0;
  auto store_paired = [&](int64_t row, int64_t c0, const uint2 (&pk)[4]) __attribute__((always_inline)) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      // lane h keeps run 2p + h and receives the other half's run 2p + h
      const uint2 give = h ? pk[2 * p] : pk[2 * p + 1];
      const uint2 keep = h ? pk[2 * p + 1] : pk[2 * p];
      const uint2 gx = lane_halves(give.x), gy = lane_halves(give.y);
      const uint2 got = h ? make_uint2(gx.x, gy.x) : make_uint2(gx.y, gy.y);
      const uint4 w = h ? make_uint4(got.x, got.y, keep.x, keep.y) : make_uint4(keep.x, keep.y, got.x, got.y);
      if (row < m)
        *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(out) + row * ld + c0 + 16 * p + 8 * h) = w;
    }
  };

  // One runtime loop over the wave's fragments keeps the epilogue code single;
  // the fragment is copied out of the accumulators by compile-time cases.
  const float alpha_u = SILU ? 1.0f / (*epi.a_global * epi.seg_w_global[0]) : (uniform ? ctab[0].alpha : 0.0f);
  const bool quant = SILU && epi.h_codes != nullptr;
  const bool track = SILU && bf16 && epi.h_amax != nullptr;   // |h| maxima of the stored bf16 values
  uint32_t hmax = 0;
  const float hg = quant ? *epi.h_global : 0.0f;
  for (int f = 0; f < NJ * MF; ++f) {
    const int jj = f / MF, i = f % MF;
    const int64_t row = m0 + wave_m * MF * 32 + i * 32 + r;
    const int lc = (wave_n * NJ + jj) * 32;                // fragment's first column in the tile
    float v[16];
    static_for<0, NJ * MF>([&](auto cc) __attribute__((always_inline)) {
      constexpr int F = decltype(cc)::value;
      if (f == F) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          if constexpr (SILU) v[e] = silu_mul(acc[F % MF][F / MF][e] * alpha_u, acc[F % MF][F / MF + NF / 2][e] * alpha_u);
          else v[e] = acc[F % MF][F / MF][e];
        }
      }
    });
    if constexpr (SILU) {
      const int64_t c0 = col_base + lc;                    // first h column of the fragment
      if (!quant) {
        if (paired_ok && c0 + 32 <= ncols) {
          uint2 pk[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) pk[q] = make_uint2(pack_bf16x2(v[4 * q], v[4 * q + 1]), pack_bf16x2(v[4 * q + 2], v[4 * q + 3]));
          store_paired(row, c0, pk);
          if (track && row < m)
            hmax = max(hmax, max(absmax_bits8(make_uint4(pk[0].x, pk[0].y, pk[1].x, pk[1].y)),
                                 absmax_bits8(make_uint4(pk[2].x, pk[2].y, pk[3].x, pk[3].y))));
        } else if (row < m) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float w4[4] = {v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
            store4(row, c0 + 8 * q + 4 * h, w4);
            if (track) {
#pragma unroll
              for (int b = 0; b < 4; ++b)     // the bf16 bits store4 wrote (columns past the output excluded)
                if (c0 + 8 * q + 4 * h + b < ncols) hmax = max(hmax, (uint32_t)f32_to_bf16_rne(w4[b]) & 0x7FFFu);
            }
          }
        }
        continue;
      }
      // h in bf16, two values per word: run q holds columns 8q + 4h .. +3
      uint32_t hb[4][2];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        hb[q][0] = pack_bf16x2(v[4 * q], v[4 * q + 1]);
        hb[q][1] = pack_bf16x2(v[4 * q + 2], v[4 * q + 3]);
      }
      // block b (columns 16b .. 16b+15) is runs q = 2b, 2b+1 of both lane halves
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const uint4 mine = make_uint4(hb[2 * b][0], hb[2 * b][1], hb[2 * b + 1][0], hb[2 * b + 1][1]);
        const uint2 mh = lane_halves(absmax_bits8(mine));
        const uint32_t mb = max(mh.x, mh.y);
        float rr;
        const uint32_t S = block_scale(mb, hg, &rr);
        uint32_t x = 0;                                    // codes of my two runs, 16 bits each
        if (S != 0) x = pack_codes4(mine.x, mine.y, rr) | (pack_codes4(mine.z, mine.w, rr) << 16);
        const uint2 xh = lane_halves(x);
        const uint32_t lo = xh.x, hi = xh.y;               // lane half 0's runs, half 1's
        const uint2 codes = make_uint2((lo & 0xFFFFu) | (hi << 16), (lo >> 16) | (hi & 0xFFFF0000u));
        const int64_t hcol = c0 + 16 * b;
        // n/2 is a multiple of 32: a fragment's columns are all inside h or all past it
        if (h == b && row < m && hcol < n / 2) {
          *reinterpret_cast<uint2*>(epi.h_codes + row * (n / 4) + hcol / 2) = codes;
          epi.h_scales[row * (n / 32) + hcol / 16] = (uint8_t)S;
        }
      }
      if (epi.h_out && row < m && c0 < n / 2) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *reinterpret_cast<uint2*>(epi.h_out + row * (n / 2) + c0 + 8 * q + 4 * h) = make_uint2(hb[q][0], hb[q][1]);
      }
    } else {
      if (paired_ok && col_base + lc + 32 <= ncols) {
        uint2 pk[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = lc + 8 * q + 4 * h;
          float w4[4];
          if (uniform) {
#pragma unroll
            for (int e = 0; e < 4; ++e) w4[e] = v[4 * q + e] * alpha_u;
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) w4[e] = apply_epilogue(ctab[c + e], v[4 * q + e]);
          }
          pk[q] = make_uint2(pack_bf16x2(w4[0], w4[1]), pack_bf16x2(w4[2], w4[3]));
        }
        store_paired(row, col_base + lc, pk);
        continue;
      }
      if (row >= m) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = lc + 8 * q + 4 * h;
        float w4[4];
        if (uniform) {
#pragma unroll
          for (int e = 0; e < 4; ++e) w4[e] = v[4 * q + e] * alpha_u;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) w4[e] = apply_epilogue(ctab[c + e], v[4 * q + e]);
        }
        store4(row, col_base + c, w4);
      }
    }
  }
  return hmax;
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
      for (int j = 0; j < NF; ++j) acc[i][j] = mfma_rows(av[i], bv[j], acc[i][j]);
  }
}

// --------------------------------------------- prefill kernel, any K ----
// Register-staged variant for K % 64 != 0 (a partial K tile at the end):
// every load is guarded and zero-filled.  With K % 32 == 16 the rows of A's
// codes are only 8-byte aligned and its scale rows have odd length, so A then
// moves in 8-byte code halves (each 16-element block guarded on its own) and
// single scale bytes.  Workgroup tile BM x BN over the whole K;
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
  static constexpr int LDS = 2 * STAGE;
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
  const bool k_aligned64 = (k & 63) == 0, k_aligned32 = (k & 31) == 0;
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
      const int64_t k0 = kt * 64 + hh * 32;
      const bool ok = q < A_CHUNKS && (m0 + row) < m && k0 < k;
      const uint8_t* p = a_codes + (m0 + row) * a_row_bytes + kt * 32 + hh * 16;
      if (k_aligned32) {
        ra[i] = ld16(p, ok);
      } else {
        const uint2 lo = ok ? *reinterpret_cast<const uint2*>(p) : make_uint2(0u, 0u);
        const uint2 hi = ok && k0 + 16 < k ? *reinterpret_cast<const uint2*>(p + 8) : make_uint2(0u, 0u);
        ra[i] = make_uint4(lo.x, lo.y, hi.x, hi.y);
      }
    }
#pragma unroll
    for (int i = 0; i < AS_PER_T; ++i) {
      const int row = t + i * NT;
      uint32_t v = 0;
      if (row < BM && (m0 + row) < m) {
        const uint8_t* p = a_scales + (m0 + row) * a_row_scales + kt * 4;
        if (k_aligned64) {
          v = *reinterpret_cast<const uint32_t*>(p);
        } else if (k_aligned32) {
          v = *reinterpret_cast<const uint16_t*>(p);
          if (kt * 64 + 32 < k) v |= (uint32_t)(*reinterpret_cast<const uint16_t*>(p + 2)) << 16;
        } else {
          for (int b = 0; b < 4; ++b)
            if (kt * 64 + 16 * b < k) v |= (uint32_t)p[b] << (8 * b);
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

  const int64_t cb = SILU ? o0 : (int64_t)blockIdx.x * BN;
  const bool uniform = !SILU && columns_uniform(epi, cb, cb + BN - 1, n);
  tile_epilogue<MF, NF, WM, WN, SILU>(acc, ctab, uniform, lane, wave_m, wave_n, m0, cb, m, n, out, epi);
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

// The body of the prefill kernels.  KW == 1: the WM x WN waves share the
// stage buffers and split the tile.  KW > 1 (split-K, WM = WN = 1): each of
// the KW waves multiplies the whole tile over its own contiguous range of K
// super-tiles through a private set of stage buffers (no barrier in the
// loop), and the partial sums are added through LDS in a fixed wave order.
template <int MF, int NF, int WM, int WN, int NSTAGE, bool SILU, int KW>
__device__ __forceinline__ void prefill_dma_tile(const uint8_t* __restrict__ a_codes,
                                                 const uint8_t* __restrict__ a_scales, int64_t m,
                                                 const uint8_t* __restrict__ w_packed, int64_t n, int64_t k,
                                                 void* __restrict__ out, const EpilogueArgs& epi, const TileMap& tmap) {
  using P = DmaShape<MF, NF, WM, WN, NSTAGE>;
  constexpr int NWAVES = P::NWAVES, BM = P::BM, BN = P::BN, NTILES = P::NTILES;
  constexpr bool SK = KW > 1;
  constexpr int NT = (SK ? KW : NWAVES) * 64;    // threads of the workgroup
  static_assert(NSTAGE == 3 || NSTAGE == 4, "3 or 4 stages");
  static_assert(!SK || (WM == 1 && WN == 1 && !SILU && KW == NSTAGE && (MF == 2 || MF == 4) && NF % 2 == 0 &&
                        MF * NF <= 16),
                "split-K: one wave per K range covers the tile; owners finish whole fragment rows or halves");
  // One LDS object per stage: the compiler can then tell that the DMA into the
  // stage being filled does not alias the reads of the stage being consumed
  // and does not wait for it before those reads.
  // (stage 0 starts 1 KB into its object: an LDS address of exactly 0 lets the
  // compiler fold the offsets into bit operations that lose the alias
  // information the DMA waits rely on)
  // (split-K: each stage object holds the KW waves' private buffers side by side)
  constexpr int SW = SK ? KW : 1;
  __shared__ __attribute__((aligned(1024))) uint8_t lds_s0[SW * P::STAGE + 1024];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_s1[SW * P::STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_s2[SW * P::STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_s3[NSTAGE > 3 ? SW * P::STAGE : 16];
  __shared__ ColumnEpilogue ctab[SILU ? 1 : BN];

  const int lane = threadIdx.x & 63, r = lane & 31, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lw = SK ? 0 : wave;                 // the wave's index within the load and tile split
  const uint32_t wbuf = SK ? (uint32_t)wave * P::STAGE : 0u;
  auto buf = [&](auto b) __attribute__((always_inline)) -> uint8_t* {
    constexpr int B = decltype(b)::value;
    if constexpr (B == 0) return lds_s0 + 1024 + wbuf;
    else if constexpr (B == 1) return lds_s1 + wbuf;
    else if constexpr (B == 2) return lds_s2 + wbuf;
    else return lds_s3 + wbuf;
  };
  const int wave_m = lw / WN, wave_n = lw % WN;
  const int64_t KT = k / kTileK;
  const int64_t KS = super_count(k);
  const int64_t ntiles_total = (n + kTileN - 1) / kTileN;
  int bx, by;
  map_tile(tmap, bx, by);
  const int64_t m0 = (int64_t)by * BM;
  // split-K: a piece wholly past m or n has nothing to store
  if constexpr (SK)
    if (m0 >= m || (int64_t)bx * BN >= n) return;
  // K steps [kb, ke) of this wave: whole super-tiles (the launcher keeps k % 256 == 0 and KS >= KW)
  const int64_t kb = SK ? kSuperTiles * (KS * wave / KW) : 0;
  const int64_t ke = SK ? kSuperTiles * (KS * (wave + 1) / KW) : KT;
  const uint32_t a_row_bytes = (uint32_t)(k / 2), a_row_scales = (uint32_t)(k / 16);
  const int64_t o0 = SILU ? (int64_t)bx * (BN / 2) : 0;
  if constexpr (!SILU) fill_column_table<BN, NT>(ctab, epi, (int64_t)bx * BN, n);

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
      const int f = (lw + i * NWAVES) % P::N_AC;
      src[i] = a_codes + kb * 32;
      voff[i] = (uint32_t)(row_of(m0 + 32 * f + r) * a_row_bytes) + h * 16;
      dst[i] = f * 1024;
    } else if (i < I_BC) {
      const int g = (lw + (i - I_AS) * NWAVES) % P::N_AS;
      src[i] = a_scales + kb * 4;
      voff[i] = (uint32_t)(row_of(m0 + 64 * g + lane) * a_row_scales);
      dst[i] = P::OFF_AS + g * 256;
    } else if (i < I_BS) {
      const int tl = (lw + (i - I_BC) * NWAVES) % P::N_BC;
      src[i] = w_packed + tile_code_off(ntile_of(tl), kb, KS);
      voff[i] = lane * 16;
      dst[i] = P::OFF_BC + tl * 1024;
    } else {
      const int p = (lw + (i - I_BS) * NWAVES) % P::N_BS;
      // the pair's two tiles (h = 0, 1) differ per lane half: the tile's base
      // offset goes in the lane part
      const int64_t o0 = tile_scale_off(ntile_of(2 * p), kb, KS, 0);
      const int64_t o1 = tile_scale_off(ntile_of(2 * p + 1), kb, KS, 0);
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
        acc[i][j] = mfma_rows(av[i], bv[j], acc[i][j]);
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
    if constexpr (!SK) __builtin_amdgcn_s_barrier();   // split-K: the stage is the wave's own
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
  int64_t kt0 = kb;
  for (; kt0 + 2 * NSTAGE - 1 < ke; kt0 += NSTAGE) {
    static_for<0, NSTAGE>([&](auto b) __attribute__((always_inline)) {
      kstep(b, true, true, std::integral_constant<int, P::LPW * (NSTAGE - 2)>{});
    });
  }
  // Tail: the last steps wait for every load in flight.
  for (; kt0 < ke; kt0 += NSTAGE) {
    static_for<0, NSTAGE>([&](auto b) __attribute__((always_inline)) {
      const int64_t kt = kt0 + decltype(b)::value;
      if (kt < ke) kstep(b, kt + 1 < ke, kt + NSTAGE < ke, std::integral_constant<int, 0>{});
    });
  }

  const int64_t cb = SILU ? o0 : (int64_t)bx * BN;
  const bool uniform = !SILU && columns_uniform(epi, cb, cb + BN - 1, n);
  if constexpr (!SK) {
    const uint32_t hm = tile_epilogue<MF, NF, WM, WN, SILU>(acc, ctab, uniform, lane, wave_m, wave_n, m0, cb, m, n,
                                                            out, epi);
    if constexpr (SILU) {
      if (epi.h_amax != nullptr) {
        const uint32_t wm = wave_max_u32(hm);
        if (lane == 0) epi.h_amax[epi.h_amax_base + (int64_t)blockIdx.x * NWAVES + wave] = wm;
      }
    }
  } else {
    // Wave v finishes OWN fragments: fragment row v (MF == 4) or half of row
    // v / 2 (MF == 2).  In G-fragment phases every other wave writes its
    // partials of v's fragments into stage object v (writer w at slot
    // w - (w > v)), and v adds the KW partials in wave order 0, 1, ..., KW - 1.
    // Every wave's last step waited for all of its loads, so after the first
    // barrier no DMA is left in flight into the stage objects.
    constexpr int OWN = MF * NF / KW, G = OWN < 2 ? OWN : 2;
    constexpr int FB = 16 * 64 * 4;                       // bytes of one fragment's partials
    static_assert((KW - 1) * G * FB <= SW * P::STAGE, "a phase's partials fit one stage object");
    auto obj = [&](auto v) __attribute__((always_inline)) -> float* {
      constexpr int V = decltype(v)::value;
      if constexpr (V == 0) return reinterpret_cast<float*>(lds_s0 + 1024);
      else if constexpr (V == 1) return reinterpret_cast<float*>(lds_s1);
      else if constexpr (V == 2) return reinterpret_cast<float*>(lds_s2);
      else return reinterpret_cast<float*>(lds_s3);
    };
    auto frag_row = [](int v) { return MF == 4 ? v : v / 2; };
    auto frag_col = [](int v) { return MF == 4 ? 0 : (v % 2) * (NF / 2); };
    floatx16 fin[1][OWN];
    __syncthreads();
    static_for<0, OWN / G>([&](auto pp) __attribute__((always_inline)) {
      constexpr int PH = decltype(pp)::value;
      static_for<0, KW>([&](auto vv) __attribute__((always_inline)) {
        constexpr int V = decltype(vv)::value;
        if (wave != V) {
          float* d = obj(vv) + (wave - (wave > V)) * G * (FB / 4);
          static_for<0, G>([&](auto gg) __attribute__((always_inline)) {
            constexpr int GI = decltype(gg)::value;
            const floatx16& a = acc[frag_row(V)][frag_col(V) + PH * G + GI];
#pragma unroll
            for (int e = 0; e < 16; ++e) d[(GI * 16 + e) * 64 + lane] = a[e];
          });
        }
      });
      __syncthreads();
      static_for<0, KW>([&](auto vv) __attribute__((always_inline)) {
        constexpr int V = decltype(vv)::value;
        if (wave == V) {
          const float* d = obj(vv);
          static_for<0, G>([&](auto gg) __attribute__((always_inline)) {
            constexpr int GI = decltype(gg)::value;
            const floatx16& mine = acc[frag_row(V)][frag_col(V) + PH * G + GI];
            floatx16 sum;
            static_for<0, KW>([&](auto ww) __attribute__((always_inline)) {
              constexpr int W = decltype(ww)::value;
              floatx16 part;
              if constexpr (W == V) {
                part = mine;
              } else {
                const float* q = d + (W - (W > V)) * G * (FB / 4) + GI * 16 * 64;
#pragma unroll
                for (int e = 0; e < 16; ++e) part[e] = q[e * 64 + lane];
              }
              if constexpr (W == 0) sum = part;
              else sum += part;
            });
            fin[0][PH * G + GI] = sum;
          });
        }
      });
      __syncthreads();
    });
    const int fr = frag_row(wave), fc = frag_col(wave);
    tile_epilogue<1, OWN, 1, 1, false>(fin, ctab + fc * 32, uniform, lane, 0, 0, m0 + fr * 32, cb + fc * 32, m, n,
                                       out, epi);
  }
}

template <int MF, int NF, int WM, int WN, int NSTAGE, bool SILU>
__global__ void __launch_bounds__(WM * WN * 64)
gemm_prefill_dma_kernel(const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales, int64_t m,
                        const uint8_t* __restrict__ w_packed, int64_t n, int64_t k, void* __restrict__ out,
                        EpilogueArgs epi, TileMap tmap) {
  prefill_dma_tile<MF, NF, WM, WN, NSTAGE, SILU, 1>(a_codes, a_scales, m, w_packed, n, k, out, epi, tmap);
}

// Split-K pieces for a launch's last, partly filled round: KW waves, each
// over a quarter of K, multiply an MF x NF-fragment piece (a cut tile) with
// the main kernel's loop, so a piece's K loop is a quarter as long.
template <int MF, int NF, int NSTAGE, int KW>
__global__ void __launch_bounds__(KW * 64)
gemm_prefill_splitk_kernel(const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales, int64_t m,
                           const uint8_t* __restrict__ w_packed, int64_t n, int64_t k, void* __restrict__ out,
                           EpilogueArgs epi, TileMap tmap) {
  prefill_dma_tile<MF, NF, 1, 1, NSTAGE, false, KW>(a_codes, a_scales, m, w_packed, n, k, out, epi, tmap);
}

// ------------------------------------------------------------ launcher ----
// Prefill tile: MF, NF (32x32 fragments per wave along M, N), WM, WN (waves), stages.
#ifndef NVFP4_PREFILL_TILE
#define NVFP4_PREFILL_TILE 4, 4, 2, 2
#endif
#ifndef NVFP4_PREFILL_STAGES
#define NVFP4_PREFILL_STAGES 4
#endif
#ifndef NVFP4_PREFILL_SPLITK
#define NVFP4_PREFILL_SPLITK 1   // 0: the last round's tiles as cut pieces only
#endif

// Compute units of the current device (a host-side attribute query).
static int cu_count() {
  int dev = 0, v = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
    return 256;
  return v;
}

// A tail piece (the tile cut into ry row bands and rx column bands) must
// itself be a valid DMA tile: whole fragments, 64-row A scale groups, weight
// tiles in pairs, and (SiLU*mul) matching gate and up halves.
template <int MF, int NF, int WM, int WN, bool SL>
constexpr bool piece_ok(int ry, int rx) {
  return MF % ry == 0 && NF % rx == 0 && (WM * (MF / ry) * 32) % 64 == 0 && (WN * (NF / rx)) % 2 == 0 &&
         (!SL || (rx == 1 && NF % 2 == 0));
}

// amax_written (SiLU*mul with epi.h_amax): receives the number of |h| partial
// maxima the launches write (one per wave), or 0 when the register-staged
// kernel runs (it writes none).
template <int MF, int NF, int WM, int WN>
static void launch_prefill(const uint8_t* ac, const uint8_t* as, int64_t m, const uint8_t* w, int64_t n,
                           int64_t k, void* out, const EpilogueArgs& epi, hipStream_t st,
                           int64_t* amax_written = nullptr) {
  if (amax_written) *amax_written = 0;
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
  // ... and the two weight tiles of a scale-pair load differ by one slab
  // (super_count(k) * kSuperBytes bytes), also a 32-bit per-lane offset.
  const bool w_fits_32 = super_count(k) * kSuperBytes < ((int64_t)1 << 32) - 1024;
  if ((k & 63) == 0 && k / kTileK >= NS && a_fits_32 && w_fits_32) {
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
        if (rem * c[i][0] * c[i][1] <= cus &&
            (epi.silu_mul ? piece_ok<MF, NF, WM, WN, true>(c[i][0], c[i][1])
                          : piece_ok<MF, NF, WM, WN, false>(c[i][0], c[i][1]))) {
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
    // the last round's |h| partial maxima follow the full rounds' (same waves per workgroup)
    EpilogueArgs epi_tail = epi;
    epi_tail.h_amax_base = epi.h_amax_base + nbig * (WM * WN);
    if (amax_written) *amax_written = (nbig + (cut ? (int64_t)tail_grid.x : 0)) * (WM * WN);
#define NVFP4_LAUNCH_PIECE(MFP, NFP, SL, GRID, MAP) \
  hipLaunchKernelGGL((gemm_prefill_dma_kernel<MFP, NFP, WM, WN, NS, SL>), GRID, block, 0, st, ac, as, m, w, n, \
                     k, out, (MAP).first > 0 ? epi_tail : epi, MAP)
    if (epi.silu_mul) {
      if constexpr (piece_ok<MF, NF, WM, WN, true>(1, 1)) {
        NVFP4_LAUNCH_PIECE(MF, NF, true, dim3((unsigned)nbig), big);
        if constexpr (piece_ok<MF, NF, WM, WN, true>(2, 1))
          if (ry == 2) NVFP4_LAUNCH_PIECE(MF / 2, NF, true, tail_grid, tail);
        if constexpr (piece_ok<MF, NF, WM, WN, true>(4, 1))
          if (ry == 4) NVFP4_LAUNCH_PIECE(MF / 4, NF, true, tail_grid, tail);
      }
    } else {
      NVFP4_LAUNCH_PIECE(MF, NF, false, dim3((unsigned)nbig), big);
      // Split-K pieces: four waves each take a quarter of K over the whole
      // piece (pieces of 4x4, 2x2 or 2x4 fragments; K in whole super-tiles,
      // at least one per wave).  Otherwise the cut pieces split the tile.
      constexpr int TM = WM * MF, TN = WN * NF;
      bool sk = false;
      if constexpr (NS == kSuperTiles && NVFP4_PREFILL_SPLITK) {
        if (cut && k % kSuperK == 0 && super_count(k) >= 4) {
#define NVFP4_LAUNCH_SPLITK(MFP, NFP)                                                                    \
  hipLaunchKernelGGL((gemm_prefill_splitk_kernel<MFP, NFP, NS, 4>), tail_grid, dim3(256), 0, st, ac, as, m, w, n, k, \
                     out, epi, tail)
          sk = true;
          if (TM == 4 * ry && TN == 4 * rx) NVFP4_LAUNCH_SPLITK(4, 4);
          else if (TM == 2 * ry && TN == 2 * rx) NVFP4_LAUNCH_SPLITK(2, 2);
          else if (TM == 2 * ry && TN == 4 * rx) NVFP4_LAUNCH_SPLITK(2, 4);
          else sk = false;
#undef NVFP4_LAUNCH_SPLITK
        }
      }
      if (!sk) {
        if constexpr (piece_ok<MF, NF, WM, WN, false>(2, 1))
          if (ry == 2 && rx == 1) NVFP4_LAUNCH_PIECE(MF / 2, NF, false, tail_grid, tail);
        if constexpr (piece_ok<MF, NF, WM, WN, false>(2, 2))
          if (ry == 2 && rx == 2) NVFP4_LAUNCH_PIECE(MF / 2, NF / 2, false, tail_grid, tail);
        if constexpr (piece_ok<MF, NF, WM, WN, false>(4, 2))
          if (ry == 4 && rx == 2) NVFP4_LAUNCH_PIECE(MF / 4, NF / 2, false, tail_grid, tail);
        if constexpr (piece_ok<MF, NF, WM, WN, false>(4, 4))
          if (ry == 4 && rx == 4) NVFP4_LAUNCH_PIECE(MF / 4, NF / 4, false, tail_grid, tail);
      }
    }
#undef NVFP4_LAUNCH_PIECE
  } else if (epi.silu_mul) {
    if constexpr (NF % 2 == 0)
      hipLaunchKernelGGL((gemm_prefill_regs_kernel<MF, NF, WM, WN, true>), grid, block, 0, st, ac, as, m, w, n, k, out, epi);
  } else {
    hipLaunchKernelGGL((gemm_prefill_regs_kernel<MF, NF, WM, WN, false>), grid, block, 0, st, ac, as, m, w, n, k, out, epi);
  }
}

// Decode launch shapes: every workgroup of a large projection must be resident
// at once (544 of them for N = 17408), so the number of waves per workgroup
// (the K split) and the register budget (waves per SIMD) are chosen together.

hipError_t launch_gemm_tiled(const uint8_t* a_codes, const uint8_t* a_scales, int64_t m, const uint8_t* w_packed,
                             int64_t n, int64_t k, void* out, const EpilogueArgs& epi, hipStream_t st) {
  launch_prefill<NVFP4_PREFILL_TILE>(a_codes, a_scales, m, w_packed, n, k, out, epi, st);
  return hipGetLastError();
}

// Partial maxima of |h|: one per wave of the prefill kernels (at most 16
// pieces of a tile, four waves each), or one per workgroup of an amax pass.
constexpr int64_t kAmaxPassParts = 1024;
int64_t silu_amax_parts_bound(int64_t m, int64_t n) {
  const int64_t tiles = ((m + 255) / 256) * ((n / 2 + 127) / 128);
  return tiles * 16 * 4 > kAmaxPassParts ? tiles * 16 * 4 : kAmaxPassParts;
}

hipError_t launch_gemm_silu_amax(const uint8_t* a_codes, const uint8_t* a_scales, int64_t m, const uint8_t* w_packed,
                                 int64_t n, int64_t k, uint16_t* h, const EpilogueArgs& epi_in, uint32_t* parts,
                                 int64_t cap, int64_t* written, hipStream_t st) {
  *written = 0;
  if (m > 64) {
    // prefill kernels: the maxima come from the epilogue
    EpilogueArgs epi = epi_in;
    epi.h_amax = parts;
    epi.h_amax_base = 0;
    launch_prefill<NVFP4_PREFILL_TILE>(a_codes, a_scales, m, w_packed, n, k, h, epi, st, written);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess || *written > 0) return e;
  } else {
    const hipError_t e = launch_gemm(a_codes, a_scales, m, w_packed, n, k, h, epi_in, st);
    if (e != hipSuccess) return e;
  }
  // decode and register-staged kernels: an amax pass over h
  int64_t np = (m * (n / 2) / 8 + 255) / 256;
  np = np < 1 ? 1 : np > kAmaxPassParts ? kAmaxPassParts : np;
  np = np > cap ? cap : np;
  *written = np;
  return launch_amax_partials(h, m, n / 2, epi_in.ld_out, parts, (int)np, st);
}

hipError_t launch_linear(const QuantSource& qs, int64_t m, const uint8_t* w_packed, int64_t n, int64_t k,
                         void* out, const EpilogueArgs& epi, hipStream_t st) {
  if (launch_gemm_decode_quantize(qs, m, w_packed, n, k, out, epi, st)) return hipGetLastError();
  const hipError_t e = launch_quantize(qs.x, m, k, qs.ld_x, qs.g, qs.dynamic != 0, qs.codes, qs.scales, st);
  if (e != hipSuccess) return e;
  return launch_gemm(qs.codes, qs.scales, m, w_packed, n, k, out, epi, st);
}

// Plain GEMMs choose between 256 x 256 tiles and 128 x 320 tiles (five
// column fragments per wave) by the rounds of one-workgroup-per-CU waves each
// needs: a 128 x 320 tile is 0.625 of the work of a 256 x 256 one, done at
// kNarrowEff of its rate (measured: 0.87); a 256 x 256 grid that leaves a
// partial last round pays about 0.4 of a round for its cut tail.  2048 x 5120
// (160 wide tiles on 256 CUs, or exactly 256 narrow ones) measured 121 ->
// 103 us with narrow tiles; 4096 x 5120 (1.25 rounds of wide tiles, or
// exactly 2 of narrow ones) stays wide: 590 against 619 us.
#ifndef NVFP4_PREFILL_NARROW
#define NVFP4_PREFILL_NARROW 1
#endif
constexpr double kNarrowEff = 0.85;
static bool narrow_tiles(int64_t m, int64_t n, const EpilogueArgs& epi) {
  if (NVFP4_PREFILL_NARROW == 0 || epi.silu_mul) return false;
  if (NVFP4_PREFILL_NARROW == 2) return true;
  const double cus = (double)cu_count();
  const double wide = (double)(((m + 255) / 256) * ((n + 255) / 256));
  const double narrow = (double)(((m + 127) / 128) * ((n + 319) / 320));
  const double r_wide = wide <= cus ? 1.0 : std::floor(wide / cus) + (std::fmod(wide, cus) > 0 ? 0.4 : 0.0);
  const double r_narrow = std::ceil(narrow / cus) * 0.625 / kNarrowEff;
  return r_narrow < r_wide;
}

hipError_t launch_gemm(const uint8_t* a_codes, const uint8_t* a_scales, int64_t m, const uint8_t* w_packed,
                       int64_t n, int64_t k, void* out, const EpilogueArgs& epi, hipStream_t st) {
  if (launch_gemm_decode(a_codes, a_scales, m, w_packed, n, k, out, epi, st)) return hipGetLastError();
  if (narrow_tiles(m, n, epi))
    launch_prefill<2, 5, 2, 2>(a_codes, a_scales, m, w_packed, n, k, out, epi, st);
  else
    launch_prefill<NVFP4_PREFILL_TILE>(a_codes, a_scales, m, w_packed, n, k, out, epi, st);
  return hipGetLastError();
}
}  // namespace nvfp4
