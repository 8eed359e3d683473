// Weight-streaming decode GEMM kernels for gfx950 (small m): the W4A4
// linear layer of the bayesiansapien page (TL;DR) at decode sizes, where the
// packed weight is read once per call and HBM bandwidth is the bound.
#include "epilogue.h"
#include "kernels.h"
#include "nvfp4_device.h"

namespace nvfp4 {

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
// Buffer resource word 3 for gfx9-family raw buffers (32-bit data format,
// no swizzle): loads past the range read zero.
constexpr int kBufferFlags = 0x00020000;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
#ifndef NVFP4_DECODE_W_AUX
#define NVFP4_DECODE_W_AUX 0
#endif
constexpr int kDecodeWAux = NVFP4_DECODE_W_AUX;
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
  // The waves' A-group areas (GA) and the final cross-wave sums share one LDS
  // buffer: the sums are written only after every wave has left its loop.
  constexpr int kRedBytes = (DW - 1) * NACC * 16 * 64 * 4;
  constexpr int kAgBytes = GA ? DW * MFD * kDecodeGroupFrag : 16;
  __shared__ __attribute__((aligned(16))) uint8_t s_lds[kRedBytes > kAgBytes ? kRedBytes : kAgBytes];
  uint8_t* const s_ag = s_lds;
  auto s_red = reinterpret_cast<float (*)[NACC][16][64]>(s_lds);
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
  // (a single 32x32 output tile would otherwise serialise every MFMA); with
  // two row fragments their two chains already alternate.
  constexpr int NSUB = MFD * NS >= 2 ? 1 : 2;
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
  // The W scale load takes the whole aligned word of row r's four block
  // scales (a 16-bit load would be widened by a VALU op that waits for it --
  // at the loop latch, for the group just issued); lane half h picks its pair
  // at use.
  const uint32_t w_lane = lane * 16, ws_lane = r * 8, ws_shift = 16 * h;
  // Weight loads: buffer loads over each slab's bytes, a constant lane offset
  // plus a wave-uniform tile offset (no per-lane 64-bit address arithmetic).
  __amdgpu_buffer_rsrc_t w_rsrc[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j)
    w_rsrc[j] = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(w_packed) + slab[j] * KS * kSuperBytes,
                                                  (short)0, (int)(KS * kSuperBytes), kBufferFlags);
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
    const int code_off = (int)tile_code_off(0, kt, KS), scale_off = (int)tile_scale_off(0, kt, KS, 0);
#pragma unroll
    for (int j = 0; j < NS; ++j) {                                 // tile offsets are wave-uniform
      const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(w_rsrc[j], w_lane, code_off, kDecodeWAux);
      T.b[j] = make_uint4(v[0], v[1], v[2], v[3]);
      T.bs[j] = __builtin_amdgcn_raw_buffer_load_b32(w_rsrc[j], ws_lane, scale_off, kDecodeWAux);
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
        bv[j] = dequant8(cw, scale_pair_f16((T.bs[j] >> (ws_shift + 8 * (s >> 1))) & 0xFFu));
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
  // The group loads are buffer loads against A's extent (m rows): the range
  // check returns zeros for rows past m, so no clamp is needed, and each load
  // takes a loop-invariant 32-bit lane offset (which alone carries the row)
  // plus the group's wave-uniform K offset.  (With clamped 64-bit addresses
  // the loop ran out of registers at three waves per SIMD, and the spill
  // reloads waited for every load in flight.)  Row i of the MFMA's A operand
  // only reaches output row i, and rows >= m are never stored.  The host
  // keeps m * k / 2 below 2^31.
  uint32_t ag_off[GA ? MFD : 1][GA ? 4 : 1], as_off[GA ? MFD : 1];
  const __amdgpu_buffer_rsrc_t ac_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(a_codes), (short)0, GA ? (int)(m * a_row_bytes) : 0, kBufferFlags);
  const __amdgpu_buffer_rsrc_t as_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(a_scales), (short)0, GA ? (int)(m * a_row_scales) : 0, kBufferFlags);
  if constexpr (GA) {
#pragma unroll
    for (int i = 0; i < MFD; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        ag_off[i][j] = (uint32_t)(i * 32 + 8 * j + (lane >> 3)) * (uint32_t)a_row_bytes + (lane & 7) * 16;
      as_off[i] = (uint32_t)(i * 32 + r) * (uint32_t)a_row_scales;
    }
  }
  auto load_agroup = [&](int64_t g0, AGroup& G) __attribute__((always_inline)) {
    if constexpr (GA) {
      g0 = g0 < kt1 - 4 ? g0 : kt1 - 4;              // groups past the wave's range: never multiplied
      const int cg = (int)(g0 * 32), sg = (int)(g0 * 4);   // wave-uniform
      auto ld = [](__amdgpu_buffer_rsrc_t rs, uint32_t off, int soff) __attribute__((always_inline)) {
        const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rs, off, soff, 0);
        return make_uint4(v[0], v[1], v[2], v[3]);
      };
#pragma unroll
      for (int i = 0; i < MFD; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) G.c[i][j] = ld(ac_rsrc, ag_off[i][j], cg);
        G.s[i] = ld(as_rsrc, as_off[i], sg);
      }
    }
  };
  // A group's loads all go out before the next multiply starts (the
  // scheduler would otherwise move some behind that group's waits).
  auto load_group = [&](int64_t g0, Tile (&T)[U], AGroup& G) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < U; ++u) load(g0 + u, T[u]);
    load_agroup(g0, G);
    __builtin_amdgcn_sched_barrier(0);
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

  // The lane's indices again, from mbcnt rather than kept live across the
  // loop (at three waves per SIMD that cost three spilled registers per lane).
  {
  const int lane = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  const int r = lane & 31, h = lane >> 5;
  floatx16 acc[MFD][NS];
#pragma unroll
  for (int i = 0; i < MFD; ++i)
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      acc[i][j] = part[i][j][0];
#pragma unroll
      for (int q = 1; q < NSUB; ++q) acc[i][j] += part[i][j][q];
    }

  if constexpr (GA) __syncthreads();                // other waves may still read their A-group areas
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
  }  // the block of the recomputed lane indices
}

// ------------------------------------------------ decode kernel, FP4 MFMA ----
// m <= 8: weight streaming on gfx950's block-scaled FP4 MFMA, applied to the
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
// reduction is needed; every (row, block slot) has a chain of its own.
//
// Streaming: one workgroup of DW waves per 32-column weight slab; the waves
// split the slab's K tiles evenly and each keeps R tiles (16 code bytes and
// the row's 4 scale bytes per lane, non-temporal) in flight, refilling a
// slot as soon as its tile is multiplied.  The waves' partial sums are added
// in LDS in a fixed order.
//
// A is staged once per workgroup into LDS: one 8-byte record (a block's 16
// codes) per (tile, block, row) plus one zero record per tile (for lanes
// whose MFMA row is empty), and the A block scales as E4M3 bytes, a lane's
// rows of a tile side by side (one LDS read per tile; the scales are widened
// to FP32 in registers).  Each lane places its record in the half of its
// 16-byte operand that its block occupies.  Its source is either the
// quantizer's codes and scales, or (QUANT) the bf16 activation itself: every
// workgroup then computes the tensor's amax and the global scale, and
// quantises the blocks with the quantizer's own routine (bit-identical to
// nvfp4_quantize); workgroup 0 also writes the codes, scales and global scale
// out.  The staging loads are issued before the first weight loads, so
// waiting for them does not wait for the weight stream.
typedef int v8i_t __attribute__((ext_vector_type(8)));

template <int MR>
struct Fp4DecodeLds {
  static constexpr int RECS = 4 * MR + 1;           // 8-byte records per K tile (last: zeros)
  __host__ __device__ static int64_t rec_bytes(int64_t kt_count) { return kt_count * RECS * 8; }
  __host__ __device__ static int64_t scale_bytes(int64_t kt_count) { return (int64_t)MR * kt_count * 4; }
};

// Three workgroups per CU (544 slabs of a 17408-column weight are then all
// resident at once on 256 CUs): at most 3 * DW / 4 waves per SIMD.
template <int DW>
constexpr int decode_fp4_waves_per_eu() { return (3 * DW + 3) / 4; }

// Workgroup barrier for LDS traffic only: waits for this wave's LDS
// operations, not for its global loads in flight (a __syncthreads() fence
// would also drain the weight stream).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// SP: A blocks staged per thread by the unrolled staging code, which must
// cover all of A unless GENERAL (a staging loop instead: any K that fits LDS,
// with conservative waits).  The two are separate kernels so that the
// unrolled one's waits for its weight tiles stay exact.
// NPW > 0: every wave has exactly NPW weight super-tiles (K / 256 == NPW * DW),
// known at compile time, so the ring below unrolls into straight code whose
// refills are unconditional: each super-tile then waits only for its own
// loads while the next R - 1 are in flight.  (With a run-time count the
// refills sit behind a branch, and the compiler's wait before the next
// super-tile conservatively drains them too, exposing a full memory round
// trip per super-tile.)
template <int MR, int DW, int R, int SP, bool QUANT, bool GENERAL, int NPW>
__global__ void __launch_bounds__(DW * 64) __attribute__((amdgpu_waves_per_eu(decode_fp4_waves_per_eu<DW>())))
gemm_decode_fp4_kernel(const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales, int64_t m,
                       const uint8_t* __restrict__ w_packed, int64_t n, int64_t k, void* __restrict__ out,
                       EpilogueArgs epi, QuantSource qs) {
  constexpr int NT = DW * 64;
  constexpr int MH = MR / 2;                     // A rows per lane: h, 2+h, ...
  using L = Fp4DecodeLds<MR>;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ uint32_t s_max[DW];

  const int t = threadIdx.x;
  const int lane = t & 63, r = lane & 31, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int64_t KS = super_count(k), KTP = KS * kSuperTiles;   // tiles incl. zero padding
  const int64_t KT = (k + kTileK - 1) / kTileK;                // tiles holding data
  const int64_t slab = blockIdx.x;
  // this wave's weight super-tiles [s0, s1)
  const int64_t s0 = NPW > 0 ? (int64_t)NPW * wave : KS * wave / DW;
  const int64_t s1 = NPW > 0 ? s0 + NPW : KS * (wave + 1) / DW;
  const int64_t slast = s1 > 0 ? s1 - 1 : 0;
  // A scale bytes: tile kt, lane half hh: rows 2i + hh, blocks q at (i * 4 + q)
  uint8_t* s_sab = smem + L::rec_bytes(KTP);

  // ---- A staging, part 1: issue the loads (unconditional: invalid items
  // read offset 0, which always exists, and are zeroed afterwards).  Item q
  // is row mm = q / (4 KTP)'s 16-element block b = q % (4 KTP).
  const uint32_t nblk = (uint32_t)(4 * KTP), nitems = (uint32_t)MR * nblk;
  const uint32_t k32 = (uint32_t)k, m32 = (uint32_t)m;
  constexpr bool fast = !GENERAL;
  static_assert(!(QUANT && GENERAL), "the quantising kernel stages A in registers");
  uint4 xa[QUANT ? SP : 1], xb[QUANT ? SP : 1];   // QUANT: the block's 16 bf16
  uint2 rc[QUANT ? 1 : SP];                       // codes of the block
  uint32_t sc[QUANT ? 1 : SP];                    // scale byte of the block
  bool iok[SP];
  // (QUANT) a calibrated global scale is read here, ahead of the weight loads:
  // waiting for a load issued after them would wait for the whole stream.
  const float g_in = QUANT ? *qs.g : 0.0f;
  auto item = [&](int i, uint32_t& mm, uint32_t& b) __attribute__((always_inline)) -> bool {
    const uint32_t q = (uint32_t)t + (uint32_t)(i * NT);
    mm = q / nblk;
    b = q - mm * nblk;
    return q < nitems && mm < m32 && b * 16 < k32;
  };
  if constexpr (fast) {
#pragma unroll
    for (int i = 0; i < SP; ++i) {
      uint32_t mm, b;
      iok[i] = item(i, mm, b);
      if constexpr (QUANT) {
        const uint16_t* p = qs.x + (iok[i] ? (int64_t)mm * qs.ld_x + b * 16 : 0);
        xa[i] = *reinterpret_cast<const uint4*>(p);
        xb[i] = *reinterpret_cast<const uint4*>(p + 8);
      } else {
        rc[i] = *reinterpret_cast<const uint2*>(a_codes + (iok[i] ? mm * (k32 / 2) + b * 8 : 0u));
        sc[i] = a_scales[iok[i] ? mm * (k32 / 16) + b : 0u];
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  // ---- weight stream: one slot per super-tile -- four tiles of 16 code
  // bytes per lane and 8 scale bytes per lane (row r's scales of tiles 2h and
  // 2h+1); the first R super-tiles of this wave go out now.
  struct Slot { uint4 b[kSuperTiles]; uint2 s; };
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
  const uint8_t* wslab = w_packed + slab * KS * kSuperBytes;   // wave-uniform
  auto load = [&](int64_t ks, Slot& S) __attribute__((always_inline)) {
    ks = ks < slast ? ks : slast;                              // past the range: never multiplied
    const uint8_t* p = wslab + ks * kSuperBytes;
#pragma unroll
    for (int u = 0; u < kSuperTiles; ++u) {
      const u32x4_t cv = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p + u * kTileCodeBytes + lane * 16));
      S.b[u] = make_uint4(cv[0], cv[1], cv[2], cv[3]);
    }
    const u32x2_t sv = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p + kSuperScaleOff + lane * 8));
    S.s = make_uint2(sv[0], sv[1]);
    // slots go out in order: the first super-tile's loads must not be
    // scheduled behind the others (its wait would then cover them all)
    __builtin_amdgcn_sched_barrier(0);
  };
  Slot ring[NPW > 0 ? R + 1 : R];
  static_for<0, R>([&](auto u) __attribute__((always_inline)) { load(s0 + decltype(u)::value, ring[decltype(u)::value]); });
  __builtin_amdgcn_sched_barrier(0);

  // ---- A staging, part 2: (QUANT) amax and global scale, then records.
  float ga;
  auto put = [&](uint32_t mm, uint32_t b, uint2 c, uint32_t S) __attribute__((always_inline)) {
    const uint32_t kt = b >> 2, qq = b & 3;
    *reinterpret_cast<uint2*>(smem + ((int64_t)kt * L::RECS + qq * MR + mm) * 8) = c;
    s_sab[((int64_t)kt * 2 + (mm & 1)) * (MH * 4) + (mm >> 1) * 4 + qq] = (uint8_t)S;
  };
  if constexpr (QUANT) {
    // (the launcher runs QUANT only when every block is one of the SP items)
    uint32_t mb = 0;
#pragma unroll
    for (int i = 0; i < SP; ++i) {
      if (!iok[i]) { xa[i] = make_uint4(0u, 0u, 0u, 0u); xb[i] = xa[i]; }
      mb = max(mb, max(absmax_bits8(xa[i]), absmax_bits8(xb[i])));
    }
    mb = wave_max_u32(mb);
    if (lane == 0) s_max[wave] = mb;
    lds_barrier();
    mb = 0;
#pragma unroll
    for (int w = 0; w < DW; ++w) mb = max(mb, s_max[w]);
    if (qs.dynamic) {
      const float amax = __uint_as_float(mb << 16);
      ga = amax > 0.0f ? kGlobalNumerator / amax : 1.0f;
    } else {
      ga = g_in;
    }
    const bool writer = blockIdx.x == 0;
    if (writer && t == 0 && qs.dynamic) *qs.g = ga;
#pragma unroll
    for (int i = 0; i < SP; ++i) {
      uint32_t mm, b;
      const bool ok = item(i, mm, b);
      if (mm < (uint32_t)MR && (uint32_t)t + (uint32_t)(i * NT) < nitems) {
        uint2 c;
        const uint32_t S = quantize_block16(xa[i], xb[i], ga, &c);
        put(mm, b, c, S);
        if (writer && ok) {
          *reinterpret_cast<uint2*>(qs.codes + (int64_t)mm * (k / 2) + b * 8) = c;
          qs.scales[(int64_t)mm * (k / 16) + b] = (uint8_t)S;
        }
      }
    }
  } else {
    ga = *epi.a_global;
    if constexpr (fast) {
#pragma unroll
      for (int i = 0; i < SP; ++i) {
        uint32_t mm, b;
        const bool ok = item(i, mm, b);
        if ((uint32_t)t + (uint32_t)(i * NT) < nitems)
          put(mm, b, ok ? rc[i] : make_uint2(0u, 0u), ok ? sc[i] : 0u);
      }
    } else {
      for (uint32_t q = t; q < nitems; q += NT) {
        const uint32_t mm = q / nblk, b = q - mm * nblk;
        const bool ok = mm < m32 && b * 16 < k32;
        uint2 c = make_uint2(0u, 0u);
        uint32_t S = 0;
        if (ok) {
          c = *reinterpret_cast<const uint2*>(a_codes + mm * (k32 / 2) + b * 8);
          S = a_scales[mm * (k32 / 16) + b];
        }
        put(mm, b, c, S);
      }
    }
  }
  for (int64_t kt = t; kt < KTP; kt += NT)
    *reinterpret_cast<uint2*>(smem + (kt * L::RECS + 4 * MR) * 8) = make_uint2(0u, 0u);
  lds_barrier();

  // ---- multiply.  This lane's A operand record within a tile: MFMA row
  // r = 4*amm + aq holds row amm's block aq, which sits in K half aq / 2 and
  // within it in the 8-byte half aq % 2.
  const int amm = r >> 2, aq = r & 3;
  const bool a_on = amm < MR && h == (aq >> 1);
  const uint32_t a_lane = a_on ? (uint32_t)((aq * MR + amm) * 8) : (uint32_t)(4 * MR * 8);
  const bool a_hi = (aq & 1) != 0;
  float y4[MH][4];
#pragma unroll
  for (int i = 0; i < MH; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) y4[i][q] = 0.0f;

  // One tile: its MFMA (issued one tile ahead), then the FP32 scale products
  // s_a * s_w applied to its per-block sums.  The MFMA of the next tile goes
  // out before this tile's products are formed, so its latency is covered by
  // this tile's VALU work.  The A scales travel as E4M3 bytes (one word per
  // row: blocks 0..3).
  typedef uint32_t sa_words_t __attribute__((ext_vector_type(MH)));
  struct Prod { floatx16 c; uint32_t sa[MH]; uint32_t ws; };
  auto tile_mfma = [&](int64_t kt, const uint4& wb, uint32_t ws, Prod& P) __attribute__((always_inline)) {
    const uint2 a2 = *reinterpret_cast<const uint2*>(smem + kt * (L::RECS * 8) + a_lane);
    const v8i_t av = {a_hi ? 0 : (int)a2.x, a_hi ? 0 : (int)a2.y, a_hi ? (int)a2.x : 0, a_hi ? (int)a2.y : 0,
                      0, 0, 0, 0};
    const v8i_t bv = {(int)wb.x, (int)wb.y, (int)wb.z, (int)wb.w, 0, 0, 0, 0};
    const floatx16 zero = {};
    P.c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, zero, 4, 4, 0, 127, 0, 127);
    if constexpr (MH == 1) {
      P.sa[0] = *reinterpret_cast<const uint32_t*>(s_sab + (kt * 2 + h) * 4);
    } else {
      const sa_words_t w = *reinterpret_cast<const sa_words_t*>(s_sab + (kt * 2 + h) * (MH * 4));
#pragma unroll
      for (int i = 0; i < MH; ++i) P.sa[i] = w[i];
    }
    P.ws = ws;
  };
  auto tile_acc = [&](const Prod& P) __attribute__((always_inline)) {
    const f32x2_t w01 = __builtin_amdgcn_cvt_pk_f32_fp8((int)P.ws, false);
    const f32x2_t w23 = __builtin_amdgcn_cvt_pk_f32_fp8((int)P.ws, true);
#pragma unroll
    for (int i = 0; i < MH; ++i) {
      const f32x2_t a01 = __builtin_amdgcn_cvt_pk_f32_fp8((int)P.sa[i], false);
      const f32x2_t a23 = __builtin_amdgcn_cvt_pk_f32_fp8((int)P.sa[i], true);
      y4[i][0] += (a01[0] * w01[0]) * P.c[4 * i + 0];
      y4[i][1] += (a01[1] * w01[1]) * P.c[4 * i + 1];
      y4[i][2] += (a23[0] * w23[0]) * P.c[4 * i + 2];
      y4[i][3] += (a23[1] * w23[1]) * P.c[4 * i + 3];
    }
  };
  // A super-tile: row r's scales of all four tiles (this lane's pair and the
  // other half's, across the wave), then its data tiles, two products in
  // flight.
  auto super_tile = [&](int64_t ks, const Slot& S) __attribute__((always_inline)) {
    const uint2 sx = lane_halves(S.s.x), sy = lane_halves(S.s.y);
    const uint32_t ws[kSuperTiles] = {sx.x, sy.x, sx.y, sy.y};
    const int64_t kt0 = ks * kSuperTiles;
    if (kt0 + kSuperTiles <= KT) {            // the common case: four data tiles
      Prod P[2];
      tile_mfma(kt0, S.b[0], ws[0], P[0]);
      tile_mfma(kt0 + 1, S.b[1], ws[1], P[1]);
      tile_acc(P[0]);
      tile_mfma(kt0 + 2, S.b[2], ws[2], P[0]);
      tile_acc(P[1]);
      tile_mfma(kt0 + 3, S.b[3], ws[3], P[1]);
      tile_acc(P[0]);
      tile_acc(P[1]);
    } else {
#pragma unroll
      for (int u = 0; u < kSuperTiles; ++u)
        if (kt0 + u < KT) {
          Prod P1;
          tile_mfma(kt0 + u, S.b[u], ws[u], P1);
          tile_acc(P1);
        }
    }
  };

  if constexpr (NPW > 0) {
    // super-tile s0 + i lives in slot i % (R + 1): the load of super-tile
    // s0 + i + R goes out before super-tile s0 + i is multiplied, so R
    // super-tiles are in flight while each one is multiplied
    static_for<0, NPW>([&](auto ii) __attribute__((always_inline)) {
      constexpr int I = decltype(ii)::value;
      if constexpr (I + R < NPW) load(s0 + I + R, ring[(I + R) % (R + 1)]);
      super_tile(s0 + I, ring[I % (R + 1)]);
    });
  } else {
    // Rounds of R super-tiles: super-tile s0 + j*R + u lives in slot u; after
    // its tiles are multiplied the slot is refilled with the super-tile R
    // further on when the wave has another round.  The first round is
    // straight code after the prologue, so its waits are exact; later rounds
    // loop.
    auto round = [&](int64_t base) __attribute__((always_inline)) {
      const bool more = base + R < s1;
      static_for<0, R>([&](auto uu) __attribute__((always_inline)) {
        constexpr int U = decltype(uu)::value;
        const int64_t ks = base + U;
        if (ks < s1) super_tile(ks, ring[U]);
        if (more) load(ks + R, ring[U]);
      });
    };
    round(s0);
    for (int64_t base = s0 + R; base < s1; base += R) round(base);
  }

  float y[MH];
#pragma unroll
  for (int i = 0; i < MH; ++i) y[i] = (y4[i][0] + y4[i][1]) + (y4[i][2] + y4[i][3]);

  // Sum the waves' partial results in LDS (reusing the A staging area).
  lds_barrier();
  float* red = reinterpret_cast<float*>(smem);
  if (wave > 0) {
#pragma unroll
    for (int i = 0; i < MH; ++i) red[((wave - 1) * MH + i) * 64 + lane] = y[i];
  }
  lds_barrier();
  if (wave != 0) return;
#pragma unroll
  for (int w = 0; w < DW - 1; ++w)
#pragma unroll
    for (int i = 0; i < MH; ++i) y[i] += red[(w * MH + i) * 64 + lane];

  const bool bf16 = epi.out_bf16 != 0;
  const int64_t col = slab * kTileN + r;
  if (col >= n) return;
  const ColumnEpilogue ce = column_epilogue(epi, col, ga);
#pragma unroll
  for (int i = 0; i < MH; ++i) {
    const int64_t row = 2 * i + h;
    if (row < m) store_out(out, bf16, row * epi.ld_out + col, apply_epilogue(ce, y[i]));
  }
}

// ------------------------------------------------------- (end of FP4 kernel)

// ------------------------------------------------ weight stream reference ----
// The decode kernels' weight stream with no arithmetic: one workgroup of four
// waves per 32-column slab, each wave reading its share of the slab's
// super-tiles (four 16-byte code loads and one 8-byte scale load per lane per
// super-tile, non-temporal), as the FP4 decode kernel does, with R = 5: every
// load of a wave (a whole K = 5120 share) in flight at once, the fastest depth
// measured for this pattern.  Each lane folds the words of its super-tiles
// into one value (XOR) that is stored only if it equals a constant, so no
// load is dead and a planted word can show that it was read.  Its time is the
// practical HBM ceiling of the decode GEMM's access pattern.
template <int R>
__global__ void __launch_bounds__(256) weight_stream_read_kernel(const uint8_t* __restrict__ w_packed, int64_t k,
                                                                 uint32_t* __restrict__ sink) {
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t KS = super_count(k);
  const int64_t s0 = KS * wave / 4, s1 = KS * (wave + 1) / 4;
  const uint8_t* wslab = w_packed + (int64_t)blockIdx.x * KS * kSuperBytes;
  uint32_t acc = 0;
  for (int64_t j = s0; j < s1; j += R) {
    u32x4_t v[R][kSuperTiles];
    u32x2_t sc[R];
#pragma unroll
    for (int u = 0; u < R; ++u) {
      const int64_t jj = j + u < s1 ? j + u : s1 - 1;
      const uint8_t* p = wslab + jj * kSuperBytes;
#pragma unroll
      for (int t = 0; t < kSuperTiles; ++t)
        v[u][t] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p + t * kTileCodeBytes + lane * 16));
      sc[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p + kSuperScaleOff + lane * 8));
    }
    // fold only the slots that hold the wave's own super-tiles: a slot
    // clamped onto the last one repeats its words, which would cancel
#pragma unroll
    for (int u = 0; u < R; ++u) {
      if (j + u >= s1) continue;
      acc ^= sc[u][0] ^ sc[u][1];
#pragma unroll
      for (int t = 0; t < kSuperTiles; ++t) acc ^= v[u][t][0] ^ v[u][t][1] ^ v[u][t][2] ^ v[u][t][3];
    }
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

#ifndef NVFP4_STREAM_READ_RING
#define NVFP4_STREAM_READ_RING 5
#endif
hipError_t launch_weight_stream_read(const uint8_t* w_packed, int64_t n, int64_t k, uint32_t* sink, hipStream_t st) {
  const int64_t slabs = (n + kTileN - 1) / kTileN;
  hipLaunchKernelGGL((weight_stream_read_kernel<NVFP4_STREAM_READ_RING>), dim3((unsigned)slabs), dim3(256), 0, st,
                     w_packed, k, sink);
  return hipGetLastError();
}

// Grouped A fetch: whole 4-tile groups per row (k % 256 == 0), 16-byte scale
// loads and 32-bit lane offsets into A.
static bool decode_group_a_ok(const uint8_t* as, int64_t m, int64_t k) {
  return k % 256 == 0 && (reinterpret_cast<uintptr_t>(as) & 15u) == 0 && m * (k / 2) < (int64_t(1) << 31);
}

// GA_ONLY: the caller has checked decode_group_a_ok, so the per-tile-fetch
// kernel of this shape is never launched (and not instantiated).
template <int MFD, bool SILU, bool ALDS, int DW, int WPE, int U, bool GA_ONLY = false>
static void launch_decode_kernel(const uint8_t* ac, const uint8_t* as, int64_t m, const uint8_t* w, int64_t n,
                                 int64_t k, void* out, const EpilogueArgs& epi, hipStream_t st) {
  const int64_t slabs = SILU ? (n / 2) / kTileN : (n + kTileN - 1) / kTileN;
  const unsigned lds = ALDS ? (unsigned)((m + 1) * ((k + kTileK - 1) / kTileK) * kTileK * 2) : 0u;
  const bool ga = !ALDS && U == 4 && decode_group_a_ok(as, m, k);
  if constexpr (!ALDS && U == 4) {
    if (GA_ONLY || ga) {
      hipLaunchKernelGGL((gemm_decode_kernel<MFD, SILU, ALDS, DW, WPE, U, true>), dim3((unsigned)slabs),
                         dim3(DW * 64), lds, st, ac, as, m, w, n, k, out, epi);
      return;
    }
  }
  if constexpr (!GA_ONLY)
    hipLaunchKernelGGL((gemm_decode_kernel<MFD, SILU, ALDS, DW, WPE, U, false>), dim3((unsigned)slabs),
                       dim3(DW * 64), lds, st, ac, as, m, w, n, k, out, epi);
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
  } else if constexpr (MFD == 2) {
    if (decode_group_a_ok(as, m, k))
      // four waves per slab, three per SIMD: the 2176 waves of a 17408-column
      // projection are all resident, at most three (a quarter of a slab's K each) per SIMD
      launch_decode_kernel<2, false, false, 4, 3, 4, true>(ac, as, m, w, n, k, out, epi, st);
    else
      // per-tile A fetch: its registers need two waves per SIMD
      launch_decode_kernel<2, false, false, 2, 2, 4>(ac, as, m, w, n, k, out, epi, st);
  } else {
    launch_decode_kernel<1, true, false, 2, 2, 4>(ac, as, m, w, n, k, out, epi, st);
  }
}

// FP4-MFMA decode: LDS for the A records and scales (reused for the K-split
// reduction); too large a K falls back to the f16 decode kernel.
#ifndef NVFP4_DECODE_FP4_WAVES
#define NVFP4_DECODE_FP4_WAVES 4
#endif
#ifndef NVFP4_DECODE_FP4_RING
#define NVFP4_DECODE_FP4_RING 2
#endif
constexpr int kDecodeFp4Waves = NVFP4_DECODE_FP4_WAVES;
constexpr int kDecodeFp4Ring = NVFP4_DECODE_FP4_RING;
// Three workgroups per CU in gfx950's 160 KB of LDS (allocation granules
// included); eight A rows at K = 5120 take 23.7 KB.
constexpr int64_t kDecodeFp4MaxLds = 52 * 1024 + 512;
// Staged A blocks per thread on the unrolled staging path: every block of A
// for K up to 8192 (m <= 2; 6144 when the kernel quantises A) or 5120
// (m <= 8).  The quantising kernel holds the staged bf16 blocks in registers
// beside the weight ring, so its ring is shorter.
template <int MR, bool QUANT>
constexpr int decode_fp4_stage() {
  constexpr int kt_max = MR <= 2 ? (QUANT ? 96 : 128) : 80;
  constexpr int nt = kDecodeFp4Waves * 64;
  return (MR * 4 * kt_max + nt - 1) / nt;
}
template <bool QUANT>
constexpr int decode_fp4_ring() { return kDecodeFp4Ring; }

template <int MR, bool QUANT>
static bool launch_decode_fp4(const uint8_t* ac, const uint8_t* as, int64_t m, const uint8_t* w, int64_t n,
                              int64_t k, void* out, const EpilogueArgs& epi, const QuantSource& qs, hipStream_t st) {
  using L = Fp4DecodeLds<MR>;
  constexpr int DW = kDecodeFp4Waves, R = decode_fp4_ring<QUANT>();
  const int64_t ks = super_count(k), ktp = ks * kSuperTiles;
  const int64_t red = (int64_t)(DW - 1) * (MR / 2) * 64 * 4;
  int64_t lds = L::rec_bytes(ktp) + L::scale_bytes(ktp);
  if (lds < red) lds = red;
  if (lds > kDecodeFp4MaxLds) return false;
  constexpr int SP = decode_fp4_stage<MR, QUANT>();
  const bool unrolled = (int64_t)MR * 4 * ktp <= (int64_t)SP * DW * 64;
  if (QUANT && !unrolled) return false;
  const int64_t slabs = (n + kTileN - 1) / kTileN;
  const dim3 grid((unsigned)slabs), block(DW * 64);
#define NVFP4_FP4_LAUNCH(GEN, NPW)                                                                              \
  hipLaunchKernelGGL((gemm_decode_fp4_kernel<MR, DW, R, SP, QUANT, GEN, NPW>), grid, block, (unsigned)lds, st, ac, as, \
                     m, w, n, k, out, epi, qs)
  // compile-time super-tiles per wave for K = 5120 and 4096 (20 and 16 super-tiles over four waves)
  if (unrolled && ks == 5 * DW) NVFP4_FP4_LAUNCH(false, 5);
  else if (unrolled && ks == 4 * DW) NVFP4_FP4_LAUNCH(false, 4);
  else if (unrolled) NVFP4_FP4_LAUNCH(false, 0);
  else if constexpr (!QUANT) NVFP4_FP4_LAUNCH(true, 0);
#undef NVFP4_FP4_LAUNCH
  return true;
}

// The FP4 path covers plain (non-SILU) GEMMs with m <= 8 (a second, gate/up,
// slab exceeds its register budget; so do eight rows when it quantises A).
template <bool QUANT>
static bool try_decode_fp4(const uint8_t* ac, const uint8_t* as, int64_t m, const uint8_t* w, int64_t n,
                           int64_t k, void* out, const EpilogueArgs& epi, const QuantSource& qs, hipStream_t st) {
  if (epi.silu_mul) return false;
  if (m <= 2) return launch_decode_fp4<2, QUANT>(ac, as, m, w, n, k, out, epi, qs, st);
  if (m <= 4) return launch_decode_fp4<4, QUANT>(ac, as, m, w, n, k, out, epi, qs, st);
  if constexpr (!QUANT) {
    if (m <= 8) return launch_decode_fp4<8, false>(ac, as, m, w, n, k, out, epi, qs, st);
  }
  return false;
}

bool launch_gemm_decode(const uint8_t* a_codes, const uint8_t* a_scales, int64_t m, const uint8_t* w_packed,
                        int64_t n, int64_t k, void* out, const EpilogueArgs& epi, hipStream_t st) {
  const QuantSource none{};
  if (m <= 8 && try_decode_fp4<false>(a_codes, a_scales, m, w_packed, n, k, out, epi, none, st)) return true;
  // The f16 decode kernel moves A in 16-byte chunks (32 elements): K % 32 == 16
  // runs the register-staged tile kernel, which reads A per 16-element block.
  if (m > 64 || k % 32 != 0) return false;
  // and addresses each weight slab through a buffer descriptor with a 32-bit range
  if (super_count(k) * kSuperBytes >= (int64_t(1) << 31)) return false;
  if (m <= 32) {
    if (epi.silu_mul) launch_decode<1, true>(a_codes, a_scales, m, w_packed, n, k, out, epi, st);
    else launch_decode<1, false>(a_codes, a_scales, m, w_packed, n, k, out, epi, st);
  } else {
    if (epi.silu_mul) launch_decode<2, true>(a_codes, a_scales, m, w_packed, n, k, out, epi, st);
    else launch_decode<2, false>(a_codes, a_scales, m, w_packed, n, k, out, epi, st);
  }
  return true;
}

bool launch_gemm_decode_quantize(const QuantSource& qs, int64_t m, const uint8_t* w_packed, int64_t n, int64_t k,
                                 void* out, const EpilogueArgs& epi, hipStream_t st) {
  // m <= 2 only: the four-row kernel's staged bf16 blocks do not fit its registers
  return m <= 2 && !epi.silu_mul && launch_decode_fp4<2, true>(qs.codes, qs.scales, m, w_packed, n, k, out, epi, qs, st);
}
}  // namespace nvfp4
