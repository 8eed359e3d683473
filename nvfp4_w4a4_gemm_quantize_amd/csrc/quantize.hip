// NVFP4 quantizer kernels for gfx950: per-tensor / per-segment amax, the
// activation quantizer (bf16 -> E2M1 codes + one E4M3 scale per 16 elements;
// bayesiansapien page, "The four-part mechanism study", first item) and the
// weight packer with one global scale per fused module (same page, "Two
// practical repairs").
//
// Memory-bound kernels: every thread moves whole 16-element blocks with
// 16-byte loads (32 B of bf16 in, 8 B of codes + 1 B of scale out), the amax
// is reduced inside a wavefront with cross-lane shuffles and across waves in
// LDS, and partial maxima from many workgroups are combined by a one-block
// finalize kernel in a fixed order (no atomics: results are bit-reproducible).
#include "kernels.h"
#include "nvfp4_device.h"

namespace nvfp4 {

constexpr int kThreads = 256;

// ------------------------------------------------------------ amax ----
// Workgroup-wide max of a per-thread value (all threads must call).
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, uint32_t* lds) {
  v = wave_max_u32(v);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) lds[wave] = v;
  __syncthreads();
  uint32_t r = 0;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) r = max(r, lds[w]);
  __syncthreads();
  return r;
}

// Partial maxima of |x| (as 15-bit bf16 magnitude patterns) over rows
// [row0, row1) of a bf16 matrix; workgroup (b, seg) writes partial[seg * gx + b].
__global__ void __launch_bounds__(kThreads)
amax_partial_kernel(const uint16_t* __restrict__ x, int64_t cols, int64_t ld, SegmentTable segs,
                    uint32_t* __restrict__ partial) {
  __shared__ uint32_t lds[kThreads / 64];
  const int seg = blockIdx.y;
  const int64_t row0 = segs.off[seg], row1 = segs.off[seg + 1];
  const int64_t vpr = cols >> 3;                     // 8 bf16 per 16-byte vector
  const int64_t nvec = (row1 - row0) * vpr;
  uint32_t m = 0;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < nvec;
       i += (int64_t)gridDim.x * kThreads) {
    const int64_t r = row0 + i / vpr, c = (i % vpr) << 3;
    uint4 v = *reinterpret_cast<const uint4*>(x + r * ld + c);
    m = max(m, absmax_bits8(v));
  }
  m = block_max_u32(m, lds);
  if (threadIdx.x == 0) partial[(int64_t)seg * gridDim.x + blockIdx.x] = m;
}

// g[seg] = 2688 / amax (1 if amax == 0) from `parts` partials per segment.
__global__ void __launch_bounds__(kThreads)
amax_finalize_kernel(const uint32_t* __restrict__ partial, int parts, int nseg, float* __restrict__ g) {
  __shared__ uint32_t lds[kThreads / 64];
  for (int s = 0; s < nseg; ++s) {
    uint32_t m = 0;
    for (int i = threadIdx.x; i < parts; i += kThreads) m = max(m, partial[s * parts + i]);
    m = block_max_u32(m, lds);
    if (threadIdx.x == 0) {
      float amax = __uint_as_float(m << 16);
      g[s] = amax > 0.0f ? kGlobalNumerator / amax : 1.0f;
    }
  }
}

// --------------------------------------------------------- quantize ----
// One thread per 16-element block, grid-stride.  Rows are [rows, cols] with
// stride ld; codes [rows, cols/2] and scales [rows, cols/16] are contiguous.
__global__ void __launch_bounds__(kThreads)
quantize_kernel(const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld,
                const float* __restrict__ gptr, uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const float g = *gptr;
  const int64_t bpr = cols >> 4;
  const int64_t nblk = rows * bpr;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < nblk;
       i += (int64_t)gridDim.x * kThreads) {
    const int64_t r = i / bpr, b = i % bpr;
    const uint4* src = reinterpret_cast<const uint4*>(x + r * ld + (b << 4));
    uint4 lo = src[0], hi = src[1];
    uint2 c;
    uint32_t S = quantize_block16(lo, hi, g, &c);
    *reinterpret_cast<uint2*>(codes + i * 8) = c;
    scales[i] = (uint8_t)S;
  }
}

// Whole small tensor in one workgroup: amax, g, then the blocks.  Saves two
// launches for decode-sized activations.  Every thread loads all its blocks
// (at most kSmallBlocksPerThread) at once and keeps them in registers for
// the quantisation, so the tensor crosses memory once, in one round trip.
constexpr int kSmallThreads = 1024;
constexpr int kSmallBlocksPerThread = 4;      // 65,536 elements in 16-element blocks over 1024 threads
__global__ void __launch_bounds__(kSmallThreads)
quantize_small_dynamic_kernel(const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld,
                              float* __restrict__ gout, uint8_t* __restrict__ codes,
                              uint8_t* __restrict__ scales) {
  __shared__ uint32_t lds[kSmallThreads / 64];
  const uint32_t bpr = (uint32_t)(cols >> 4), nblk = (uint32_t)rows * bpr;
  uint4 lo[kSmallBlocksPerThread], hi[kSmallBlocksPerThread];
  uint32_t m = 0;
#pragma unroll
  for (int j = 0; j < kSmallBlocksPerThread; ++j) {
    // unconditional loads (past the end: the last block again, left out of the max)
    const uint32_t q = min(threadIdx.x + (uint32_t)j * kSmallThreads, nblk - 1);
    const uint4* src = reinterpret_cast<const uint4*>(x + (int64_t)(q / bpr) * ld + ((q % bpr) << 4));
    lo[j] = src[0];
    hi[j] = src[1];
  }
#pragma unroll
  for (int j = 0; j < kSmallBlocksPerThread; ++j)
    if (threadIdx.x + (uint32_t)j * kSmallThreads < nblk) m = max(m, max(absmax_bits8(lo[j]), absmax_bits8(hi[j])));
  m = block_max_u32(m, lds);
  const float amax = __uint_as_float(m << 16);
  const float g = amax > 0.0f ? kGlobalNumerator / amax : 1.0f;
  if (threadIdx.x == 0) *gout = g;
#pragma unroll
  for (int j = 0; j < kSmallBlocksPerThread; ++j) {
    const uint32_t q = threadIdx.x + (uint32_t)j * kSmallThreads;
    if (q < nblk) {
      uint2 c;
      const uint32_t S = quantize_block16(lo[j], hi[j], g, &c);
      *reinterpret_cast<uint2*>(codes + (int64_t)q * 8) = c;
      scales[q] = (uint8_t)S;
    }
  }
}

// ------------------------------------------------------------ packer ----
__device__ __forceinline__ int segment_of(const SegmentTable& t, int64_t row) {
  int s = 0;
  while (s + 1 < t.num && row >= t.off[s + 1]) ++s;
  return s;
}

// One thread per (row, 16-block) of the padded [Np, Kp] weight: quantise with
// the row's segment scale (zeros in the padding) and scatter into the tiles.
__global__ void __launch_bounds__(kThreads)
pack_kernel(const uint16_t* __restrict__ w, int64_t n, int64_t k, int64_t np, int64_t kp,
            SegmentTable segs, const float* __restrict__ seg_g, uint8_t* __restrict__ packed) {
  const int64_t bpr = kp >> 4;
  const int64_t ks = kp / kSuperK;
  const int64_t total = np * bpr;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * kThreads) {
    const int64_t row = i / bpr, b = i % bpr;
    uint2 c = make_uint2(0u, 0u);
    uint32_t S = 0;
    if (row < n && (b << 4) < k) {
      const float g = seg_g[segment_of(segs, row)];
      const uint4* src = reinterpret_cast<const uint4*>(w + row * k + (b << 4));
      S = quantize_block16(src[0], src[1], g, &c);
    }
    const int64_t nt = row / kTileN, cc = row % kTileN;
    const int64_t kt = b >> 2, bin = b & 3;        // block within the 64-wide tile
    const int64_t lane = cc + kTileN * (bin >> 1);
    *reinterpret_cast<uint2*>(packed + tile_code_off(nt, kt, ks) + lane * 16 + (bin & 1) * 8) = c;
    packed[tile_scale_off(nt, kt, ks, cc) + bin] = (uint8_t)S;
  }
}

__global__ void __launch_bounds__(kThreads)
unpack_kernel(const uint8_t* __restrict__ packed, int64_t n, int64_t k, int64_t np, int64_t kp,
              uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int64_t bpr = k >> 4;
  const int64_t ks = kp / kSuperK;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n * bpr;
       i += (int64_t)gridDim.x * kThreads) {
    const int64_t row = i / bpr, b = i % bpr;
    const int64_t nt = row / kTileN, cc = row % kTileN;
    const int64_t kt = b >> 2, bin = b & 3;
    const int64_t lane = cc + kTileN * (bin >> 1);
    *reinterpret_cast<uint2*>(codes + row * (k / 2) + b * 8) =
        *reinterpret_cast<const uint2*>(packed + tile_code_off(nt, kt, ks) + lane * 16 + (bin & 1) * 8);
    scales[row * bpr + b] = packed[tile_scale_off(nt, kt, ks, cc) + bin];
  }
}

// ------------------------------------------------------ E2M1 encoder ----
// The quantizer's E2M1 encoder applied to caller-given FP32 values, one code
// (0..15) per byte: exposes the exact device routine for verification.
// Values 2j and 2j+1 share one conversion (operand slots a and b), written to
// byte position j % 4, so every slot and position the quantizer uses is run.
__global__ void __launch_bounds__(kThreads)
e2m1_encode_kernel(const float* __restrict__ q, int64_t n, uint8_t* __restrict__ codes) {
  const int64_t pairs = (n + 1) / 2;
  for (int64_t j = (int64_t)blockIdx.x * kThreads + threadIdx.x; j < pairs; j += (int64_t)gridDim.x * kThreads) {
    const float a = q[2 * j], b = 2 * j + 1 < n ? q[2 * j + 1] : 0.0f;
    uint32_t w;
    switch (j & 3) {
      case 0: w = e2m1_pair<0>(0u, a, b); break;
      case 1: w = e2m1_pair<1>(0u, a, b) >> 8; break;
      case 2: w = e2m1_pair<2>(0u, a, b) >> 16; break;
      default: w = e2m1_pair<3>(0u, a, b) >> 24; break;
    }
    codes[2 * j] = (uint8_t)(w & 0xFu);
    if (2 * j + 1 < n) codes[2 * j + 1] = (uint8_t)((w >> 4) & 0xFu);
  }
}

// ---------------------------------------------------------- launchers ----
static int grid_for(int64_t items, int64_t cap) {
  int64_t g = (items + kThreads - 1) / kThreads;
  if (g > cap) g = cap;
  return (int)(g < 1 ? 1 : g);
}

constexpr int64_t kSmallElems = (int64_t)kSmallThreads * kSmallBlocksPerThread * 16;   // one-workgroup dynamic path
constexpr int kMaxPartials = 1024;

hipError_t launch_quantize(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, float* g,
                           bool dynamic, uint8_t* codes, uint8_t* scales, hipStream_t st) {
  const int64_t nblk = rows * (cols / 16);
  if (dynamic && rows * cols <= kSmallElems) {
    hipLaunchKernelGGL(quantize_small_dynamic_kernel, dim3(1), dim3(kSmallThreads), 0, st,
                       x, rows, cols, ld, g, codes, scales);
    return hipGetLastError();
  }
  if (dynamic) {
    // Partials live in the codes buffer (rows*cols/2 bytes), overwritten later.
    int64_t cap = (rows * cols / 2) / 4;
    int parts = grid_for(rows * cols / 8, kMaxPartials);
    if (parts > cap) parts = (int)cap;
    SegmentTable one{};
    one.num = 1;
    one.off[0] = 0;
    one.off[1] = rows;
    uint32_t* partial = reinterpret_cast<uint32_t*>(codes);
    hipLaunchKernelGGL(amax_partial_kernel, dim3(parts, 1), dim3(kThreads), 0, st, x, cols, ld, one, partial);
    hipLaunchKernelGGL(amax_finalize_kernel, dim3(1), dim3(kThreads), 0, st, partial, parts, 1, g);
  }
  hipLaunchKernelGGL(quantize_kernel, dim3(grid_for(nblk, 8192)), dim3(kThreads), 0, st,
                     x, rows, cols, ld, g, codes, scales);
  return hipGetLastError();
}

hipError_t launch_amax_partials(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, uint32_t* parts,
                                int nparts, hipStream_t st) {
  SegmentTable one{};
  one.num = 1;
  one.off[0] = 0;
  one.off[1] = rows;
  hipLaunchKernelGGL(amax_partial_kernel, dim3(nparts, 1), dim3(kThreads), 0, st, x, cols, ld, one, parts);
  return hipGetLastError();
}

hipError_t launch_quantize_from_parts(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld,
                                      const uint32_t* parts, int64_t nparts, float* g, uint8_t* codes,
                                      uint8_t* scales, hipStream_t st) {
  hipLaunchKernelGGL(amax_finalize_kernel, dim3(1), dim3(kThreads), 0, st, parts, (int)nparts, 1, g);
  const int64_t nblk = rows * (cols / 16);
  hipLaunchKernelGGL(quantize_kernel, dim3(grid_for(nblk, 8192)), dim3(kThreads), 0, st,
                     x, rows, cols, ld, g, codes, scales);
  return hipGetLastError();
}

hipError_t launch_pack(const uint16_t* w, int64_t n, int64_t k, const SegmentTable& segs, float* seg_g,
                       bool dynamic, uint8_t* packed, hipStream_t st) {
  const int64_t np = round_up(n, kTileN), kp = round_up(k, kSuperK);
  if (dynamic) {
    // Partials in the packed buffer (>= 1152 bytes), overwritten by the pack.
    int64_t cap = (np * kp / 2) / 4 / segs.num;
    int parts = (int)(cap < 256 ? cap : 256);
    uint32_t* partial = reinterpret_cast<uint32_t*>(packed);
    hipLaunchKernelGGL(amax_partial_kernel, dim3(parts, segs.num), dim3(kThreads), 0, st,
                       w, k, k, segs, partial);
    hipLaunchKernelGGL(amax_finalize_kernel, dim3(1), dim3(kThreads), 0, st, partial, parts, segs.num, seg_g);
  }
  hipLaunchKernelGGL(pack_kernel, dim3(grid_for(np * (kp / 16), 16384)), dim3(kThreads), 0, st,
                     w, n, k, np, kp, segs, seg_g, packed);
  return hipGetLastError();
}

hipError_t launch_unpack(const uint8_t* packed, int64_t n, int64_t k, uint8_t* codes, uint8_t* scales,
                         hipStream_t st) {
  const int64_t np = round_up(n, kTileN), kp = round_up(k, kSuperK);
  hipLaunchKernelGGL(unpack_kernel, dim3(grid_for(n * (k / 16), 16384)), dim3(kThreads), 0, st,
                     packed, n, k, np, kp, codes, scales);
  return hipGetLastError();
}

hipError_t launch_e2m1_encode(const float* q, int64_t n, uint8_t* codes, hipStream_t st) {
  hipLaunchKernelGGL(e2m1_encode_kernel, dim3(grid_for((n + 1) / 2, 8192)), dim3(kThreads), 0, st, q, n, codes);
  return hipGetLastError();
}

}  // namespace nvfp4
