// Gated delta-rule recurrence of a Gated DeltaNet layer on gfx950: the
// second workload of the path, fed by the fused in-projection (its q, k, v
// columns and the sigmoid / decay gate columns).  The pages give the rule's
// behaviour, not a formula -- a write replaces the state's component along
// the key (bayesiansapien page, "The four-part mechanism study", third
// item); per value head h, with key head h / (Hv / Hk) and state S [128, 128]
// (row = value index, column = key index):
//     k^ = k / sqrt(|k|^2 + 1e-6),  q^ likewise,  alpha = exp(g),
//     u = alpha S k^,  c = beta (v - u),  S <- alpha S + c k^T,  o = S q^.
// Since the dot products are taken on the state before the step,
//     u_i = alpha (S_i . k^),  o_i = alpha (S_i . q^) + c_i (k^ . q^),
// both dots of a row come from one pass over the old state.
//
// Scaled state: within a segment of 8 steps the registers hold S^ = S / A,
// A = the product of the segment's decays so far, so that a step is
//     u = A (S^ . k^),  c = beta (v - u),  o = A (S^ . q^) + c (k^ . q^),
//     S^ <- S^ + (c / A) k^,
// one multiply-add per element instead of a multiply and a multiply-add; at
// the segment's end S = A S^ is restored.  The stage holds beta v (exact: both
// are bf16) and beta A, so the write coefficient c = beta v - (beta A)(S^.k^)
// is a single multiply-add (likewise beta alpha for the unscaled update).  Floating point being scale-free,
// this changes only which products are rounded: the state's effective decay
// per step is the ratio of two consecutive rounded A, within a few units of
// roundoff of alpha.  A chunk whose decays all lie in [2^-12, 2^12] keeps A
// and 1 / A within [2^-96, 2^96]; any other chunk (a near-total reset, a
// growing gate, NaN) runs the unscaled update.
//
// Work split: the recurrence is sequential in time and independent per state
// row, so a workgroup owns 32 rows of one head's state in registers for the
// whole sequence (4 workgroups per head, 8 waves each: with 48 heads one
// workgroup per CU and two waves per SIMD, and each head's keys and queries
// normalised by 4 workgroups rather than 8).  16 lanes share a row, each holding
// 8 of its 128 columns (4j..4j+3 and 64+4j..64+4j+3 for lane j, so the 16
// lanes' 16-byte LDS reads of a key are contiguous); the row's dot products
// are summed across those lanes with DPP.  Inputs are staged 64 time steps at
// a time (155 KB of LDS for both buffers; a workgroup of 8 waves at this
// register count holds a CU alone anyway) through double-buffered LDS, which
// halves the chunk-boundary barriers of 32-step chunks: while a chunk is being consumed the
// next one is loaded into registers, then converted -- keys and queries to
// normalised fp32 (their norms reduced once per step per workgroup), gates to
// (alpha, beta, k^.q^, A, 1/A) -- and written to the other buffer; within a
// chunk each step's LDS operands are read during the step before.  ALU-bound:
// about 7 * 128^2 flops per head per token.  (Layouts with one wave per SIMD
// -- 8 lanes x 16 columns per row, or two rows per lane -- balance the SIMDs
// at 48 heads but issue less well from a lone wave and measured slower.)
#include <type_traits>

#include "kernels.h"
#include "nvfp4_device.h"

namespace nvfp4 {

namespace {

constexpr int kD = 128;          // key and value dimension of a head
constexpr int kRows = 32;        // state rows per workgroup
constexpr int kThreads = 16 * kRows;   // 4 rows x 16 lanes per wave
constexpr int kChunk = 64;       // time steps per LDS stage
constexpr int kSeg = 8;          // time steps per segment of the scaled state
constexpr float kRangeLo = 0x1p-12f, kRangeHi = 0x1p12f;   // decays that keep A within [2^-96, 2^96]
static_assert(kChunk % kSeg == 0 && (kSeg & (kSeg - 1)) == 0, "segments tile a chunk");
// Staging maps: key/query pieces (8 bf16) are 16 per step, kThreads / 16
// steps per pass; value rows move 8 bf16 per item; outputs are two per thread.
constexpr int kStepsPerPass = kThreads / 16;
constexpr int kKqPasses = kChunk / kStepsPerPass;
constexpr int kVParts = kRows / 8;
static_assert(kChunk % kStepsPerPass == 0 && kRows % 8 == 0 && kChunk * kVParts <= kThreads, "staging maps");
constexpr int kOutPerThread = kChunk * kRows / kThreads, kOutStepStride = kThreads / kRows;
static_assert(kChunk * kRows % kThreads == 0, "outputs per thread");
constexpr float kNormEps = 1e-6f;

struct Stage {
  float kn[kChunk][kD];     // normalised keys
  float qn[kChunk][kD];     // normalised queries
  float v[kChunk][kRows];   // beta times this workgroup's value rows (exact: both are bf16)
  float4 gs[kChunk];        // scaled update: A (decay product since the step's 8-step segment began), 1 / A, beta A, k^ . q^
  float4 gu[kChunk];        // plain update: alpha, beta alpha, k^ . q^, unused
  int scaled;               // every decay of the chunk within [2^-12, 2^12]
};

__device__ __forceinline__ float bf16f(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
// Sum over the 16 lanes of a DPP row; every lane gets the same bits (each
// step adds the same two values in either order).
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp<0xB1>(x);    // quad_perm [1, 0, 3, 2]
  x += dpp<0x4E>(x);    // quad_perm [2, 3, 0, 1]
  x += dpp<0x141>(x);   // row_half_mirror
  x += dpp<0x140>(x);   // row_mirror
  return x;
}

// Registers holding one chunk's raw inputs between its global loads and its
// conversion into a Stage.  Thread t carries key and query pieces (8 bf16) of
// steps t/16 + p * kStepsPerPass, piece t%16; threads < kChunk * kVParts 8
// bf16 of a value row (step t / kVParts, part t % kVParts); threads < kChunk
// the two gates of step t.
struct Raw {
  uint4 k[kKqPasses], q[kKqPasses], v;
  uint32_t beta, g, vbeta;   // vbeta: the write strength of the value item's step
};

}  // namespace

__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 2)))
gdn_recurrence_kernel(GdnArgs a) {
  __shared__ Stage st[2];
  __shared__ float obuf[kChunk][kRows];
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int lr = lane & 15;                     // lane within the row
  const int rloc = wave * 4 + (lane >> 4);      // row within the workgroup
  const int groups = kD / kRows;
  const int h = blockIdx.x / groups;
  const int i0 = (blockIdx.x % groups) * kRows;
  const int hk = h / (a.hv / a.hk);
  const int64_t T = a.T;
  const int64_t nchunks = (T + kChunk - 1) / kChunk;

  const int c0 = 4 * lr, c1 = 64 + 4 * lr;      // this lane's columns
  float s[8];
  if (a.s_init) {
    const float* p = a.s_init + ((int64_t)h * kD + i0 + rloc) * kD;
    const float4 x = *reinterpret_cast<const float4*>(p + c0), y = *reinterpret_cast<const float4*>(p + c1);
    s[0] = x.x; s[1] = x.y; s[2] = x.z; s[3] = x.w; s[4] = y.x; s[5] = y.y; s[6] = y.z; s[7] = y.w;
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) s[j] = 0.0f;
  }

  // Loop-invariant parts of this thread's element offsets; a chunk adds its
  // first step times the leading dimension (a workgroup-uniform value).
  const int64_t koff = (int64_t)(t >> 4) * a.ld_k + hk * kD + 8 * (t & 15);
  const int64_t qoff = (int64_t)(t >> 4) * a.ld_q + hk * kD + 8 * (t & 15);
  const int64_t voff = (int64_t)(t / kVParts) * a.ld_v + (int64_t)h * kD + i0 + 8 * (t % kVParts);
  const int64_t boff = (int64_t)t * a.ld_beta + h, goff = (int64_t)t * a.ld_g + h;
  const int64_t vboff = (int64_t)(t / kVParts) * a.ld_beta + h;
  auto load = [&](int64_t chunk, Raw& R) __attribute__((always_inline)) {
    const int64_t t0 = chunk * kChunk;
    if (t0 + kChunk <= T) {
#pragma unroll
      for (int p = 0; p < kKqPasses; ++p) {
        R.k[p] = *reinterpret_cast<const uint4*>(a.k + (t0 + kStepsPerPass * p) * a.ld_k + koff);
        R.q[p] = *reinterpret_cast<const uint4*>(a.q + (t0 + kStepsPerPass * p) * a.ld_q + qoff);
      }
      if (t < kChunk * kVParts) {
        R.v = *reinterpret_cast<const uint4*>(a.v + t0 * a.ld_v + voff);
        R.vbeta = a.beta[t0 * a.ld_beta + vboff];
      }
      if (t < kChunk) {
        R.beta = a.beta[t0 * a.ld_beta + boff];
        R.g = a.g[t0 * a.ld_g + goff];
      }
      return;
    }
    // the last, partial chunk: steps past the end read the last step again
#pragma unroll
    for (int p = 0; p < kKqPasses; ++p) {
      int64_t step = t0 + p * kStepsPerPass + (t >> 4);
      step = step < T ? step : T - 1;
      const int col = hk * kD + 8 * (t & 15);
      R.k[p] = *reinterpret_cast<const uint4*>(a.k + step * a.ld_k + col);
      R.q[p] = *reinterpret_cast<const uint4*>(a.q + step * a.ld_q + col);
    }
    if (t < kChunk * kVParts) {
      int64_t step = t0 + t / kVParts;
      step = step < T ? step : T - 1;
      R.v = *reinterpret_cast<const uint4*>(a.v + step * a.ld_v + (int64_t)h * kD + i0 + 8 * (t % kVParts));
      R.vbeta = a.beta[step * a.ld_beta + h];
    }
    if (t < kChunk) {
      int64_t step = t0 + t;
      step = step < T ? step : T - 1;
      R.beta = a.beta[step * a.ld_beta + h];
      R.g = a.g[step * a.ld_g + h];
    }
  };
  auto unpack8 = [](const uint4& u, float (&f)[8]) __attribute__((always_inline)) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[2 * e] = bf16f(w[e] & 0xFFFFu);
      f[2 * e + 1] = bf16f(w[e] >> 16);
    }
  };
  auto store = [&](const Raw& R, Stage& S) __attribute__((always_inline)) {
#pragma unroll
    for (int p = 0; p < kKqPasses; ++p) {
      const int step = p * kStepsPerPass + (t >> 4), pc = t & 15;
      float kf[8], qf[8];
      unpack8(R.k[p], kf);
      unpack8(R.q[p], qf);
      float kk = 0.0f, qq = 0.0f, kq = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        kk = fmaf(kf[e], kf[e], kk);
        qq = fmaf(qf[e], qf[e], qq);
        kq = fmaf(kf[e], qf[e], kq);
      }
      kk = row_sum16(kk);
      qq = row_sum16(qq);
      kq = row_sum16(kq);
      // hardware reciprocal square root (within 1 ulp; the sums are >= eps, normal)
      const float nk = __builtin_amdgcn_rsqf(kk + kNormEps), nq = __builtin_amdgcn_rsqf(qq + kNormEps);
      float4* kd = reinterpret_cast<float4*>(&S.kn[step][8 * pc]);
      float4* qd = reinterpret_cast<float4*>(&S.qn[step][8 * pc]);
      kd[0] = make_float4(kf[0] * nk, kf[1] * nk, kf[2] * nk, kf[3] * nk);
      kd[1] = make_float4(kf[4] * nk, kf[5] * nk, kf[6] * nk, kf[7] * nk);
      qd[0] = make_float4(qf[0] * nq, qf[1] * nq, qf[2] * nq, qf[3] * nq);
      qd[1] = make_float4(qf[4] * nq, qf[5] * nq, qf[6] * nq, qf[7] * nq);
      if (pc == 0) {
        const float kqn = kq * nk * nq;
        S.gs[step].w = kqn;
        S.gu[step].z = kqn;
      }
    }
    if (t < kChunk * kVParts) {
      float vf[8];
      unpack8(R.v, vf);
      const float bv = bf16f(R.vbeta & 0xFFFFu);
      float4* vd = reinterpret_cast<float4*>(&S.v[t / kVParts][8 * (t % kVParts)]);
      vd[0] = make_float4(vf[0] * bv, vf[1] * bv, vf[2] * bv, vf[3] * bv);
      vd[1] = make_float4(vf[4] * bv, vf[5] * bv, vf[6] * bv, vf[7] * bv);
    }
    if (t < kChunk) {
      const float alpha = expf(bf16f(R.g & 0xFFFFu));
      const float beta = bf16f(R.beta & 0xFFFFu);
      S.gu[t].x = alpha;
      S.gu[t].y = beta * alpha;
      // product of the decays from the segment's first step to this one
      float A = alpha;
#pragma unroll
      for (int off = 1; off < kSeg; off <<= 1) {
        const float y = __shfl_up(A, off, kSeg);
        if ((t & (kSeg - 1)) >= off) A *= y;
      }
      S.gs[t].x = A;
      S.gs[t].y = __builtin_amdgcn_rcpf(A);      // within 1 ulp
      S.gs[t].z = beta * A;
      const bool in_range = alpha >= kRangeLo && alpha <= kRangeHi;    // false for NaN
      const uint64_t out = __ballot(!in_range);
      if (t == 0) S.scaled = out == 0;
    }
  };

  const int64_t ooff = (int64_t)(t / kRows) * a.ld_o + (int64_t)h * kD + i0 + (t % kRows);
  Raw R;
  load(0, R);
  store(R, st[0]);
  __syncthreads();
  for (int64_t c = 0; c < nchunks; ++c) {
    if (c + 1 < nchunks) load(c + 1, R);
    const Stage& S = st[c & 1];
    const int cnt = (int)(T - c * kChunk < kChunk ? T - c * kChunk : kChunk);
    // One time step for this lane's eight state elements, scaled (S^ = S / A)
    // or not.  Every lane of a row holds the row's output (identical bits), so
    // all of them write it.
    struct In { float4 ka, kb, qa, qb, g; float vi; };
    auto fetch = [&](int step, auto scaled_tag) __attribute__((always_inline)) {
      In x;
      x.ka = reinterpret_cast<const float4*>(S.kn[step])[lr];
      x.kb = reinterpret_cast<const float4*>(S.kn[step])[16 + lr];
      x.qa = reinterpret_cast<const float4*>(S.qn[step])[lr];
      x.qb = reinterpret_cast<const float4*>(S.qn[step])[16 + lr];
      x.g = decltype(scaled_tag)::value ? S.gs[step] : S.gu[step];
      x.vi = S.v[step][rloc];
      return x;
    };
    auto compute = [&](int step, const In& x, auto scaled_tag) __attribute__((always_inline)) {
      constexpr bool kScaled = decltype(scaled_tag)::value;
      const float4 ka = x.ka, kb = x.kb, qa = x.qa, qb = x.qb, g = x.g;
      const float bvi = x.vi;           // beta v
      float sk0 = s[0] * ka.x, sq0 = s[0] * qa.x;
      sk0 = fmaf(s[1], ka.y, sk0); sq0 = fmaf(s[1], qa.y, sq0);
      sk0 = fmaf(s[2], ka.z, sk0); sq0 = fmaf(s[2], qa.z, sq0);
      sk0 = fmaf(s[3], ka.w, sk0); sq0 = fmaf(s[3], qa.w, sq0);
      sk0 = fmaf(s[4], kb.x, sk0); sq0 = fmaf(s[4], qb.x, sq0);
      sk0 = fmaf(s[5], kb.y, sk0); sq0 = fmaf(s[5], qb.y, sq0);
      sk0 = fmaf(s[6], kb.z, sk0); sq0 = fmaf(s[6], qb.z, sq0);
      sk0 = fmaf(s[7], kb.w, sk0); sq0 = fmaf(s[7], qb.w, sq0);
      const float sk = row_sum16(sk0), sq = row_sum16(sq0);
      const float kv[8] = {ka.x, ka.y, ka.z, ka.w, kb.x, kb.y, kb.z, kb.w};
      if constexpr (kScaled) {
        // g = (A, 1/A, beta A, k^.q^): c = beta v - beta A (S^.k^)
        const float cw = fmaf(-g.z, sk, bvi);
        obuf[step][rloc] = fmaf(g.x, sq, cw * g.w);
        const float d = cw * g.y;
#pragma unroll
        for (int j = 0; j < 8; ++j) s[j] = fmaf(d, kv[j], s[j]);
        if ((step & (kSeg - 1)) == kSeg - 1) {
#pragma unroll
          for (int j = 0; j < 8; ++j) s[j] *= g.x;
        }
      } else {
        // g = (alpha, beta alpha, k^.q^, -): c = beta v - beta alpha (S.k^)
        const float alpha = g.x;
        const float cw = fmaf(-g.y, sk, bvi);
        obuf[step][rloc] = fmaf(alpha, sq, cw * g.z);
#pragma unroll
        for (int j = 0; j < 8; ++j) s[j] = fmaf(alpha, s[j], cw * kv[j]);
      }
    };
    auto run_full = [&](auto scaled_tag) __attribute__((always_inline)) {
      In cur = fetch(0, scaled_tag);
#pragma unroll
      for (int step = 0; step < kChunk; ++step) {
        In nxt;
        if (step + 1 < kChunk) nxt = fetch(step + 1, scaled_tag);
        asm volatile("" ::: "memory");
        compute(step, cur, scaled_tag);
        cur = nxt;
      }
    };
    if (cnt == kChunk && __builtin_amdgcn_readfirstlane(S.scaled)) {
      run_full(std::true_type{});
    } else if (cnt == kChunk) {
      run_full(std::false_type{});
    } else {
      for (int step = 0; step < cnt; ++step) compute(step, fetch(step, std::false_type{}), std::false_type{});
    }
    __syncthreads();
    if (c + 1 < nchunks) store(R, st[(c + 1) & 1]);
    // this chunk's outputs: kChunk x kRows values, two per thread (steps
    // t/kRows and kChunk/2 + t/kRows, row t%kRows)
#pragma unroll
    for (int e = 0; e < kOutPerThread; ++e) {
      const int step = t / kRows + kOutStepStride * e, r = t % kRows;
      if (step < cnt) {
        const int64_t off = (c * kChunk + kOutStepStride * e) * a.ld_o + ooff;
        const float val = obuf[step][r];
        if (a.o_bf16) reinterpret_cast<uint16_t*>(a.o)[off] = f32_to_bf16_rne(val);
        else reinterpret_cast<float*>(a.o)[off] = val;
      }
    }
    __syncthreads();
  }
  if (a.s_final) {
    float* p = a.s_final + ((int64_t)h * kD + i0 + rloc) * kD;
    *reinterpret_cast<float4*>(p + c0) = make_float4(s[0], s[1], s[2], s[3]);
    *reinterpret_cast<float4*>(p + c1) = make_float4(s[4], s[5], s[6], s[7]);
  }
}

hipError_t launch_gdn_recurrence(const GdnArgs& a, hipStream_t st) {
  const unsigned blocks = (unsigned)(a.hv * (kD / kRows));
  hipLaunchKernelGGL(gdn_recurrence_kernel, dim3(blocks), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace nvfp4
