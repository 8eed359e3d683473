// Host-only check of the C ABI layer (abi.cpp + validate.cpp), built by
// tests/test_abi_cpu.py with AddressSanitizer and UndefinedBehaviorSanitizer
// and no GPU code: the kernel launchers are replaced here by stubs that
// record each call.  Every case calls an entry point with fake device
// addresses and checks the status it returns, that a rejected call reaches no
// launcher, and that an accepted one reaches the right launcher with the
// arguments the header documents (segment table, per-segment gates, SiLU*mul
// and output flags).  Prints "abi host check: N cases ok" and exits 0, or
// names the first failing case and exits 1.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../include/nvfp4.h"
#include "../nvfp4_w4a4_gemm_quantize_amd/csrc/kernels.h"

namespace {

struct Call {
  const char* fn = nullptr;
  int count = 0;
  int64_t m = -1, n = -1, k = -1, rows = -1, cols = -1;
  bool dynamic = false;
  nvfp4::EpilogueArgs epi{};
  nvfp4::SegmentTable segs{};
  nvfp4::GdnArgs gdn{};
};
Call g_call;

void record(const char* fn) {
  g_call.fn = fn;
  g_call.count++;
}

int g_cases = 0;
void fail(const char* what, int line) {
  fprintf(stderr, "abi host check FAILED at line %d: %s\n", line, what);
  exit(1);
}
#define CHECK(cond) \
  do {              \
    if (!(cond)) fail(#cond, __LINE__); \
  } while (0)

// Expect status `want` and, for a launch, exactly one call of launcher `fn`
// (fn == nullptr: no launcher may be reached).
void expect(int rc, int want, const char* fn, const char* what, int line) {
  ++g_cases;
  if (rc != want) {
    fprintf(stderr, "status %d, expected %d\n", rc, want);
    fail(what, line);
  }
  const bool ok = fn == nullptr ? g_call.count == 0 : g_call.count == 1 && strcmp(g_call.fn, fn) == 0;
  if (!ok) fail(what, line);
}
#define EXPECT(call, want, fn) expect((g_call = Call{}, (call)), (want), (fn), #call, __LINE__)

void* const A16 = reinterpret_cast<void*>(0x10000);   // a 16-byte aligned fake device address
void* const MIS = reinterpret_cast<void*>(0x10004);   // a misaligned one
const char* const NONE = nullptr;

}  // namespace

// ------------------------------------------------------ launcher stubs ----
namespace nvfp4 {
hipError_t launch_quantize(const uint16_t*, int64_t rows, int64_t cols, int64_t, float*, bool dynamic, uint8_t*,
                           uint8_t*, hipStream_t) {
  record("quantize");
  g_call.rows = rows;
  g_call.cols = cols;
  g_call.dynamic = dynamic;
  return hipSuccess;
}
hipError_t launch_e2m1_encode(const float*, int64_t n, uint8_t*, hipStream_t) {
  record("e2m1");
  g_call.n = n;
  return hipSuccess;
}
hipError_t launch_pack(const uint16_t*, int64_t n, int64_t k, const SegmentTable& segs, float*, bool dynamic,
                       uint8_t*, hipStream_t) {
  record("pack");
  g_call.n = n;
  g_call.k = k;
  g_call.segs = segs;
  g_call.dynamic = dynamic;
  return hipSuccess;
}
hipError_t launch_unpack(const uint8_t*, int64_t n, int64_t k, uint8_t*, uint8_t*, hipStream_t) {
  record("unpack");
  g_call.n = n;
  g_call.k = k;
  return hipSuccess;
}
hipError_t launch_gemm(const uint8_t*, const uint8_t*, int64_t m, const uint8_t*, int64_t n, int64_t k, void*,
                       const EpilogueArgs& epi, hipStream_t) {
  record("gemm");
  g_call.m = m;
  g_call.n = n;
  g_call.k = k;
  g_call.epi = epi;
  return hipSuccess;
}
hipError_t launch_gemm_tiled(const uint8_t*, const uint8_t*, int64_t m, const uint8_t*, int64_t n, int64_t k, void*,
                             const EpilogueArgs& epi, hipStream_t) {
  record("gemm_tiled");
  g_call.m = m;
  g_call.n = n;
  g_call.k = k;
  g_call.epi = epi;
  return hipSuccess;
}
hipError_t launch_linear(const QuantSource& qs, int64_t m, const uint8_t*, int64_t n, int64_t k, void*,
                         const EpilogueArgs& epi, hipStream_t) {
  record("linear");
  g_call.m = m;
  g_call.n = n;
  g_call.k = k;
  g_call.epi = epi;
  g_call.dynamic = qs.dynamic != 0;
  g_call.rows = qs.ld_x;
  return hipSuccess;
}
hipError_t launch_weight_stream_read(const uint8_t*, int64_t n, int64_t k, uint32_t*, hipStream_t) {
  record("stream_read");
  g_call.n = n;
  g_call.k = k;
  return hipSuccess;
}
int64_t silu_amax_parts_bound(int64_t m, int64_t n) { return m * n / 64 + 1024; }
hipError_t launch_gemm_silu_amax(const uint8_t*, const uint8_t*, int64_t m, const uint8_t*, int64_t n, int64_t k,
                                 uint16_t*, const EpilogueArgs& epi, uint32_t*, int64_t, int64_t* written,
                                 hipStream_t) {
  record("gemm_silu_amax");
  g_call.m = m;
  g_call.n = n;
  g_call.k = k;
  g_call.epi = epi;
  *written = 77;
  return hipSuccess;
}
hipError_t launch_quantize_from_parts(const uint16_t*, int64_t rows, int64_t cols, int64_t, const uint32_t*,
                                      int64_t nparts, float*, uint8_t*, uint8_t*, hipStream_t) {
  record("quantize_parts");
  g_call.rows = rows;
  g_call.cols = cols;
  g_call.n = nparts;
  return hipSuccess;
}
hipError_t launch_gdn_recurrence(const GdnArgs& a, hipStream_t) {
  record("gdn");
  g_call.gdn = a;
  return hipSuccess;
}
}  // namespace nvfp4

// ----------------------------------------------------------------- cases ----
static int gemm(int64_t m, int64_t n, int64_t k, int epi = NVFP4_EPI_NONE, int dt = NVFP4_OUT_BF16,
                int64_t ld = -1, void* ac = A16, void* out = A16) {
  const int64_t cols = epi == NVFP4_EPI_SILU_MUL ? n / 2 : n;
  return gemm_w4a4(static_cast<const uint8_t*>(ac), static_cast<const uint8_t*>(A16), static_cast<const float*>(A16),
                   m, A16, static_cast<const float*>(A16), n, k, out, dt, ld < 0 ? cols : ld, epi, nullptr);
}

static int fused(int64_t m, int64_t n, int64_t k, int nseg, const int64_t* offs, const int* epis,
                 const void* alog = A16) {
  return gemm_w4a4_fused_segments(static_cast<const uint8_t*>(A16), static_cast<const uint8_t*>(A16),
                                  static_cast<const float*>(A16), m, A16, n, k, nseg, offs,
                                  static_cast<const float*>(A16), epis, static_cast<const float*>(alog),
                                  static_cast<const float*>(A16), A16, NVFP4_OUT_BF16, n, nullptr);
}

int main() {
  const uint16_t* X = static_cast<const uint16_t*>(A16);
  float* G = static_cast<float*>(A16);
  uint8_t* B = static_cast<uint8_t*>(A16);

  // quantize
  EXPECT(nvfp4_quantize(X, 4, 64, 64, G, 1, B, B, nullptr), 0, "quantize");
  CHECK(g_call.rows == 4 && g_call.cols == 64 && g_call.dynamic);
  EXPECT(nvfp4_quantize(X, 4, 5136, 5136, G, 0, B, B, nullptr), 0, "quantize");
  CHECK(!g_call.dynamic);
  EXPECT(nvfp4_quantize(X, 0, 64, 64, nullptr, 1, nullptr, nullptr, nullptr), 0, NONE);
  EXPECT(nvfp4_quantize(X, 4, 24, 24, G, 1, B, B, nullptr), NVFP4_ESHAPE, NONE);
  EXPECT(nvfp4_quantize(X, 4, 64, 32, G, 1, B, B, nullptr), NVFP4_ESHAPE, NONE);
  EXPECT(nvfp4_quantize(nullptr, 4, 64, 64, G, 1, B, B, nullptr), NVFP4_EINVAL, NONE);
  EXPECT(nvfp4_quantize(static_cast<const uint16_t*>(MIS), 4, 64, 64, G, 1, B, B, nullptr), NVFP4_EALIGN, NONE);
  EXPECT(nvfp4_quantize(X, 4, 64, 68, G, 1, B, B, nullptr), NVFP4_EALIGN, NONE);

  // E2M1 encoder
  EXPECT(nvfp4_e2m1_encode(static_cast<const float*>(A16), 1000, B, nullptr), 0, "e2m1");
  CHECK(g_call.n == 1000);
  EXPECT(nvfp4_e2m1_encode(nullptr, 0, nullptr, nullptr), 0, NONE);
  EXPECT(nvfp4_e2m1_encode(static_cast<const float*>(A16), -1, B, nullptr), NVFP4_ESHAPE, NONE);
  EXPECT(nvfp4_e2m1_encode(reinterpret_cast<const float*>(0x10002), 8, B, nullptr), NVFP4_EALIGN, NONE);

  // pack / unpack
  CHECK(nvfp4_packed_weight_bytes(17408, 5120) == (size_t)17408 * 5120 * 9 / 16);
  CHECK(nvfp4_packed_weight_bytes(100, 80) == (size_t)128 * 256 * 9 / 16);
  CHECK(nvfp4_packed_weight_bytes(64, 24) == 0 && nvfp4_packed_weight_bytes(-1, 64) == 0);
  const int64_t seg3[4] = {0, 32, 40, 100};
  const size_t pb = nvfp4_packed_weight_bytes(100, 80);
  EXPECT(nvfp4_pack_weights(X, 100, 80, 3, seg3, G, 1, A16, pb, nullptr), 0, "pack");
  CHECK(g_call.segs.num == 3 && g_call.segs.off[0] == 0 && g_call.segs.off[1] == 32 && g_call.segs.off[3] == 100);
  EXPECT(nvfp4_pack_weights(X, 100, 80, 3, seg3, G, 1, A16, pb - 1, nullptr), NVFP4_ESIZE, NONE);
  const int64_t bad[3] = {0, 70, 64};
  EXPECT(nvfp4_pack_weights(X, 64, 80, 2, bad, G, 1, A16, pb, nullptr), NVFP4_ESHAPE, NONE);
  EXPECT(nvfp4_pack_weights(X, 64, 80, 17, seg3, G, 1, A16, pb, nullptr), NVFP4_EINVAL, NONE);
  EXPECT(nvfp4_pack_weights(X, 64, 80, 1, nullptr, G, 1, A16, pb, nullptr), NVFP4_EINVAL, NONE);
  EXPECT(nvfp4_unpack_weights_linear(A16, 100, 80, B, B, nullptr), 0, "unpack");
  EXPECT(nvfp4_unpack_weights_linear(A16, 100, 72, B, B, nullptr), NVFP4_ESHAPE, NONE);

  // gemm_w4a4
  EXPECT(gemm(1, 17408, 5120), 0, "gemm");
  CHECK(g_call.m == 1 && g_call.n == 17408 && g_call.k == 5120 && g_call.epi.segs.num == 1 &&
        g_call.epi.segs.off[1] == 17408 && g_call.epi.out_bf16 == 1 && g_call.epi.silu_mul == 0 &&
        g_call.epi.ld_out == 17408);
  EXPECT(gemm(4096, 34816, 5120, NVFP4_EPI_SILU_MUL), 0, "gemm");
  CHECK(g_call.epi.silu_mul == 1 && g_call.epi.ld_out == 17408 && g_call.epi.h_codes == nullptr);
  EXPECT(gemm(3, 64, 48, NVFP4_EPI_NONE, NVFP4_OUT_F32), 0, "gemm");      // K = 16 (mod 32)
  CHECK(g_call.epi.out_bf16 == 0 && g_call.k == 48);
  EXPECT(gemm(3, 64, 16), 0, "gemm");
  EXPECT(gemm(0, 64, 128, NVFP4_EPI_NONE, NVFP4_OUT_BF16, -1, nullptr, nullptr), 0, NONE);
  EXPECT(gemm(3, 64, 40), NVFP4_ESHAPE, NONE);
  EXPECT(gemm(3, 96, 128, NVFP4_EPI_SILU_MUL), NVFP4_ESHAPE, NONE);
  EXPECT(gemm(3, 128, 128, NVFP4_EPI_NONE, NVFP4_OUT_BF16, 100), NVFP4_ESHAPE, NONE);
  EXPECT(gemm(3, 128, 128, 5), NVFP4_EINVAL, NONE);
  EXPECT(gemm(3, 128, 128, NVFP4_EPI_NONE, 7), NVFP4_EINVAL, NONE);
  EXPECT(gemm(3, 128, 128, NVFP4_EPI_NONE, NVFP4_OUT_BF16, -1, MIS), NVFP4_EALIGN, NONE);
  EXPECT(gemm(3, 128, 128, NVFP4_EPI_NONE, NVFP4_OUT_F32, -1, A16, reinterpret_cast<void*>(0x10002)),
         NVFP4_EALIGN, NONE);
  EXPECT(gemm_w4a4(B, B, G, 3, A16, nullptr, 64, 64, A16, 1, 64, 0, nullptr), NVFP4_EINVAL, NONE);

  // nvfp4_linear: the quantiser's and the GEMM's rules together
  auto lin = [&](int64_t m, int64_t n, int64_t k, int64_t ld_x, int epi, const void* x, float* g, uint8_t* codes) {
    return nvfp4_linear(static_cast<const uint16_t*>(x), m, k, ld_x, g, 1, codes, B, A16, G, n, A16,
                        NVFP4_OUT_BF16, epi == NVFP4_EPI_SILU_MUL ? n / 2 : n, epi, nullptr);
  };
  EXPECT(lin(1, 17408, 5120, 5120, NVFP4_EPI_NONE, X, G, B), 0, "linear");
  CHECK(g_call.m == 1 && g_call.n == 17408 && g_call.k == 5120 && g_call.dynamic && g_call.rows == 5120 &&
        g_call.epi.a_global == G && g_call.epi.seg_w_global == G && g_call.epi.segs.off[1] == 17408);
  EXPECT(lin(8, 34816, 5120, 5128, NVFP4_EPI_SILU_MUL, X, G, B), 0, "linear");
  CHECK(g_call.epi.silu_mul == 1 && g_call.epi.ld_out == 17408);
  EXPECT(lin(0, 64, 128, 128, NVFP4_EPI_NONE, X, G, B), 0, NONE);
  EXPECT(lin(1, 64, 40, 40, NVFP4_EPI_NONE, X, G, B), NVFP4_ESHAPE, NONE);
  EXPECT(lin(1, 64, 128, 132, NVFP4_EPI_NONE, X, G, B), NVFP4_EALIGN, NONE);    // rows of x 16-byte aligned
  EXPECT(lin(1, 96, 128, 128, NVFP4_EPI_SILU_MUL, X, G, B), NVFP4_ESHAPE, NONE);
  EXPECT(lin(1, 64, 128, 128, 4, X, G, B), NVFP4_EINVAL, NONE);
  EXPECT(lin(1, 64, 128, 128, NVFP4_EPI_NONE, MIS, G, B), NVFP4_EALIGN, NONE);
  EXPECT(lin(1, 64, 128, 128, NVFP4_EPI_NONE, X, nullptr, B), NVFP4_EINVAL, NONE);
  EXPECT(lin(1, 64, 128, 128, NVFP4_EPI_NONE, X, G, static_cast<uint8_t*>(MIS)), NVFP4_EALIGN, NONE);

  // gemm_w4a4_fused_segments: six modules with gates
  const int64_t offs[7] = {0, 2048, 4096, 10240, 16384, 16432, 16480};
  const int epis[6] = {NVFP4_SEG_NONE, NVFP4_SEG_NONE, NVFP4_SEG_NONE, NVFP4_SEG_NONE, NVFP4_SEG_SIGMOID,
                       NVFP4_SEG_GDN_DECAY};
  EXPECT(fused(4096, 16480, 5120, 6, offs, epis), 0, "gemm");
  CHECK(g_call.epi.segs.num == 6 && g_call.epi.segs.off[6] == 16480 && g_call.epi.seg_epi[4] == NVFP4_SEG_SIGMOID &&
        g_call.epi.seg_epi[5] == NVFP4_SEG_GDN_DECAY && g_call.epi.a_log == A16 && g_call.epi.silu_mul == 0);
  EXPECT(fused(4096, 16480, 5120, 6, offs, epis, nullptr), NVFP4_EINVAL, NONE);   // decay needs A_log
  const int two_decay[2] = {NVFP4_SEG_GDN_DECAY, NVFP4_SEG_GDN_DECAY};
  const int64_t offs2[3] = {0, 64, 128};
  EXPECT(fused(64, 128, 128, 2, offs2, two_decay), NVFP4_EUNSUPPORTED, NONE);
  const int bad_epi[2] = {0, 9};
  EXPECT(fused(64, 128, 128, 2, offs2, bad_epi), NVFP4_EINVAL, NONE);
  EXPECT(fused(64, 128, 80, 2, offs2, epis), 0, "gemm");
  EXPECT(fused(64, 120, 128, 2, offs2, epis), NVFP4_ESHAPE, NONE);

  // gemm_w4a4_silu_mul_quantize: always the tiled kernels
  EXPECT(gemm_w4a4_silu_mul_quantize(B, B, G, 8, A16, G, 34816, 5120, G, B, B, nullptr, nullptr), 0, "gemm_tiled");
  CHECK(g_call.epi.silu_mul == 1 && g_call.epi.h_codes == B && g_call.epi.h_out == nullptr && g_call.epi.ld_out == 17408);
  EXPECT(gemm_w4a4_silu_mul_quantize(B, B, G, 8, A16, G, 96, 5120, G, B, B, nullptr, nullptr), NVFP4_ESHAPE, NONE);
  EXPECT(gemm_w4a4_silu_mul_quantize(B, B, G, 8, A16, G, 128, 5120, nullptr, B, B, nullptr, nullptr), NVFP4_EINVAL,
         NONE);
  EXPECT(gemm_w4a4_silu_mul_quantize(B, B, G, 8, A16, G, 128, 5120, G, reinterpret_cast<uint8_t*>(0x10008), B,
                                     nullptr, nullptr),
         NVFP4_EALIGN, NONE);

  // gdn_recurrence
  EXPECT(gdn_recurrence(X, 256, X, 256, X, 768, X, 6, X, 6, 10, 2, 6, 128, nullptr, nullptr, A16, 0, 768, nullptr), 0,
         "gdn");
  CHECK(g_call.gdn.T == 10 && g_call.gdn.hk == 2 && g_call.gdn.hv == 6 && g_call.gdn.o_bf16 == 0);
  EXPECT(gdn_recurrence(X, 256, X, 256, X, 768, X, 6, X, 6, 10, 2, 5, 128, nullptr, nullptr, A16, 0, 768, nullptr),
         NVFP4_ESHAPE, NONE);
  EXPECT(gdn_recurrence(X, 256, X, 256, X, 768, X, 6, X, 6, 10, 2, 6, 64, nullptr, nullptr, A16, 0, 768, nullptr),
         NVFP4_EUNSUPPORTED, NONE);
  EXPECT(gdn_recurrence(X, 260, X, 256, X, 768, X, 6, X, 6, 10, 2, 6, 128, nullptr, nullptr, A16, 0, 768, nullptr),
         NVFP4_EALIGN, NONE);

  // gemm_w4a4_silu_mul_amax and nvfp4_quantize_amax_parts
  {
    uint16_t* const H = static_cast<uint16_t*>(A16);
    uint32_t* const P = static_cast<uint32_t*>(A16);
    const int64_t cap = nvfp4_silu_amax_parts(300, 128);
    int64_t wr = -1;
    EXPECT(gemm_w4a4_silu_mul_amax(B, B, G, 300, A16, G, 128, 5120, H, 64, P, cap, &wr, nullptr), 0, "gemm_silu_amax");
    CHECK(wr == 77 && g_call.m == 300 && g_call.epi.silu_mul == 1 && g_call.epi.out_bf16 == 1 && g_call.epi.ld_out == 64);
    EXPECT(gemm_w4a4_silu_mul_amax(B, B, G, 300, A16, G, 128, 5120, H, 64, P, cap - 1, &wr, nullptr), NVFP4_ESHAPE,
           NONE);
    EXPECT(gemm_w4a4_silu_mul_amax(B, B, G, 300, A16, G, 96, 5120, H, 64, P, cap, &wr, nullptr), NVFP4_ESHAPE, NONE);
    EXPECT(gemm_w4a4_silu_mul_amax(B, B, G, 300, A16, G, 128, 5120, H, 64, P, cap, nullptr, nullptr), NVFP4_EINVAL,
           NONE);
    EXPECT(gemm_w4a4_silu_mul_amax(B, B, G, 300, A16, G, 128, 5120, H, 68, P, cap, &wr, nullptr), NVFP4_EALIGN, NONE);
    wr = -1;
    EXPECT(gemm_w4a4_silu_mul_amax(nullptr, nullptr, nullptr, 0, nullptr, nullptr, 128, 5120, nullptr, 64, nullptr, 0,
                                   &wr, nullptr),
           0, NONE);
    CHECK(wr == 0);
    EXPECT(nvfp4_quantize_amax_parts(H, 300, 64, 64, P, 5, static_cast<float*>(A16), B, B, nullptr), 0,
           "quantize_parts");
    CHECK(g_call.rows == 300 && g_call.cols == 64 && g_call.n == 5);
    EXPECT(nvfp4_quantize_amax_parts(H, 300, 64, 64, P, 0, static_cast<float*>(A16), B, B, nullptr), NVFP4_ESHAPE,
           NONE);
    EXPECT(nvfp4_quantize_amax_parts(H, 300, 64, 64, nullptr, 5, static_cast<float*>(A16), B, B, nullptr),
           NVFP4_EINVAL, NONE);
  }

  // weight stream reference
  EXPECT(nvfp4_weight_stream_read(A16, 17408, 5120, static_cast<uint32_t*>(A16), nullptr), 0, "stream_read");
  CHECK(g_call.n == 17408 && g_call.k == 5120);
  EXPECT(nvfp4_weight_stream_read(A16, 17408, 5128, static_cast<uint32_t*>(A16), nullptr), NVFP4_ESHAPE, NONE);
  EXPECT(nvfp4_weight_stream_read(MIS, 17408, 5120, static_cast<uint32_t*>(A16), nullptr), NVFP4_EALIGN, NONE);

  // status strings
  for (int s = 0; s >= -6; --s) CHECK(nvfp4_status_string(s) != nullptr && strlen(nvfp4_status_string(s)) > 0);
  CHECK(strcmp(nvfp4_status_string(123), "unknown status") == 0);
  CHECK(nvfp4_last_hip_error() == 0);

  printf("abi host check: %d cases ok\n", g_cases);
  return 0;
}
