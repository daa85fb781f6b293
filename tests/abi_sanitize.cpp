// Host-only driver for the C ABI layer (fp8_fine_grained_fp8bq_amd/csrc/api.cpp)
// built with AddressSanitizer and UndefinedBehaviorSanitizer (g++, no GPU
// code): it runs the argument-validation paths of every entry point, and the
// accepted calls through to stand-ins for the kernel launchers, against stub
// HIP device queries that report either no device or one gfx950. Any memory
// error or undefined behaviour (an overflowing size product, an out-of-range
// shift, a bad read of the group offsets) aborts the run with the sanitizer's
// report. Built and run by tests/test_abi_sanitized.py.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "fp8bq.h"

// ---- stand-ins for the HIP device queries the ABI layer makes ----------------
static bool g_have_device = false;
static int g_launches = 0;

extern "C" hipError_t hipGetDevice(int* d) {
  if (!g_have_device) return hipErrorNoDevice;
  *d = 0;
  return hipSuccess;
}
extern "C" hipError_t hipGetDevicePropertiesR0600(hipDeviceProp_tR0600* p, int) {
  std::memset(p, 0, sizeof(*p));
  std::strcpy(p->gcnArchName, "gfx950:sramecc+:xnack-");
  return hipSuccess;
}
extern "C" hipError_t hipGetLastError(void) { return hipSuccess; }
extern "C" const char* hipGetErrorString(hipError_t) { return "stub"; }

// ---- stand-ins for the launchers: record the call, check what reached them ----
namespace fp8bq {
#define LAUNCHED() (++g_launches, hipSuccess)
hipError_t launch_quant_act_rows(const uint16_t*, int64_t rows, int64_t cols, int64_t, uint8_t*, int64_t, float*,
                                 int64_t lds, bool, hipStream_t) {
  if (rows <= 0 || cols % 128 || lds < rows) std::abort();
  return LAUNCHED();
}
hipError_t launch_quant_act_cols(const uint16_t*, int64_t rows, int64_t cols, int64_t, uint8_t*, int64_t, float*,
                                 int64_t, bool, hipStream_t) {
  if (rows % 128 || cols % 128) std::abort();
  return LAUNCHED();
}
hipError_t launch_quant_w(const uint16_t*, int64_t n, int64_t k, int64_t, uint8_t*, int64_t, float*, int64_t,
                          uint8_t*, int64_t, bool, hipStream_t) {
  if (n % 128 || k % 128) std::abort();
  return LAUNCHED();
}
hipError_t launch_requant_t(const uint8_t*, int64_t rows, int64_t cols, int64_t, const float*, int64_t, uint8_t*,
                            int64_t, float*, int64_t, bool, hipStream_t) {
  if (rows % 128 || cols % 128) std::abort();
  return LAUNCHED();
}
hipError_t launch_cache_e5m6(const uint16_t*, int64_t rows, int64_t cols, int64_t ldx, uint8_t*, int64_t ldq, float*,
                             int64_t lds, hipStream_t) {
  if (rows <= 0 || cols % 128 || ldx < cols || ldq < cols / 2 * 3 || lds < rows) std::abort();
  return LAUNCHED();
}
hipError_t launch_uncache_e5m6(const uint8_t*, int64_t rows, int64_t cols, int64_t ldq, const float*, int64_t lds,
                               uint16_t*, int64_t ldy, hipStream_t) {
  if (rows <= 0 || cols % 128 || ldy < cols || ldq < cols / 2 * 3 || lds < rows) std::abort();
  return LAUNCHED();
}
hipError_t launch_requant_e5m6_t(const uint8_t*, int64_t rows, int64_t cols, int64_t ldq, const float*, int64_t lds,
                                  uint8_t*, int64_t ldqt, float*, int64_t ldst, hipStream_t) {
  if (rows <= 0 || rows % 128 || cols % 128 || ldq < cols / 2 * 3 || ldqt < rows || lds < rows || ldst < cols)
    std::abort();
  return LAUNCHED();
}
hipError_t launch_gemm(int kind, int64_t, int64_t n, int64_t k, const uint8_t*, int64_t, const float*, int64_t,
                       const uint8_t*, int64_t, const float*, int64_t, void*, int64_t, bool, hipStream_t) {
  if (kind < 0 || kind > 2 || n % 128 || k % 128) std::abort();
  return LAUNCHED();
}
hipError_t launch_gemm_quant(int kind, int64_t, int64_t n, int64_t k, const uint8_t*, int64_t, const float*,
                             int64_t, const uint8_t*, int64_t, const float*, int64_t, uint16_t*, int64_t, uint8_t*,
                             int64_t, float*, int64_t, bool, bool, hipStream_t) {
  if (kind < 0 || kind > 1 || n % 128 || k % 128) std::abort();
  return LAUNCHED();
}
hipError_t launch_grouped_gemm(int groups, const int64_t* row_off, int64_t, int64_t, const uint8_t*, int64_t,
                               const float*, int64_t, const uint8_t*, int64_t, const float*, int64_t, uint16_t*,
                               int64_t, bool, hipStream_t) {
  for (int e = 0; e < groups; ++e)
    if (row_off[e + 1] < row_off[e] || row_off[e] % 128) std::abort();
  return LAUNCHED();
}
int64_t grouped_gemm_decode_workspace(int groups, const int64_t* row_off, int64_t n, int64_t k) {
  // the library's rule: counters, then both K halves' partial sums of the split experts' 16-row subtiles
  int64_t t = 0;
  for (int e = 0; e < groups; ++e)
    if (row_off[e + 1] - row_off[e] > 32) t += (row_off[e + 1] - row_off[e] + 15) / 16;
  if (t == 0 || k / 128 < 2 || n / 128 > 256) return 0;
  return 256 * 256 * 4 + 2 * t * 16 * n * 4;
}
hipError_t launch_grouped_gemm_decode_noalloc(int groups, const int64_t* row_off, int64_t n, int64_t k,
                                              const uint8_t*, int64_t, const float*, int64_t, const uint8_t*,
                                              int64_t, const float*, int64_t, uint16_t*, int64_t, hipStream_t) {
  const int64_t need = grouped_gemm_decode_workspace(groups, row_off, n, k);
  if (need <= 0 || need > ((int64_t)32 << 20)) std::abort();   // the scratch: 32 MiB
  return LAUNCHED();
}
hipError_t launch_grouped_gemm_decode(int groups, const int64_t* row_off, int64_t n, int64_t k, const uint8_t*,
                                      int64_t, const float*, int64_t, const uint8_t*, int64_t, const float*,
                                      int64_t, uint16_t*, int64_t, void* workspace, hipStream_t) {
  for (int e = 0; e < groups; ++e)
    if (row_off[e + 1] < row_off[e] || row_off[e + 1] - row_off[e] > 256) std::abort();
  if (workspace && grouped_gemm_decode_workspace(groups, row_off, n, k) == 0) std::abort();
  return LAUNCHED();
}
}  // namespace fp8bq

// ---- the checks ----------------------------------------------------------------
static int g_fail = 0;
#define EXPECT(call, want)                                                                              \
  do {                                                                                                  \
    const int got_ = (call);                                                                            \
    if (got_ != (want)) {                                                                               \
      std::printf("line %d: %s returned %d, expected %d (%s)\n", __LINE__, #call, got_, (want),        \
                  fp8bq_last_error());                                                                  \
      ++g_fail;                                                                                         \
    }                                                                                                   \
    if (got_ != FP8BQ_OK && std::strlen(fp8bq_last_error()) == 0) {                                     \
      std::printf("line %d: empty error message\n", __LINE__);                                          \
      ++g_fail;                                                                                         \
    }                                                                                                   \
  } while (0)

// stand-in device addresses: aligned, never dereferenced by the ABI layer
static void* P(uintptr_t a) { return reinterpret_cast<void*>(a); }
static float* F(uintptr_t a) { return reinterpret_cast<float*>(a); }
static const uintptr_t A16 = 0x10000, B16 = 0x20000, S4 = 0x30000, O16 = 0x40000, Q16 = 0x50000;

static void validation() {
  // fp8bq_quant_act_1x128
  EXPECT(fp8bq_quant_act_1x128(nullptr, 256, 1024, 1024, 0, P(B16), 1024, F(S4), 256, nullptr), FP8BQ_E_INVAL);
  EXPECT(fp8bq_quant_act_1x128(P(A16), 0, 1024, 1024, 0, P(B16), 1024, F(S4), 256, nullptr), FP8BQ_E_INVAL);
  EXPECT(fp8bq_quant_act_1x128(P(A16), 256, 1024, 1024, 2, P(B16), 1024, F(S4), 256, nullptr), FP8BQ_E_INVAL);
  EXPECT(fp8bq_quant_act_1x128(P(A16), 256, 1024, 1000, 0, P(B16), 1024, F(S4), 256, nullptr), FP8BQ_E_INVAL);
  EXPECT(fp8bq_quant_act_1x128(P(A16), 256, 1000, 1000, 0, P(B16), 1000, F(S4), 256, nullptr), FP8BQ_E_SHAPE);
  EXPECT(fp8bq_quant_act_1x128(P(A16 + 2), 256, 1024, 1024, 0, P(B16), 1024, F(S4), 256, nullptr), FP8BQ_E_ALIGN);
  EXPECT(fp8bq_quant_act_1x128(P(A16), (int64_t)1 << 30, 8192, 8192, 0, P(B16), 8192, F(S4), (int64_t)1 << 30,
                               nullptr), FP8BQ_E_SHAPE);
  EXPECT(fp8bq_quant_act_1x128(P(A16), INT64_MAX / 2, 1 << 20, 1 << 20, 0, P(B16), 1 << 20, F(S4), INT64_MAX / 2,
                               nullptr), FP8BQ_E_SHAPE);
  EXPECT(fp8bq_quant_act_1x128(P(A16), 200, 1024, 1024, 1, P(B16), 256, F(S4), 1024, nullptr), FP8BQ_E_SHAPE);
  EXPECT(fp8bq_quant_act_1x128(P(A16), 256, 1024, 1024, 1, P(B16), 200, F(S4), 1024, nullptr), FP8BQ_E_INVAL);
  // fp8bq_quant_w_128x128
  EXPECT(fp8bq_quant_w_128x128(P(A16), 0, 384, 384, P(B16), 384, F(S4), 3, P(O16), 256, 0, nullptr), FP8BQ_E_INVAL);
  EXPECT(fp8bq_quant_w_128x128(P(A16), 200, 384, 384, P(B16), 384, F(S4), 3, P(O16), 256, 0, nullptr), FP8BQ_E_SHAPE);
  EXPECT(fp8bq_quant_w_128x128(P(A16), 256, 384, 384, P(B16), 384, F(S4), 2, P(O16), 256, 0, nullptr), FP8BQ_E_INVAL);
  EXPECT(fp8bq_quant_w_128x128(P(A16), 256, 384, 384, P(B16), 384, F(S4), 3, P(O16), 128, 0, nullptr), FP8BQ_E_INVAL);
  EXPECT(fp8bq_quant_w_128x128(P(A16), 256, 384, 384, P(B16), 384, F(S4), 3, P(O16 + 1), 256, 0, nullptr), FP8BQ_E_ALIGN);
  EXPECT(fp8bq_quant_w_128x128(P(A16), 256, 384, 384, P(B16), 384, F(S4), 3, P(O16), 256, 0x20, nullptr), FP8BQ_E_INVAL);
  EXPECT(fp8bq_quant_w_128x128(P(A16), INT64_MAX - 127, INT64_MAX - 127, INT64_MAX - 127, P(B16), INT64_MAX - 127,
                               F(S4), INT64_MAX, nullptr, 0, 0, nullptr), FP8BQ_E_SHAPE);
  // fp8bq_cache_e5m6_1x128 / fp8bq_uncache_e5m6_1x128
  EXPECT(fp8bq_cache_e5m6_1x128(nullptr, 100, 384, 384, P(B16), 576, F(S4), 100, nullptr), FP8BQ_E_INVAL);
  EXPECT(fp8bq_cache_e5m6_1x128(P(A16), 100, 300, 384, P(B16), 576, F(S4), 100, nullptr), FP8BQ_E_SHAPE);
  EXPECT(fp8bq_cache_e5m6_1x128(P(A16), 100, 384, 384, P(B16), 560, F(S4), 100, nullptr), FP8BQ_E_INVAL);
  EXPECT(fp8bq_cache_e5m6_1x128(P(A16), 100, 384, 384, P(B16 + 4), 576, F(S4), 100, nullptr), FP8BQ_E_ALIGN);
  EXPECT(fp8bq_uncache_e5m6_1x128(P(B16), 100, 384, 576, F(S4), 99, P(A16), 384, nullptr), FP8BQ_E_INVAL);
  EXPECT(fp8bq_uncache_e5m6_1x128(P(B16), 100, 384, 584, F(S4), 100, P(A16), 384, nullptr), FP8BQ_E_ALIGN);
  {
    const int64_t huge = INT64_MAX - 127;
    // 1.5 * cols past INT64_MAX: rejected on ldq without forming the product
    EXPECT(fp8bq_cache_e5m6_1x128(P(A16), huge, huge / 128 * 128, INT64_MAX / 8 * 8, P(B16), INT64_MAX / 16 * 16,
                                  F(S4), huge, nullptr), FP8BQ_E_INVAL);
    // rows or the tile count past the grid
    EXPECT(fp8bq_cache_e5m6_1x128(P(A16), huge, 1024, 1024, P(B16), 1536, F(S4), huge, nullptr), FP8BQ_E_SHAPE);
    EXPECT(fp8bq_uncache_e5m6_1x128(P(B16), 1024, INT64_MAX / 3 / 128 * 128, INT64_MAX / 16 * 16, F(S4), 1024,
                                    P(A16), INT64_MAX / 8 * 8, nullptr), FP8BQ_E_SHAPE);
  }
  // fp8bq_requant_e5m6_t_128x1
  EXPECT(fp8bq_requant_e5m6_t_128x1(nullptr, 256, 384, 576, F(S4), 256, P(B16), 256, F(S4 + 4096), 384, nullptr),
         FP8BQ_E_INVAL);
  EXPECT(fp8bq_requant_e5m6_t_128x1(P(A16), 200, 384, 576, F(S4), 256, P(B16), 256, F(S4 + 4096), 384, nullptr),
         FP8BQ_E_SHAPE);
  EXPECT(fp8bq_requant_e5m6_t_128x1(P(A16), 256, 384, 560, F(S4), 256, P(B16), 256, F(S4 + 4096), 384, nullptr),
         FP8BQ_E_INVAL);
  EXPECT(fp8bq_requant_e5m6_t_128x1(P(A16), 256, 384, 576, F(S4), 255, P(B16), 256, F(S4 + 4096), 384, nullptr),
         FP8BQ_E_INVAL);
  EXPECT(fp8bq_requant_e5m6_t_128x1(P(A16), 256, 384, 576, F(S4), 256, P(B16), 256, F(S4 + 4096), 383, nullptr),
         FP8BQ_E_INVAL);
  EXPECT(fp8bq_requant_e5m6_t_128x1(P(A16), 256, 384, 584, F(S4), 256, P(B16), 256, F(S4 + 4096), 384, nullptr),
         FP8BQ_E_ALIGN);
  EXPECT(fp8bq_requant_e5m6_t_128x1(P(A16), 256, 384, 576, F(S4), 256, P(B16 + 4), 256, F(S4 + 4096), 384, nullptr),
         FP8BQ_E_ALIGN);
  {
    const int64_t huge = INT64_MAX / 128 * 128;
    // 1.5 * cols past INT64_MAX: rejected on ldq without forming the product
    EXPECT(fp8bq_requant_e5m6_t_128x1(P(A16), 128, huge, INT64_MAX / 16 * 16, F(S4), 128, P(B16), 128, F(S4),
                                      huge, nullptr), FP8BQ_E_INVAL);
    // row or column blocks past the grid
    EXPECT(fp8bq_requant_e5m6_t_128x1(P(A16), huge, 128, 192, F(S4), huge, P(B16), huge, F(S4), 128, nullptr),
           FP8BQ_E_SHAPE);
    EXPECT(fp8bq_requant_e5m6_t_128x1(P(A16), 128, 128 * 65536, 192 * 65536, F(S4), 128, P(B16), 128, F(S4),
                                      128 * 65536, nullptr), FP8BQ_E_SHAPE);
  }
  // fp8bq_requant_t_128x1
  EXPECT(fp8bq_requant_t_128x1(nullptr, 256, 384, 384, F(S4), 256, P(B16), 256, F(S4 + 4096), 384, 0, nullptr), FP8BQ_E_INVAL);
  EXPECT(fp8bq_requant_t_128x1(P(A16), 200, 384, 384, F(S4), 256, P(B16), 256, F(S4 + 4096), 384, 0, nullptr), FP8BQ_E_SHAPE);
  EXPECT(fp8bq_requant_t_128x1(P(A16), 256, 384, 256, F(S4), 256, P(B16), 256, F(S4 + 4096), 384, 0, nullptr), FP8BQ_E_INVAL);
  EXPECT(fp8bq_requant_t_128x1(P(A16), 256, 384, 384, F(S4 + 2), 256, P(B16), 256, F(S4 + 4096), 384, 0, nullptr), FP8BQ_E_ALIGN);
  EXPECT(fp8bq_requant_t_128x1(P(A16), 128, 128 * 65536, 128 * 65536, F(S4), 128, P(B16), 128, F(S4 + 4096),
                               128 * 65536, 0, nullptr), FP8BQ_E_SHAPE);
  // fp8bq_gemm, every op
  for (int op = 0; op < 3; ++op) {
    const int64_t ldsb = op == 0 ? 8 : op == 1 ? 3 : 384;
    EXPECT(fp8bq_gemm(3, 300, 384, 1024, P(A16), 1024, F(S4), 300, P(B16), 1024, F(S4), ldsb, P(O16), 384, nullptr), FP8BQ_E_INVAL);
    EXPECT(fp8bq_gemm(op, 300, 384, 1024, nullptr, 1024, F(S4), 300, P(B16), 1024, F(S4), ldsb, P(O16), 384, nullptr), FP8BQ_E_INVAL);
    EXPECT(fp8bq_gemm(op, 300, 384, 1000, P(A16), 1008, F(S4), 300, P(B16), 1008, F(S4), ldsb, P(O16), 384, nullptr), FP8BQ_E_SHAPE);
    EXPECT(fp8bq_gemm(op, 300, 200, 1024, P(A16), 1024, F(S4), 300, P(B16), 1024, F(S4), ldsb, P(O16), 208, nullptr), FP8BQ_E_SHAPE);
    EXPECT(fp8bq_gemm(op, 300, 384, 1024, P(A16), 1024, F(S4), 299, P(B16), 1024, F(S4), ldsb, P(O16), 384, nullptr), FP8BQ_E_INVAL);
    EXPECT(fp8bq_gemm(op, 300, 384, 1024, P(A16), 1024, F(S4), 300, P(B16), 1024, F(S4), ldsb - 1, P(O16), 384, nullptr), FP8BQ_E_INVAL);
    EXPECT(fp8bq_gemm(op, 300, 384, 1024, P(A16), 1032, F(S4), 300, P(B16), 1024, F(S4), ldsb, P(O16), 384, nullptr), FP8BQ_E_ALIGN);
    EXPECT(fp8bq_gemm(op, 300, 384, 1024, P(A16), 1024, F(S4), 300, P(B16), 1024, F(S4), ldsb, P(O16), 383, nullptr), FP8BQ_E_INVAL);
    EXPECT(fp8bq_gemm(op | 0x20, 300, 384, 1024, P(A16), 1024, F(S4), 300, P(B16), 1024, F(S4), ldsb, P(O16), 384, nullptr), FP8BQ_E_INVAL);
    EXPECT(fp8bq_gemm(op, INT64_MAX / 4, 1 << 20, 1 << 20, P(A16), 1 << 20, F(S4), INT64_MAX / 4, P(B16), 1 << 20,
                      F(S4), (int64_t)1 << 22, P(O16), 1 << 20, nullptr), FP8BQ_E_SHAPE);
  }
  // fp8bq_gemm_quant
  EXPECT(fp8bq_gemm_quant(2, 300, 384, 1024, P(A16), 1024, F(S4), 300, P(B16), 1024, F(S4), 384, P(O16), 384, P(Q16),
                          384, F(S4), 300, 0, nullptr), FP8BQ_E_INVAL);
  EXPECT(fp8bq_gemm_quant(0, 300, 384, 1024, P(A16), 1024, F(S4), 300, P(B16), 1024, F(S4), 8, P(O16), 384, nullptr,
                          384, F(S4), 300, 0, nullptr), FP8BQ_E_INVAL);
  EXPECT(fp8bq_gemm_quant(0, 300, 384, 1024, P(A16), 1024, F(S4), 300, P(B16), 1024, F(S4), 8, P(O16), 384, P(Q16),
                          368, F(S4), 300, 0, nullptr), FP8BQ_E_INVAL);
  EXPECT(fp8bq_gemm_quant(0, 300, 384, 1024, P(A16), 1024, F(S4), 300, P(B16), 1024, F(S4), 8, P(O16), 384, P(Q16 + 4),
                          384, F(S4), 300, 0, nullptr), FP8BQ_E_ALIGN);
  // grouped
  const int64_t off_ok[3] = {0, 256, 512}, off_neg[3] = {0, 256, 128}, off_odd[3] = {0, 100, 512};
  EXPECT(fp8bq_grouped_gemm(0, off_ok, 2048, 7168, P(A16), 7168, F(S4), 512, P(B16), 7168, F(S4), 56, P(O16), 2048, 0, nullptr), FP8BQ_E_INVAL);
  EXPECT(fp8bq_grouped_gemm(2, nullptr, 2048, 7168, P(A16), 7168, F(S4), 512, P(B16), 7168, F(S4), 56, P(O16), 2048, 0, nullptr), FP8BQ_E_INVAL);
  EXPECT(fp8bq_grouped_gemm(2, off_neg, 2048, 7168, P(A16), 7168, F(S4), 512, P(B16), 7168, F(S4), 56, P(O16), 2048, 0, nullptr), FP8BQ_E_SHAPE);
  EXPECT(fp8bq_grouped_gemm(2, off_odd, 2048, 7168, P(A16), 7168, F(S4), 512, P(B16), 7168, F(S4), 56, P(O16), 2048, 0, nullptr), FP8BQ_E_SHAPE);
  EXPECT(fp8bq_grouped_gemm(2, off_ok, 2048, 7168, P(A16), 7168, F(S4), 500, P(B16), 7168, F(S4), 56, P(O16), 2048, 0, nullptr), FP8BQ_E_INVAL);
  const int64_t doff_ok[3] = {0, 30, 50}, doff_big[3] = {0, 257, 300};
  EXPECT(fp8bq_grouped_gemm_decode(2, doff_big, 2048, 7168, P(A16), 7168, F(S4), 512, P(B16), 7168, F(S4), 56, P(O16), 2048, 0, nullptr), FP8BQ_E_SHAPE);
  EXPECT(fp8bq_grouped_gemm_decode(2, doff_ok, 2000, 7168, P(A16), 7168, F(S4), 512, P(B16), 7168, F(S4), 56, P(O16), 2000, 0, nullptr), FP8BQ_E_SHAPE);
  EXPECT(fp8bq_grouped_gemm_decode(2, doff_ok, 2048, 7168, P(A16 + 8), 7168, F(S4), 512, P(B16), 7168, F(S4), 56, P(O16), 2048, 0, nullptr), FP8BQ_E_ALIGN);
  // the workspace form: size query, missing / small / misaligned workspace
  {
    const int64_t big[3] = {0, 217, 260};                  // one expert above 32 rows: split
    int64_t need = -1;
    EXPECT(fp8bq_grouped_gemm_decode_workspace_size(2, big, 2048, 7168, nullptr), FP8BQ_E_INVAL);
    EXPECT(fp8bq_grouped_gemm_decode_workspace_size(2, doff_big, 2048, 7168, &need), FP8BQ_E_SHAPE);
    EXPECT(fp8bq_grouped_gemm_decode_workspace_size(2, big, 2000, 7168, &need), FP8BQ_E_SHAPE);
    EXPECT(fp8bq_grouped_gemm_decode_workspace_size(2, big, 2048, 7168, &need), FP8BQ_OK);
    if (need != 262144 + 2 * 17 * 16 * 2048 * 4) { std::printf("workspace size %lld\n", (long long)need); ++g_fail; }
    EXPECT(fp8bq_grouped_gemm_decode_workspace_size(2, doff_ok, 2048, 7168, &need), FP8BQ_OK);
    if (need != 0) { std::printf("workspace size %lld for small experts\n", (long long)need); ++g_fail; }
    const int64_t w = 262144 + 2 * 17 * 16 * 2048 * 4;
    EXPECT(fp8bq_grouped_gemm_decode_ws(2, big, 2048, 7168, P(A16), 7168, F(S4), 512, P(B16), 7168, F(S4), 56, P(O16),
                                        2048, nullptr, w, 0, nullptr), FP8BQ_E_INVAL);
    EXPECT(fp8bq_grouped_gemm_decode_ws(2, big, 2048, 7168, P(A16), 7168, F(S4), 512, P(B16), 7168, F(S4), 56, P(O16),
                                        2048, P(Q16), w - 1, 0, nullptr), FP8BQ_E_INVAL);
    EXPECT(fp8bq_grouped_gemm_decode_ws(2, big, 2048, 7168, P(A16), 7168, F(S4), 512, P(B16), 7168, F(S4), 56, P(O16),
                                        2048, P(Q16 + 8), w, 0, nullptr), FP8BQ_E_ALIGN);
    EXPECT(fp8bq_grouped_gemm_decode_ws(2, big, 2048, 7168, P(A16), 7168, F(S4), 512, P(B16), 7168, F(S4), 56, P(O16),
                                        2048, P(Q16), w, 1, nullptr), FP8BQ_E_INVAL);
  }
  // the allocation-free form: a launch whose workspace exceeds the scratch is refused
  {
    int64_t big8[9];
    for (int e = 0; e <= 8; ++e) big8[e] = 256 * (int64_t)e;     // 8 x 256 rows at n = 4096: 64 MiB of partial sums
    EXPECT(fp8bq_grouped_gemm_decode_noalloc(8, big8, 4096, 7168, P(A16), 7168, F(S4), 2048, P(B16), 7168, F(S4), 56,
                                             P(O16), 4096, 0, nullptr), FP8BQ_E_SHAPE);
    EXPECT(fp8bq_grouped_gemm_decode_noalloc(8, big8, 4096, 7168, P(A16), 7168, F(S4), 2048, P(B16), 7168, F(S4), 56,
                                             P(O16), 4096, 1, nullptr), FP8BQ_E_INVAL);
  }
  // sizes whose products do not fit in 64 bits
  const int64_t huge = INT64_MAX - 127;
  EXPECT(fp8bq_grouped_gemm_decode(2, doff_ok, huge / 128 * 128, 7168, P(A16), 7168, F(S4), 512, P(B16), 7168,
                                   F(S4), 56, P(O16), INT64_MAX / 64 * 64, 0, nullptr), FP8BQ_E_SHAPE);
  EXPECT(fp8bq_grouped_gemm(2, off_ok, huge / 128 * 128, 7168, P(A16), 7168, F(S4), 512, P(B16), 7168, F(S4), 56,
                            P(O16), INT64_MAX / 64 * 64, 0, nullptr), FP8BQ_E_SHAPE);
  EXPECT(fp8bq_quant_act_1x128(P(A16), huge, huge / 128 * 128, huge / 128 * 128, 0, P(B16), huge / 128 * 128, F(S4),
                               huge, nullptr), FP8BQ_E_SHAPE);
  EXPECT(fp8bq_quant_act_1x128(P(A16), huge / 128 * 128, huge / 128 * 128, huge / 128 * 128, 1, P(B16),
                               huge / 128 * 128, F(S4), huge / 128 * 128, nullptr), FP8BQ_E_SHAPE);
  EXPECT(fp8bq_gemm(0, huge, huge / 128 * 128, huge / 128 * 128, P(A16), huge / 128 * 128, F(S4), huge, P(B16),
                    huge / 128 * 128, F(S4), INT64_MAX, P(O16), INT64_MAX / 64 * 64, nullptr), FP8BQ_E_SHAPE);
  EXPECT(fp8bq_gemm_quant(0, huge, huge / 128 * 128, 1024, P(A16), 1024, F(S4), huge, P(B16), 1024, F(S4), INT64_MAX,
                          P(O16), INT64_MAX / 64 * 64, P(Q16), INT64_MAX / 64 * 64, F(S4), huge, 0, nullptr), FP8BQ_E_SHAPE);
}

// calls that pass validation: E_DEVICE without a device, OK through the launchers with one
static void accepted(int want) {
  EXPECT(fp8bq_quant_act_1x128(P(A16), 256, 1024, 1024, 0, P(B16), 1024, F(S4), 256, nullptr), want);
  EXPECT(fp8bq_quant_act_1x128(P(A16), 256, 1024, 1024, 1 | FP8BQ_SCALE_POW2, P(B16), 256, F(S4), 1024, nullptr), want);
  EXPECT(fp8bq_quant_w_128x128(P(A16), 256, 384, 384, P(B16), 384, F(S4), 3, nullptr, 0, 0, nullptr), want);
  EXPECT(fp8bq_requant_t_128x1(P(A16), 256, 384, 384, F(S4), 256, P(B16), 256, F(S4 + 4096), 384, 0, nullptr), want);
  EXPECT(fp8bq_requant_t_128x1(P(A16), 256, 384, 384, F(S4), 256, P(B16), 256, F(S4 + 4096), 384, FP8BQ_SCALE_POW2,
                               nullptr), want);
  EXPECT(fp8bq_cache_e5m6_1x128(P(A16), 100, 384, 384, P(B16), 576, F(S4), 100, nullptr), want);
  EXPECT(fp8bq_uncache_e5m6_1x128(P(B16), 100, 384, 576, F(S4), 100, P(A16), 384, nullptr), want);
  EXPECT(fp8bq_requant_e5m6_t_128x1(P(A16), 256, 384, 576, F(S4), 256, P(B16), 256, F(S4 + 4096), 384, nullptr), want);
  for (int op = 0; op < 3; ++op) {
    const int64_t ldsb = op == 0 ? 8 : op == 1 ? 3 : 384;
    EXPECT(fp8bq_gemm(op, 300, 384, 1024, P(A16), 1024, F(S4), 300, P(B16), 1024, F(S4), ldsb, P(O16), 384, nullptr), want);
    EXPECT(fp8bq_gemm(op | FP8BQ_SCALE_POW2, 300, 384, 1024, P(A16), 1024, F(S4), 300, P(B16), 1024, F(S4), ldsb,
                      P(O16), 384, nullptr), want);
  }
  EXPECT(fp8bq_gemm_quant(1, 300, 384, 1024, P(A16), 1024, F(S4), 300, P(B16), 1024, F(S4), 3, nullptr, 384, P(Q16),
                          384, F(S4), 300, FP8BQ_SCALE_POW2, nullptr), want);
  int64_t off[257];
  for (int e = 0; e <= 256; ++e) off[e] = 128 * (int64_t)e;
  EXPECT(fp8bq_grouped_gemm(256, off, 2048, 7168, P(A16), 7168, F(S4), 32768, P(B16), 7168, F(S4), 56, P(O16), 2048,
                            0, nullptr), want);
  int64_t doff[257];
  for (int e = 0; e <= 256; ++e) doff[e] = 7 * (int64_t)e;
  const int64_t doff_ok_small[3] = {0, 30, 50};
  EXPECT(fp8bq_grouped_gemm_decode(256, doff, 2048, 7168, P(A16), 7168, F(S4), 1792, P(B16), 7168, F(S4), 56,
                                   P(O16), 2048, 0, nullptr), want);
  int64_t doff2[257];
  for (int e = 0; e <= 256; ++e) doff2[e] = 256 * (int64_t)e;      // 256 experts of 256 rows: all split
  const int64_t w2 = 262144 + 2 * 4096 * 16 * (int64_t)2048 * 4;
  EXPECT(fp8bq_grouped_gemm_decode_ws(256, doff2, 2048, 7168, P(A16), 7168, F(S4), 65536, P(B16), 7168, F(S4), 56,
                                      P(O16), 2048, P(Q16), w2, 0, nullptr), want);
  EXPECT(fp8bq_grouped_gemm_decode_ws(2, doff_ok_small, 2048, 7168, P(A16), 7168, F(S4), 512, P(B16), 7168, F(S4), 56,
                                      P(O16), 2048, nullptr, 0, 0, nullptr), want);       // nothing split: no workspace
  const int64_t dmix[9] = {0, 217, 396, 516, 609, 684, 741, 810, 853};     // the 256-token decode step: fits
  EXPECT(fp8bq_grouped_gemm_decode_noalloc(8, dmix, 2048, 7168, P(A16), 7168, F(S4), 853, P(B16), 7168, F(S4), 56,
                                           P(O16), 2048, 0, nullptr), want);
  EXPECT(fp8bq_grouped_gemm_decode_noalloc(2, doff_ok_small, 2048, 7168, P(A16), 7168, F(S4), 512, P(B16), 7168,
                                           F(S4), 56, P(O16), 2048, 0, nullptr), want);
}

int main() {
  validation();
  g_have_device = false;
  accepted(FP8BQ_E_DEVICE);
  const int before = g_launches;
  g_have_device = true;
  accepted(FP8BQ_OK);
  validation();   // again, past the cached device check
  std::printf("abi_sanitize: %d failed checks, %d launches reached\n", g_fail, g_launches - before);
  return g_fail != 0 || g_launches == before;
}
