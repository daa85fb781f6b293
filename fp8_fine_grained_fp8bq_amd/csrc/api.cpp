// C-ABI entry points of libfp8bq: argument validation (host only, before any
// HIP call), the device check, and dispatch to the kernel launchers.
// The operations and their layouts are specified in include/fp8bq.h.
#include "../../include/fp8bq.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "internal.h"

static_assert(FP8BQ_DECODE_NOALLOC_SCRATCH_BYTES == fp8bq::kNoAllocScratchBytes, "scratch size in the header");

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr int kMaxDevices = 64;
std::atomic<int> g_arch[kMaxDevices];   // 0 unknown, 1 gfx950, 2 other

// Current device must exist and be gfx950. The arch lookup is cached per device.
int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return fail(FP8BQ_E_DEVICE, "no HIP device available");
  }
  if (dev >= kMaxDevices) return fail(FP8BQ_E_DEVICE, "device index %d out of range", dev);
  int st = g_arch[dev].load(std::memory_order_acquire);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      (void)hipGetLastError();
      return fail(FP8BQ_E_DEVICE, "hipGetDeviceProperties failed for device %d", dev);
    }
    st = (strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_arch[dev].store(st, std::memory_order_release);
    if (st == 2) return fail(FP8BQ_E_DEVICE, "device %d is %s, this library is built for gfx950", dev, prop.gcnArchName);
  }
  if (st != 1) return fail(FP8BQ_E_DEVICE, "device %d is not gfx950", dev);
  return FP8BQ_OK;
}

// a * b >= limit for a, b >= 1, without forming the product (callers pass
// user-supplied sizes, whose product may not fit in int64)
bool product_at_least(int64_t a, int64_t b, int64_t limit) { return a > (limit - 1) / b; }

// ceil(a / d) for a >= 1 without overflowing a + d - 1
int64_t ceil_div(int64_t a, int64_t d) { return (a - 1) / d + 1; }

int launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(FP8BQ_E_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  return FP8BQ_OK;
}

constexpr int64_t kMaxTiles = (int64_t)1 << 31;

}  // namespace

extern "C" {

const char* fp8bq_last_error(void) { return g_err; }

const char* fp8bq_version(void) { return "fp8bq 0.1 (gfx950)"; }

int fp8bq_quant_act_1x128(const void* x, int64_t rows, int64_t cols, int64_t ldx, int mode_flags,
                          void* q, int64_t ldq, float* s, int64_t lds, void* stream) {
  if (!x || !q || !s) return fail(FP8BQ_E_INVAL, "quant_act: null pointer");
  if (rows <= 0 || cols <= 0) return fail(FP8BQ_E_INVAL, "quant_act: rows and cols must be positive");
  const bool pow2 = (mode_flags & FP8BQ_SCALE_POW2) != 0;
  const int mode = mode_flags & ~FP8BQ_SCALE_POW2;
  if (mode != FP8BQ_ACT_ROWWISE && mode != FP8BQ_ACT_COLWISE)
    return fail(FP8BQ_E_INVAL, "quant_act: mode must be ROWWISE (0) or COLWISE (1), optionally | SCALE_POW2, got %d", mode_flags);
  if (ldx < cols) return fail(FP8BQ_E_INVAL, "quant_act: ldx (%lld) < cols (%lld)", (long long)ldx, (long long)cols);
  if (cols % 128) return fail(FP8BQ_E_SHAPE, "quant_act: cols (%lld) must be a multiple of 128", (long long)cols);
  if (mode == FP8BQ_ACT_ROWWISE) {
    if (ldq < cols) return fail(FP8BQ_E_INVAL, "quant_act: ldq < cols");
    if (lds < rows) return fail(FP8BQ_E_INVAL, "quant_act: lds < rows");
    if (rows >= kMaxTiles || product_at_least(ceil_div(rows, 32), cols / 128, kMaxTiles))
      return fail(FP8BQ_E_SHAPE, "quant_act: too large");
  } else {
    if (rows % 128) return fail(FP8BQ_E_SHAPE, "quant_act: column-wise mode needs rows (%lld) to be a multiple of 128", (long long)rows);
    if (ldq < rows) return fail(FP8BQ_E_INVAL, "quant_act: ldq < rows (transposed output)");
    if (lds < cols) return fail(FP8BQ_E_INVAL, "quant_act: lds < cols");
    // grid: rows / 128 row blocks (x) by cols / 128 column blocks (y)
    if (cols / 128 > 65535 || rows / 128 > ((int64_t)1 << 31) - 1) return fail(FP8BQ_E_SHAPE, "quant_act: too large");
  }
  if (!aligned(x, 16) || !aligned(q, 16) || !aligned(s, 4))
    return fail(FP8BQ_E_ALIGN, "quant_act: x and q must be 16-byte aligned, s 4-byte aligned");
  if (ldx % 8 || ldq % 16) return fail(FP8BQ_E_ALIGN, "quant_act: ldx must be a multiple of 8 and ldq of 16");
  if (int st = check_device()) return st;
  hipStream_t str = reinterpret_cast<hipStream_t>(stream);
  if (mode == FP8BQ_ACT_ROWWISE)
    return launched(fp8bq::launch_quant_act_rows(static_cast<const uint16_t*>(x), rows, cols, ldx,
                                                 static_cast<uint8_t*>(q), ldq, s, lds, pow2, str), "quant_act");
  return launched(fp8bq::launch_quant_act_cols(static_cast<const uint16_t*>(x), rows, cols, ldx,
                                               static_cast<uint8_t*>(q), ldq, s, lds, pow2, str), "quant_act");
}

static int check_e5m6(const char* who, const void* a, const void* b, const float* s, int64_t rows, int64_t cols,
                      int64_t ld16, int64_t ldq, int64_t lds) {
  if (!a || !b || !s) return fail(FP8BQ_E_INVAL, "%s: null pointer", who);
  if (rows <= 0 || cols <= 0) return fail(FP8BQ_E_INVAL, "%s: rows and cols must be positive", who);
  if (cols % 128) return fail(FP8BQ_E_SHAPE, "%s: cols (%lld) must be a multiple of 128", who, (long long)cols);
  if (ld16 < cols) return fail(FP8BQ_E_INVAL, "%s: bf16 leading dimension < cols", who);
  if (ldq / 3 < cols / 2) return fail(FP8BQ_E_INVAL, "%s: ldq (bytes) < 1.5 * cols", who);   // ldq < 3 (cols / 2)
  if (lds < rows) return fail(FP8BQ_E_INVAL, "%s: lds < rows", who);
  // the kernels run 16 rows of one 128-column chunk per workgroup: the grid holds ceil(rows / 16) * (cols / 128)
  if (rows >= kMaxTiles || product_at_least(ceil_div(rows, 16), cols / 128, kMaxTiles))
    return fail(FP8BQ_E_SHAPE, "%s: too large", who);
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(s, 4))
    return fail(FP8BQ_E_ALIGN, "%s: bf16 and code buffers must be 16-byte aligned, s 4-byte aligned", who);
  if (ld16 % 8 || ldq % 16) return fail(FP8BQ_E_ALIGN, "%s: bf16 ld must be a multiple of 8 and ldq of 16", who);
  return check_device();
}

int fp8bq_cache_e5m6_1x128(const void* x, int64_t rows, int64_t cols, int64_t ldx, void* q, int64_t ldq, float* s,
                           int64_t lds, void* stream) {
  if (int st = check_e5m6("cache_e5m6", x, q, s, rows, cols, ldx, ldq, lds)) return st;
  return launched(fp8bq::launch_cache_e5m6(static_cast<const uint16_t*>(x), rows, cols, ldx, static_cast<uint8_t*>(q),
                                           ldq, s, lds, reinterpret_cast<hipStream_t>(stream)), "cache_e5m6");
}

int fp8bq_uncache_e5m6_1x128(const void* q, int64_t rows, int64_t cols, int64_t ldq, const float* s, int64_t lds,
                             void* y, int64_t ldy, void* stream) {
  if (int st = check_e5m6("uncache_e5m6", y, q, s, rows, cols, ldy, ldq, lds)) return st;
  return launched(fp8bq::launch_uncache_e5m6(static_cast<const uint8_t*>(q), rows, cols, ldq, s, lds,
                                             static_cast<uint16_t*>(y), ldy, reinterpret_cast<hipStream_t>(stream)),
                  "uncache_e5m6");
}

int fp8bq_requant_e5m6_t_128x1(const void* q, int64_t rows, int64_t cols, int64_t ldq, const float* s, int64_t lds,
                                void* qt, int64_t ldqt, float* st, int64_t ldst, void* stream) {
  if (!q || !s || !qt || !st) return fail(FP8BQ_E_INVAL, "requant_e5m6_t: null pointer");
  if (rows <= 0 || cols <= 0) return fail(FP8BQ_E_INVAL, "requant_e5m6_t: rows and cols must be positive");
  if (rows % 128 || cols % 128)
    return fail(FP8BQ_E_SHAPE, "requant_e5m6_t: rows (%lld) and cols (%lld) must be multiples of 128", (long long)rows,
                (long long)cols);
  if (ldq / 3 < cols / 2) return fail(FP8BQ_E_INVAL, "requant_e5m6_t: ldq (bytes) < 1.5 * cols");
  if (ldqt < rows) return fail(FP8BQ_E_INVAL, "requant_e5m6_t: ldqt must be >= rows");
  if (lds < rows || ldst < cols) return fail(FP8BQ_E_INVAL, "requant_e5m6_t: lds must be >= rows and ldst >= cols");
  if (cols / 128 > 65535 || rows / 128 > ((int64_t)1 << 31) - 1) return fail(FP8BQ_E_SHAPE, "requant_e5m6_t: too large");
  if (!aligned(q, 16) || !aligned(qt, 16) || !aligned(s, 4) || !aligned(st, 4))
    return fail(FP8BQ_E_ALIGN, "requant_e5m6_t: q and qt must be 16-byte aligned, scales 4-byte aligned");
  if (ldq % 16 || ldqt % 16) return fail(FP8BQ_E_ALIGN, "requant_e5m6_t: ldq and ldqt must be multiples of 16");
  if (int stt = check_device()) return stt;
  return launched(fp8bq::launch_requant_e5m6_t(static_cast<const uint8_t*>(q), rows, cols, ldq, s, lds,
                                               static_cast<uint8_t*>(qt), ldqt, st, ldst,
                                               reinterpret_cast<hipStream_t>(stream)), "requant_e5m6_t");
}

int fp8bq_requant_t_128x1(const void* q, int64_t rows, int64_t cols, int64_t ldq, const float* s, int64_t lds,
                          void* qt, int64_t ldqt, float* st, int64_t ldst, int flags, void* stream) {
  if (!q || !s || !qt || !st) return fail(FP8BQ_E_INVAL, "requant_t: null pointer");
  if (flags & ~FP8BQ_SCALE_POW2) return fail(FP8BQ_E_INVAL, "requant_t: unknown flags %d", flags);
  if (rows <= 0 || cols <= 0) return fail(FP8BQ_E_INVAL, "requant_t: rows and cols must be positive");
  if (ldq < cols || ldqt < rows) return fail(FP8BQ_E_INVAL, "requant_t: ldq must be >= cols and ldqt >= rows");
  if (lds < rows || ldst < cols) return fail(FP8BQ_E_INVAL, "requant_t: lds must be >= rows and ldst >= cols");
  if (rows % 128 || cols % 128)
    return fail(FP8BQ_E_SHAPE, "requant_t: rows (%lld) and cols (%lld) must be multiples of 128", (long long)rows, (long long)cols);
  if (cols / 128 > 65535 || rows / 128 > ((int64_t)1 << 31) - 1) return fail(FP8BQ_E_SHAPE, "requant_t: too large");
  if (!aligned(q, 16) || !aligned(qt, 16) || !aligned(s, 4) || !aligned(st, 4))
    return fail(FP8BQ_E_ALIGN, "requant_t: q and qt must be 16-byte aligned, scales 4-byte aligned");
  if (ldq % 16 || ldqt % 16) return fail(FP8BQ_E_ALIGN, "requant_t: ldq and ldqt must be multiples of 16");
  if (int stt = check_device()) return stt;
  return launched(fp8bq::launch_requant_t(static_cast<const uint8_t*>(q), rows, cols, ldq, s, lds,
                                          static_cast<uint8_t*>(qt), ldqt, st, ldst, (flags & FP8BQ_SCALE_POW2) != 0,
                                          reinterpret_cast<hipStream_t>(stream)), "requant_t");
}

int fp8bq_quant_w_128x128(const void* w, int64_t n, int64_t k, int64_t ldw, void* q, int64_t ldq,
                          float* s, int64_t lds, void* qt, int64_t ldqt, int flags, void* stream) {
  if (!w || !q || !s) return fail(FP8BQ_E_INVAL, "quant_w: null pointer");
  if (flags & ~FP8BQ_SCALE_POW2) return fail(FP8BQ_E_INVAL, "quant_w: unknown flags %d", flags);
  if (n <= 0 || k <= 0) return fail(FP8BQ_E_INVAL, "quant_w: n and k must be positive");
  if (ldw < k || ldq < k) return fail(FP8BQ_E_INVAL, "quant_w: ldw and ldq must be >= k");
  if (lds < k / 128) return fail(FP8BQ_E_INVAL, "quant_w: lds must be >= k / 128");
  if (qt && ldqt < n) return fail(FP8BQ_E_INVAL, "quant_w: ldqt must be >= n");
  if (n % 128 || k % 128) return fail(FP8BQ_E_SHAPE, "quant_w: n (%lld) and k (%lld) must be multiples of 128", (long long)n, (long long)k);
  if (n / 128 > 65535 || k / 128 > ((int64_t)1 << 31) - 1) return fail(FP8BQ_E_SHAPE, "quant_w: too large");
  if (!aligned(w, 16) || !aligned(q, 16) || !aligned(s, 4) || (qt && !aligned(qt, 16)))
    return fail(FP8BQ_E_ALIGN, "quant_w: w, q, qt must be 16-byte aligned, s 4-byte aligned");
  if (ldw % 8 || ldq % 16 || (qt && ldqt % 16))
    return fail(FP8BQ_E_ALIGN, "quant_w: ldw must be a multiple of 8, ldq and ldqt of 16");
  if (int st = check_device()) return st;
  return launched(fp8bq::launch_quant_w(static_cast<const uint16_t*>(w), n, k, ldw, static_cast<uint8_t*>(q),
                                        ldq, s, lds, static_cast<uint8_t*>(qt), ldqt,
                                        (flags & FP8BQ_SCALE_POW2) != 0,
                                        reinterpret_cast<hipStream_t>(stream)), "quant_w");
}

namespace {

int check_gemm_common(const char* who, int64_t m, int64_t n, int64_t k, const void* a, int64_t lda,
                      const float* sa, const void* b, int64_t ldb, const float* sb, const void* out,
                      int64_t ldo, int out_elem_bytes) {
  if (!a || !b || !sa || !sb || !out) return fail(FP8BQ_E_INVAL, "%s: null pointer", who);
  if (m <= 0 || n <= 0 || k <= 0) return fail(FP8BQ_E_INVAL, "%s: m, n, k must be positive", who);
  if (lda < k || ldb < k) return fail(FP8BQ_E_INVAL, "%s: lda and ldb must be >= k", who);
  if (ldo < n) return fail(FP8BQ_E_INVAL, "%s: ldo must be >= n", who);
  if (k % 128 || n % 128) return fail(FP8BQ_E_SHAPE, "%s: k (%lld) and n (%lld) must be multiples of 128", who, (long long)k, (long long)n);
  if (product_at_least(ceil_div(m, 256), ceil_div(n, 128), kMaxTiles)) return fail(FP8BQ_E_SHAPE, "%s: too many tiles", who);
  if (lda >= ((int64_t)1 << 23) || ldb >= ((int64_t)1 << 23))
    return fail(FP8BQ_E_SHAPE, "%s: lda and ldb must be below 2^23 (256 rows within 2 GiB)", who);
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(out, 16) || !aligned(sa, 4) || !aligned(sb, 4))
    return fail(FP8BQ_E_ALIGN, "%s: a, b, out must be 16-byte aligned, scales 4-byte aligned", who);
  if (lda % 16 || ldb % 16 || ((ldo % 16) * out_elem_bytes) % 16)
    return fail(FP8BQ_E_ALIGN, "%s: lda, ldb must be multiples of 16 and ldo*sizeof(out) of 16 bytes", who);
  return FP8BQ_OK;
}

}  // namespace

int fp8bq_gemm(int op_flags, int64_t m, int64_t n, int64_t k, const void* a, int64_t lda, const float* sa,
               int64_t ldsa, const void* b, int64_t ldb, const float* sb, int64_t ldsb, void* out,
               int64_t ldo, void* stream) {
  const bool pow2 = (op_flags & FP8BQ_SCALE_POW2) != 0;
  const int op = op_flags & ~FP8BQ_SCALE_POW2;
  if (op != FP8BQ_FPROP && op != FP8BQ_DGRAD && op != FP8BQ_WGRAD)
    return fail(FP8BQ_E_INVAL, "gemm: op must be FPROP (0), DGRAD (1) or WGRAD (2), optionally | SCALE_POW2, got %d",
                op_flags);
  if (int st = check_gemm_common("gemm", m, n, k, a, lda, sa, b, ldb, sb, out, ldo, op == FP8BQ_WGRAD ? 4 : 2))
    return st;
  if (ldsa < m) return fail(FP8BQ_E_INVAL, "gemm: ldsa must be >= m");
  if (op == FP8BQ_FPROP && ldsb < k / 128) return fail(FP8BQ_E_INVAL, "gemm: FPROP ldsb must be >= k / 128");
  if (op == FP8BQ_DGRAD && ldsb < n / 128) return fail(FP8BQ_E_INVAL, "gemm: DGRAD ldsb must be >= n / 128");
  if (op == FP8BQ_WGRAD && ldsb < n) return fail(FP8BQ_E_INVAL, "gemm: WGRAD ldsb must be >= n");
  if (int st = check_device()) return st;
  return launched(fp8bq::launch_gemm(op, m, n, k, static_cast<const uint8_t*>(a), lda, sa, ldsa,
                                     static_cast<const uint8_t*>(b), ldb, sb, ldsb, out, ldo, pow2,
                                     reinterpret_cast<hipStream_t>(stream)), "gemm");
}

int fp8bq_gemm_quant(int op_flags, int64_t m, int64_t n, int64_t k, const void* a, int64_t lda,
                     const float* sa, int64_t ldsa, const void* b, int64_t ldb, const float* sb, int64_t ldsb,
                     void* out, int64_t ldo, void* q, int64_t ldq, float* s, int64_t lds, int qflags,
                     void* stream) {
  const bool pow2 = (op_flags & FP8BQ_SCALE_POW2) != 0;
  const int op = op_flags & ~FP8BQ_SCALE_POW2;
  if (op != FP8BQ_FPROP && op != FP8BQ_DGRAD)
    return fail(FP8BQ_E_INVAL, "gemm_quant: op must be FPROP (0) or DGRAD (1), optionally | SCALE_POW2, got %d",
                op_flags);
  if (qflags & ~FP8BQ_SCALE_POW2) return fail(FP8BQ_E_INVAL, "gemm_quant: unknown qflags %d", qflags);
  if (!q || !s) return fail(FP8BQ_E_INVAL, "gemm_quant: null q or s");
  // the bf16 output is optional: validate it when given, else the checks run on q
  if (int st = check_gemm_common("gemm_quant", m, n, k, a, lda, sa, b, ldb, sb, out ? out : q,
                                 out ? ldo : n, 2))
    return st;
  if (ldsa < m) return fail(FP8BQ_E_INVAL, "gemm_quant: ldsa must be >= m");
  if (op == FP8BQ_FPROP && ldsb < k / 128) return fail(FP8BQ_E_INVAL, "gemm_quant: FPROP ldsb must be >= k / 128");
  if (op == FP8BQ_DGRAD && ldsb < n / 128) return fail(FP8BQ_E_INVAL, "gemm_quant: DGRAD ldsb must be >= n / 128");
  if (ldq < n) return fail(FP8BQ_E_INVAL, "gemm_quant: ldq must be >= n");
  if (lds < m) return fail(FP8BQ_E_INVAL, "gemm_quant: lds must be >= m");
  if (!aligned(q, 16) || ldq % 16 || !aligned(s, 4))
    return fail(FP8BQ_E_ALIGN, "gemm_quant: q must be 16-byte aligned with ldq a multiple of 16, s 4-byte aligned");
  if (int st = check_device()) return st;
  return launched(fp8bq::launch_gemm_quant(op, m, n, k, static_cast<const uint8_t*>(a), lda, sa, ldsa,
                                           static_cast<const uint8_t*>(b), ldb, sb, ldsb,
                                           static_cast<uint16_t*>(out), ldo, static_cast<uint8_t*>(q), ldq, s, lds,
                                           pow2, (qflags & FP8BQ_SCALE_POW2) != 0,
                                           reinterpret_cast<hipStream_t>(stream)),
                  "gemm_quant");
}

int fp8bq_grouped_gemm(int32_t groups, const int64_t* row_off, int64_t n, int64_t k, const void* a,
                       int64_t lda, const float* sa, int64_t ldsa, const void* b, int64_t ldb,
                       const float* sb, int64_t ldsb, void* out, int64_t ldo, int flags, void* stream) {
  if (flags & ~FP8BQ_SCALE_POW2) return fail(FP8BQ_E_INVAL, "grouped_gemm: unknown flags %d", flags);
  if (groups < 1 || groups > fp8bq::kMaxGroups)
    return fail(FP8BQ_E_INVAL, "grouped_gemm: groups must be in [1, %d], got %d", fp8bq::kMaxGroups, groups);
  if (!row_off) return fail(FP8BQ_E_INVAL, "grouped_gemm: null row_off");
  if (row_off[0] != 0) return fail(FP8BQ_E_SHAPE, "grouped_gemm: row_off[0] must be 0");
  for (int e = 0; e < groups; ++e) {
    if (row_off[e + 1] < row_off[e]) return fail(FP8BQ_E_SHAPE, "grouped_gemm: row_off must be non-decreasing (at %d)", e);
    if (row_off[e + 1] % 128) return fail(FP8BQ_E_SHAPE, "grouped_gemm: row_off[%d] = %lld is not a multiple of 128", e + 1, (long long)row_off[e + 1]);
  }
  const int64_t m = row_off[groups];
  if (m / 128 >= ((int64_t)1 << 30)) return fail(FP8BQ_E_SHAPE, "grouped_gemm: too many rows");
  if (int st = check_gemm_common("grouped_gemm", m > 0 ? m : 1, n, k, a, lda, sa, b, ldb, sb, out, ldo, 2))
    return st;
  if (ldsa < m) return fail(FP8BQ_E_INVAL, "grouped_gemm: ldsa must be >= m");
  if (ldsb < k / 128) return fail(FP8BQ_E_INVAL, "grouped_gemm: ldsb must be >= k / 128");
  if (int st = check_device()) return st;
  if (m == 0) return FP8BQ_OK;
  return launched(fp8bq::launch_grouped_gemm(groups, row_off, n, k, static_cast<const uint8_t*>(a), lda, sa, ldsa,
                                             static_cast<const uint8_t*>(b), ldb, sb, ldsb,
                                             static_cast<uint16_t*>(out), ldo, (flags & FP8BQ_SCALE_POW2) != 0,
                                             reinterpret_cast<hipStream_t>(stream)),
                  "grouped_gemm");
}

// Offsets of a decode-shape launch: G in range, row_off[0] == 0,
// non-decreasing, at most kMaxDecodeRows rows per expert.
static int check_decode_offsets(const char* who, int32_t groups, const int64_t* row_off) {
  if (groups < 1 || groups > fp8bq::kMaxGroups)
    return fail(FP8BQ_E_INVAL, "%s: groups must be in [1, %d], got %d", who, fp8bq::kMaxGroups, groups);
  if (!row_off) return fail(FP8BQ_E_INVAL, "%s: null row_off", who);
  if (row_off[0] != 0) return fail(FP8BQ_E_SHAPE, "%s: row_off[0] must be 0", who);
  for (int e = 0; e < groups; ++e) {
    const int64_t rows = row_off[e + 1] - row_off[e];
    if (rows < 0) return fail(FP8BQ_E_SHAPE, "%s: row_off must be non-decreasing (at %d)", who, e);
    if (rows > fp8bq::kMaxDecodeRows)
      return fail(FP8BQ_E_SHAPE, "%s: group %d has %lld rows, at most %d", who, e, (long long)rows,
                  fp8bq::kMaxDecodeRows);
  }
  return FP8BQ_OK;
}

static int check_decode(const char* who, int32_t groups, const int64_t* row_off, int64_t n, int64_t k,
                        const void* a, int64_t lda, const float* sa, int64_t ldsa, const void* b, int64_t ldb,
                        const float* sb, int64_t ldsb, void* out, int64_t ldo, int flags) {
  if (flags != 0) return fail(FP8BQ_E_INVAL, "%s: flags must be 0, got %d", who, flags);
  if (int st = check_decode_offsets(who, groups, row_off)) return st;
  const int64_t m = row_off[groups];
  if (int st = check_gemm_common(who, m > 0 ? m : 1, n, k, a, lda, sa, b, ldb, sb, out, ldo, 2)) return st;
  if (product_at_least(groups, n / 64, (int64_t)1 << 31)) return fail(FP8BQ_E_SHAPE, "%s: too many column slices", who);
  if (ldsa < m) return fail(FP8BQ_E_INVAL, "%s: ldsa must be >= m", who);
  if (ldsb < k / 128) return fail(FP8BQ_E_INVAL, "%s: ldsb must be >= k / 128", who);
  return FP8BQ_OK;
}

int fp8bq_grouped_gemm_decode(int32_t groups, const int64_t* row_off, int64_t n, int64_t k, const void* a,
                              int64_t lda, const float* sa, int64_t ldsa, const void* b, int64_t ldb,
                              const float* sb, int64_t ldsb, void* out, int64_t ldo, int flags, void* stream) {
  if (int st = check_decode("grouped_gemm_decode", groups, row_off, n, k, a, lda, sa, ldsa, b, ldb, sb, ldsb, out,
                            ldo, flags))
    return st;
  if (int st = check_device()) return st;
  if (row_off[groups] == 0) return FP8BQ_OK;
  return launched(fp8bq::launch_grouped_gemm_decode(groups, row_off, n, k, static_cast<const uint8_t*>(a), lda, sa,
                                                    ldsa, static_cast<const uint8_t*>(b), ldb, sb, ldsb,
                                                    static_cast<uint16_t*>(out), ldo, nullptr,
                                                    reinterpret_cast<hipStream_t>(stream)),
                  "grouped_gemm_decode");
}

int fp8bq_grouped_gemm_decode_workspace_size(int32_t groups, const int64_t* row_off, int64_t n, int64_t k,
                                             int64_t* bytes) {
  if (!bytes) return fail(FP8BQ_E_INVAL, "grouped_gemm_decode_workspace_size: null bytes");
  if (int st = check_decode_offsets("grouped_gemm_decode_workspace_size", groups, row_off)) return st;
  if (n <= 0 || k <= 0 || n % 128 || k % 128)
    return fail(FP8BQ_E_SHAPE, "grouped_gemm_decode_workspace_size: n and k must be positive multiples of 128");
  if (product_at_least(groups, n / 64, (int64_t)1 << 31))
    return fail(FP8BQ_E_SHAPE, "grouped_gemm_decode_workspace_size: too many column slices");
  *bytes = fp8bq::grouped_gemm_decode_workspace(groups, row_off, n, k);
  return FP8BQ_OK;
}

int fp8bq_grouped_gemm_decode_ws(int32_t groups, const int64_t* row_off, int64_t n, int64_t k, const void* a,
                                 int64_t lda, const float* sa, int64_t ldsa, const void* b, int64_t ldb,
                                 const float* sb, int64_t ldsb, void* out, int64_t ldo, void* workspace,
                                 int64_t workspace_bytes, int flags, void* stream) {
  if (int st = check_decode("grouped_gemm_decode_ws", groups, row_off, n, k, a, lda, sa, ldsa, b, ldb, sb, ldsb, out,
                            ldo, flags))
    return st;
  const int64_t need = fp8bq::grouped_gemm_decode_workspace(groups, row_off, n, k);
  if (need > 0 && !workspace) return fail(FP8BQ_E_INVAL, "grouped_gemm_decode_ws: null workspace (%lld bytes needed)", (long long)need);
  if (need > 0 && workspace_bytes < need)
    return fail(FP8BQ_E_INVAL, "grouped_gemm_decode_ws: workspace of %lld bytes, %lld needed", (long long)workspace_bytes,
                (long long)need);
  if (need > 0 && !aligned(workspace, 16)) return fail(FP8BQ_E_ALIGN, "grouped_gemm_decode_ws: workspace must be 16-byte aligned");
  if (int st = check_device()) return st;
  if (row_off[groups] == 0) return FP8BQ_OK;
  return launched(fp8bq::launch_grouped_gemm_decode(groups, row_off, n, k, static_cast<const uint8_t*>(a), lda, sa,
                                                    ldsa, static_cast<const uint8_t*>(b), ldb, sb, ldsb,
                                                    static_cast<uint16_t*>(out), ldo, need > 0 ? workspace : nullptr,
                                                    reinterpret_cast<hipStream_t>(stream)),
                  "grouped_gemm_decode_ws");
}

int fp8bq_grouped_gemm_decode_noalloc(int32_t groups, const int64_t* row_off, int64_t n, int64_t k, const void* a,
                                      int64_t lda, const float* sa, int64_t ldsa, const void* b, int64_t ldb,
                                      const float* sb, int64_t ldsb, void* out, int64_t ldo, int flags,
                                      void* stream) {
  if (int st = check_decode("grouped_gemm_decode_noalloc", groups, row_off, n, k, a, lda, sa, ldsa, b, ldb, sb, ldsb,
                            out, ldo, flags))
    return st;
  const int64_t need = fp8bq::grouped_gemm_decode_workspace(groups, row_off, n, k);
  if (need > fp8bq::kNoAllocScratchBytes)
    return fail(FP8BQ_E_SHAPE,
                "grouped_gemm_decode_noalloc: these experts need %lld bytes of scratch, the library holds %lld per "
                "device (pass a workspace to fp8bq_grouped_gemm_decode_ws instead)",
                (long long)need, (long long)fp8bq::kNoAllocScratchBytes);
  if (int st = check_device()) return st;
  if (row_off[groups] == 0) return FP8BQ_OK;
  const hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  return launched(need > 0
                      ? fp8bq::launch_grouped_gemm_decode_noalloc(groups, row_off, n, k, static_cast<const uint8_t*>(a),
                                                                  lda, sa, ldsa, static_cast<const uint8_t*>(b), ldb,
                                                                  sb, ldsb, static_cast<uint16_t*>(out), ldo, hs)
                      : fp8bq::launch_grouped_gemm_decode(groups, row_off, n, k, static_cast<const uint8_t*>(a), lda,
                                                          sa, ldsa, static_cast<const uint8_t*>(b), ldb, sb, ldsb,
                                                          static_cast<uint16_t*>(out), ldo, nullptr, hs),
                  "grouped_gemm_decode_noalloc");
}

}  // extern "C"
