// Internal declarations shared by the host entry points and the kernel files.
// Nothing here is part of the C ABI (include/fp8bq.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8bq {

// Launchers. Arguments have been validated by the entry points; each returns
// the hipError_t of its launch.
// pow2: power-of-two scales (otherwise s = absmax / 448).
hipError_t launch_quant_act_rows(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                                 uint8_t* q, int64_t ldq, float* s, int64_t lds, bool pow2, hipStream_t st);
hipError_t launch_quant_act_cols(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                                 uint8_t* qt, int64_t ldq, float* s, int64_t lds, bool pow2, hipStream_t st);
hipError_t launch_quant_w(const uint16_t* w, int64_t n, int64_t k, int64_t ldw, uint8_t* q,
                          int64_t ldq, float* s, int64_t lds, uint8_t* qt, int64_t ldqt,
                          bool pow2, hipStream_t st);
// pow2_hint: the caller's scales are powers of two (same result, faster kernel).
hipError_t launch_requant_t(const uint8_t* q, int64_t rows, int64_t cols, int64_t ldq, const float* s,
                            int64_t lds, uint8_t* qt, int64_t ldqt, float* st, int64_t ldst, bool pow2_hint,
                            hipStream_t stream);

// E5M6 activation cache: bf16 [rows, cols] -> packed 12-bit codes (1.5 B per
// element, ldq in bytes) + chunk-major power-of-two scales, and back to bf16.
hipError_t launch_cache_e5m6(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, uint8_t* q, int64_t ldq,
                             float* s, int64_t lds, hipStream_t st);
hipError_t launch_uncache_e5m6(const uint8_t* q, int64_t rows, int64_t cols, int64_t ldq, const float* s,
                               int64_t lds, uint16_t* y, int64_t ldy, hipStream_t st);
// E5M6 cache -> transposed 128x1 FP8 tiles with power-of-two scales.
hipError_t launch_requant_e5m6_t(const uint8_t* q, int64_t rows, int64_t cols, int64_t ldq, const float* s,
                                  int64_t lds, uint8_t* qt, int64_t ldqt, float* st, int64_t ldst, hipStream_t stream);

enum GemmKind { KIND_FPROP = 0, KIND_DGRAD = 1, KIND_WGRAD = 2 };

hipError_t launch_gemm(int kind, int64_t m, int64_t n, int64_t k, const uint8_t* a, int64_t lda,
                       const float* sa, int64_t ldsa, const uint8_t* b, int64_t ldb,
                       const float* sb, int64_t ldsb, void* out, int64_t ldo, bool pow2, hipStream_t st);

// Largest group count the grouped GEMM accepts (offsets travel as kernel arguments).
constexpr int kMaxGroups = 256;
constexpr int kMaxDecodeRows = 256;   // rows per group of the decode-shape grouped GEMM
// Split decode workspace: one counter per (expert, 128-column slice) at a fixed
// place, for up to kDecodeSlices slices (n <= 32768), then the partial sums.
constexpr int kDecodeSlices = 256;
constexpr int64_t kDecodeCounterBytes = (int64_t)kMaxGroups * kDecodeSlices * 4;

// The same with a quantised copy of the bf16 output (FPROP / DGRAD only):
// q [m, n] (ldq) with chunk-major 1x128 scales sq[c * ldsq + row]; out may be
// null. out_pow2 selects power-of-two output scales.
hipError_t launch_gemm_quant(int kind, int64_t m, int64_t n, int64_t k, const uint8_t* a, int64_t lda,
                             const float* sa, int64_t ldsa, const uint8_t* b, int64_t ldb, const float* sb,
                             int64_t ldsb, uint16_t* out, int64_t ldo, uint8_t* q, int64_t ldq, float* sq,
                             int64_t ldsq, bool pow2, bool out_pow2, hipStream_t st);
hipError_t launch_grouped_gemm(int groups, const int64_t* row_off, int64_t n, int64_t k,
                               const uint8_t* a, int64_t lda, const float* sa, int64_t ldsa,
                               const uint8_t* b, int64_t ldb, const float* sb, int64_t ldsb,
                               uint16_t* out, int64_t ldo, bool pow2, hipStream_t st);
// Grouped Fprop for decode-sized experts (each at most 256 rows, any count):
// row_off host array of groups + 1 row offsets. workspace: null, or at least
// grouped_gemm_decode_workspace() bytes whose counters are zero (every call
// leaves them zero); with it, experts of more than 32 rows run as 128-column,
// half-K workgroup pairs.
hipError_t launch_grouped_gemm_decode(int groups, const int64_t* row_off, int64_t n, int64_t k,
                                      const uint8_t* a, int64_t lda, const float* sa, int64_t ldsa,
                                      const uint8_t* b, int64_t ldb, const float* sb, int64_t ldsb,
                                      uint16_t* out, int64_t ldo, void* workspace, hipStream_t st);
// Bytes of workspace the split form needs (0: nothing would be split).
int64_t grouped_gemm_decode_workspace(int groups, const int64_t* row_off, int64_t n, int64_t k);
// The split form with the library's own scratch (kNoAllocScratchBytes per
// device, a static device array) as its workspace: allocates nothing. The
// caller has checked that the workspace it needs fits.
constexpr int64_t kNoAllocScratchBytes = (int64_t)32 << 20;
hipError_t launch_grouped_gemm_decode_noalloc(int groups, const int64_t* row_off, int64_t n, int64_t k,
                                              const uint8_t* a, int64_t lda, const float* sa, int64_t ldsa,
                                              const uint8_t* b, int64_t ldb, const float* sb, int64_t ldsb,
                                              uint16_t* out, int64_t ldo, hipStream_t st);

}  // namespace fp8bq
