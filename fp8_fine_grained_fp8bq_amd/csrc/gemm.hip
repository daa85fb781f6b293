// Launcher of the block-scaled FP8 GEMM (fp8bq_gemm): the VALU-promotion
// kernel for general scales (256 x 256 tiles; 256 x 128 when there are too few
// of those to fill the CUs; 256 x 224 when those finish the walk sooner), the
// scaled-MFMA kernel for power-of-two scales.
#include "gemm_kernels.h"

namespace fp8bq {

// GEMMs with at most this many 256 x 256 tiles (half the CUs or fewer) run
// with 256 x 128 tiles instead: twice the workgroups, each with half the work.
constexpr int64_t kNarrowTiles = 128;

// 256 x 224 tiles when they finish the persistent walk in less time than
// 256 x 256 tiles: rounds of the walk (tiles / CUs, rounded up) times the
// tile's share of a 256 x 256 tile's work (7/8). A backward GEMM with
// n = 7168 and m = 4096 has 448 tiles of 256 x 256 (2 rounds on 256 CUs) or
// 512 of 256 x 224 (2 rounds of 7/8: 1.75); with m = 2048, 224 (one round,
// 32 CUs idle) or 256 (one round of 7/8).
bool prefer_224(int64_t m, int64_t n, int cus) {
  const int64_t tm = (m + BM - 1) / BM;
  const int64_t r256 = (tm * ((n + 255) / 256) + cus - 1) / cus;
  const int64_t r224 = (tm * ((n + 223) / 224) + cus - 1) / cus;
  return r224 * 7 < r256 * 8;
}

hipError_t launch_gemm(int kind, int64_t m, int64_t n, int64_t k, const uint8_t* a, int64_t lda,
                       const float* sa, int64_t ldsa, const uint8_t* b, int64_t ldb,
                       const float* sb, int64_t ldsb, void* out, int64_t ldo, bool pow2, hipStream_t st) {
  GroupArgs g;
  g.groups = 0;
  const int64_t tiles256 = ((m + BM - 1) / BM) * ((n + BN - 1) / BN);
  if (!pow2 && tiles256 <= kNarrowTiles) {
    constexpr int kNarrow = 128;
    GemmArgs p = make_args(m, n, k, a, lda, sa, ldsa, b, ldb, sb, ldsb, out, ldo, kNarrow);
    const dim3 grid((unsigned)persistent_grid(p.tiles_m * p.tiles_n)), block(kBlock);
    switch (kind) {
      case KIND_FPROP: hipLaunchKernelGGL((gemm_kernel<KIND_FPROP, false, kWM, kWN, kLd, 0, kNarrow>), grid, block, 0, st, p, g); break;
      case KIND_DGRAD: hipLaunchKernelGGL((gemm_kernel<KIND_DGRAD, false, kWM, kWN, kLd, 0, kNarrow>), grid, block, 0, st, p, g); break;
      default:         hipLaunchKernelGGL((gemm_kernel<KIND_WGRAD, false, kWM, kWN, kLd, 0, kNarrow>), grid, block, 0, st, p, g); break;
    }
    return hipGetLastError();
  }
  if (!pow2 && prefer_224(m, n, persistent_grid(1 << 30))) {
    constexpr int kT = 224;
    GemmArgs p = make_args(m, n, k, a, lda, sa, ldsa, b, ldb, sb, ldsb, out, ldo, kT);
    const dim3 grid((unsigned)persistent_grid(p.tiles_m * p.tiles_n)), block(kBlock);
    switch (kind) {
      case KIND_FPROP: hipLaunchKernelGGL((gemm_kernel<KIND_FPROP, false, kWM, kWN, kLd, 0, kT>), grid, block, 0, st, p, g); break;
      case KIND_DGRAD: hipLaunchKernelGGL((gemm_kernel<KIND_DGRAD, false, kWM, kWN, kLd, 0, kT>), grid, block, 0, st, p, g); break;
      default:         hipLaunchKernelGGL((gemm_kernel<KIND_WGRAD, false, kWM, kWN, kLd, 0, kT>), grid, block, 0, st, p, g); break;
    }
    return hipGetLastError();
  }
  GemmArgs p = make_args(m, n, k, a, lda, sa, ldsa, b, ldb, sb, ldsb, out, ldo);
  const dim3 grid((unsigned)persistent_grid(p.tiles_m * p.tiles_n)), block(kBlock);
  if (pow2) {
    const dim3 block4(256);
    switch (kind) {
      case KIND_FPROP: hipLaunchKernelGGL((gemm_pow2_kernel<KIND_FPROP, false>), grid, block4, 0, st, p, g); break;
      case KIND_DGRAD: hipLaunchKernelGGL((gemm_pow2_kernel<KIND_DGRAD, false>), grid, block4, 0, st, p, g); break;
      default:         hipLaunchKernelGGL((gemm_pow2_kernel<KIND_WGRAD, false>), grid, block4, 0, st, p, g); break;
    }
    return hipGetLastError();
  }
  switch (kind) {
    case KIND_FPROP: hipLaunchKernelGGL((gemm_kernel<KIND_FPROP, false, kWM, kWN, kLd>), grid, block, 0, st, p, g); break;
    case KIND_DGRAD: hipLaunchKernelGGL((gemm_kernel<KIND_DGRAD, false, kWM, kWN, kLd>), grid, block, 0, st, p, g); break;
    default:         hipLaunchKernelGGL((gemm_kernel<KIND_WGRAD, false, kWM, kWN, kLd>), grid, block, 0, st, p, g); break;
  }
  return hipGetLastError();
}

}  // namespace fp8bq
