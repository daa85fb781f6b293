// Launcher of the block-scaled FP8 GEMM (fp8bq_gemm): the VALU-promotion
// kernel for general scales, the scaled-MFMA kernel for power-of-two scales.
#include "gemm_kernels.h"

namespace fp8bq {

hipError_t launch_gemm(int kind, int64_t m, int64_t n, int64_t k, const uint8_t* a, int64_t lda,
                       const float* sa, int64_t ldsa, const uint8_t* b, int64_t ldb,
                       const float* sb, int64_t ldsb, void* out, int64_t ldo, bool pow2, hipStream_t st) {
  GemmArgs p = make_args(m, n, k, a, lda, sa, ldsa, b, ldb, sb, ldsb, out, ldo);
  GroupArgs g;
  g.groups = 0;
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
