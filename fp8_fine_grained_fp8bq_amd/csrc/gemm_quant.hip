// Launcher of the GEMM whose epilogue also quantises its bf16 output
// (fp8bq_gemm_quant): the same kernels with the quantising epilogue.
#include "gemm_kernels.h"

namespace fp8bq {

hipError_t launch_gemm_quant(int kind, int64_t m, int64_t n, int64_t k, const uint8_t* a, int64_t lda,
                             const float* sa, int64_t ldsa, const uint8_t* b, int64_t ldb, const float* sb,
                             int64_t ldsb, uint16_t* out, int64_t ldo, uint8_t* q, int64_t ldq, float* sq,
                             int64_t ldsq, bool pow2, bool out_pow2, hipStream_t st) {
  GemmArgs p = make_args(m, n, k, a, lda, sa, ldsa, b, ldb, sb, ldsb, out, ldo);
  p.q = q; p.ldq = ldq; p.sq = sq; p.ldsq = ldsq;
  GroupArgs g;
  g.groups = 0;
  const dim3 grid((unsigned)persistent_grid(p.tiles_m * p.tiles_n)), block(kBlock);
  const bool dg = kind == KIND_DGRAD;
  if (pow2) {
    const dim3 block4(256);
    if (out_pow2) {
      if (dg) hipLaunchKernelGGL((gemm_pow2_kernel<KIND_DGRAD, false, 2>), grid, block4, 0, st, p, g);
      else    hipLaunchKernelGGL((gemm_pow2_kernel<KIND_FPROP, false, 2>), grid, block4, 0, st, p, g);
    } else {
      if (dg) hipLaunchKernelGGL((gemm_pow2_kernel<KIND_DGRAD, false, 1>), grid, block4, 0, st, p, g);
      else    hipLaunchKernelGGL((gemm_pow2_kernel<KIND_FPROP, false, 1>), grid, block4, 0, st, p, g);
    }
    return hipGetLastError();
  }
  if (out_pow2) {
    if (dg) hipLaunchKernelGGL((gemm_kernel<KIND_DGRAD, false, kWM, kWN, kLd, 2>), grid, block, 0, st, p, g);
    else    hipLaunchKernelGGL((gemm_kernel<KIND_FPROP, false, kWM, kWN, kLd, 2>), grid, block, 0, st, p, g);
  } else {
    if (dg) hipLaunchKernelGGL((gemm_kernel<KIND_DGRAD, false, kWM, kWN, kLd, 1>), grid, block, 0, st, p, g);
    else    hipLaunchKernelGGL((gemm_kernel<KIND_FPROP, false, kWM, kWN, kLd, 1>), grid, block, 0, st, p, g);
  }
  return hipGetLastError();
}

}  // namespace fp8bq
