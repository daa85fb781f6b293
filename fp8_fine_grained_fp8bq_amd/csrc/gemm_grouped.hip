// Launcher of the grouped (per-expert) Fprop (fp8bq_grouped_gemm).
#include "gemm_kernels.h"

namespace fp8bq {

hipError_t launch_grouped_gemm(int groups, const int64_t* row_off, int64_t n, int64_t k,
                               const uint8_t* a, int64_t lda, const float* sa, int64_t ldsa,
                               const uint8_t* b, int64_t ldb, const float* sb, int64_t ldsb,
                               uint16_t* out, int64_t ldo, bool pow2, hipStream_t st) {
  GroupArgs g;
  g.groups = groups;
  int tiles = 0;
  for (int e = 0; e < groups; ++e) {
    g.tile_prefix[e] = tiles;
    g.row_off128[e] = (int)(row_off[e] / 128);
    tiles += (int)((row_off[e + 1] - row_off[e] + BM - 1) / BM);
  }
  g.tile_prefix[groups] = tiles;
  g.row_off128[groups] = (int)(row_off[groups] / 128);
  GemmArgs p = make_args(row_off[groups], n, k, a, lda, sa, ldsa, b, ldb, sb, ldsb, out, ldo);
  p.tiles_m = tiles;
  if (tiles == 0) return hipSuccess;   // every group empty: nothing to compute
  const dim3 grid((unsigned)persistent_grid(p.tiles_m * p.tiles_n)), block(kBlock);
  if (pow2)
    hipLaunchKernelGGL((gemm_pow2_kernel<KIND_FPROP, true>), grid, dim3(256), 0, st, p, g);
  else
    hipLaunchKernelGGL((gemm_kernel<KIND_FPROP, true, kWM, kWN, kLd>), grid, block, 0, st, p, g);
  return hipGetLastError();
}

}  // namespace fp8bq
