// Block-scaled FP8 GEMM with per-128-K-chunk promotion into FP32, for gfx950.
//
//   out[i][j] = sum_c P_c[i][j] * sa(i, c) * sb(j, c),
//   P_c[i][j] = sum_{k in chunk c} a[i][k] * b[j][k]     (E4M3 x E4M3, exact products)
//
// This is the FP8 GEMM of the DeepSeek-V3 report (Chinese translation), section
// 3.3.2 "increasing accumulation precision" and Figure 7b: every N_C = 128
// K-elements the matrix-core partial sum is promoted to FP32 registers, where
// it is multiplied by both operands' group scales and added (the tech note
// "DeepSeek-V3 FP8 dynamic quantisation": out += MMA(FP8 x, FP8 w) * s_x * s_w).
// On the pages' hardware the promotion moves partial sums from tensor cores to
// CUDA cores; on CDNA4 the MFMA writes its result straight into VGPRs, so the
// "promotion" is one VALU FMA per output per chunk into a second accumulator.
//
// Design (MI355X / gfx950):
//  * One v_mfma_f32_16x16x128_f8f6f4 covers a whole 128-K chunk of a 16x16
//    tile, so each chunk's partial sum is a fresh MFMA result (C = 0) that is
//    folded into the FP32 accumulator with acc = fma(P, scale, acc).
//  * The weight tile is the MFMA's first operand and the activation tile its
//    second, so a lane's four result registers are four consecutive output
//    columns j of one output row i: one activation scale per (lane, 16-row
//    subtile) per chunk and 8-byte (bf16) / 16-byte (fp32) output stores.
//  * Workgroup tile 256 x 256, 8 waves (2 per SIMD) of 64 (i) x 128 (j):
//    128 accumulator VGPRs per lane, 32 MFMAs per wave per chunk.
//  * Operands stream global -> LDS with global_load_lds_dwordx4 (no VGPR
//    staging), two 66 KB stages (A 32 KB, B 32 KB, scales 2 KB), one barrier
//    per chunk; the next chunk's loads run under the current chunk's MFMAs.
//  * LDS rows are 128 bytes (one chunk); the 16-byte slots of row r are
//    XOR-swizzled by (r & 7) so the MFMA operand reads spread over the banks.
//  * Workgroups are remapped so that each XCD (own L2) gets a contiguous range
//    of output tiles, walked in groups of 8 row-tiles: the blocks resident on
//    one XCD share activation and weight panels in its L2.
#include "internal.h"

namespace fp8bq {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int BM = 256, BN = 256, BK = 128;
constexpr int kThreads = 512;
constexpr int kWavesM = 4, kWavesN = 2;
constexpr int WM = BM / kWavesM;   // 64
constexpr int WN = BN / kWavesN;   // 128
constexpr int TM = WM / 16;        // 4
constexpr int TN = WN / 16;        // 8
constexpr int kABytes = BM * BK;
constexpr int kBBytes = BN * BK;
constexpr int kSaOff = kABytes + kBBytes;
constexpr int kSbOff = kSaOff + BM * 4;
constexpr int kStage = kSbOff + BN * 4;
constexpr int kGroupM = 8;
constexpr int kXcds = 8;

static_assert(kWavesM * kWavesN * 64 == kThreads, "wave grid");
static_assert(WN == 128, "one weight block column per wave");

struct GemmArgs {
  int64_t m, n, k;
  const uint8_t* a; int64_t lda;
  const float* sa; int64_t ldsa;
  const uint8_t* b; int64_t ldb;
  const float* sb; int64_t ldsb;
  void* out; int64_t ldo;
  int tiles_m, tiles_n;
};

struct GroupArgs {
  int groups;
  int tile_prefix[kMaxGroups + 1];   // first row-tile of each group
  int row_off128[kMaxGroups + 1];    // row offsets in units of 128 rows
};

// Global -> LDS DMA (gfx950 global_load_lds_dword[x4]): lane i's bytes land at
// M0 + i * size. Issued from inline asm so that the compiler does not guard
// every later LDS read with a wait for these loads; the kernel waits itself
// (vmcnt(0) + barrier before a stage is read). Every vector memory load in the
// K-loop goes through these helpers, so vmcnt counts exactly them.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
// M0 is reserved by the compiler; on gfx950 only LDS DMA reads it and the
// compiler itself never keeps a value there across these statements.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* gbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"(gbase), "s"(lds) : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* gbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1"
               :: "v"(voff), "s"(gbase), "s"(lds) : "memory", "m0");
}
#pragma clang diagnostic pop

// Tile position: logical tile index after the XCD remap and the grouped walk.
__device__ __forceinline__ void tile_coords(int tiles_m, int tiles_n, int& tm, int& tn) {
  const int T = tiles_m * tiles_n;
  const int w = blockIdx.x;
  const int q = T / kXcds, r = T % kXcds;
  const int xcd = w % kXcds, local = w / kXcds;
  const int logical = xcd * q + (xcd < r ? xcd : r) + local;
  const int per_group = kGroupM * tiles_n;
  const int group = logical / per_group;
  const int first_m = group * kGroupM;
  const int gsize = min(tiles_m - first_m, kGroupM);
  const int in_group = logical - group * per_group;
  tm = first_m + in_group % gsize;
  tn = in_group / gsize;
}

// One K-chunk of the wave's 64 x 128 tile from one LDS stage: per 16x16 subtile
// one MFMA (fresh partial sum of the chunk) and four FMAs folding it into the
// FP32 accumulator. The two waves sharing a SIMD overlap one's MFMAs with the
// other's FMAs.
template <int KIND>
__device__ __forceinline__ void compute_chunk(const uint8_t* __restrict__ As, v4f (&acc)[TM][TN],
                                              int wave_m, int wave_n, int l16, int lq, int off0,
                                              int off1) {
  const uint8_t* Bs = As + kABytes;
  const float* Sa = reinterpret_cast<const float*>(As + kSaOff);
  const float* Sb = reinterpret_cast<const float*>(As + kSbOff);

  float sc[TM];
#pragma unroll
  for (int i = 0; i < TM; ++i) sc[i] = Sa[wave_m * WM + i * 16 + l16];
  if constexpr (KIND != KIND_WGRAD) {
    const float sbv = Sb[wave_n];
#pragma unroll
    for (int i = 0; i < TM; ++i) sc[i] *= sbv;
  }

  v8i af[TM];
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const uint8_t* rowp = As + (wave_m * WM + i * 16) * BK;
    const uint4 x0 = *reinterpret_cast<const uint4*>(rowp + off0);
    const uint4 x1 = *reinterpret_cast<const uint4*>(rowp + off1);
    af[i] = v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
  }
  auto load_b = [&](int j) {
    const uint8_t* rowp = Bs + (wave_n * WN + j * 16) * BK;
    const uint4 y0 = *reinterpret_cast<const uint4*>(rowp + off0);
    const uint4 y1 = *reinterpret_cast<const uint4*>(rowp + off1);
    return v8i{(int)y0.x, (int)y0.y, (int)y0.z, (int)y0.w, (int)y1.x, (int)y1.y, (int)y1.z, (int)y1.w};
  };
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const v8i bf = load_b(j);
    v4f sbj;
    if constexpr (KIND == KIND_WGRAD) sbj = *reinterpret_cast<const v4f*>(Sb + wave_n * WN + j * 16 + 4 * lq);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const v4f pc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf, af[i], zero, 0, 0, 0, 0, 0, 0);
      if constexpr (KIND == KIND_WGRAD) {
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(pc[r] * sbj[r], sc[i], acc[i][j][r]);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(pc[r], sc[i], acc[i][j][r]);
      }
    }
  }
}

template <int KIND, bool GROUPED>
__global__ __launch_bounds__(kThreads) void gemm_kernel(GemmArgs p, GroupArgs g) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kStage];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wave_m = wave % kWavesM;
  const int wave_n = wave / kWavesM;
  const int l16 = lane & 15, lq = lane >> 4;

  int tmi, tni;
  tile_coords(p.tiles_m, p.tiles_n, tmi, tni);

  // Row range of this tile, and the weight (and its scales) it multiplies.
  int64_t m0, m_end;
  const uint8_t* bmat = p.b;
  const float* sbm = p.sb;
  if constexpr (GROUPED) {
    int lo = 0, hi = g.groups;             // find e: tile_prefix[e] <= tmi < tile_prefix[e+1]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (g.tile_prefix[mid] <= tmi) lo = mid; else hi = mid;
    }
    const int e = lo;
    m0 = (int64_t)g.row_off128[e] * 128 + (int64_t)(tmi - g.tile_prefix[e]) * BM;
    m_end = min(m0 + BM, (int64_t)g.row_off128[e + 1] * 128);
    bmat += (int64_t)e * p.n * p.ldb;
    sbm += (int64_t)e * (p.n / 128) * p.ldsb;
  } else {
    m0 = (int64_t)tmi * BM;
    m_end = min(m0 + BM, p.m);
  }
  const int64_t n0 = (int64_t)tni * BN;
  const int64_t n_end = min(n0 + BN, p.n);
  const int nc = (int)(p.k / BK);

  // ---- per-thread load descriptors (global -> LDS) -------------------------
  // Instruction i of wave w covers tile rows [64 i + 8 w, +8); lane ln fills row
  // 64 i + 8 w + ln / 8, physical slot ln % 8, i.e. logical slot (ln % 8) ^ (row & 7).
  // Offsets are 32-bit relative to the tile's first row (the host checks that
  // 256 rows of either operand span less than 2 GiB).
  const uint8_t* a_tile = p.a + m0 * p.lda;
  const uint8_t* b_tile = bmat + n0 * p.ldb;
  uint32_t a_off[4], b_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 64 * i + 8 * wave + (lane >> 3);
    const int gslot = (lane & 7) ^ (row & 7);
    const int64_t ar = min(m0 + row, m_end - 1) - m0;
    const int64_t br = min(n0 + row, n_end - 1) - n0;
    a_off[i] = (uint32_t)(ar * p.lda + gslot * 16);
    b_off[i] = (uint32_t)(br * p.ldb + gslot * 16);
  }
  // Scales: waves 0-3 fetch 64 activation scales each; wave 4 (block scales) or
  // waves 4-7 (row scales) the weight side. s_base advances s_step floats per chunk.
  const float* s_base;
  uint32_t s_off;
  int64_t s_step;
  if (wave < 4) {
    s_base = p.sa + m0;
    s_off = (uint32_t)(min(m0 + 64 * wave + lane, m_end - 1) - m0) * 4u;
    s_step = p.ldsa;
  } else if (KIND == KIND_WGRAD) {
    s_base = sbm + n0;
    s_off = (uint32_t)(min(n0 + 64 * (wave - 4) + lane, n_end - 1) - n0) * 4u;
    s_step = p.ldsb;
  } else {
    // two 128-column weight blocks per tile; lanes beyond 0 read block 1 (clamped)
    const int64_t blk0 = n0 / 128;
    const int64_t blk = min(blk0 + (lane < 1 ? 0 : 1), n_end / 128 - 1) - blk0;
    if (KIND == KIND_FPROP) { s_base = sbm + blk0 * p.ldsb; s_off = (uint32_t)(blk * p.ldsb) * 4u; s_step = 1; }
    else                    { s_base = sbm + blk0;          s_off = (uint32_t)blk * 4u;            s_step = p.ldsb; }
  }
  const bool loads_scales = wave < 4 || KIND == KIND_WGRAD || wave == 4;
  const uint32_t s_lds = wave < 4 ? kSaOff + 256 * wave : kSbOff + 256 * (wave - 4);
  const uint32_t smem_lds = lds_addr(smem);

  auto issue = [&](int c) {
    const uint32_t base = smem_lds + (uint32_t)((c & 1) * kStage);
    const uint8_t* ak = a_tile + (int64_t)c * BK;
    const uint8_t* bk = b_tile + (int64_t)c * BK;
#pragma unroll
    for (int i = 0; i < 4; ++i) dma16(ak, a_off[i], base + (64 * i + 8 * wave) * BK);
#pragma unroll
    for (int i = 0; i < 4; ++i) dma16(bk, b_off[i], base + kABytes + (64 * i + 8 * wave) * BK);
    if (loads_scales) dma4(s_base + c * s_step, s_off, base + s_lds);
  };

  v4f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // LDS byte offset of this lane's operand slice inside a 16-row subtile whose
  // first row is a multiple of 16: row r = base + l16, logical slots 2 lq, 2 lq + 1.
  const int sw = l16 & 7;
  const int off0 = l16 * BK + (((2 * lq) ^ sw) * 16);
  const int off1 = l16 * BK + (((2 * lq + 1) ^ sw) * 16);

  // Chunk c lives in stage c % 2. After the barrier at the top of step c every
  // wave has finished step c - 1, so stage (c + 1) % 2 can be refilled.
  issue(0);
#pragma clang loop unroll(disable)
  for (int c = 0; c < nc; ++c) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (c + 1 < nc) issue(c + 1);
    compute_chunk<KIND>(smem + (c & 1) * kStage, acc, wave_m, wave_n, l16, lq, off0, off1);
  }

  // ---- epilogue: lane holds out[row][col .. col+3] for each (i, j) ---------
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int64_t row = m0 + wave_m * WM + i * 16 + l16;
    if (row >= m_end) continue;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int64_t col = n0 + wave_n * WN + j * 16 + 4 * lq;
      if (col >= n_end) continue;
      if constexpr (KIND == KIND_WGRAD) {
        float* o = reinterpret_cast<float*>(p.out) + row * p.ldo + col;
        *reinterpret_cast<v4f*>(o) = acc[i][j];
      } else {
        uint32_t h[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const uint32_t u = __float_as_uint(acc[i][j][r]);
          h[r] = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;   // round to nearest even (finite)
        }
        uint16_t* o = reinterpret_cast<uint16_t*>(p.out) + row * p.ldo + col;
        *reinterpret_cast<uint2*>(o) = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
      }
    }
  }
}

GemmArgs make_args(int64_t m, int64_t n, int64_t k, const uint8_t* a, int64_t lda, const float* sa,
                   int64_t ldsa, const uint8_t* b, int64_t ldb, const float* sb, int64_t ldsb,
                   void* out, int64_t ldo) {
  GemmArgs p;
  p.m = m; p.n = n; p.k = k;
  p.a = a; p.lda = lda; p.sa = sa; p.ldsa = ldsa;
  p.b = b; p.ldb = ldb; p.sb = sb; p.ldsb = ldsb;
  p.out = out; p.ldo = ldo;
  p.tiles_m = (int)((m + BM - 1) / BM);
  p.tiles_n = (int)((n + BN - 1) / BN);
  return p;
}

}  // namespace

hipError_t launch_gemm(int kind, int64_t m, int64_t n, int64_t k, const uint8_t* a, int64_t lda,
                       const float* sa, int64_t ldsa, const uint8_t* b, int64_t ldb,
                       const float* sb, int64_t ldsb, void* out, int64_t ldo, hipStream_t st) {
  GemmArgs p = make_args(m, n, k, a, lda, sa, ldsa, b, ldb, sb, ldsb, out, ldo);
  GroupArgs g;
  g.groups = 0;
  const dim3 grid((unsigned)(p.tiles_m * p.tiles_n)), block(kThreads);
  switch (kind) {
    case KIND_FPROP: hipLaunchKernelGGL((gemm_kernel<KIND_FPROP, false>), grid, block, 0, st, p, g); break;
    case KIND_DGRAD: hipLaunchKernelGGL((gemm_kernel<KIND_DGRAD, false>), grid, block, 0, st, p, g); break;
    default:         hipLaunchKernelGGL((gemm_kernel<KIND_WGRAD, false>), grid, block, 0, st, p, g); break;
  }
  return hipGetLastError();
}

hipError_t launch_grouped_gemm(int groups, const int64_t* row_off, int64_t n, int64_t k,
                               const uint8_t* a, int64_t lda, const float* sa, int64_t ldsa,
                               const uint8_t* b, int64_t ldb, const float* sb, int64_t ldsb,
                               uint16_t* out, int64_t ldo, hipStream_t st) {
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
  const dim3 grid((unsigned)(p.tiles_m * p.tiles_n)), block(kThreads);
  hipLaunchKernelGGL((gemm_kernel<KIND_FPROP, true>), grid, block, 0, st, p, g);
  return hipGetLastError();
}

}  // namespace fp8bq
