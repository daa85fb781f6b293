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
//  * Workgroup tile 256 x 256, 8 waves (two per SIMD) of 64 x 128: 128
//    accumulator VGPRs per lane (the promotion FMAs need the accumulator in the
//    256 VGPRs the VALU can address, which rules out 128 x 128 wave tiles),
//    24 KB of LDS operand reads per wave per chunk.
//  * Operands stream global -> LDS with global_load_lds_dwordx4 (no VGPR
//    staging), two 66 KB stages (A 32 KB, B 32 KB, scales 2 KB), one barrier
//    per chunk; the next chunk's loads run under the current chunk's MFMAs.
//  * LDS rows are 128 bytes (one chunk); the 16-byte slot s of row r is stored
//    at slot s ^ (r & 7) ^ ((r >> 3) & 1). An operand read has 16 lanes on 16
//    consecutive rows at one logical slot; measured on gfx950, ds_read_b128
//    runs at full LDS bandwidth only if rows r and r + 8 also land in different
//    slots (an (r & 7) swizzle alone halves it).
//  * Persistent workgroups, one per CU; each XCD (own L2) walks a contiguous
//    range of output tiles in groups of 8 row-tiles, so the blocks resident on
//    one XCD share activation and weight panels in its L2. The next tile's
//    first chunk is fetched during the current tile's last chunk.
#include "internal.h"

namespace fp8bq {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int BM = 256, BN = 256, BK = 128;
constexpr int kABytes = BM * BK;
constexpr int kBBytes = BN * BK;
constexpr int kSaOff = kABytes + kBBytes;
constexpr int kSbOff = kSaOff + BM * 4;
constexpr int kStage = kSbOff + BN * 4;
constexpr int kGroupM = 8;
constexpr int kXcds = 8;

template <int WAVES_M, int WAVES_N, int LOADERS>
struct Cfg {
  static constexpr int kWaves = WAVES_M * WAVES_N;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int WM = BM / WAVES_M;
  static constexpr int WN = BN / WAVES_N;
  static constexpr int TM = WM / 16;
  static constexpr int TN = WN / 16;
  static constexpr int kLoaders = LOADERS;                 // waves that issue the operand loads
  static constexpr int kRowsPerRound = 8 * kLoaders;       // one dwordx4 DMA per wave covers 8 rows
  static constexpr int kRounds = BM / kRowsPerRound;
  static_assert(WN == 128, "one weight block column per wave");
  static_assert(BM == BN && BM % kRowsPerRound == 0, "tile / wave grid");
  static_assert(kWaves == 8, "scale loaders: four 64-lane dword DMAs per side");
};

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
// compiler itself never keeps a value there across these statements (the
// build passes -Wno-inline-asm for this clobber).
__device__ __forceinline__ void dma16(const void* gbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"(gbase), "s"(lds) : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* gbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1"
               :: "v"(voff), "s"(gbase), "s"(lds) : "memory", "m0");
}

// A pointer every lane holds the same value of, moved to scalar registers
// (the LDS-DMA helpers take their base address in SGPRs).
template <class T>
__device__ __forceinline__ T* uniform_ptr(T* ptr) {
  const uint64_t v = (uint64_t)(uintptr_t)ptr;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (T*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// Physical-slot XOR of LDS row r (see the layout note at the top).
__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

__device__ __forceinline__ v8i frag(const uint8_t* rowp, int off0, int off1) {
  const uint4 x0 = *reinterpret_cast<const uint4*>(rowp + off0);
  const uint4 x1 = *reinterpret_cast<const uint4*>(rowp + off1);
  return v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
}

// Folds one chunk's MFMA result into the FP32 accumulator with the chunk's
// scales: acc += P * (s_a * s_b). FPROP / DGRAD pass the product of the row's
// activation scale and the weight block scale in sc; WGRAD has a row scale per
// output row (sc) and a column scale per output column (sbj).
// The empty asm pins the fold where it is written: without it the compiler
// sinks the folds of a whole chunk below the mid-chunk barrier, keeping every
// MFMA result of the chunk live at once.
template <int KIND>
__device__ __forceinline__ void fold(v4f& acc, const v4f& pc, float sc, const v4f& sbj) {
  if constexpr (KIND == KIND_WGRAD) {
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] = __builtin_fmaf(pc[r] * sbj[r], sc, acc[r]);
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] = __builtin_fmaf(pc[r], sc, acc[r]);
  }
  asm volatile("" : "+v"(acc));
}

// One output tile: its row / column ranges and the weight (with scales) it uses.
struct Tile {
  int64_t m0, m_end, n0, n_end;
  const uint8_t* b;
  const float* sb;
};

template <bool GROUPED>
__device__ __forceinline__ Tile make_tile(const GemmArgs& p, const GroupArgs& g, int logical) {
  const int per_group = kGroupM * p.tiles_n;
  const int group = logical / per_group;
  const int first_m = group * kGroupM;
  const int gsize = min(p.tiles_m - first_m, kGroupM);
  const int in_group = logical - group * per_group;
  const int tmi = first_m + in_group % gsize;
  const int tni = in_group / gsize;
  Tile t;
  t.b = p.b;
  t.sb = p.sb;
  if constexpr (GROUPED) {
    int lo = 0, hi = g.groups;             // find e: tile_prefix[e] <= tmi < tile_prefix[e+1]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (g.tile_prefix[mid] <= tmi) lo = mid; else hi = mid;
    }
    const int e = lo;
    t.m0 = (int64_t)g.row_off128[e] * 128 + (int64_t)(tmi - g.tile_prefix[e]) * BM;
    t.m_end = min(t.m0 + BM, (int64_t)g.row_off128[e + 1] * 128);
    t.b += (int64_t)e * p.n * p.ldb;
    t.sb += (int64_t)e * (p.n / 128) * p.ldsb;
  } else {
    t.m0 = (int64_t)tmi * BM;
    t.m_end = min(t.m0 + BM, p.m);
  }
  t.n0 = (int64_t)tni * BN;
  t.n_end = min(t.n0 + BN, p.n);
  return t;
}

// Persistent kernel: each workgroup owns one CU and walks a strided list of
// output tiles. Workgroup w runs on XCD w % 8 (hardware round-robin); the
// tiles of XCD x are a contiguous range of the grouped walk, shared out among
// that XCD's workgroups, so blocks resident on one XCD (one L2) work on
// neighbouring tiles. The first chunk of the next tile is fetched during the
// current tile's last chunk, so the pipeline fills once per workgroup.
template <int KIND, bool GROUPED, int WAVES_M, int WAVES_N, int LOADERS>
__global__ __launch_bounds__((Cfg<WAVES_M, WAVES_N, LOADERS>::kThreads)) void gemm_kernel(GemmArgs p, GroupArgs g) {
  using C = Cfg<WAVES_M, WAVES_N, LOADERS>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kStage];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wave_m = wave % WAVES_M;
  const int wave_n = wave / WAVES_M;
  const int l16 = lane & 15, lq = lane >> 4;

  // this workgroup's tiles: logical start + local + nper * k, k = 0, 1, ...
  const int G = gridDim.x, w = blockIdx.x;
  const int T = p.tiles_m * p.tiles_n;
  const int x = w % kXcds, local = w / kXcds;
  const int nper = G / kXcds + (x < G % kXcds ? 1 : 0);
  const int count = T / kXcds + (x < T % kXcds ? 1 : 0);
  const int start = x * (T / kXcds) + min(x, T % kXcds);
  if (local >= count) return;                                  // uniform: no tile for this workgroup
  const int my_tiles = (count - local + nper - 1) / nper;
  const int nc = (int)(p.k / BK);
  const int total = my_tiles * nc;

  // ---- global -> LDS load geometry -----------------------------------------
  // Loader wave w (w < kLoaders) fills, in round i, tile rows
  // i * kRowsPerRound + 8 w + ln / 8 (lane ln), 16 bytes at physical slot
  // ln % 8, i.e. logical slot (ln % 8) ^ swz(row); with an even number of
  // loaders swz(row) = (ln / 8) ^ (w & 1) in every round, so a lane's slot is
  // fixed and only its row moves. The lane's byte offset from the tile's
  // first row is computed per load; rows past the end of the operand repeat
  // its last row (their results are never stored). Offsets are 32-bit (the
  // host checks that 256 rows of either operand span less than 2 GiB).
  // Scales: waves 0-3 bring 64 activation scales each; waves 4-7 bring 64
  // column scales each (WGRAD), or wave 4 brings the tile's two weight block
  // scales (lane 0 the first block, lane 1 the second, which is the first
  // again when the tile has only one).
  static_assert(C::kLoaders % 2 == 0, "fixed slot per lane");
  const uint32_t lrow = 8 * wave + (lane >> 3);
  const uint32_t g16 = (uint32_t)(((lane & 7) ^ (lane >> 3) ^ (wave & 1)) * 16);
  uint32_t s_off = 0, a_last = 0, b_last = 0;
  auto set_offsets = [&](const Tile& t) {
    a_last = (uint32_t)(t.m_end - t.m0 - 1);
    b_last = (uint32_t)(t.n_end - t.n0 - 1);
    const int q4 = wave & 3;
    if (wave < 4) {
      s_off = (uint32_t)(min(t.m0 + 64 * q4 + lane, t.m_end - 1) - t.m0) * 4u;
    } else if constexpr (KIND == KIND_WGRAD) {
      s_off = (uint32_t)(min(t.n0 + 64 * q4 + lane, t.n_end - 1) - t.n0) * 4u;
    } else {
      const int64_t blk0 = t.n0 / 128;
      const int64_t blk1 = min(blk0 + 1, t.n_end / 128 - 1) - blk0;
      const int64_t bsel = lane < 1 ? 0 : blk1;
      s_off = (uint32_t)(KIND == KIND_FPROP ? bsel * p.ldsb : bsel) * 4u;
    }
  };
  auto row_off = [&](int i, uint32_t last, uint32_t ld) {
    return min((uint32_t)(i * C::kRowsPerRound) + lrow, last) * ld + g16;
  };

  // ---- global -> LDS cursor: runs two steps ahead of the MFMAs -------------
  // Step s is chunk s % nc of the workgroup's (s / nc)-th tile and lives in
  // stage s % 2. The cursor (dtk, dc) is the next step to load; d_ak, d_bk,
  // d_sk point at its chunk of A, B and the wave's scale vector. A step goes
  // out as kParts load instructions per wave, issued one per MFMA by part(q)
  // so that no wave stalls on a burst of loads. After the last step the
  // cursor stays put: the remaining loads repeat that step into a stage no
  // one reads any more (the kernel waits for them before it ends), which
  // keeps every load unconditional.
  constexpr int kParts = 2 * C::kRounds + 1;
  int dtk = 0, dc = 0;
  const uint8_t* d_ak;
  const uint8_t* d_bk;
  const float* d_sk;
  // per-step advance of the wave's scale pointer: activation scales are
  // chunk-major; FPROP block scales are contiguous along K, DGRAD's and the
  // WGRAD column scales chunk-major
  const int64_t s_step = wave < 4 ? p.ldsa : (KIND == KIND_FPROP ? 1 : p.ldsb);
  auto cursor_tile = [&]() {
    const Tile t = make_tile<GROUPED>(p, g, start + local + nper * dtk);
    set_offsets(t);
    d_ak = p.a + t.m0 * p.lda;
    d_bk = t.b + t.n0 * p.ldb;
    if (wave < 4) d_sk = p.sa + t.m0;
    else if constexpr (KIND == KIND_WGRAD) d_sk = t.sb + t.n0;
    else if constexpr (KIND == KIND_FPROP) d_sk = t.sb + (t.n0 / 128) * p.ldsb;
    else d_sk = t.sb + t.n0 / 128;
  };
  auto advance = [&]() {
    if (dc + 1 < nc) {
      ++dc;
      d_ak += BK;
      d_bk += BK;
      d_sk += s_step;
    } else if (dtk + 1 < my_tiles) {
      dc = 0;
      ++dtk;
      cursor_tile();
    }
  };
  cursor_tile();
  auto part = [&](int q, int st) {
    const uint32_t base = lds_addr(smem) + (uint32_t)(st * kStage);
    if (q < 2 * C::kRounds) {
      if (wave >= C::kLoaders) return;
      if (q < C::kRounds)
        dma16(d_ak, row_off(q, a_last, (uint32_t)p.lda), base + (q * C::kRowsPerRound + 8 * wave) * BK);
      else
        dma16(d_bk, row_off(q - C::kRounds, b_last, (uint32_t)p.ldb),
              base + kABytes + ((q - C::kRounds) * C::kRowsPerRound + 8 * wave) * BK);
    } else if (wave < 4 || KIND == KIND_WGRAD) {
      dma4(uniform_ptr(d_sk), s_off, base + (wave < 4 ? kSaOff : kSbOff) + 256 * (wave & 3));
    } else if (wave == 4) {
      // FPROP / DGRAD: the tile's two weight block scales; a load's cost
      // follows its active lanes, so only two lanes take part
      if (lane < 2) dma4(uniform_ptr(d_sk), s_off, base + kSbOff);
    }
  };

  // LDS byte offset of this lane's operand slice inside a 16-row subtile whose
  // first row is a multiple of 16: row r = base + l16, logical slots 2 lq, 2 lq + 1.
  const int sw = swz(l16);   // the subtile's first row is a multiple of 16
  const int off0 = l16 * BK + (((2 * lq) ^ sw) * 16);
  const int off1 = l16 * BK + (((2 * lq + 1) ^ sw) * 16);

  // Fragments and scales of one step, read from its stage: the wave's TM
  // activation subtiles, the first weight subtile and the per-row scale
  // products of the chunk.
  auto read_scales = [&](const uint8_t* stage, float (&sc)[C::TM]) {
    const float* Sa = reinterpret_cast<const float*>(stage + kSaOff);
    const float* Sb = reinterpret_cast<const float*>(stage + kSbOff);
#pragma unroll
    for (int i = 0; i < C::TM; ++i) sc[i] = Sa[wave_m * C::WM + i * 16 + l16];
    if constexpr (KIND != KIND_WGRAD) {
      const float sbv = Sb[wave_n];
#pragma unroll
      for (int i = 0; i < C::TM; ++i) sc[i] *= sbv;
    }
  };
  auto wgrad_col_scales = [&](const uint8_t* stage, int j) {
    return *reinterpret_cast<const v4f*>(stage + kSbOff + 4 * (wave_n * C::WN + j * 16 + 4 * lq));
  };
  auto a_frag = [&](const uint8_t* stage, int i) { return frag(stage + (wave_m * C::WM + i * 16) * BK, off0, off1); };
  auto b_frag = [&](const uint8_t* stage, int j) {
    return frag(stage + kABytes + (wave_n * C::WN + j * 16) * BK, off0, off1);
  };

#pragma unroll
  for (int q = 0; q < kParts; ++q) part(q, 0);
  advance();
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
#pragma unroll
  for (int q = 0; q < kParts; ++q) part(q, 1);
  advance();

  // Weight fragments are read kBAhead columns before their MFMAs (one column
  // for WGRAD, whose column scales take the registers). bw[0] is the current
  // column's, bw[q] the one q columns on; the barrier precedes column kBarCol,
  // the first whose look-ahead read falls into the next step's stage.
  constexpr int kBAhead = KIND == KIND_WGRAD ? 1 : 3;
  constexpr int kBarCol = C::TN - kBAhead;
  v8i bw[kBAhead + 1];
#pragma unroll
  for (int q = 0; q < kBAhead; ++q) bw[q] = b_frag(smem, q);
  v8i af[C::TM];
#pragma unroll
  for (int i = 0; i < C::TM; ++i) af[i] = a_frag(smem, i);
  float sc[C::TM], scp[C::TM], scn[C::TM];
  read_scales(smem, sc);

  v4f acc[C::TM][C::TN];
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  // MFMA results waiting to be folded: the result of the chunk's t-th MFMA
  // (t = j * TM + i) sits in pend[t % 4] until it is folded kLag MFMAs later,
  // so a fold never waits for the matrix core. The last kLag results of a
  // chunk are folded during the next chunk's first MFMAs with that chunk's
  // scales (scp), or before the epilogue at the end of a tile.
  constexpr int kNT = C::TM * C::TN;
  constexpr int kLag = 3;
  static_assert(kNT % 4 == 0 && kNT > kLag, "result ring");
  static_assert(kLag <= C::TM, "a column's folds finish within the next column");
  v4f pend[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) pend[q] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < C::TM; ++i) scp[i] = 0.f;
  v4f sbj[2] = {v4f{0.f, 0.f, 0.f, 0.f}, v4f{0.f, 0.f, 0.f, 0.f}};
  const v4f zero = {0.f, 0.f, 0.f, 0.f};

  // Step s: weight columns 0 .. TN-2 from stage s % 2 with fragments already in
  // registers; then the barrier (every wave has read all of stage s % 2, and
  // step s + 1 has landed in the other stage), the DMA of step s + 2 into
  // stage s % 2, and the last column's MFMAs while the fragments of step s + 1
  // are read (each activation fragment right after its last use).
  int s = 0;
#pragma clang loop unroll(disable)
  for (int tk = 0; tk < my_tiles; ++tk) {
#pragma clang loop unroll(disable)
    for (int c = 0; c < nc; ++c, ++s) {
      const uint8_t* stage = smem + (s & 1) * kStage;
      const uint8_t* nstage = smem + ((s + 1) & 1) * kStage;
#pragma unroll
      for (int j = 0; j < C::TN; ++j) {
        if (j == kBarCol) {
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          __syncthreads();
          read_scales(nstage, scn);
        }
        bw[kBAhead] = j + kBAhead < C::TN ? b_frag(stage, j + kBAhead) : b_frag(nstage, j + kBAhead - C::TN);
        // WGRAD column scales of column j (the last column's are read before
        // the barrier, below: after it the stage is being refilled)
        if constexpr (KIND == KIND_WGRAD) {
          if (j + 1 < C::TN) sbj[j & 1] = wgrad_col_scales(stage, j);
        }
#pragma unroll
        for (int i = 0; i < C::TM; ++i) {
          const int t = j * C::TM + i;
          pend[t % 4] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bw[0], af[i], zero, 0, 0, 0, 0, 0, 0);
          if (t >= kLag) {
            const int u = t - kLag;
            fold<KIND>(acc[u % C::TM][u / C::TM], pend[u % 4], sc[u % C::TM], sbj[(u / C::TM) & 1]);
          } else {
            const int u = t - kLag + kNT;   // previous chunk, last column
            fold<KIND>(acc[u % C::TM][C::TN - 1], pend[u % 4], scp[u % C::TM], sbj[(C::TN - 1) & 1]);
          }
          if (j + 1 == C::TN) af[i] = a_frag(nstage, i);
          // column TN-2's last MFMA: the folds of column TN-3 are done, so its
          // slot takes the last column's scales
          if constexpr (KIND == KIND_WGRAD) {
            if (j + 2 == C::TN && i + 1 == C::TM) sbj[(j + 1) & 1] = wgrad_col_scales(stage, j + 1);
          }
          // the cursor's step into stage s % 2 (free since the barrier): its
          // loads spread evenly over the MFMAs after the barrier, then the
          // cursor moves on
          {
            constexpr int kFirst = C::TM * kBarCol;
            constexpr int kSlots = kNT - kFirst;
            if (t >= kFirst) {
#pragma unroll
              for (int q = 0; q < kParts; ++q)
                if (q * kSlots / kParts == t - kFirst) part(q, s & 1);
            }
            if (t + 1 == kNT) advance();
          }
          // keep this order: one MFMA, the fold of the result kLag MFMAs old,
          // then the reads due here (no result waits for the matrix core, and
          // MFMA results never pile up in registers)
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int q = 0; q < kBAhead; ++q) bw[q] = bw[q + 1];
      }
#pragma unroll
      for (int i = 0; i < C::TM; ++i) { scp[i] = sc[i]; sc[i] = scn[i]; }
    }

    // ---- tile done: remaining folds (scales of the tile's last chunk, now in
    // scp), epilogue; the next tile's first folds then add zeros ------------
#pragma unroll
    for (int u = kNT - kLag; u < kNT; ++u)
      fold<KIND>(acc[u % C::TM][u / C::TM], pend[u % 4], scp[u % C::TM], sbj[(u / C::TM) & 1]);
#pragma unroll
    for (int i = 0; i < C::TM; ++i) scp[i] = 0.f;
    const Tile cur = make_tile<GROUPED>(p, g, start + local + nper * tk);
#pragma unroll
    for (int i = 0; i < C::TM; ++i) {
      const int64_t row = cur.m0 + wave_m * C::WM + i * 16 + l16;
#pragma unroll
      for (int j = 0; j < C::TN; ++j) {
        const int64_t col = cur.n0 + wave_n * C::WN + j * 16 + 4 * lq;
        if (row < cur.m_end && col < cur.n_end) {
          if constexpr (KIND == KIND_WGRAD) {
            float* o = reinterpret_cast<float*>(p.out) + row * p.ldo + col;
            *reinterpret_cast<v4f*>(o) = acc[i][j];
          } else {
            // v_cvt_pk_bf16_f32 rounds to nearest even (equal to the integer
            // rounding on every finite fp32, checked exhaustively on gfx950)
            const bf16x2 lo = __builtin_convertvector((f32x2){acc[i][j][0], acc[i][j][1]}, bf16x2);
            const bf16x2 hi = __builtin_convertvector((f32x2){acc[i][j][2], acc[i][j][3]}, bf16x2);
            uint2 packed;
            __builtin_memcpy(&packed.x, &lo, 4);
            __builtin_memcpy(&packed.y, &hi, 4);
            uint16_t* o = reinterpret_cast<uint16_t*>(p.out) + row * p.ldo + col;
            *reinterpret_cast<uint2*>(o) = packed;
          }
        }
        acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
      }
    }
  }
  // the repeated loads after the last step must land before the workgroup's
  // LDS is released
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
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

constexpr int kWM = 4;   // 4 x 2 waves of 64 x 128: the accumulator must stay within the
constexpr int kWN = 2;   // 256 VGPRs the VALU can address, with room for fragments
#ifndef FP8BQ_LOADERS
#define FP8BQ_LOADERS 8
#endif
constexpr int kLd = FP8BQ_LOADERS;   // waves issuing the operand loads
constexpr int kBlock = Cfg<kWM, kWN, kLd>::kThreads;

// One workgroup per CU (the LDS stages take most of a CU's 160 KB): as many
// workgroups as CUs, or as tiles when there are fewer tiles.
int persistent_grid(int tiles) {
  static int cus = [] {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    return n;
  }();
  return tiles < cus ? tiles : cus;
}

}  // namespace

hipError_t launch_gemm(int kind, int64_t m, int64_t n, int64_t k, const uint8_t* a, int64_t lda,
                       const float* sa, int64_t ldsa, const uint8_t* b, int64_t ldb,
                       const float* sb, int64_t ldsb, void* out, int64_t ldo, hipStream_t st) {
  GemmArgs p = make_args(m, n, k, a, lda, sa, ldsa, b, ldb, sb, ldsb, out, ldo);
  GroupArgs g;
  g.groups = 0;
  const dim3 grid((unsigned)persistent_grid(p.tiles_m * p.tiles_n)), block(kBlock);
  switch (kind) {
    case KIND_FPROP: hipLaunchKernelGGL((gemm_kernel<KIND_FPROP, false, kWM, kWN, kLd>), grid, block, 0, st, p, g); break;
    case KIND_DGRAD: hipLaunchKernelGGL((gemm_kernel<KIND_DGRAD, false, kWM, kWN, kLd>), grid, block, 0, st, p, g); break;
    default:         hipLaunchKernelGGL((gemm_kernel<KIND_WGRAD, false, kWM, kWN, kLd>), grid, block, 0, st, p, g); break;
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
  const dim3 grid((unsigned)persistent_grid(p.tiles_m * p.tiles_n)), block(kBlock);
  hipLaunchKernelGGL((gemm_kernel<KIND_FPROP, true, kWM, kWN, kLd>), grid, block, 0, st, p, g);
  return hipGetLastError();
}

}  // namespace fp8bq
