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

constexpr int BM = 256, BN = 256, BK = 128;
constexpr int kABytes = BM * BK;
constexpr int kBBytes = BN * BK;
constexpr int kSaOff = kABytes + kBBytes;
constexpr int kSbOff = kSaOff + BM * 4;
constexpr int kStage = kSbOff + BN * 4;
constexpr int kGroupM = 8;
constexpr int kXcds = 8;

template <int WAVES_M, int WAVES_N>
struct Cfg {
  static constexpr int kWaves = WAVES_M * WAVES_N;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int WM = BM / WAVES_M;
  static constexpr int WN = BN / WAVES_N;
  static constexpr int TM = WM / 16;
  static constexpr int TN = WN / 16;
  static constexpr int kRowsPerRound = 8 * kWaves;        // one dwordx4 DMA per wave covers 8 rows
  static constexpr int kRounds = BM / kRowsPerRound;
  static_assert(WN == 128, "one weight block column per wave");
  static_assert(BM == BN && BM % kRowsPerRound == 0, "tile / wave grid");
  static_assert(kWaves == 4 || kWaves == 8, "scale loaders: four 64-lane dword DMAs per side");
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

// Physical-slot XOR of LDS row r (see the layout note at the top).
__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

__device__ __forceinline__ v8i frag(const uint8_t* rowp, int off0, int off1) {
  const uint4 x0 = *reinterpret_cast<const uint4*>(rowp + off0);
  const uint4 x1 = *reinterpret_cast<const uint4*>(rowp + off1);
  return v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
}

// Per-chunk promotion state carried across the barrier: the last weight
// subtile's MFMA results of a chunk are folded at the start of the next chunk,
// after the barrier, so those MFMAs keep the matrix core busy while the waves
// synchronise.
// WGRAD folds every column inside its chunk: it needs two VALU ops per output
// and per-column row scales, and the carry would not fit in its registers.
template <int KIND, class C>
struct Carry {
  static constexpr bool kUsed = KIND != KIND_WGRAD;
  v4f p[C::TM];      // partial sums of subtile column TN - 1, not yet folded
  float sc[C::TM];   // the chunk's activation scale times the weight block scale
  v4f sbj;           // unused (kept so that fold() has one signature)
};

template <int KIND, class C>
__device__ __forceinline__ void fold(v4f& acc, const v4f& pc, float sc, const v4f& sbj) {
  if constexpr (KIND == KIND_WGRAD) {
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] = __builtin_fmaf(pc[r] * sbj[r], sc, acc[r]);
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] = __builtin_fmaf(pc[r], sc, acc[r]);
  }
}

// One K-chunk of the wave's WM x WN tile from one LDS stage: per 16x16
// subtile one MFMA (the chunk's partial sum) and four FMAs folding it into the
// FP32 accumulator with the chunk's scales. `after_reads` runs once the
// fragment reads are issued (it issues the next chunk's DMA). Folds lag one
// MFMA behind, so the matrix core always has work queued while the VALU folds.
template <int KIND, class C, bool HAVE_CARRY, class AfterReads>
__device__ __forceinline__ void compute_chunk(const uint8_t* __restrict__ As, v4f (&acc)[C::TM][C::TN],
                                              Carry<KIND, C>& carry, int wave_m, int wave_n, int l16,
                                              int lq, int off0, int off1, AfterReads after_reads) {
  const uint8_t* Bs = As + kABytes;
  const float* Sa = reinterpret_cast<const float*>(As + kSaOff);
  const float* Sb = reinterpret_cast<const float*>(As + kSbOff);

  v8i af[C::TM];
#pragma unroll
  for (int i = 0; i < C::TM; ++i) af[i] = frag(As + (wave_m * C::WM + i * 16) * BK, off0, off1);
  v8i bcur = frag(Bs + (wave_n * C::WN) * BK, off0, off1);
  float sc[C::TM];
#pragma unroll
  for (int i = 0; i < C::TM; ++i) sc[i] = Sa[wave_m * C::WM + i * 16 + l16];
  if constexpr (KIND != KIND_WGRAD) {
    const float sbv = Sb[wave_n];
#pragma unroll
    for (int i = 0; i < C::TM; ++i) sc[i] *= sbv;
  }
  after_reads();

  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  v4f sbj[2];
  v4f prev = zero;
  // MFMAs in linear order t = j * TM + i; after MFMA t the result of t - 1 is
  // folded, unless t - 1 lies in the last column (carried to the next chunk).
#pragma unroll
  for (int j = 0; j < C::TN; ++j) {
    v8i bnext = bcur;
    if (j + 1 < C::TN) bnext = frag(Bs + (wave_n * C::WN + (j + 1) * 16) * BK, off0, off1);
    if constexpr (KIND == KIND_WGRAD)
      sbj[j & 1] = *reinterpret_cast<const v4f*>(Sb + wave_n * C::WN + j * 16 + 4 * lq);
#pragma unroll
    for (int i = 0; i < C::TM; ++i) {
      const v4f pc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bcur, af[i], zero, 0, 0, 0, 0, 0, 0);
      if constexpr (HAVE_CARRY && Carry<KIND, C>::kUsed) {
        if (j == 0) fold<KIND, C>(acc[i][C::TN - 1], carry.p[i], carry.sc[i], carry.sbj);
      }
      const int t = j * C::TM + i;
      if (t >= 1) {
        const int pj = (t - 1) / C::TM, pi = (t - 1) % C::TM;
        if (!Carry<KIND, C>::kUsed || pj < C::TN - 1) fold<KIND, C>(acc[pi][pj], prev, sc[pi], sbj[pj & 1]);
      }
      if (Carry<KIND, C>::kUsed && j == C::TN - 1) carry.p[i] = pc;
      prev = pc;
    }
    bcur = bnext;
  }
  if constexpr (Carry<KIND, C>::kUsed) {
#pragma unroll
    for (int i = 0; i < C::TM; ++i) carry.sc[i] = sc[i];
  } else {
    fold<KIND, C>(acc[C::TM - 1][C::TN - 1], prev, sc[C::TM - 1], sbj[(C::TN - 1) & 1]);
  }
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
template <int KIND, bool GROUPED, int WAVES_M, int WAVES_N>
__global__ __launch_bounds__((Cfg<WAVES_M, WAVES_N>::kThreads)) void gemm_kernel(GemmArgs p, GroupArgs g) {
  using C = Cfg<WAVES_M, WAVES_N>;
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

  // ---- per-thread load descriptors (global -> LDS) -------------------------
  // Round i of wave w covers tile rows [i * kRowsPerRound + 8 w, +8); lane ln
  // fills row ... + ln / 8, physical slot ln % 8, i.e. logical slot
  // (ln % 8) ^ swz(row). Offsets are 32-bit relative to the tile's first
  // row (the host checks that 256 rows of either operand span less than 2 GiB);
  // rows past the end of the operand repeat its last row (their results are
  // never stored).
  uint32_t a_off[C::kRounds], b_off[C::kRounds];
  auto set_offsets = [&](const Tile& t) {
#pragma unroll
    for (int i = 0; i < C::kRounds; ++i) {
      const int row = i * C::kRowsPerRound + 8 * wave + (lane >> 3);
      const int gslot = (lane & 7) ^ swz(row);
      const int64_t ar = min(t.m0 + row, t.m_end - 1) - t.m0;
      const int64_t br = min(t.n0 + row, t.n_end - 1) - t.n0;
      a_off[i] = (uint32_t)(ar * p.lda + gslot * 16);
      b_off[i] = (uint32_t)(br * p.ldb + gslot * 16);
    }
  };
  // Chunk c of tile t into LDS stage st. Scales: four dword DMAs of 64 lanes
  // bring the tile's 256 activation scales (waves take turns); the weight side
  // is four more for row scales (WGRAD) or one for the two block scales of the
  // tile (FPROP / DGRAD).
  auto issue = [&](const Tile& t, int c, int st) {
    const uint32_t base = lds_addr(smem) + (uint32_t)(st * kStage);
    const uint8_t* ak = p.a + t.m0 * p.lda + (int64_t)c * BK;
    const uint8_t* bk = t.b + t.n0 * p.ldb + (int64_t)c * BK;
#pragma unroll
    for (int i = 0; i < C::kRounds; ++i) dma16(ak, a_off[i], base + (i * C::kRowsPerRound + 8 * wave) * BK);
#pragma unroll
    for (int i = 0; i < C::kRounds; ++i) dma16(bk, b_off[i], base + kABytes + (i * C::kRowsPerRound + 8 * wave) * BK);
#pragma unroll
    for (int q4 = wave; q4 < 4; q4 += C::kWaves) {
      const uint32_t ro = (uint32_t)(min(t.m0 + 64 * q4 + lane, t.m_end - 1) - t.m0) * 4u;
      dma4(p.sa + t.m0 + (int64_t)c * p.ldsa, ro, base + kSaOff + 256 * q4);
    }
    if constexpr (KIND == KIND_WGRAD) {
#pragma unroll
      for (int q4 = wave; q4 < 4; q4 += C::kWaves) {
        const uint32_t co = (uint32_t)(min(t.n0 + 64 * q4 + lane, t.n_end - 1) - t.n0) * 4u;
        dma4(t.sb + t.n0 + (int64_t)c * p.ldsb, co, base + kSbOff + 256 * q4);
      }
    } else if (wave == C::kWaves - 1) {
      // lane 0 -> the tile's first 128-column block, every other lane -> its
      // second (the first again when the tile has only one)
      const int64_t blk0 = t.n0 / 128;
      const int64_t blk1 = min(blk0 + 1, t.n_end / 128 - 1) - blk0;
      const int64_t b = lane < 1 ? 0 : blk1;
      if constexpr (KIND == KIND_FPROP)
        dma4(t.sb + blk0 * p.ldsb + c, (uint32_t)(b * p.ldsb) * 4u, base + kSbOff);
      else
        dma4(t.sb + blk0 + (int64_t)c * p.ldsb, (uint32_t)b * 4u, base + kSbOff);
    }
  };

  v4f acc[C::TM][C::TN];
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // LDS byte offset of this lane's operand slice inside a 16-row subtile whose
  // first row is a multiple of 16: row r = base + l16, logical slots 2 lq, 2 lq + 1.
  const int sw = swz(l16);   // the subtile's first row is a multiple of 16
  const int off0 = l16 * BK + (((2 * lq) ^ sw) * 16);
  const int off1 = l16 * BK + (((2 * lq + 1) ^ sw) * 16);

  // Step s handles chunk c = s % nc of the workgroup's (s / nc)-th tile from
  // stage s % 2. After the barrier at the top of step s every wave has finished
  // step s - 1, so stage (s + 1) % 2 may be refilled: with the next chunk of the
  // same tile, or with chunk 0 of the next tile during a tile's last chunk.
  // The carried column is zero at a tile's first chunk, so folding it there is
  // a no-op and every step runs the same code.
  Carry<KIND, C> carry;
#pragma unroll
  for (int i = 0; i < C::TM; ++i) {
    carry.p[i] = v4f{0.f, 0.f, 0.f, 0.f};
    carry.sc[i] = 0.f;
  }
  carry.sbj = v4f{0.f, 0.f, 0.f, 0.f};
  int tk = 0;
  Tile cur = make_tile<GROUPED>(p, g, start + local);
  Tile nxt = cur;
  set_offsets(cur);
  issue(cur, 0, 0);
  int c = 0;
#pragma clang loop unroll(disable)
  for (int s = 0; s < total; ++s) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const bool last = c + 1 == nc;
    const bool more = !last || tk + 1 < my_tiles;
    if (last && more) {
      nxt = make_tile<GROUPED>(p, g, start + local + nper * (tk + 1));
      set_offsets(nxt);                        // the current tile issues no more loads
    }
    const Tile& tt = last ? nxt : cur;
    const int cc = last ? 0 : c + 1;
    compute_chunk<KIND, C, true>(smem + (s & 1) * kStage, acc, carry, wave_m, wave_n, l16, lq, off0, off1,
                                 [&] { if (more) issue(tt, cc, (s + 1) & 1); });
    if (!last) {
      ++c;
      continue;
    }

    // ---- tile done: last column's fold, epilogue, next tile ----------------
    if constexpr (Carry<KIND, C>::kUsed) {
#pragma unroll
      for (int i = 0; i < C::TM; ++i) {
        fold<KIND, C>(acc[i][C::TN - 1], carry.p[i], carry.sc[i], carry.sbj);
        carry.p[i] = v4f{0.f, 0.f, 0.f, 0.f};
      }
    }
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
        acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
      }
    }
    c = 0;
    ++tk;
    cur = nxt;
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

constexpr int kWM = 4;   // 4 x 2 waves of 64 x 128: the accumulator must stay within the
constexpr int kWN = 2;   // 256 VGPRs the VALU can address, with room for fragments
constexpr int kBlock = Cfg<kWM, kWN>::kThreads;

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
    case KIND_FPROP: hipLaunchKernelGGL((gemm_kernel<KIND_FPROP, false, kWM, kWN>), grid, block, 0, st, p, g); break;
    case KIND_DGRAD: hipLaunchKernelGGL((gemm_kernel<KIND_DGRAD, false, kWM, kWN>), grid, block, 0, st, p, g); break;
    default:         hipLaunchKernelGGL((gemm_kernel<KIND_WGRAD, false, kWM, kWN>), grid, block, 0, st, p, g); break;
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
  hipLaunchKernelGGL((gemm_kernel<KIND_FPROP, true, kWM, kWN>), grid, block, 0, st, p, g);
  return hipGetLastError();
}

}  // namespace fp8bq
