// Block-scaled FP8 GEMM with per-128-K-chunk promotion into FP32, for gfx950:
// the kernels (templates), included by the files that instantiate and launch
// them (gemm.hip, gemm_quant.hip, gemm_grouped.hip).
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
//    subtile) per chunk; the epilogue regroups pairs of lanes so that every
//    lane stores 16 bytes (bf16 and fp32 alike).
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
//  * Persistent workgroups, one per CU, walking output tiles in groups of 8
//    row-tiles; an XCD's 32 workgroups take 32 consecutive tiles at a time
//    (an 8 x 4 block sharing panels in its L2) and the eight XCDs neighbouring
//    blocks (sharing panels in the MALL). The next tile's first chunk is
//    fetched during the current tile's last chunk.
#pragma once

#include "internal.h"
#include "fp8_codec.h"

namespace fp8bq {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Workgroup tile: BM rows x TBN columns, TBN = 256 (BN); 128 for GEMMs with
// too few 256 x 256 tiles to fill the CUs; 224 where 256-column tiles would
// leave the last round of the persistent walk partly idle (n = 7168 = 32 x 224:
// a backward GEMM's 448 tiles of 256 x 256 take two rounds on 256 CUs, its 512
// tiles of 256 x 224 two rounds of 7/8 the work).
constexpr int BM = 256, BN = 256, BK = 128;
// One LDS stage: the A and B tiles of a K-chunk, BM activation scales, and
// room for 256 weight-side scales (column scales of WGRAD, else the tile's
// weight block scales).
template <int TBN>
struct Stage {
  static constexpr int kABytes = BM * BK;
  static constexpr int kBBytes = TBN * BK;
  static constexpr int kSaOff = kABytes + kBBytes;
  static constexpr int kSbOff = kSaOff + BM * 4;
  static constexpr int kStage = kSbOff + 256 * 4;
};
constexpr int kABytes = Stage<BN>::kABytes;
constexpr int kSaOff = Stage<BN>::kSaOff;
constexpr int kSbOff = Stage<BN>::kSbOff;
constexpr int kStage = Stage<BN>::kStage;
constexpr int kGroupM = 8;
constexpr int kXcds = 8;

template <int WAVES_M, int WAVES_N, int TBN = BN>
struct Cfg {
  static constexpr int kWaves = WAVES_M * WAVES_N;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int WM = BM / WAVES_M;
  static constexpr int WN = TBN / WAVES_N;
  static constexpr int TM = WM / 16;
  static constexpr int TN = WN / 16;
  // a wave's columns lie in one weight block column, except with 224-column tiles
  // (waves of 112 columns), whose waves may straddle two blocks
  static_assert(WN <= 128 && (128 % WN == 0 || WN == 112), "wave columns against 128-column weight blocks");
};

struct GemmArgs {
  int64_t m, n, k;
  const uint8_t* a; int64_t lda;
  const float* sa; int64_t ldsa;
  const uint8_t* b; int64_t ldb;
  const float* sb; int64_t ldsb;
  void* out; int64_t ldo;
  uint8_t* q; int64_t ldq;     // optional quantised copy of the output (1x128 tiles)
  float* sq; int64_t ldsq;     // and its chunk-major scales
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
// build passes -Wno-inline-asm for this clobber). An SALU write of M0 needs
// one wait state before an LDS DMA reads it (the compiler puts an s_nop 0
// there for its own LDS-DMA builtins; its hazard check cannot see inside an
// asm block, so each block carries the s_nop itself). tests/test_lds_dma_m0.py
// checks the built code objects: every M0 use is this write, wait, DMA triple.
__device__ __forceinline__ void dma16(const void* gbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"(gbase), "s"(lds) : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* gbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
               :: "v"(voff), "s"(gbase), "s"(lds) : "memory", "m0");
}
// A 4-byte LDS DMA through a raw buffer resource (lane i's bytes to M0 + 4 i).
__device__ __forceinline__ void dma4_buf(const u32x4& rsrc, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds"
               :: "v"(voff), "s"(rsrc), "s"(lds) : "memory", "m0");
}
// The same 16-byte LDS DMA through a raw buffer resource (base, byte bound):
// a lane whose offset (VGPR, no scalar offset, no thread-id addressing) is at
// or past the bound reads nothing from memory and its bytes come back as
// zeros.
__device__ __forceinline__ void dma16_buf(const u32x4& rsrc, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :: "v"(voff), "s"(rsrc), "s"(lds) : "memory", "m0");
}
// Raw buffer resource over [base, end) (bound capped at 4 GiB - 1: offsets
// stay below 2 GiB), all words uniform.
__device__ __forceinline__ u32x4 make_rsrc(const uint8_t* base, const uint8_t* end) {
  const uint64_t b = (uint64_t)(uintptr_t)base;
  const uint64_t n = end > base ? (uint64_t)(end - base) : 0;
  u32x4 r;
  r.x = __builtin_amdgcn_readfirstlane((uint32_t)b);
  r.y = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32) & 0xFFFFu);   // stride 0: raw
  r.z = __builtin_amdgcn_readfirstlane(n > 0xFFFFFFFFull ? 0xFFFFFFFFu : (uint32_t)n);
  r.w = 0x00020000u;
  return r;
}
// Moves a resource's base on by d bytes (d below its bound).
__device__ __forceinline__ void bump_rsrc(u32x4& r, uint32_t d) {
  const uint64_t b = (((uint64_t)r.y << 32) | r.x) + d;
  r.x = (uint32_t)b;
  r.y = (uint32_t)(b >> 32);
  r.z = r.z == 0xFFFFFFFFu ? r.z : r.z - d;
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

template <bool GROUPED, int TBN = BN>
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
    // the group table is read with scalar loads, which complete out of order
    // with LDS reads: wait for them here, or every later LDS wait the compiler
    // places would have to wait for everything
    __builtin_amdgcn_s_waitcnt(0xC07F);
  } else {
    t.m0 = (int64_t)tmi * BM;
    t.m_end = min(t.m0 + BM, p.m);
  }
  t.n0 = (int64_t)tni * TBN;
  t.n_end = min(t.n0 + TBN, p.n);
  return t;
}

// This workgroup's share of the persistent tile walk. Workgroup w runs on XCD
// x = w % 8 (hardware round-robin) as its local = w / 8-th workgroup. With a
// grid of 8 C workgroups (C per XCD), the grouped walk is cut into chunks of C
// consecutive tiles dealt to the XCDs in turn (chunk c to XCD c % 8), one tile
// per workgroup: at any time the eight XCDs work on eight consecutive chunks,
// which share operand panels (in the large fprop the same 8 row-tiles of A, in a
// grouped MoE GEMM mostly one expert's weight) in the MALL. A grid that is not
// a multiple of 8 (fewer tiles than CUs) gives XCD x a contiguous range of the
// walk instead. Either way the
// workgroup's tiles are logical indices start + local + nper * t,
// t = 0 .. my_tiles - 1.
struct Walk {
  int start, local, nper, my_tiles, nc, total;
};

__device__ __forceinline__ Walk make_walk(const GemmArgs& p) {
  Walk wk;
  const int G = gridDim.x, w = blockIdx.x;
  const int T = p.tiles_m * p.tiles_n;
  const int x = w % kXcds;
  wk.local = w / kXcds;
  wk.nper = G / kXcds + (x < G % kXcds ? 1 : 0);
  if (G % kXcds == 0) {
    const int C = G / kXcds;
    wk.start = x * C;
    wk.nper = kXcds * C;
    const int first = wk.start + wk.local;
    wk.my_tiles = first < T ? (T - 1 - first) / wk.nper + 1 : 0;
  } else {
    const int count = T / kXcds + (x < T % kXcds ? 1 : 0);
    wk.start = x * (T / kXcds) + min(x, T % kXcds);
    wk.my_tiles = wk.local < count ? (count - wk.local + wk.nper - 1) / wk.nper : 0;
  }
  wk.nc = (int)(p.k / BK);
  wk.total = wk.my_tiles * wk.nc;
  return wk;
}

// ---- epilogue ----------------------------------------------------------------
// bf16 pair of four accumulators (round to nearest even: hardware
// v_cvt_pk_bf16_f32, equal to the integer rounding on every finite fp32).
__device__ __forceinline__ uint2 pack_bf16x4(const v4f& v) {
  const bf16x2 lo = __builtin_convertvector((f32x2){v[0], v[1]}, bf16x2);
  const bf16x2 hi = __builtin_convertvector((f32x2){v[2], v[3]}, bf16x2);
  uint2 r;
  __builtin_memcpy(&r.x, &lo, 4);
  __builtin_memcpy(&r.y, &hi, 4);
  return r;
}

// Two subtiles' bf16 results (A of subtile j, B of subtile j + 1; lane: row
// l16, columns 4 lq .. 4 lq + 3) regrouped between lanes lq and lq ^ 1 into
// 16 contiguous bytes per lane: even lanes take columns 4 lq .. 4 lq + 7 of
// subtile j, odd lanes columns 4 lq - 4 .. 4 lq + 3 of subtile j + 1. Stores
// cost per active lane, so 16-byte lanes halve the epilogue's store work.
// Returns the 16 bytes; they go to the lane's own column of subtile j (even
// lanes) or 12 columns on from it (odd lanes).
// v_permlane16_swap_b32 (gfx950) exchanges the odd 16-lane rows of its first
// operand with the even rows of its second: with A first and B second, even
// rows end with (own A, partner's A) and odd rows with (partner's B, own B),
// which is the regrouping itself, with no lane index, select or LDS crossbar.
__device__ __forceinline__ uint4 pair16(uint2 A, uint2 B) {
  const auto x = __builtin_amdgcn_permlane16_swap(A.x, B.x, false, false);
  const auto y = __builtin_amdgcn_permlane16_swap(A.y, B.y, false, false);
  return make_uint4(x[0], y[0], x[1], y[1]);
}

// The lane's index within its wave, recomputed where it is used: the inline
// asm cannot be moved or merged, so the compiler does not hoist lane-dependent
// epilogue and tile-change offsets out of the K-loop and keep them live through
// it (the 256-column kernels spilled them to scratch, and every reload waited
// for all loads in flight).
__device__ __forceinline__ int lane_fresh() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// The codes of four subtiles of one output row (d[k]: columns 16 k + 4 lq ..
// 16 k + 4 lq + 3 of subtile group g, from lane lq of the row) transposed
// between the row's four lanes, which sit in the wave's four 16-lane rows:
// lane lq ends with the 16 codes of subtile 4 g + lq, one 16-byte store
// instead of four 4-byte ones. Two v_permlane16_swap_b32 (odd rows of the first
// operand <-> even rows of the second) leave every lane with index lq & 1 of
// both lanes of its row pair, for subtiles lq & 1 and 2 + (lq & 1); two
// v_permlane32_swap_b32 (rows 2, 3 of the first <-> rows 0, 1 of the second)
// then bring the other pair's values, in source-lane order on every lane.
__device__ __forceinline__ uint4 codes16(const uint32_t (&d)[4]) {
  const auto xy = __builtin_amdgcn_permlane16_swap(d[0], d[1], false, false);
  const auto zw = __builtin_amdgcn_permlane16_swap(d[2], d[3], false, false);
  const auto p0 = __builtin_amdgcn_permlane32_swap(xy[0], zw[0], false, false);
  const auto p1 = __builtin_amdgcn_permlane32_swap(xy[1], zw[1], false, false);
  return make_uint4(p0[0], p1[0], p0[1], p1[1]);
}

// Largest of a value over the four lanes l16 + 16 lq of an output row.
__device__ __forceinline__ uint32_t row_max4(uint32_t v) {
  const auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = umax(a[0], a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return umax(b[0], b[1]);
}

// Stores a wave's TM x TN subtiles (lane: output row l16 of subtile i, columns
// 4 lq .. 4 lq + 3 of subtile j) as bf16 or fp32. Full bf16 tiles store 16
// bytes per lane (pair16) with one row pointer per subtile row; edge tiles
// check every row and column.
template <int KIND, int TM, int TN, int TBN>
__device__ __forceinline__ void store_tile(const GemmArgs& p, const Tile& cur, const v4f (&acc)[TM][TN],
                                           int64_t row0, int64_t col0, int lq) {
  auto put = [&](int64_t row, int64_t col, const v4f& v) {
    if constexpr (KIND == KIND_WGRAD) {
      *reinterpret_cast<v4f*>(reinterpret_cast<float*>(p.out) + row * p.ldo + col) = v;
    } else {
      *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.out) + row * p.ldo + col) = pack_bf16x4(v);
    }
  };
  if (cur.m_end - cur.m0 == BM && cur.n_end - cur.n0 == TBN) {   // uniform
    if constexpr (KIND == KIND_WGRAD) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) put(row0 + i * 16, col0 + j * 16, acc[i][j]);
    } else {
      const bool odd = (lq & 1) != 0;
#pragma unroll
      for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int jp = 0; jp < TN / 2; ++jp) {
          const uint4 v = pair16(pack_bf16x4(acc[i][2 * jp]), pack_bf16x4(acc[i][2 * jp + 1]));
          const int64_t col = col0 + 2 * jp * 16 + (odd ? 12 : 0);
          *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(p.out) + (row0 + i * 16) * p.ldo + col) = v;
        }
        if constexpr (TN % 2 != 0) put(row0 + i * 16, col0 + (TN - 1) * 16, acc[i][TN - 1]);   // 112-column waves
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        if (row0 + i * 16 < cur.m_end && col0 + j * 16 < cur.n_end) put(row0 + i * 16, col0 + j * 16, acc[i][j]);
  }
}

// Producer fusion (report section 3.5.2, "online quantization support": the
// activations a GEMM consumes are otherwise read from HBM, quantised, written
// back and read again): the epilogue also quantises its bf16 output as the
// next GEMM's activation operand, 1x128 tiles along each output row. A wave's
// 128 output columns are one tile per row, held by the four lanes l16 + 16 lq
// (32 values each): each lane takes the max of its bf16 magnitudes, two lane
// exchanges give the tile's, and scale and codes come from the quantisers'
// codec (fp8_codec.h) applied to the same bf16 values, so q / sq equal
// fp8bq_quant_act_1x128 of the bf16 output bit for bit. The codes are
// transposed among the row's lanes (codes16) into 16-byte stores. The bf16
// output itself is written only when p.out is set. grp is the tile's
// 128-column group.
template <bool POW2, int TM, int TN>
__device__ __forceinline__ void store_tile_q(const GemmArgs& p, const Tile& cur, const v4f (&acc)[TM][TN],
                                             int64_t row0, int64_t col0, int64_t grp, int lq) {
  static_assert(TN * 16 == 128, "one 1x128 tile per output row per wave");
  if (grp * 128 >= cur.n_end) return;            // uniform: the wave's columns lie past n
  const bool bf_out = p.out != nullptr;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int64_t row = row0 + i * 16;
    uint2 w[TN];
    uint32_t amax = 0;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const bf16x2 lo = __builtin_convertvector((f32x2){acc[i][j][0], acc[i][j][1]}, bf16x2);
      const bf16x2 hi = __builtin_convertvector((f32x2){acc[i][j][2], acc[i][j][3]}, bf16x2);
      __builtin_memcpy(&w[j].x, &lo, 4);
      __builtin_memcpy(&w[j].y, &hi, 4);
      amax = umax(amax, umax(mag_max2(w[j].x), mag_max2(w[j].y)));
    }
    amax = row_max4(amax);
    const TileScale ts = group_scale<POW2>(amax);
    uint32_t code[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j)
      code[j] = encode4<POW2>(bf_lo(w[j].x), bf_hi(w[j].x), bf_lo(w[j].y), bf_hi(w[j].y), ts);
    // lane exchanges (every lane of the wave takes part) before the row check
    uint4 c16[TN / 4], b16[TN / 2];
#pragma unroll
    for (int g = 0; g < TN / 4; ++g) {
      const uint32_t d[4] = {code[4 * g], code[4 * g + 1], code[4 * g + 2], code[4 * g + 3]};
      c16[g] = codes16(d);
    }
    if (bf_out) {
#pragma unroll
      for (int jp = 0; jp < TN / 2; ++jp) b16[jp] = pair16(w[2 * jp], w[2 * jp + 1]);
    }
    if (row < cur.m_end) {
      const int64_t gcol = col0 - 4 * lq;       // the wave's first column
#pragma unroll
      for (int g = 0; g < TN / 4; ++g)
        *reinterpret_cast<uint4*>(p.q + row * p.ldq + gcol + 16 * (4 * g + lq)) = c16[g];
      if (bf_out) {
#pragma unroll
        for (int jp = 0; jp < TN / 2; ++jp)
          *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(p.out) + row * p.ldo + col0 + 2 * jp * 16 +
                                    ((lq & 1) ? 12 : 0)) = b16[jp];
      }
      if (lq == 0) p.sq[grp * p.ldsq + row] = ts.s;
    }
  }
}

// Epilogue of a tile: plain store, or (QMODE 1: s = absmax / 448, 2: power of
// two) with the quantised copy of the output.
template <int KIND, int QMODE, int TM, int TN, int TBN = BN>
__device__ __forceinline__ void epilogue(const GemmArgs& p, const Tile& cur, const v4f (&acc)[TM][TN],
                                         int64_t row0, int64_t n_wave, int lq) {
  static_assert(QMODE == 0 || TBN == BN, "quantised output: 256-column tiles");
  if constexpr (QMODE == 0)
    store_tile<KIND, TM, TN, TBN>(p, cur, acc, row0, n_wave + 4 * lq, lq);
  else
    store_tile_q<QMODE == 2, TM, TN>(p, cur, acc, row0, n_wave + 4 * lq, n_wave / 128, lq);
}

// ---- global -> LDS loads ----------------------------------------------------
// Loader wave w (w < LOADERS) fills, in round i, tile rows
// i * kRowsPerRound + 8 w + ln / 8 (lane ln), 16 bytes at physical slot
// ln % 8, i.e. logical slot (ln % 8) ^ swz(row); with an even number of
// loaders swz(row) = (ln / 8) ^ (w & 1) in every round, so a lane's slot is
// fixed and only its row moves. The lane's byte offset from the tile's first
// row in each round is the same for every step and every tile, so it is
// computed once; the operand tiles are read through raw buffer resources whose
// base is the step's chunk of the tile's first row and whose bound is the end
// of the operand, so rows past the end read as zeros (their results are never
// stored). Offsets are 32-bit (the host checks that 256 rows of either operand
// span less than 2 GiB).
// Scales are brought by eight "scale waves" of 64 lanes (each real wave plays
// 8 / WAVES of them): scale waves 0-3 bring 64 activation scales each; 4-7
// bring 64 column scales each (WGRAD), or scale wave 4 brings the tile's two
// weight block scales (lane 0 the first block, lane 1 the second, which is the
// first again when the tile has only one).
//
// The cursor (dtk, dc) is the next step to load: step s is chunk s % nc of the
// workgroup's (s / nc)-th tile and lives in stage s % 2; rs_a, rs_b and d_sk
// address its chunk of A, B and the scale vectors. A step goes out as kParts load
// instructions per wave, part(0 .. kParts-1), and then advance() moves the
// cursor on. After the last step the cursor stays put: further loads repeat
// that step into a stage no one reads any more (the kernels wait for them
// before they end), which keeps every load unconditional.
template <int KIND, bool GROUPED, int WAVES, int LOADERS, int TBN = BN>
struct Loader {
  using S = Stage<TBN>;
  static constexpr int kRowsPerRound = 8 * LOADERS;      // one dwordx4 load per wave covers 8 rows
  static constexpr int kRounds = BM / kRowsPerRound;     // of A; then kRoundsB of B
  static constexpr int kRoundsB = (TBN + kRowsPerRound - 1) / kRowsPerRound;   // the last may be partial
  static constexpr int kScaleWaves = 8 / WAVES;
  static constexpr int kParts = kRounds + kRoundsB + kScaleWaves;
  static_assert(LOADERS % 2 == 0 && LOADERS <= WAVES && BM % kRowsPerRound == 0 && TBN % 8 == 0, "load rounds");
  static_assert(WAVES == 4 || WAVES == 8, "scale waves");

  const GemmArgs& p;
  const GroupArgs& g;
  const Walk& wk;
  const uint32_t smem_base;
  const int wave, lane;
  const uint32_t lrow, g16;
  uint32_t voff_a[kRounds], voff_b[kRoundsB];
  uint32_t s_off[kScaleWaves];
  int64_t s_step[kScaleWaves];
  const float* d_sk[kScaleWaves];
  u32x4 rs_a, rs_b;
  int dtk = 0, dc = 0;

  __device__ __forceinline__ Loader(const GemmArgs& p_, const GroupArgs& g_, const Walk& wk_, uint32_t smem_base_,
                                    int wave_, int lane_)
      : p(p_), g(g_), wk(wk_), smem_base(smem_base_), wave(wave_), lane(lane_),
        lrow(8 * wave_ + (lane_ >> 3)), g16((uint32_t)(((lane_ & 7) ^ (lane_ >> 3) ^ (wave_ & 1)) * 16)) {
#pragma unroll
    for (int v = 0; v < kScaleWaves; ++v) {
      // per-step advance of a scale pointer: activation scales are chunk-major;
      // FPROP block scales are contiguous along K, DGRAD's and the WGRAD column
      // scales chunk-major
      const int sw = wave + v * WAVES;
      s_step[v] = sw < 4 ? p.ldsa : (KIND == KIND_FPROP ? 1 : p.ldsb);
    }
#pragma unroll
    for (int i = 0; i < kRounds; ++i) voff_a[i] = ((uint32_t)(i * kRowsPerRound) + lrow) * (uint32_t)p.lda + g16;
#pragma unroll
    for (int i = 0; i < kRoundsB; ++i) voff_b[i] = ((uint32_t)(i * kRowsPerRound) + lrow) * (uint32_t)p.ldb + g16;
    cursor_tile();
  }

  __device__ __forceinline__ void cursor_tile() {
    const Tile t = make_tile<GROUPED, TBN>(p, g, wk.start + wk.local + wk.nper * dtk);
    const int ln = lane_fresh();   // not `lane`: its 64-bit offsets would be kept live through the K-loop
    rs_a = make_rsrc(p.a + t.m0 * p.lda, p.a + (p.m - 1) * p.lda + p.k);
    rs_b = make_rsrc(t.b + t.n0 * p.ldb, t.b + (p.n - 1) * p.ldb + p.k);
#pragma unroll
    for (int v = 0; v < kScaleWaves; ++v) {
      const int sw = wave + v * WAVES, q4 = sw & 3;
      if (sw < 4) {
        s_off[v] = (uint32_t)(min(t.m0 + 64 * q4 + ln, t.m_end - 1) - t.m0) * 4u;
        d_sk[v] = p.sa + t.m0;
      } else if constexpr (KIND == KIND_WGRAD) {
        s_off[v] = (uint32_t)(min(t.n0 + 64 * q4 + ln, t.n_end - 1) - t.n0) * 4u;
        d_sk[v] = t.sb + t.n0;
      } else {
          // the tile's columns span blocks blk0 .. blk0 + last (last <= 2): lane l
        // brings block blk0 + min(l, last)
        const int64_t blk0 = t.n0 / 128;
        const int64_t last = (t.n_end - 1) / 128 - blk0;
        const int64_t bsel = TBN % 128 == 0 ? (ln < 1 ? 0 : last) : min((int64_t)ln, last);
        s_off[v] = (uint32_t)(KIND == KIND_FPROP ? bsel * p.ldsb : bsel) * 4u;
        d_sk[v] = KIND == KIND_FPROP ? t.sb + blk0 * p.ldsb : t.sb + blk0;
      }
    }
  }

  __device__ __forceinline__ void advance() {
    if (dc + 1 < wk.nc) {
      ++dc;
      bump_rsrc(rs_a, BK);
      bump_rsrc(rs_b, BK);
#pragma unroll
      for (int v = 0; v < kScaleWaves; ++v) d_sk[v] += s_step[v];
    } else if (dtk + 1 < wk.my_tiles) {
      dc = 0;
      ++dtk;
      cursor_tile();
    }
  }

  // L2 prefetch of the cursor's step (8 waves): one 4-byte LDS DMA per lane, one
  // lane per 128-byte line of the step's chunk, waves 0-3 the 256 activation
  // rows, 4-7 the weight rows; the bytes land in a scratch area nobody reads.
  // Issued right after advance(), it reaches L2 one step before that step's own
  // loads, which then hit there.
  __device__ __forceinline__ void prefetch(uint32_t junk) const {
    static_assert(WAVES == 8, "prefetch rows: 8 waves");
    if (wave < 4) dma4_buf(rs_a, (uint32_t)(wave * 64 + lane) * (uint32_t)p.lda, junk);
    else dma4_buf(rs_b, (uint32_t)((wave - 4) * 64 + lane) * (uint32_t)p.ldb, junk);
  }

  // Load instruction q of the cursor's step into stage st.
  __device__ __forceinline__ void part(int q, int st) const {
    const uint32_t base = smem_base + (uint32_t)(st * S::kStage);
    if (q < kRounds + kRoundsB) {
      if constexpr (LOADERS < WAVES) {
        if (wave >= LOADERS) return;
      }
      if (q < kRounds) {
        dma16_buf(rs_a, voff_a[q], base + (q * kRowsPerRound + 8 * wave) * BK);
      } else {
        // a partial last round (224-column tiles): waves whose rows lie past the
        // tile load nothing (uniform per wave)
        if constexpr (TBN % kRowsPerRound != 0) {
          if ((q - kRounds) * kRowsPerRound + 8 * wave >= TBN) return;
        }
        dma16_buf(rs_b, voff_b[q - kRounds], base + S::kABytes + ((q - kRounds) * kRowsPerRound + 8 * wave) * BK);
      }
      return;
    }
    const int v = q - kRounds - kRoundsB, sw = wave + v * WAVES;
    // with four waves, scale wave v of wave w is w (activations) or w + 4
    const bool act = WAVES == 4 ? v == 0 : sw < 4;
    if (act || KIND == KIND_WGRAD) {
      dma4(uniform_ptr(d_sk[v]), s_off[v], base + (act ? S::kSaOff : S::kSbOff) + 256 * (sw & 3));
    } else if (sw == 4) {
      // FPROP / DGRAD: the tile's weight block scales (up to three); a load's
      // cost follows its active lanes, so only three lanes take part
      if (lane < (TBN % 128 == 0 ? 2 : 3)) dma4(uniform_ptr(d_sk[v]), s_off[v], base + S::kSbOff);
    }
  }
};

// Persistent kernel with promotion on the VALU: each workgroup owns one CU and
// walks its tiles (make_walk); the first chunk of the next tile is fetched
// during the current tile's last chunks, so the pipeline fills once per
// workgroup.
template <int KIND, bool GROUPED, int WAVES_M, int WAVES_N, int LOADERS, int QMODE = 0, int TBN = BN>
__global__ __launch_bounds__((Cfg<WAVES_M, WAVES_N, TBN>::kThreads)) void gemm_kernel(GemmArgs p, GroupArgs g) {
  using C = Cfg<WAVES_M, WAVES_N, TBN>;
  using S = Stage<TBN>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * S::kStage];
  // Grouped (MoE) GEMMs prefetch each step's chunk into L2 one step ahead. Their
  // activations come from HBM, and their steps take 3833 cycles against 3138 with
  // no loads at all; the prefetch takes the MoE workload from 712-724 to 705-708 us
  // (three rounds of each). The large fprop's and the backward GEMMs' operands sit
  // in the MALL (their loads cost 2% of a step), and there the prefetch costs 2-4%.
  // After each step's loads every wave issues exactly one prefetch, which the
  // barrier's wait lets stay in flight (loads complete in issue order).
#ifdef FP8BQ_PREFETCH_ALL
  constexpr bool kPF = true;
#else
  constexpr bool kPF = GROUPED;
#endif
  __shared__ uint32_t pf_junk[64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wave_m = wave % WAVES_M;
  const int wave_n = wave / WAVES_M;
  const int l16 = lane & 15, lq = lane >> 4;

  const Walk wk = make_walk(p);
  if (wk.my_tiles == 0) return;                                // uniform: no tile for this workgroup
  const int my_tiles = wk.my_tiles, nc = wk.nc;
  Loader<KIND, GROUPED, C::kWaves, LOADERS, TBN> ld(p, g, wk, lds_addr(smem), wave, lane);
  constexpr int kParts = decltype(ld)::kParts;

  // LDS byte offset of this lane's operand slice inside a 16-row subtile whose
  // first row is a multiple of 16: row r = base + l16, logical slots 2 lq, 2 lq + 1.
  const int sw = swz(l16);   // the subtile's first row is a multiple of 16
  const int off0 = l16 * BK + (((2 * lq) ^ sw) * 16);
  const int off1 = l16 * BK + (((2 * lq + 1) ^ sw) * 16);

  // Fragments and scales of one step, read from its stage: the wave's TM
  // activation subtiles, the first weight subtile and the per-row scale
  // products of the chunk.
  // With 224-column tiles (FPROP / DGRAD) a wave's 112 columns may straddle two
  // weight blocks: column subtiles j < jb take block b0's scale (sc), the others
  // block b1's (sc1). `off` is the wave's first column counted from its tile's
  // first block (n0 % 128 + wave_n * WN), wave-uniform.
  constexpr bool kMB = KIND != KIND_WGRAD && (TBN % 128) != 0;
  auto wave_off = [&](int tk_) -> int {
    if constexpr (kMB) {
      const int64_t n0 = make_tile<GROUPED, TBN>(p, g, wk.start + wk.local + wk.nper * tk_).n0;
      return (int)(n0 % 128) + wave_n * C::WN;
    } else {
      return 0;
    }
  };
  auto read_scales = [&](const uint8_t* stage, float (&sc)[C::TM], float (&sc1)[C::TM], int& jb, int off) {
    const float* Sa = reinterpret_cast<const float*>(stage + S::kSaOff);
    const float* Sb = reinterpret_cast<const float*>(stage + S::kSbOff);
#pragma unroll
    for (int i = 0; i < C::TM; ++i) sc[i] = Sa[wave_m * C::WM + i * 16 + l16];
    if constexpr (kMB) {
      const int b0 = off >> 7, b1 = (off + C::WN - 1) >> 7;
      jb = ((b0 + 1) * 128 - off) >> 4;                  // >= TN: one block only
      const float s0 = Sb[b0], s1 = Sb[b1];
#pragma unroll
      for (int i = 0; i < C::TM; ++i) { sc1[i] = sc[i] * s1; sc[i] *= s0; }
    } else if constexpr (KIND != KIND_WGRAD) {
      const float sbv = Sb[wave_n * C::WN / 128];   // the weight block of the wave's columns
#pragma unroll
      for (int i = 0; i < C::TM; ++i) sc[i] *= sbv;
    }
  };
  auto wgrad_col_scales = [&](const uint8_t* stage, int j) {
    return *reinterpret_cast<const v4f*>(stage + S::kSbOff + 4 * (wave_n * C::WN + j * 16 + 4 * lq));
  };
  auto a_frag = [&](const uint8_t* stage, int i) { return frag(stage + (wave_m * C::WM + i * 16) * BK, off0, off1); };
  auto b_frag = [&](const uint8_t* stage, int j) {
    return frag(stage + S::kABytes + (wave_n * C::WN + j * 16) * BK, off0, off1);
  };

#pragma unroll
  for (int q = 0; q < kParts; ++q) ld.part(q, 0);
  ld.advance();
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
#pragma unroll
  for (int q = 0; q < kParts; ++q) ld.part(q, 1);
  ld.advance();
  if constexpr (kPF) ld.prefetch(lds_addr(pf_junk));

  // Weight fragments are read kBAhead columns before their MFMAs (one column
  // for WGRAD, whose column scales take the registers). The earlier the
  // barrier sits in the step, the less the waves lose waiting at it (measured:
  // four columns ahead is 2% faster than three; in the grouped and the
  // output-quantising kernels 1.5% and 1%, although they then spill one
  // register per step). bw[0] is the current
  // column's, bw[q] the one q columns on; the barrier precedes column kBarCol,
  // the first whose look-ahead read falls into the next step's stage.
  // With four columns per wave (128-column tiles) two columns ahead keep the
  // barrier mid-step.
  constexpr int kBAhead = KIND == KIND_WGRAD ? 1 : C::TN < 8 ? C::TN / 2 : 4;
  constexpr int kBarCol = C::TN - kBAhead;
  v8i bw[kBAhead + 1];
#pragma unroll
  for (int q = 0; q < kBAhead; ++q) bw[q] = b_frag(smem, q);
  v8i af[C::TM];
#pragma unroll
  for (int i = 0; i < C::TM; ++i) af[i] = a_frag(smem, i);
  float sc[C::TM], scp[C::TM], scn[C::TM], sc1[C::TM], scn1[C::TM];
  int jb = C::TN, jbn = C::TN;
  int off_cur = wave_off(0), off_nxt = off_cur;
  read_scales(smem, sc, sc1, jb, off_cur);
  // The compiler tracks at most 15 outstanding LDS reads; with more in flight
  // where a loop iteration begins it waits for all of them before the first
  // MFMA. This wait and the one at the last column keep the count it carries
  // into the loop below that.
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)

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
  // WGRAD, odd TN (224-column tiles): the last column and the next chunk's
  // column 0 share a slot of sbj, so the last column's scales are kept here
  // for its folds that run during the next chunk (or after the tile)
  v4f sbjp = {0.f, 0.f, 0.f, 0.f};
  auto last_col_scales = [&]() -> const v4f& {
    if constexpr (C::TN % 2 != 0) return sbjp;
    else return sbj[(C::TN - 1) & 1];
  };
  const v4f zero = {0.f, 0.f, 0.f, 0.f};

  // Step s: weight columns 0 .. TN-2 from stage s % 2 with fragments already in
  // registers; then the barrier (every wave has read all of stage s % 2, and
  // step s + 1 has landed in the other stage), the DMA of step s + 2 into
  // stage s % 2, and the last column's MFMAs while the fragments of step s + 1
  // are read (each activation fragment right after its last use).
  int s = 0;
#pragma clang loop unroll(disable)
  for (int tk = 0; tk < my_tiles; ++tk) {
    if constexpr (kMB) {
      if (tk > 0) off_cur = off_nxt;
      off_nxt = tk + 1 < my_tiles ? wave_off(tk + 1) : off_cur;
    }
#pragma clang loop unroll(disable)
    for (int c = 0; c < nc; ++c, ++s) {
      const uint8_t* stage = smem + (s & 1) * S::kStage;
      const uint8_t* nstage = smem + ((s + 1) & 1) * S::kStage;
#pragma unroll
      for (int j = 0; j < C::TN; ++j) {
        if (j == kBarCol) {
          if constexpr (kPF) asm volatile("s_waitcnt vmcnt(1)" ::: "memory");   // all but the prefetch
          else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          __syncthreads();
          read_scales(nstage, scn, scn1, jbn, c + 1 < nc ? off_cur : off_nxt);
        }
        // last column: everything read before the previous column's weight
        // fragment has landed (read at least a column ago)
        if (j + 1 == C::TN) __builtin_amdgcn_s_waitcnt(0xC07F | (2 << 8));
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
            const float su = kMB ? (u / C::TM < jb ? sc[u % C::TM] : sc1[u % C::TM]) : sc[u % C::TM];
            fold<KIND>(acc[u % C::TM][u / C::TM], pend[u % 4], su, sbj[(u / C::TM) & 1]);
          } else {
            const int u = t - kLag + kNT;   // previous chunk, last column
            fold<KIND>(acc[u % C::TM][C::TN - 1], pend[u % 4], scp[u % C::TM], last_col_scales());
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
                if (q * kSlots / kParts == t - kFirst) ld.part(q, s & 1);
            }
            if (t + 1 == kNT) {
              ld.advance();
              if constexpr (kPF) ld.prefetch(lds_addr(pf_junk));
            }
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
      for (int i = 0; i < C::TM; ++i) {
        // the previous chunk's last column keeps its scale for its lagged folds
        scp[i] = kMB ? (C::TN - 1 < jb ? sc[i] : sc1[i]) : sc[i];
        sc[i] = scn[i];
        if constexpr (kMB) sc1[i] = scn1[i];
      }
      if constexpr (kMB) jb = jbn;
      if constexpr (KIND == KIND_WGRAD && C::TN % 2 != 0) sbjp = sbj[(C::TN - 1) & 1];
    }

    // ---- tile done: remaining folds (scales of the tile's last chunk, now in
    // scp), epilogue; the next tile's first folds then add zeros ------------
#pragma unroll
    for (int u = kNT - kLag; u < kNT; ++u)
      fold<KIND>(acc[u % C::TM][u / C::TM], pend[u % 4], scp[u % C::TM], last_col_scales());
#pragma unroll
    for (int i = 0; i < C::TM; ++i) scp[i] = 0.f;
    const Tile cur = make_tile<GROUPED, TBN>(p, g, wk.start + wk.local + wk.nper * tk);
    const int el = lane_fresh();
    epilogue<KIND, QMODE, C::TM, C::TN, TBN>(p, cur, acc, cur.m0 + wave_m * C::WM + (el & 15), cur.n0 + wave_n * C::WN,
                                             el >> 4);
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
      for (int j = 0; j < C::TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  }
  // the repeated loads after the last step must land before the workgroup's
  // LDS is released
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// ---------------------------------------------------------------------------
// Power-of-two scales applied by the matrix unit.
// v_mfma_scale_f32_16x16x128_f8f6f4 takes one E8M0 exponent byte per lane for
// each operand: lane l scales row l % 16 of its operand over K-block l / 16
// (probed on gfx950). With power-of-two scales s = 2^k the byte is the fp32
// exponent field (k + 127; 0 for the subnormal 2^-127) and every K-block of a
// row carries its tile's scale, so the instruction itself multiplies each
// product by s_a * s_b — the "MMA with group scaling" the report asks hardware
// for (section 3.5.2) — and adds the scaled chunk sum into the FP32 accumulator
// (C = acc), which it does block by block (8 products at a time) rather than
// with one rounding. No VALU promotion is left, so the accumulator can live in
// the AGPRs: 128 x 128 wave tiles (256 accumulators), 4 waves (one per SIMD),
// workgroup tile 256 x 256, the same stages, loads and tile walk as above.
// ---------------------------------------------------------------------------
// Position t of the row / column pass order over an n x n grid of MFMAs:
// row 0, column 0 (what is left of it), row 1, column 1, ...; end_a / end_b
// name the operand whose last use this is (-1 if none).
struct PassCell { int i, j, end_a, end_b; };
constexpr PassCell pass_cell(int t, int n) {
  int pos = 0;
  for (int k = 0; k < n; ++k) {
    for (int j = k; j < n; ++j, ++pos)
      if (pos == t) return {k, j, j == n - 1 ? k : -1, (j == n - 1 && k == n - 1) ? k : -1};
    for (int i = k + 1; i < n; ++i, ++pos)
      if (pos == t) return {i, k, -1, i == n - 1 ? k : -1};
  }
  return {-1, -1, -1, -1};
}
// Position of the last MFMA that uses activation (weight) fragment k.
constexpr int death_a(int k, int n) {
  for (int t = 0; t < n * n; ++t) if (pass_cell(t, n).end_a == k) return t;
  return -1;
}
constexpr int death_b(int k, int n) {
  for (int t = 0; t < n * n; ++t) if (pass_cell(t, n).end_b == k) return t;
  return -1;
}
constexpr int cmax(int a, int b) { return a > b ? a : b; }
// LDS reads (two per fragment) that the pass order issues after the MFMAs at
// positions lo < t < hi.
constexpr int frag_reads_between(int lo, int hi, int n) {
  int r = 0;
  for (int t = lo + 1; t < hi; ++t) {
    const PassCell c = pass_cell(t, n);
    r += 2 * ((c.end_a >= 0) + (c.end_b >= 0));
  }
  return r;
}
template <class F, int... T>
__device__ __forceinline__ void for_each_const(F&& f, std::integer_sequence<int, T...>) {
  (f(std::integral_constant<int, T>{}), ...);
}

// The scaled MFMA as a statement with its accumulator tied (destination = C):
// written through the builtin, the register allocator moves accumulators
// between AGPRs around the loop when all 256 hold them, costing copies and
// hazard waits. It also fixes the MFMA's place in the schedule. The compiler
// no longer sees the instruction's hazards, so it carries them itself: two
// wait states ahead of it cover a VALU write of any of its operands just
// before (the scale exponents, the cleared accumulators); reading results
// needs mfma_results_ready().
__device__ __forceinline__ void mfma_scaled(v4f& acc, const v8i& a, const v8i& b, int sa, int sb) {
  asm volatile("s_nop 1\n\tv_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0]"
               : "+a"(acc) : "v"(a), "v"(b), "v"(sa), "v"(sb));
}
// Wait states between the last MFMAs and any other read of their results (more
// than the longest XDL write-to-read requirement); the scheduling barrier keeps
// every later instruction below them.
__device__ __forceinline__ void mfma_results_ready() {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ int e8m0(float s) { return (int)((__float_as_uint(s) >> 23) & 0xFFu); }

template <int KIND, bool GROUPED, int QMODE = 0>
__global__ __launch_bounds__(256) void gemm_pow2_kernel(GemmArgs p, GroupArgs g) {
  constexpr int WAVES_M = 2, WM = 128, WN = 128, TM = WM / 16, TN = WN / 16, kNT = TM * TN;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kStage];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wave_m = wave % WAVES_M;
  const int wave_n = wave / WAVES_M;
  const int l16 = lane & 15, lq = lane >> 4;

  const Walk wk = make_walk(p);
  if (wk.my_tiles == 0) return;                                // uniform: no tile for this workgroup
  const int my_tiles = wk.my_tiles, nc = wk.nc, total = wk.total;
  Loader<KIND, GROUPED, 4, 4> ld(p, g, wk, lds_addr(smem), wave, lane);
  constexpr int kParts = decltype(ld)::kParts;

  const int sw = swz(l16);
  const int off0 = l16 * BK + (((2 * lq) ^ sw) * 16);
  const int off1 = l16 * BK + (((2 * lq + 1) ^ sw) * 16);
  auto a_frag = [&](const uint8_t* stage, int i) { return frag(stage + (wave_m * WM + i * 16) * BK, off0, off1); };
  auto b_frag = [&](const uint8_t* stage, int j) {
    return frag(stage + kABytes + (wave_n * WN + j * 16) * BK, off0, off1);
  };
  // Exponent bytes of one step: ea[i] of this lane's activation row in subtile
  // i; eb[j] of its weight row in subtile j (one block scale per wave except
  // for WGRAD's row scales).
  // Scales of one step: ra[i] of this lane's activation row in subtile i; rb[j]
  // of its weight row in subtile j (one block scale per wave except for
  // WGRAD's row scales). The MFMA takes their exponent bytes.
  auto read_scales = [&](const uint8_t* stage, float (&ra)[TM], float (&rb)[TN]) {
    const float* Sa = reinterpret_cast<const float*>(stage + kSaOff);
    const float* Sb = reinterpret_cast<const float*>(stage + kSbOff);
#pragma unroll
    for (int i = 0; i < TM; ++i) ra[i] = Sa[wave_m * WM + i * 16 + l16];
    if constexpr (KIND == KIND_WGRAD) {
#pragma unroll
      for (int j = 0; j < TN; ++j) rb[j] = Sb[wave_n * WN + j * 16 + l16];
    } else {
      const float v = Sb[wave_n];
#pragma unroll
      for (int j = 0; j < TN; ++j) rb[j] = v;
    }
  };

#pragma unroll
  for (int q = 0; q < kParts; ++q) ld.part(q, 0);
  ld.advance();
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
#pragma unroll
  for (int q = 0; q < kParts; ++q) ld.part(q, 1);
  ld.advance();

  // A step's fragments all sit in registers before it starts. Its 64 MFMAs
  // run row 0, column 0, row 1, column 1, ... (each pass over what is left of
  // that row or column), so activation fragment k is dead after the row-k
  // pass and weight fragment k after the column-k pass; the next step's copy
  // of each is read into the same registers right then, which spreads the
  // step's 16 fragment reads over the step instead of bunching them at its
  // end. The stage a step was read from is therefore free once the step
  // begins; the one barrier per step (after the row-0 pass, before the first
  // read of the next stage) makes it free for every wave and the previous
  // step's loads visible, and the loads of step s + 2 into stage s % 2 spread
  // over kSlots MFMAs after it, leaving them the rest of the step to land.
#ifndef FP8BQ_P2_SLOTS
#define FP8BQ_P2_SLOTS 40
#endif
  constexpr int kFirst = TN;   // the barrier follows the row-0 pass
  constexpr int kSlots = FP8BQ_P2_SLOTS;
  static_assert(TM == TN, "the row / column pass order assumes square wave tiles");
  static_assert(kFirst + kSlots <= kNT, "loads must be issued within the step");
  // The compiler tracks at most 15 outstanding LDS reads; with more in
  // flight where a loop iteration begins it waits for all of them before the
  // first MFMA, which would expose the latency of the step's last reads. An
  // explicit wait late in each step (for reads issued at least kDrainLag
  // MFMAs earlier) keeps the count it carries across the loop below that.
  constexpr int kDrainAt = kNT - 5, kDrainLag = 8;
  constexpr int kExpReady = kFirst + 12;   // scales are read right after the barrier
  constexpr int kDrainCnt = frag_reads_between(kDrainAt - kDrainLag, kDrainAt, TM) +
                            2 * (pass_cell(kDrainAt, TM).end_a >= 0);
  static_assert(kDrainCnt + frag_reads_between(kDrainAt, kNT, TM) + 2 * (pass_cell(kDrainAt, TM).end_b >= 0) <= 14,
                "reads in flight at the end of a step must stay countable");
  v8i af[TM], bf[TN];
#pragma unroll
  for (int i = 0; i < TM; ++i) af[i] = a_frag(smem, i);
#pragma unroll
  for (int j = 0; j < TN; ++j) bf[j] = b_frag(smem, j);
  int ea[TM], eb[TN];
  float ran[TM], rbn[TN];
  read_scales(smem, ran, rbn);
#pragma unroll
  for (int i = 0; i < TM; ++i) ea[i] = e8m0(ran[i]);
#pragma unroll
  for (int j = 0; j < TN; ++j) eb[j] = e8m0(rbn[j]);
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the prologue's reads, for the same reason

  v4f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  int s = 0;
  // wait_loads: the step's barrier also waits for this wave's loads of the
  // next stage; a tile's first step skips that, its epilogue waited for them
  // before storing, so the stores stay in flight until the next step.
  auto step = [&](bool wait_loads) {
    const uint8_t* nstage = smem + ((s + 1) & 1) * kStage;
    for_each_const([&](auto tc) {
      constexpr int t = decltype(tc)::value;
      constexpr PassCell c = pass_cell(t, TM);
      mfma_scaled(acc[c.i][c.j], bf[c.j], af[c.i], eb[c.j], ea[c.i]);
      if constexpr (t >= kFirst && t < kFirst + kSlots) {
#pragma unroll
        for (int q = 0; q < kParts; ++q)
          if (q * kSlots / kParts == t - kFirst) ld.part(q, s & 1);
      }
      if constexpr (t + 1 == kNT) ld.advance();
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (c.end_a >= 0) {
        if constexpr (c.end_a == 0) {
          if (wait_loads) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          __syncthreads();
          read_scales(nstage, ran, rbn);
        }
        af[c.end_a] = a_frag(nstage, c.end_a);
      }
      // the next step's exponent of row (column) k replaces this step's once
      // both its last use has passed and the scale read has had time to land
      for_each_const([&](auto kc) {
        constexpr int k = decltype(kc)::value;
        if constexpr (cmax(death_a(k, TM), kExpReady) == t) ea[k] = e8m0(ran[k]);
        if constexpr (cmax(death_b(k, TN), kExpReady) == t) eb[k] = e8m0(rbn[k]);
      }, std::make_integer_sequence<int, TM>{});
      if constexpr (t == kDrainAt) __builtin_amdgcn_s_waitcnt(0xC07F | (kDrainCnt << 8));
      if constexpr (c.end_b >= 0) bf[c.end_b] = b_frag(nstage, c.end_b);
    }, std::make_integer_sequence<int, kNT>{});
    ++s;
  };

#pragma clang loop unroll(disable)
  for (int tk = 0; tk < my_tiles; ++tk) {
#pragma clang loop unroll(disable)
    for (int c = 0; c < nc; ++c) step(c != 0 || tk == 0);
    mfma_results_ready();
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the loads the next tile's first step reads

    // ---- tile done: epilogue --------------------------------------------------
    const Tile cur = make_tile<GROUPED>(p, g, wk.start + wk.local + wk.nper * tk);
    const int el = lane_fresh();
    epilogue<KIND, QMODE, TM, TN>(p, cur, acc, cur.m0 + wave_m * WM + (el & 15), cur.n0 + wave_n * WN, el >> 4);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  }
  // the repeated loads after the last step must land before the workgroup's
  // LDS is released
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  (void)total;
}

GemmArgs make_args(int64_t m, int64_t n, int64_t k, const uint8_t* a, int64_t lda, const float* sa,
                   int64_t ldsa, const uint8_t* b, int64_t ldb, const float* sb, int64_t ldsb,
                   void* out, int64_t ldo, int tbn = BN) {
  GemmArgs p;
  p.m = m; p.n = n; p.k = k;
  p.a = a; p.lda = lda; p.sa = sa; p.ldsa = ldsa;
  p.b = b; p.ldb = ldb; p.sb = sb; p.ldsb = ldsb;
  p.out = out; p.ldo = ldo;
  p.q = nullptr; p.ldq = 0; p.sq = nullptr; p.ldsq = 0;
  p.tiles_m = (int)((m + BM - 1) / BM);
  p.tiles_n = (int)((n + tbn - 1) / tbn);
  return p;
}

constexpr int kWM = 4;   // 4 x 2 waves of 64 x 128: the accumulator must stay within the
constexpr int kWN = 2;   // 256 VGPRs the VALU can address, with room for fragments
#ifndef FP8BQ_LOADERS
#define FP8BQ_LOADERS 8
#endif
constexpr int kLd = FP8BQ_LOADERS;   // waves issuing the operand loads
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
}  // namespace fp8bq
