// Online fine-grained E4M3 quantisers for gfx950 (MI355X).
//
// What they compute (DeepSeek-V3 report, Chinese translation, section 3.3.2
// "fine-grained quantization" / "online quantization", Figure 7a; tech note
// "DeepSeek-V3 FP8 dynamic quantisation", fine-grained quantization formulas):
// per 1x128 activation tile, 128x1 token-direction tile (section 3.3.3 / 3.5.2)
// or 128x128 weight block, s = fl32(absmax / 448) and q = E4M3(fl32(x / s)),
// rounded to nearest even, sign kept, s = 0 and +-0 codes for an all-zero group.
//
// These kernels are HBM-bound streams (read 2 B, write 1 B per element). The
// per-element arithmetic (fp8_codec.h) is kept small so it hides under the
// memory traffic; absmax is reduced across a tile's lanes with DPP row
// permutations.
#include "internal.h"
#include "fp8_codec.h"

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

namespace fp8bq {
namespace {

// Max of v over the 16 lanes of each DPP row; every lane of the row receives it.
__device__ __forceinline__ uint32_t row16_max(uint32_t v) {
  v = umax(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, true));   // quad_perm [1,0,3,2]
  v = umax(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, true));   // quad_perm [2,3,0,1]
  v = umax(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, true));  // row_half_mirror
  v = umax(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, true));  // row_mirror
  return v;
}

// Max over aligned groups of 8 lanes.
__device__ __forceinline__ uint32_t lane8_max(uint32_t v) {
  v = umax(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, true));
  v = umax(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, true));
  v = umax(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, true));
  return v;
}

// Largest of v over lanes l and l ^ 16 (xor16_max) or l and l ^ 32
// (xor32_max): gfx950's v_permlane16_swap_b32 exchanges the odd 16-lane rows of
// its first operand with the even rows of its second, v_permlane32_swap_b32 the
// upper half of the first with the lower half of the second; with v as both
// operands, the two results are v and its partner (one VALU instruction
// instead of a round trip through the LDS crossbar).
__device__ __forceinline__ uint32_t xor16_max(uint32_t v) {
  const auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return umax(a[0], a[1]);
}
__device__ __forceinline__ uint32_t xor32_max(uint32_t v) {
  const auto a = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return umax(a[0], a[1]);
}

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Packed (two 16-bit lanes per dword) max of the bf16 magnitudes of 8 dwords;
// returns the largest of the 16 magnitudes.
__device__ __forceinline__ uint32_t mag_max16(const uint4 a, const uint4 b) {
  auto m = [](uint32_t w) { return __builtin_bit_cast(u16x2, w & 0x7FFF7FFFu); };
  const u16x2 r = __builtin_elementwise_max(
      __builtin_elementwise_max(__builtin_elementwise_max(m(a.x), m(a.y)), __builtin_elementwise_max(m(a.z), m(a.w))),
      __builtin_elementwise_max(__builtin_elementwise_max(m(b.x), m(b.y)), __builtin_elementwise_max(m(b.z), m(b.w))));
  return umax(r.x, r.y);
}

// Eight bf16 (packed in four dwords) -> eight codes.
template <bool POW2>
__device__ __forceinline__ uint2 encode8(const uint4 w, const TileScale& t) {
  uint2 r;
  r.x = encode4<POW2>(bf_lo(w.x), bf_hi(w.x), bf_lo(w.y), bf_hi(w.y), t);
  r.y = encode4<POW2>(bf_lo(w.z), bf_hi(w.z), bf_lo(w.w), bf_hi(w.w), t);
  return r;
}

// ---------------------------------------------------------------------------
// 1x128 row-wise activation tiles.
// One tile per aligned group of 8 lanes (each lane 16 bf16 = 32 B, stored as
// 16 codes = 16 B), and each lane takes two neighbouring tiles of its row, both
// loaded before any arithmetic. A 256-thread block covers 32 rows of two
// column tiles: each load instruction reads 8 runs of 256 B, and a wave's 8
// scales per tile land in 32 contiguous bytes of the chunk-major scale array.
// Block b takes tile pair b % pairs of row group b / pairs: consecutive blocks
// read neighbouring 512-byte pieces of the same rows (with one tile per block,
// blocks walking along the rows were 12% faster on gfx950 than blocks walking
// down a column of tiles). Two tiles per lane: 55.3-56.2 against 56.0-57.1 us
// for one on X [16384, 7168] cold (rotated runs on one box), four: 55.9-57.4; a
// layout whose load instructions each read a 2 KB run of one row: 57.7 us.
// With an odd number of tiles per row, the last pair's second tile is its first.
// ---------------------------------------------------------------------------
constexpr int kRowThreads = 256;
constexpr int kRowsPerBlock = (kRowThreads / 64) * 8;

template <bool POW2>
__global__ __launch_bounds__(kRowThreads) void quant_act_rows_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, int rows, int tpr, uint8_t* __restrict__ q, int64_t ldq,
    float* __restrict__ s, int64_t lds) {
  const int lane = threadIdx.x & 63;
  const int l8 = lane & 7;
  const int pairs = (tpr + 1) / 2;
  const int group = (int)(blockIdx.x / (unsigned)pairs);
  const int pc = (int)(blockIdx.x - (unsigned)group * (unsigned)pairs);
  const int col0 = 2 * pc, col1 = min(2 * pc + 1, tpr - 1);
  const int r = group * kRowsPerBlock + (threadIdx.x >> 3);
  const int row = r < rows ? r : rows - 1;
  const uint16_t* p0 = x + (int64_t)row * ldx + col0 * 128 + l8 * 16;
  const uint16_t* p1 = x + (int64_t)row * ldx + col1 * 128 + l8 * 16;
  const uint4 v0 = *reinterpret_cast<const uint4*>(p0);
  const uint4 v1 = *reinterpret_cast<const uint4*>(p0 + 8);
  const uint4 w0 = *reinterpret_cast<const uint4*>(p1);
  const uint4 w1 = *reinterpret_cast<const uint4*>(p1 + 8);
  const TileScale ts = group_scale<POW2>(lane8_max(mag_max16(v0, v1)));
  const TileScale tt = group_scale<POW2>(lane8_max(mag_max16(w0, w1)));
  const uint2 a = encode8<POW2>(v0, ts), b = encode8<POW2>(v1, ts);
  const uint2 c = encode8<POW2>(w0, tt), d = encode8<POW2>(w1, tt);
  if (r < rows) {
    *reinterpret_cast<uint4*>(q + (int64_t)row * ldq + col0 * 128 + l8 * 16) = make_uint4(a.x, a.y, b.x, b.y);
    if (l8 == 0) s[(int64_t)col0 * lds + row] = ts.s;
    if (col1 != col0) {
      *reinterpret_cast<uint4*>(q + (int64_t)row * ldq + col1 * 128 + l8 * 16) = make_uint4(c.x, c.y, d.x, d.y);
      if (l8 == 0) s[(int64_t)col1 * lds + row] = tt.s;
    }
  }
}

// ---------------------------------------------------------------------------
// 128x1 column-wise tiles, written transposed.
// A 256-thread block stages 128 rows x 64 columns of bf16 (16 KB) in LDS: 8
// lanes per row load its 128 bytes, 32 rows at a time, so each thread has four
// 16-byte loads in flight. Thread t then owns columns 2 (t / 8), 2 (t / 8) + 1
// and rows [16 (t % 8), +16): it reduces each column's absmax with its 7
// neighbours (one aligned group of 8 lanes), encodes its 16 rows of each column
// and writes them as 16 contiguous bytes of the transposed output, so every
// output row of the block is one full 128-byte line. Half-width blocks (16 KB
// of LDS instead of 32) let 8 blocks share a CU instead of 5, which fills the
// memory pipeline better through the launch's last blocks: on X [4096, 7168]
// (interleaved runs on one box) 18.9-19.3 us against 19.8-19.9 us for 128
// columns per block, with byte-identical output; on X [16384, 7168] 61.9-62.3
// us against 62.8-63.2 us. (A first 64-column version
// staged dword by dword ran at 64% of 8 TB/s on X [16384, 7168].)
// LDS: the 16-byte unit u (columns 8u .. 8u + 7) of staged row r sits at unit
// u ^ ((r / 16) % 8). The LDS serves 128 bytes per clock, 32 lanes of a 4-byte
// read or 8 lanes of a 16-byte store at a time; a column read (32 lanes: 4
// column pairs of one unit, 8 rows 16 apart) then touches 32 distinct banks,
// and a staging store (8 lanes on one row) 8 distinct units.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int cols_swz(int r) { return (r >> 4) & 7; }

template <bool POW2>
__global__ __launch_bounds__(256) void quant_act_cols_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, uint8_t* __restrict__ qt, int64_t ldq,
    float* __restrict__ s, int64_t lds) {
  __shared__ uint4 tile[128 * 8];   // 128 rows x 8 units of 16 bytes (64 columns)
  const int t = threadIdx.x;
  const int64_t r0 = (int64_t)blockIdx.x * 128;
  const int64_t c0 = (int64_t)blockIdx.y * 64;
  const int l8 = t & 7, rs = t >> 3;
  uint4 in[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    in[j] = *reinterpret_cast<const uint4*>(x + (r0 + 32 * j + rs) * ldx + c0 + l8 * 8);
#pragma unroll
  for (int j = 0; j < 4; ++j) tile[(32 * j + rs) * 8 + (l8 ^ cols_swz(32 * j + rs))] = in[j];
  __syncthreads();

  const int p = t >> 3, seg = t & 7;   // columns 2p, 2p + 1; rows 16 seg .. + 15
  const uint32_t* lt = reinterpret_cast<const uint32_t*>(tile);
  uint32_t w[16];
  uint32_t m0 = 0u, m1 = 0u;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int row = seg * 16 + i;
    w[i] = lt[row * 32 + (((p >> 2) ^ cols_swz(row)) << 2) + (p & 3)];
    m0 = umax(m0, w[i] & 0x7FFFu);
    m1 = umax(m1, (w[i] >> 16) & 0x7FFFu);
  }
  const TileScale t0 = group_scale<POW2>(lane8_max(m0)), t1 = group_scale<POW2>(lane8_max(m1));
  uint4 o0, o1;
  o0.x = encode4<POW2>(bf_lo(w[0]), bf_lo(w[1]), bf_lo(w[2]), bf_lo(w[3]), t0);
  o0.y = encode4<POW2>(bf_lo(w[4]), bf_lo(w[5]), bf_lo(w[6]), bf_lo(w[7]), t0);
  o0.z = encode4<POW2>(bf_lo(w[8]), bf_lo(w[9]), bf_lo(w[10]), bf_lo(w[11]), t0);
  o0.w = encode4<POW2>(bf_lo(w[12]), bf_lo(w[13]), bf_lo(w[14]), bf_lo(w[15]), t0);
  o1.x = encode4<POW2>(bf_hi(w[0]), bf_hi(w[1]), bf_hi(w[2]), bf_hi(w[3]), t1);
  o1.y = encode4<POW2>(bf_hi(w[4]), bf_hi(w[5]), bf_hi(w[6]), bf_hi(w[7]), t1);
  o1.z = encode4<POW2>(bf_hi(w[8]), bf_hi(w[9]), bf_hi(w[10]), bf_hi(w[11]), t1);
  o1.w = encode4<POW2>(bf_hi(w[12]), bf_hi(w[13]), bf_hi(w[14]), bf_hi(w[15]), t1);
  *reinterpret_cast<uint4*>(qt + (c0 + 2 * p) * ldq + r0 + seg * 16) = o0;
  *reinterpret_cast<uint4*>(qt + (c0 + 2 * p + 1) * ldq + r0 + seg * 16) = o1;
  if (seg == 0) {
    float* sp = s + (int64_t)blockIdx.x * lds + c0 + 2 * p;
    sp[0] = t0.s;
    sp[1] = t1.s;
  }
}

// ---------------------------------------------------------------------------
// Transposing re-quantisation of an FP8 activation cache (1x128 -> 128x1).
// The report's backward step (section 3.5.2, "support for transposed GEMM"):
// read the forward pass's FP8 codes and 1x128 scales, dequantise, transpose
// and quantise again into 128x1 tiles; for these activations every scale is an
// integral power of two (section 3.3.3), so the conversion adds no error of its
// own where the row scale is not below the new one.
// x_hat = dec(q) * s is formed in float64, where it is exact for any binary32
// scale (4 + 24 significant bits), or in binary32 where that is exact too (see
// the kernel); the new scale is 2^k with k the smallest
// exponent such that the 128x1 group's absmax is at most 448 * 2^k (E8M0
// range, 2^-127 for an all-zero group); the code is E4M3(fl32(x_hat * 2^-k)),
// the product exact in float64 and rounded once to binary32.
// One 256-thread block per 128 x 128 block of the cache: the codes are staged
// in LDS; thread (p, seg) takes columns 4p .. 4p + 3 of rows 16 seg .. 16 seg +
// 15, so each of its four output rows gets 16 consecutive bytes; the column
// maxima meet across the 8 lanes that share p.
// LDS: staged row r at 128 r bytes; its 16-byte unit u (codes 16u .. 16u + 15)
// sits at unit u ^ ((r / 16) % 8). A column read (one dword per lane; over 32
// lanes p takes four consecutive values within one unit and seg 0..7) then
// touches 32 distinct dwords of one 128-byte stripe of banks, and a staging
// store (8 lanes on one row) the 8 units of that row. (Rows padded to 33
// dwords instead put the rows 16 seg of four row groups on the same banks: a
// 4-way conflict in every read.)
// ---------------------------------------------------------------------------
__device__ __forceinline__ int req_unit(int u, int r) { return u ^ ((r >> 4) & 7); }

// The four E4M3 codes of a word as floats (exact; hardware conversion).
__device__ __forceinline__ void dec4(uint32_t w, float (&f)[4]) {
  f[0] = __builtin_amdgcn_cvt_f32_fp8((int)w, 0);
  f[1] = __builtin_amdgcn_cvt_f32_fp8((int)w, 1);
  f[2] = __builtin_amdgcn_cvt_f32_fp8((int)w, 2);
  f[3] = __builtin_amdgcn_cvt_f32_fp8((int)w, 3);
}

// A 64-bit value moved between lanes by one DPP pattern (both halves alike).
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t b) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, CTRL, 0xF, 0xF, true);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), CTRL, 0xF, 0xF, true);
  return ((uint64_t)hi << 32) | lo;
}

// Largest of a non-negative double over an aligned group of 8 lanes. For
// non-negative doubles the order is that of their bit patterns as unsigned
// integers, so the rounds of lane8_max (partners lane ^ 1, lane ^ 2, then the
// group's mirror) apply to the patterns, in VALU and DPP instead of the LDS
// crossbar.
__device__ __forceinline__ double dmax_lane8(double v) {
  uint64_t b = (uint64_t)__double_as_longlong(v);
  uint64_t o = dpp_u64<0xB1>(b);
  b = o > b ? o : b;
  o = dpp_u64<0x4E>(b);
  b = o > b ? o : b;
  o = dpp_u64<0x141>(b);
  b = o > b ? o : b;
  return __longlong_as_double((long long)b);
}

// The same for a binary32 a >= 0: a = 1.f * 2^(E - 127) with 448 = 1.75 * 2^8
// (a zero or subnormal a gives k <= -134, clamped to -127, as in float64).
__device__ __forceinline__ int pow2_exponent_f32(float a) {
  const uint32_t b = __float_as_uint(a);
  const int k = (int)(b >> 23) - 135 + ((b & 0x7FFFFFu) > 0x600000u ? 1 : 0);
  return max(-127, min(127, k));
}

// k = smallest integer with a <= 448 * 2^k, clamped to [-127, 127]; a >= 0.
__device__ __forceinline__ int pow2_exponent_f64(double a) {
  const uint64_t b = (uint64_t)__double_as_longlong(a);
  const int e = (int)((b >> 52) & 0x7FF);
  const uint64_t m = b & 0xFFFFFFFFFFFFFull;
  const int k = e - 1031 + (m > 0xC000000000000ull ? 1 : 0);   // 448 = 1.75 * 2^8
  return max(-127, min(127, k));
}

// POW2_HINT: the caller's scales are powers of two (FP8BQ_SCALE_POW2): blocks
// whose row scales all qualify take a binary32 path (below); the others, and
// every block without the hint, the float64 path. The results are the same.
template <bool POW2_HINT>
__global__ __launch_bounds__(256) void requant_t_kernel(
    const uint8_t* __restrict__ q, int64_t ldq, const float* __restrict__ s, int64_t lds,
    uint8_t* __restrict__ qt, int64_t ldqt, float* __restrict__ st, int64_t ldst) {
  __shared__ uint4 tile[128 * 8];   // 128 rows x 8 units of 16 bytes
  const int t = threadIdx.x;
  // row blocks vary fastest: consecutive blocks write neighbouring 128-byte
  // pieces of the same transposed rows (6% faster than column blocks fastest)
  const int64_t r0 = (int64_t)blockIdx.x * 128, c0 = (int64_t)blockIdx.y * 128;

#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = i * 32 + (t >> 3);
    tile[row * 8 + req_unit(t & 7, row)] =
        *reinterpret_cast<const uint4*>(q + (r0 + row) * ldq + c0 + (t & 7) * 16);
  }
  const int p = t >> 3, seg = t & 7;
  const float* srow = s + (int64_t)blockIdx.y * lds + r0 + seg * 16;
  float sf[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) sf[i] = srow[i];
  __syncthreads();

  uint32_t w[16];
#pragma unroll
  for (int i = 0; i < 16; ++i)   // dword p of row 16 seg + i: dword p % 4 of logical unit p / 4
    w[i] = reinterpret_cast<const uint32_t*>(tile)[(seg * 16 + i) * 32 + req_unit(p >> 2, seg * 16) * 4 + (p & 3)];

  // Row scales that are powers of two 2^e with -117 <= e <= 118 (the forward
  // pass's activation scales, report section 3.3.3): dec(q) * s then has at
  // most 4 significant bits and lies in binary32's normal range (|dec(q)| <=
  // 448 < 2^9, and its smallest nonzero magnitude 2^-9 times 2^-117 is
  // 2^-126), so binary32 forms x_hat exactly, and with it the column maxima
  // and x_hat * 2^-k (exact, or below 2^-126, where it encodes to a signed
  // zero whether rounded or flushed): the float64 path's values, at a fraction
  // of its cost. A wave takes this path when every lane's scales qualify.
  // Output row b of the thread (column 4p + b) is byte b of every w[i].
  auto emit = [&](int b, auto&& value) {
    uint4 o;
    uint32_t* const op = reinterpret_cast<uint32_t*>(&o);
#pragma unroll
    for (int g = 0; g < 4; ++g)
      op[g] = cvt4(value(4 * g, b), value(4 * g + 1, b), value(4 * g + 2, b), value(4 * g + 3, b));
    *reinterpret_cast<uint4*>(qt + (c0 + 4 * p + b) * ldqt + r0 + seg * 16) = o;
  };
  // reform(): tells the compiler that w may have changed, so that a pass forms
  // its values again instead of keeping an earlier pass's live (and decoding
  // shared by two branches is not hoisted above them)
  auto reform = [&]() {
#pragma unroll
    for (int i = 0; i < 16; ++i) asm volatile("" : "+v"(w[i]));
  };
  auto dec1 = [&](int i, int b) {   // (b is a constant once unrolled: one conversion)
    const int x = (int)w[i];
    return b == 0 ? __builtin_amdgcn_cvt_f32_fp8(x, 0) : b == 1 ? __builtin_amdgcn_cvt_f32_fp8(x, 1)
         : b == 2 ? __builtin_amdgcn_cvt_f32_fp8(x, 2) : __builtin_amdgcn_cvt_f32_fp8(x, 3);
  };
  // float64 path, pass 1: the column maxima of |x_hat|, exact
  auto f64_max = [&](int (&k)[4]) {
    double cmax[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float d[4];
      dec4(w[i], d);
#pragma unroll
      for (int b = 0; b < 4; ++b) cmax[b] = fmax(cmax[b], fabs((double)d[b] * (double)sf[i]));
    }
#pragma unroll
    for (int b = 0; b < 4; ++b) k[b] = pow2_exponent_f64(dmax_lane8(cmax[b]));
  };
  int k[4];
  bool fast = POW2_HINT;
  if constexpr (POW2_HINT) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t b = __float_as_uint(sf[i]);
      fast = fast && (b & 0x807FFFFFu) == 0u && (b >> 23) - 10u <= 235u;   // exponent field 10 .. 245
    }
    fast = __builtin_amdgcn_ballot_w64(!fast) == 0;   // wave-uniform
  }
  if (fast) {
    // binary32 path: pass 2 forms x_hat again, output row by output row,
    // encoding four values at a time (57 registers where keeping pass 1's
    // values, or sharing them with the other branch, took 173-228)
    reform();
    float cmax[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float d[4];
      dec4(w[i], d);
#pragma unroll
      for (int b = 0; b < 4; ++b) cmax[b] = fmaxf(cmax[b], fabsf(d[b] * sf[i]));   // exact
    }
#pragma unroll
    for (int b = 0; b < 4; ++b) k[b] = pow2_exponent_f32(__uint_as_float(lane8_max(__float_as_uint(cmax[b]))));
    reform();
#pragma unroll
    for (int b = 0; b < 4; ++b) emit(b, [&](int i, int bb) { return ldexpf(dec1(i, bb) * sf[i], -k[bb]); });
  } else if constexpr (POW2_HINT) {
    // a hinted launch whose block has other scales: float64, forming x_hat
    // again in pass 2 (keeping the registers of the binary32 path's kernel)
    reform();
    f64_max(k);
    reform();
#pragma unroll
    for (int b = 0; b < 4; ++b)   // exact product, one rounding
      emit(b, [&](int i, int bb) { return (float)ldexp((double)dec1(i, bb) * (double)sf[i], -k[bb]); });
  } else {
    // float64 path: pass 2 scales the products of pass 1, which the compiler
    // keeps live (148-175 registers; forming them again is 13% slower, the
    // path being bound by its float64 arithmetic)
    f64_max(k);
    float v[4][16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float d[4];
      dec4(w[i], d);
#pragma unroll
      for (int b = 0; b < 4; ++b) v[b][i] = (float)ldexp((double)d[b] * (double)sf[i], -k[b]);   // exact, one rounding
    }
#pragma unroll
    for (int b = 0; b < 4; ++b) emit(b, [&](int i, int bb) { return v[bb][i]; });
  }
  if (seg == 0) {
    float4 sc;
    float* scp = reinterpret_cast<float*>(&sc);
#pragma unroll
    for (int b = 0; b < 4; ++b)
      scp[b] = k[b] >= -126 ? __uint_as_float((uint32_t)(k[b] + 127) << 23) : __uint_as_float(0x00400000u);
    float* sp = st + (int64_t)blockIdx.x * ldst + c0 + 4 * p;
    sp[0] = sc.x; sp[1] = sc.y; sp[2] = sc.z; sp[3] = sc.w;
  }
}

// ---------------------------------------------------------------------------
// 128x128 weight blocks. One 256-thread block per weight block: each thread
// holds 64 elements (8 rows x 8 columns) in registers, so the block is read
// from HBM once; the absmax goes DPP row -> cross-row shuffles -> LDS.
// Optionally the codes are staged in LDS and written transposed as well.
// ---------------------------------------------------------------------------
constexpr int kWStride = 132;   // bytes per staged code row (128 + 4 pad, keeps dword alignment)

__device__ __forceinline__ uint32_t byte_perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

template <bool POW2>
__global__ __launch_bounds__(256) void quant_w_kernel(
    const uint16_t* __restrict__ w, int64_t ldw, uint8_t* __restrict__ q, int64_t ldq,
    float* __restrict__ s, int64_t lds, uint8_t* __restrict__ qt, int64_t ldqt) {
  __shared__ uint32_t wmax[4];
  __shared__ uint32_t codes[128 * kWStride / 4];
  const int t = threadIdx.x;
  const int64_t n0 = (int64_t)blockIdx.y * 128, k0 = (int64_t)blockIdx.x * 128;
  const int r = t >> 4, c8 = (t & 15) * 8;

  uint4 v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    v[i] = *reinterpret_cast<const uint4*>(w + (n0 + r + 16 * i) * ldw + k0 + c8);

  uint32_t m = umax(umax(mag_max16(v[0], v[1]), mag_max16(v[2], v[3])),
                    umax(mag_max16(v[4], v[5]), mag_max16(v[6], v[7])));
  m = row16_max(m);
  m = xor32_max(xor16_max(m));
  if ((t & 63) == 0) wmax[t >> 6] = m;
  __syncthreads();
  m = umax(umax(wmax[0], wmax[1]), umax(wmax[2], wmax[3]));
  const TileScale ts = group_scale<POW2>(m);
  if (t == 0) s[(int64_t)blockIdx.y * lds + blockIdx.x] = ts.s;

#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint2 c = encode8<POW2>(v[i], ts);
    *reinterpret_cast<uint2*>(q + (n0 + r + 16 * i) * ldq + k0 + c8) = c;
    if (qt) {
      uint32_t* dst = codes + ((r + 16 * i) * kWStride + c8) / 4;
      dst[0] = c.x;
      dst[1] = c.y;
    }
  }
  if (!qt) return;   // uniform over the block
  __syncthreads();

  // Thread t transposes the 16 (n) x 4 (k) byte sub-block at n = 16 (t / 32),
  // k = 4 (t % 32) and writes 4 rows of 16 bytes of the [k, n] copy.
  const int kq = t & 31, nb = t >> 5;
  uint32_t d[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) d[i] = codes[((nb * 16 + i) * kWStride) / 4 + kq];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    // byte j of d[4g .. 4g+3] -> dword g of output row j
    uint32_t o[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const uint32_t sel01 = (uint32_t)(j) | ((uint32_t)(j + 4) << 8);           // byte j of lo, byte j of hi
      const uint32_t a = byte_perm(d[4 * g + 1], d[4 * g + 0], sel01 | 0x0C0C0000u);
      const uint32_t b = byte_perm(d[4 * g + 3], d[4 * g + 2], sel01 | 0x0C0C0000u);
      o[g] = (a & 0xFFFFu) | (b << 16);
    }
    *reinterpret_cast<uint4*>(qt + (k0 + 4 * kq + j) * ldqt + n0 + 16 * nb) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

// Weight blocks without the transposed copy: a workgroup quantises two
// neighbouring 128x128 blocks along k. Lane l takes 32 contiguous bytes (16
// values) of one row: row 4 i + l / 16 of its wave's 32, block (l / 8) % 2,
// columns 16 (l % 8) .. + 15; it stores 16 bytes of codes per row, so each
// load and store instruction of a wave touches four rows of both blocks. Absmax per block: DPP
// over each group of 8 lanes, lanes l ^ 16 and l ^ 32 (the other rows), then
// the four waves through LDS. A k with an odd number of blocks leaves the
// second block of the last workgroup empty: its lanes re-read the first block
// and store nothing. Measured on W [18432, 7168] (interleaved runs on one box):
// 64.3-65.0 us against 64.9-65.6 us for 16-byte loads and 8-byte stores per
// lane, and 65.8 us for one block per workgroup; the plain read-2-bytes /
// write-1-byte stream takes 60.7 us.
template <bool POW2>
__global__ __launch_bounds__(256) void quant_w2_kernel(
    const uint16_t* __restrict__ w, int64_t ldw, int kblocks, uint8_t* __restrict__ q, int64_t ldq,
    float* __restrict__ s, int64_t lds) {
  __shared__ uint32_t wmax[4][2];
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int rg = lane >> 4, half = (lane >> 3) & 1, l8 = lane & 7;
  const int kb = 2 * (int)blockIdx.x + half;
  const bool ok = kb < kblocks;
  const int64_t n0 = (int64_t)blockIdx.y * 128;
  const int64_t col = (int64_t)(ok ? kb : kb - 1) * 128 + l8 * 16;
  uint4 v[8][2];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint16_t* pp = w + (n0 + wv * 32 + 4 * i + rg) * ldw + col;
    v[i][0] = *reinterpret_cast<const uint4*>(pp);
    v[i][1] = *reinterpret_cast<const uint4*>(pp + 8);
  }
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = umax(m, mag_max16(v[i][0], v[i][1]));
  m = xor32_max(xor16_max(lane8_max(m)));
  if (lane == 0) wmax[wv][0] = m;
  if (lane == 8) wmax[wv][1] = m;
  __syncthreads();
  m = umax(umax(wmax[0][half], wmax[1][half]), umax(wmax[2][half], wmax[3][half]));
  const TileScale ts = group_scale<POW2>(m);
  if (!ok) return;
  if (t == 0 || t == 8) s[(int64_t)blockIdx.y * lds + kb] = ts.s;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint2 a = encode8<POW2>(v[i][0], ts), b = encode8<POW2>(v[i][1], ts);
    *reinterpret_cast<uint4*>(q + (n0 + wv * 32 + 4 * i + rg) * ldq + col) = make_uint4(a.x, a.y, b.x, b.y);
  }
}

// ---------------------------------------------------------------------------
// E5M6 activation cache (report section 3.3.3, low-precision activations,
// item 1: the inputs of the Linear after attention are cached in a custom
// 12-bit E5M6 format, in 1x128 tiles with power-of-two scaling factors).
// E5M6: 1 sign, 5 exponent (bias 15), 6 mantissa bits, the binary16 layout
// without its four lowest mantissa bits; subnormals m * 2^-20; largest finite
// value 65024. Tile scale s = 2^k, k the smallest integer with absmax <=
// 65024 * 2^k, clamped to [-127, 127]; codes E5M6(x * 2^-k), rounded to
// nearest even once (the product is exact). Codes are packed two per 3 bytes,
// little-endian in the 24-bit group, so a tile is 192 contiguous bytes.
// ---------------------------------------------------------------------------

// k of the tile from its bf16 absmax bits (no sign). absmax = f * 2^(e - 127)
// with f = 1 + m / 128; 65024 = (127/64) * 2^15, so k = e - 142, plus one when
// f > 127/64 (m = 127). A zero or subnormal absmax is at most 65024 * 2^-127.
__device__ __forceinline__ int e5m6_tile_exponent(uint32_t amax16) {
  const int e = (int)(amax16 >> 7);
  if (e == 0) return -127;
  const int k = e - 142 + ((amax16 & 0x7Fu) == 0x7Fu ? 1 : 0);
  return k < -127 ? -127 : k;
}

// 2^j as a float for j in [-127, 127] (2^-127 is subnormal).
__device__ __forceinline__ float exp2_int(int j) {
  return j >= -126 ? __uint_as_float((uint32_t)(j + 127) << 23) : __uint_as_float(0x00400000u);
}

// E5M6 code of v, |v| <= 65024: round to nearest even, sign kept. Normal
// range (|v| >= 2^-14): the fp32 mantissa rounded to 6 bits (a carry moves
// into the exponent), exponent rebiased 127 -> 15; below it, the nearest
// multiple of 2^-20 (64 of them is the smallest normal, whose code is 64).
__device__ __forceinline__ uint32_t e5m6_code(float v) {
  const uint32_t b = __float_as_uint(v);
  const uint32_t sign = (b >> 20) & 0x800u;
  const uint32_t mag = b & 0x7FFFFFFFu;
  const uint32_t cn = ((mag + 0xFFFFu + ((mag >> 17) & 1u)) >> 17) - (112u << 6);
  const uint32_t cs = (uint32_t)__builtin_rintf(__uint_as_float(mag) * 1048576.0f);   // exact product
  return (mag >= 0x38800000u ? cn : cs) | sign;   // both formed: no divergent branch
}

// Value of an E5M6 code (exponent field 31 is never written).
__device__ __forceinline__ float e5m6_value(uint32_t c) {
  const uint32_t e = (c >> 6) & 31u, m = c & 63u;
  const float f = e ? __uint_as_float(((e + 112u) << 23) | (m << 17)) : (float)m * 0x1p-20f;
  return __uint_as_float(__float_as_uint(f) | ((c & 0x800u) << 20));
}

// A tile per 16-lane DPP row, 8 elements per lane: a lane loads 16 B of bf16
// and stores its 12 code bytes next to its neighbours', so one store
// instruction writes each tile's 192 bytes contiguously (with 24-byte lanes,
// three 8-byte stores each covering every third piece of the tile ran the
// cache at 83 us on X [16384, 7168]). A 256-thread block covers 16 rows of one
// 128-column chunk (4 per wave).
constexpr int kE5RowsPerBlock = kRowThreads / 16;

__device__ __forceinline__ uint32_t mag_max8(const uint4 a) {
  auto m = [](uint32_t w) { return __builtin_bit_cast(u16x2, w & 0x7FFF7FFFu); };
  const u16x2 r = __builtin_elementwise_max(__builtin_elementwise_max(m(a.x), m(a.y)),
                                            __builtin_elementwise_max(m(a.z), m(a.w)));
  return umax(r.x, r.y);
}

typedef short i16x2 __attribute__((ext_vector_type(2)));

// Codes of two bf16 values (one dword w, magnitudes m = w & 0x7FFF7FFF) under
// the tile scale 2^k, on the fast path: each value zero or, scaled, in E5M6's
// normal range (bf16 exponent at least k + 113), and k >= -111. With a
// power-of-two scale the code is then the bf16 magnitude with its lowest
// mantissa bit rounded off (to nearest, ties to even; a carry moves into the
// exponent) and the exponent rebiased by -(k + 112) (off = (k + 112) << 6 in
// both halves); a zero gives a negative difference, clamped to 0, and the sign
// bits move from bit 15 to bit 11. Two values per 32-bit instruction, with
// packed 16-bit arithmetic. Returns the 24-bit group (low value in bits 0..11).
__device__ __forceinline__ uint32_t e5m6_pair_fast(uint32_t w, uint32_t m, u16x2 off) {
  const u16x2 q = __builtin_bit_cast(u16x2, m) >> (u16x2){1, 1};
  const uint32_t tie = m & __builtin_bit_cast(uint32_t, q) & 0x00010001u;   // dropped bit 1 and q odd
  const u16x2 cm = q + __builtin_bit_cast(u16x2, tie);
  const i16x2 c = __builtin_elementwise_max(__builtin_bit_cast(i16x2, (u16x2)(cm - off)), (i16x2){0, 0});
  const uint32_t code = __builtin_bit_cast(uint32_t, c) | ((w >> 4) & 0x08000800u);
  return (code & 0x0FFFu) | ((code >> 4) & 0x00FFF000u);
}

// A thread takes NT neighbouring tiles of its row (NT = 2 when the row has an
// even number of tiles: two loads in flight per lane, as in the FP8 kernel).
// A wave whose values all qualify for e5m6_pair_fast (the usual case: E5M6
// subnormals lie 28 binades below a tile's absmax) encodes them with it; any
// other wave uses the general codec for that tile (half the VALU instructions
// per value on the fast path, which ran the kernel at 73% of 8 TB/s before).
template <int NT>
__global__ __launch_bounds__(kRowThreads) void cache_e5m6_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, int rows, int tpr, uint8_t* __restrict__ q, int64_t ldq,
    float* __restrict__ s, int64_t lds) {
  const int l16 = threadIdx.x & 15;
  const int groups = tpr / NT;
  const int group = (int)(blockIdx.x / (unsigned)groups);
  const int col0 = (int)(blockIdx.x - (unsigned)group * (unsigned)groups) * NT;
  const int r = group * kE5RowsPerBlock + (threadIdx.x >> 4);
  const int row = r < rows ? r : rows - 1;
  uint4 v[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
    v[t] = *reinterpret_cast<const uint4*>(x + (int64_t)row * ldx + (col0 + t) * 128 + l16 * 8);
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int k = e5m6_tile_exponent(row16_max(mag_max8(v[t])));
    const uint32_t w[4] = {v[t].x, v[t].y, v[t].z, v[t].w};
    uint32_t m[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) m[i] = w[i] & 0x7FFF7FFFu;
    // fast path: every non-zero magnitude at least (k + 113) << 7 (m - 1 wraps a
    // zero to 0xFFFF), k >= -111
    const u16x2 one = {1, 1};
    const u16x2 mn = __builtin_elementwise_min(
        __builtin_elementwise_min(__builtin_bit_cast(u16x2, m[0]) - one, __builtin_bit_cast(u16x2, m[1]) - one),
        __builtin_elementwise_min(__builtin_bit_cast(u16x2, m[2]) - one, __builtin_bit_cast(u16x2, m[3]) - one));
    const uint32_t mn16 = mn.x < mn.y ? mn.x : mn.y;
    const bool ok = k >= -111 && mn16 >= (uint32_t)(((k + 113) << 7) - 1);
    uint32_t pr[4];   // element pairs (2i, 2i + 1) as 24-bit groups
    if (__builtin_amdgcn_ballot_w64(!ok) == 0) {   // uniform per wave
      const unsigned short o = (unsigned short)((k + 112) << 6);
      const u16x2 off = {o, o};
#pragma unroll
      for (int i = 0; i < 4; ++i) pr[i] = e5m6_pair_fast(w[i], m[i], off);
    } else {
      const float inv = exp2_int(-k);
#pragma unroll
      for (int i = 0; i < 4; ++i) pr[i] = e5m6_code(bf_lo(w[i]) * inv) | (e5m6_code(bf_hi(w[i]) * inv) << 12);
    }
    if (r < rows) {
      *reinterpret_cast<uint3*>(q + (int64_t)row * ldq + (col0 + t) * 192 + l16 * 12) =
          make_uint3(pr[0] | (pr[1] << 24), (pr[1] >> 8) | (pr[2] << 16), (pr[2] >> 16) | (pr[3] << 8));
      if (l16 == 0) s[(int64_t)(col0 + t) * lds + row] = exp2_int(k);
    }
  }
}

template <int NT>
__global__ __launch_bounds__(kRowThreads) void uncache_e5m6_kernel(
    const uint8_t* __restrict__ q, int64_t ldq, const float* __restrict__ s, int64_t lds, int rows, int tpr,
    uint16_t* __restrict__ y, int64_t ldy) {
  const int l16 = threadIdx.x & 15;
  const int groups = tpr / NT;
  const int group = (int)(blockIdx.x / (unsigned)groups);
  const int col0 = (int)(blockIdx.x - (unsigned)group * (unsigned)groups) * NT;
  const int r = group * kE5RowsPerBlock + (threadIdx.x >> 4);
  if (r >= rows) return;
  uint3 in[NT];
  float sc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    in[t] = *reinterpret_cast<const uint3*>(q + (int64_t)r * ldq + (col0 + t) * 192 + l16 * 12);
    sc[t] = s[(int64_t)(col0 + t) * lds + r];
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const uint3 i = in[t];
    const uint32_t pr[4] = {i.x & 0xFFFFFFu, (i.x >> 24) | ((i.y & 0xFFFFu) << 8),
                            (i.y >> 16) | ((i.z & 0xFFu) << 16), i.z >> 8};
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // exact products (7 significant bits times a power of two within range),
      // then one rounding to bf16
      const bf16x2 h = __builtin_convertvector(
          (f32x2){e5m6_value(pr[j] & 0xFFFu) * sc[t], e5m6_value(pr[j] >> 12) * sc[t]}, bf16x2);
      __builtin_memcpy(&o[j], &h, 4);
    }
    *reinterpret_cast<uint4*>(y + (int64_t)r * ldy + (col0 + t) * 128 + l16 * 8) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

// ---------------------------------------------------------------------------
// E5M6 cache -> 128x1 FP8 tiles (the backward use of the cache: its 1x128
// tiles become the 128x1 tiles of the weight-gradient operand). x_hat =
// E5M6(code) * 2^kc exactly; per 128 rows of one column, k = the smallest
// integer with absmax <= 448 * 2^k (within [-127, 127]) and codes
// E4M3(fl32(x_hat * 2^-k)); the output scale is 2^k.
//
// All in fp32. A code shifted left by 4 is the IEEE binary16 pattern of its
// value, so one half-to-float conversion decodes it (exactly, subnormals
// included). y = value * 2^(kc - 2) is exact: y has at most 7 significant
// bits, its smallest possible quantum is 2^-20 * 2^-127 * 2^-2 = 2^-149 and its
// magnitude stays below 2^16 * 2^113 * 2^-2 = 2^127 (a bf16 input keeps kc <=
// 113; the 2^-2 is what keeps the largest cached value, up to 2^128, finite).
// The column absmax is then a plain fp32 max over y, and the code input is
// ldexp(y, 2 - k): exact unless it falls below 2^-126, where every value
// encodes to a signed E4M3 zero anyway.
//
// One 256-thread block per 128 x 128 block of values (a 128-row x 192-byte
// piece of the cache). Staging: 16 lanes per row, each loading 12 bytes (8
// codes) and storing them as 8 binary16 patterns (16 bytes) to LDS. Then
// thread (p, seg) takes columns 4p .. 4p + 3 of rows 16 seg .. 16 seg + 15,
// as in the FP8 re-quantisation above.
// LDS tile: row r at 256 r bytes; the 8-byte unit u (codes 4u .. 4u + 3) sits
// at unit u ^ e5_swz(r >> 4). Over any 16 lanes of a read (p in {2i, 2i+1},
// seg 0..7) the units are 16 distinct ones of 16 consecutive aligned units,
// and over 32 lanes 32 distinct units: every read is free of bank conflicts.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int e5_swz(int seg) { return (seg << 1) ^ ((seg & 1) << 4); }

// Smallest k with a <= 448 * 2^k from y = a / 4 (a >= 0, y exact), within
// [-127, 127]. y = f * 2^(E - 127): k = E - 133, plus one when f > 1.75.
__device__ __forceinline__ int pow2_exponent_y4(float y) {
  const uint32_t b = __float_as_uint(y);
  const int k = (int)(b >> 23) - 133 + ((b & 0x7FFFFFu) > 0x600000u ? 1 : 0);
  return max(-127, min(127, k));
}

__device__ __forceinline__ float half_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)(w & 0xFFFFu));
}
__device__ __forceinline__ float half_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)(w >> 16));
}

__global__ __launch_bounds__(256) void requant_e5m6_t_kernel(
    const uint8_t* __restrict__ q, int64_t ldq, const float* __restrict__ s, int64_t lds,
    uint8_t* __restrict__ qt, int64_t ldqt, float* __restrict__ st, int64_t ldst) {
  __shared__ uint4 tile[128 * 16];   // 128 rows x 16 units of 16 bytes
  const int t = threadIdx.x;
  const int64_t r0 = (int64_t)blockIdx.x * 128, c0 = (int64_t)blockIdx.y * 128;
  const int l16 = t & 15, rs = t >> 4;

  uint3 in[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
    in[j] = *reinterpret_cast<const uint3*>(q + (r0 + 16 * j + rs) * ldq + blockIdx.y * 192 + l16 * 12);
  const int p = t >> 3, seg = t & 7;
  float sc[16];   // 2^(kc - 2) of the 16 rows (exact: the cache scales are powers of two)
  const float* srow = s + (int64_t)blockIdx.y * lds + r0 + seg * 16;
#pragma unroll
  for (int i = 0; i < 16; ++i) sc[i] = srow[i] * 0.25f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint3 v = in[j];
    const uint32_t pr[4] = {v.x & 0xFFFFFFu, (v.x >> 24) | ((v.y & 0xFFFFu) << 8),
                            (v.y >> 16) | ((v.z & 0xFFu) << 16), v.z >> 8};
    uint32_t h[4];   // codes 2i, 2i + 1 as binary16 patterns (code << 4) in the low / high half
#pragma unroll
    for (int i = 0; i < 4; ++i) h[i] = ((pr[i] << 4) & 0xFFF0u) | ((pr[i] << 8) & 0xFFF00000u);
    // row 16 j + rs, units 2 l16 and 2 l16 + 1 -> 16-byte slot l16 ^ (e5_swz(j) / 2)
    tile[(16 * j + rs) * 16 + (l16 ^ (e5_swz(j) >> 1))] = make_uint4(h[0], h[1], h[2], h[3]);
  }
  __syncthreads();

  const uint2* lt = reinterpret_cast<const uint2*>(tile);
  float y[16][4];
  float cmax[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint2 w = lt[(seg * 16 + i) * 32 + (p ^ e5_swz(seg))];
    y[i][0] = half_lo(w.x) * sc[i];
    y[i][1] = half_hi(w.x) * sc[i];
    y[i][2] = half_lo(w.y) * sc[i];
    y[i][3] = half_hi(w.y) * sc[i];
#pragma unroll
    for (int b = 0; b < 4; ++b) cmax[b] = fmaxf(cmax[b], fabsf(y[i][b]));
  }
  int k[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) k[b] = pow2_exponent_y4(__uint_as_float(lane8_max(__float_as_uint(cmax[b]))));
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int n = 2 - k[b];
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = __builtin_amdgcn_ldexpf(y[i][b], n);
    uint4 o;
    o.x = cvt4(v[0], v[1], v[2], v[3]);
    o.y = cvt4(v[4], v[5], v[6], v[7]);
    o.z = cvt4(v[8], v[9], v[10], v[11]);
    o.w = cvt4(v[12], v[13], v[14], v[15]);
    *reinterpret_cast<uint4*>(qt + (c0 + 4 * p + b) * ldqt + r0 + seg * 16) = o;
  }
  if (seg == 0) {
    float* sp = st + (int64_t)blockIdx.x * ldst + c0 + 4 * p;
#pragma unroll
    for (int b = 0; b < 4; ++b) sp[b] = exp2_int(k[b]);
  }
}

}  // namespace

hipError_t launch_quant_act_rows(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                                 uint8_t* q, int64_t ldq, float* s, int64_t lds, bool pow2, hipStream_t st) {
  const int tpr = (int)(cols / 128);
  const dim3 grid((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock * ((tpr + 1) / 2)));
  if (pow2)
    hipLaunchKernelGGL(quant_act_rows_kernel<true>, grid, dim3(kRowThreads), 0, st, x, ldx, (int)rows, tpr, q, ldq, s, lds);
  else
    hipLaunchKernelGGL(quant_act_rows_kernel<false>, grid, dim3(kRowThreads), 0, st, x, ldx, (int)rows, tpr, q, ldq, s, lds);
  return hipGetLastError();
}

hipError_t launch_quant_act_cols(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                                 uint8_t* qt, int64_t ldq, float* s, int64_t lds, bool pow2, hipStream_t st) {
  dim3 grid((unsigned)(rows / 128), (unsigned)(cols / 64));
  if (pow2)
    hipLaunchKernelGGL(quant_act_cols_kernel<true>, grid, dim3(256), 0, st, x, ldx, qt, ldq, s, lds);
  else
    hipLaunchKernelGGL(quant_act_cols_kernel<false>, grid, dim3(256), 0, st, x, ldx, qt, ldq, s, lds);
  return hipGetLastError();
}

hipError_t launch_requant_t(const uint8_t* q, int64_t rows, int64_t cols, int64_t ldq, const float* s,
                            int64_t lds, uint8_t* qt, int64_t ldqt, float* st, int64_t ldst, bool pow2_hint,
                            hipStream_t stream) {
  dim3 grid((unsigned)(rows / 128), (unsigned)(cols / 128));
  if (pow2_hint)
    hipLaunchKernelGGL(requant_t_kernel<true>, grid, dim3(256), 0, stream, q, ldq, s, lds, qt, ldqt, st, ldst);
  else
    hipLaunchKernelGGL(requant_t_kernel<false>, grid, dim3(256), 0, stream, q, ldq, s, lds, qt, ldqt, st, ldst);
  return hipGetLastError();
}

hipError_t launch_requant_e5m6_t(const uint8_t* q, int64_t rows, int64_t cols, int64_t ldq, const float* s,
                                  int64_t lds, uint8_t* qt, int64_t ldqt, float* st, int64_t ldst, hipStream_t stream) {
  dim3 grid((unsigned)(rows / 128), (unsigned)(cols / 128));
  hipLaunchKernelGGL(requant_e5m6_t_kernel, grid, dim3(256), 0, stream, q, ldq, s, lds, qt, ldqt, st, ldst);
  return hipGetLastError();
}

hipError_t launch_quant_w(const uint16_t* w, int64_t n, int64_t k, int64_t ldw, uint8_t* q,
                          int64_t ldq, float* s, int64_t lds, uint8_t* qt, int64_t ldqt,
                          bool pow2, hipStream_t st) {
  if (qt == nullptr) {
    const int kblocks = (int)(k / 128);
    const dim3 grid2((unsigned)((kblocks + 1) / 2), (unsigned)(n / 128));
    if (pow2)
      hipLaunchKernelGGL(quant_w2_kernel<true>, grid2, dim3(256), 0, st, w, ldw, kblocks, q, ldq, s, lds);
    else
      hipLaunchKernelGGL(quant_w2_kernel<false>, grid2, dim3(256), 0, st, w, ldw, kblocks, q, ldq, s, lds);
    return hipGetLastError();
  }
  dim3 grid((unsigned)(k / 128), (unsigned)(n / 128));
  if (pow2)
    hipLaunchKernelGGL(quant_w_kernel<true>, grid, dim3(256), 0, st, w, ldw, q, ldq, s, lds, qt, ldqt);
  else
    hipLaunchKernelGGL(quant_w_kernel<false>, grid, dim3(256), 0, st, w, ldw, q, ldq, s, lds, qt, ldqt);
  return hipGetLastError();
}

hipError_t launch_cache_e5m6(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, uint8_t* q, int64_t ldq,
                             float* s, int64_t lds, hipStream_t st) {
  const int tpr = (int)(cols / 128);
  const int nt = tpr % 4 == 0 ? 4 : tpr % 2 == 0 ? 2 : 1;
  const dim3 grid((unsigned)((rows + kE5RowsPerBlock - 1) / kE5RowsPerBlock * (tpr / nt)));
  if (nt == 4)
    hipLaunchKernelGGL(cache_e5m6_kernel<4>, grid, dim3(kRowThreads), 0, st, x, ldx, (int)rows, tpr, q, ldq, s, lds);
  else if (nt == 2)
    hipLaunchKernelGGL(cache_e5m6_kernel<2>, grid, dim3(kRowThreads), 0, st, x, ldx, (int)rows, tpr, q, ldq, s, lds);
  else
    hipLaunchKernelGGL(cache_e5m6_kernel<1>, grid, dim3(kRowThreads), 0, st, x, ldx, (int)rows, tpr, q, ldq, s, lds);
  return hipGetLastError();
}

hipError_t launch_uncache_e5m6(const uint8_t* q, int64_t rows, int64_t cols, int64_t ldq, const float* s,
                               int64_t lds, uint16_t* y, int64_t ldy, hipStream_t st) {
  const int tpr = (int)(cols / 128);
  const int nt = tpr % 4 == 0 ? 4 : tpr % 2 == 0 ? 2 : 1;
  const dim3 grid((unsigned)((rows + kE5RowsPerBlock - 1) / kE5RowsPerBlock * (tpr / nt)));
  if (nt == 4)
    hipLaunchKernelGGL(uncache_e5m6_kernel<4>, grid, dim3(kRowThreads), 0, st, q, ldq, s, lds, (int)rows, tpr, y, ldy);
  else if (nt == 2)
    hipLaunchKernelGGL(uncache_e5m6_kernel<2>, grid, dim3(kRowThreads), 0, st, q, ldq, s, lds, (int)rows, tpr, y, ldy);
  else
    hipLaunchKernelGGL(uncache_e5m6_kernel<1>, grid, dim3(kRowThreads), 0, st, q, ldq, s, lds, (int)rows, tpr, y, ldy);
  return hipGetLastError();
}

}  // namespace fp8bq
