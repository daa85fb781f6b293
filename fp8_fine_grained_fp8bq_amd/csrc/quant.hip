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
// per-element arithmetic is kept small so it hides under the memory traffic:
//
//  * absmax is an integer max over the bf16 magnitude bits (bits & 0x7fff
//    order like the values for finite inputs), reduced across a tile's lanes
//    with DPP row permutations;
//  * the exact quotient fl32(x / s) is needed only to pick an E4M3 code. With
//    r = fl32(1 / s), rlo = fl32(r (1 - 2^-20)), rhi = fl32(r (1 + 2^-20)), the
//    products x*rlo and x*rhi bracket fl32(x / s) strictly (each of r, rlo/rhi
//    and the product is within 2^-24 relative, so x*rlo <= (x/s)(1 - 0.81*2^-20)
//    < fl32(x/s) and symmetrically for rhi, for x / s in fp32's normal range;
//    below it all three encode to a signed zero). The conversion is monotone,
//    so when both brackets give the same code it is the code of fl32(x / s).
//    Otherwise (about 3 elements in 10^5) the lane recomputes with the
//    correctly-rounded division. Tiles whose scale is below 2^-100 (where
//    1 / s may overflow) always take the division.
//  * v_cvt_pk_fp8_f32 rounds to nearest even, keeps the sign of zero and handles
//    fp32 denormals like the E4M3 definition on every finite input below 448,
//    and returns 448 for inputs in [448, 464]. No quotient here exceeds 450
//    (|x| <= absmax, and s = fl32(absmax / 448) is within 2^-24 relative unless
//    it is a binary32 subnormal, within 0.4% then), so no clamp is needed.
#include "internal.h"

namespace fp8bq {
namespace {

constexpr float kFmax = 448.0f;
constexpr float kFastScaleMin = 0x1p-100f;

__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

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

// Magnitude bits of the two bf16 in a dword, max of the pair, as a 16-bit value.
__device__ __forceinline__ uint32_t mag_max2(uint32_t w) {
  return umax(w & 0x7FFFu, (w >> 16) & 0x7FFFu);
}

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ uint32_t cvt4(float a, float b, float c, float d) {
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
  return (uint32_t)r;
}

struct TileScale {
  float s, rlo, rhi;
  bool fast;
};

// Scale of a group from the magnitude bits (upper 16 bits of an fp32) of its absmax.
__device__ __forceinline__ TileScale make_scale(uint32_t amax_bits16) {
  TileScale t;
  const float amax = __uint_as_float(amax_bits16 << 16);
  t.s = amax / kFmax;                      // correctly rounded binary32 division
  if (t.s == 0.0f) {
    t.rlo = t.rhi = 0.0f;                  // +-0 * 0 keeps the sign of zero
    t.fast = true;
  } else {
    t.fast = t.s >= kFastScaleMin;
    const float r = t.fast ? 1.0f / t.s : 0.0f;
    t.rlo = r * (1.0f - 0x1p-20f);
    t.rhi = r * (1.0f + 0x1p-20f);
  }
  return t;
}

// Encodes four values (one output dword); `exact` codes are computed only when
// the brackets disagree.
__device__ __forceinline__ uint32_t encode4(float f0, float f1, float f2, float f3, const TileScale& t) {
  const uint32_t lo = cvt4(f0 * t.rlo, f1 * t.rlo, f2 * t.rlo, f3 * t.rlo);
  const uint32_t hi = cvt4(f0 * t.rhi, f1 * t.rhi, f2 * t.rhi, f3 * t.rhi);
  if (__builtin_expect(t.fast && lo == hi, 1)) return lo;
  return cvt4(f0 / t.s, f1 / t.s, f2 / t.s, f3 / t.s);
}

// Eight bf16 (packed in four dwords) -> eight codes.
__device__ __forceinline__ uint2 encode8(const uint4 w, const TileScale& t) {
  uint2 r;
  r.x = encode4(bf_lo(w.x), bf_hi(w.x), bf_lo(w.y), bf_hi(w.y), t);
  r.y = encode4(bf_lo(w.z), bf_hi(w.z), bf_lo(w.w), bf_hi(w.w), t);
  return r;
}

// ---------------------------------------------------------------------------
// 1x128 row-wise activation tiles.
// One 16-lane DPP row holds one tile (each lane 8 bf16 = 16 B); a wave handles
// kRowU x 4 consecutive tiles of the flattened [rows, cols/128] grid, so every
// load instruction of a wave reads 1 KB of consecutive tiles.
// ---------------------------------------------------------------------------
constexpr int kRowU = 2;
constexpr int kRowThreads = 256;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// 16-byte load / 8-byte store, optionally marked non-temporal (streamed once).
__device__ __forceinline__ uint4 load16(const void* p, bool nt) {
  const u32x4* q = reinterpret_cast<const u32x4*>(p);
  const u32x4 v = nt ? __builtin_nontemporal_load(q) : *q;
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store8(void* p, uint2 v, bool nt) {
  u32x2* q = reinterpret_cast<u32x2*>(p);
  const u32x2 w = {v.x, v.y};
  if (nt) __builtin_nontemporal_store(w, q); else *q = w;
}

template <int U, bool NT>
__global__ __launch_bounds__(kRowThreads) void quant_act_rows_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, int tiles_per_row, int ntiles,
    uint8_t* __restrict__ q, int64_t ldq, float* __restrict__ s, int64_t lds) {
  const int lane = threadIdx.x & 63;
  const int grp = lane >> 4, l16 = lane & 15;
  const int wave = blockIdx.x * (kRowThreads / 64) + (threadIdx.x >> 6);
  const int t0 = wave * (4 * U);

  uint4 v[U];
  int row[U], col[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    int t = t0 + u * 4 + grp;
    t = t < ntiles ? t : ntiles - 1;
    row[u] = t / tiles_per_row;
    col[u] = t - row[u] * tiles_per_row;
    v[u] = load16(x + (int64_t)row[u] * ldx + col[u] * 128 + l16 * 8, NT);
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    uint32_t m = umax(umax(mag_max2(v[u].x), mag_max2(v[u].y)), umax(mag_max2(v[u].z), mag_max2(v[u].w)));
    m = row16_max(m);
    const TileScale ts = make_scale(m);
    const uint2 codes = encode8(v[u], ts);
    const int t = t0 + u * 4 + grp;
    if (t < ntiles) {
      store8(q + (int64_t)row[u] * ldq + col[u] * 128 + l16 * 8, codes, NT);
      if (l16 == 0) s[(int64_t)col[u] * lds + row[u]] = ts.s;
    }
  }
}

// ---------------------------------------------------------------------------
// 128x1 column-wise tiles, written transposed.
// A 256-thread block stages 128 rows x 64 columns of bf16 in LDS. Thread t
// then owns column pair p = t / 8 and rows [16 (t % 8), +16): it reduces both
// columns' absmax with its 7 neighbours (one aligned group of 8 lanes), encodes
// its 16 rows of each column and writes them as 16 contiguous bytes of the
// transposed output, so each wave writes 128-byte runs of 16 output rows.
// ---------------------------------------------------------------------------
constexpr int kColBlockCols = 64;
constexpr int kColLdsStride = kColBlockCols / 2 + 1;   // dwords per staged row (+1 pad)

__global__ __launch_bounds__(256) void quant_act_cols_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, uint8_t* __restrict__ qt, int64_t ldq,
    float* __restrict__ s, int64_t lds) {
  __shared__ uint32_t tile[128 * kColLdsStride];
  const int t = threadIdx.x;
  const int64_t r0 = (int64_t)blockIdx.y * 128;
  const int64_t c0 = (int64_t)blockIdx.x * kColBlockCols;

#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = i * 32 + (t >> 3);
    const int d = (t & 7) * 4;
    const uint4 w = *reinterpret_cast<const uint4*>(x + (r0 + row) * ldx + c0 + d * 2);
    uint32_t* dst = tile + row * kColLdsStride + d;
    dst[0] = w.x; dst[1] = w.y; dst[2] = w.z; dst[3] = w.w;
  }
  __syncthreads();

  const int p = t >> 3, seg = t & 7;
  uint32_t w[16];
  uint32_t mlo = 0, mhi = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    w[i] = tile[(seg * 16 + i) * kColLdsStride + p];
    mlo = umax(mlo, w[i] & 0x7FFFu);
    mhi = umax(mhi, (w[i] >> 16) & 0x7FFFu);
  }
  mlo = lane8_max(mlo);
  mhi = lane8_max(mhi);
  const TileScale slo = make_scale(mlo), shi = make_scale(mhi);

  uint4 clo, chi;
  clo.x = encode4(bf_lo(w[0]), bf_lo(w[1]), bf_lo(w[2]), bf_lo(w[3]), slo);
  clo.y = encode4(bf_lo(w[4]), bf_lo(w[5]), bf_lo(w[6]), bf_lo(w[7]), slo);
  clo.z = encode4(bf_lo(w[8]), bf_lo(w[9]), bf_lo(w[10]), bf_lo(w[11]), slo);
  clo.w = encode4(bf_lo(w[12]), bf_lo(w[13]), bf_lo(w[14]), bf_lo(w[15]), slo);
  chi.x = encode4(bf_hi(w[0]), bf_hi(w[1]), bf_hi(w[2]), bf_hi(w[3]), shi);
  chi.y = encode4(bf_hi(w[4]), bf_hi(w[5]), bf_hi(w[6]), bf_hi(w[7]), shi);
  chi.z = encode4(bf_hi(w[8]), bf_hi(w[9]), bf_hi(w[10]), bf_hi(w[11]), shi);
  chi.w = encode4(bf_hi(w[12]), bf_hi(w[13]), bf_hi(w[14]), bf_hi(w[15]), shi);

  const int64_t col = c0 + 2 * p;
  *reinterpret_cast<uint4*>(qt + col * ldq + r0 + seg * 16) = clo;
  *reinterpret_cast<uint4*>(qt + (col + 1) * ldq + r0 + seg * 16) = chi;
  if (seg == 0) {
    float* sp = s + (int64_t)blockIdx.y * lds + col;
    sp[0] = slo.s;
    sp[1] = shi.s;
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

  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    m = umax(m, umax(umax(mag_max2(v[i].x), mag_max2(v[i].y)), umax(mag_max2(v[i].z), mag_max2(v[i].w))));
  m = row16_max(m);
  m = umax(m, (uint32_t)__shfl_xor((int)m, 16));
  m = umax(m, (uint32_t)__shfl_xor((int)m, 32));
  if ((t & 63) == 0) wmax[t >> 6] = m;
  __syncthreads();
  m = umax(umax(wmax[0], wmax[1]), umax(wmax[2], wmax[3]));
  const TileScale ts = make_scale(m);
  if (t == 0) s[(int64_t)blockIdx.y * lds + blockIdx.x] = ts.s;

#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint2 c = encode8(v[i], ts);
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

}  // namespace

hipError_t launch_quant_act_rows(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                                 uint8_t* q, int64_t ldq, float* s, int64_t lds, hipStream_t st) {
  const int tiles_per_row = (int)(cols / 128);
  const int ntiles = (int)(rows * tiles_per_row);
  const int per_block = (kRowThreads / 64) * 4 * kRowU;
  const int blocks = (ntiles + per_block - 1) / per_block;
  hipLaunchKernelGGL((quant_act_rows_kernel<kRowU, false>), dim3(blocks), dim3(kRowThreads), 0, st, x,
                     ldx, tiles_per_row, ntiles, q, ldq, s, lds);
  return hipGetLastError();
}

hipError_t launch_quant_act_cols(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                                 uint8_t* qt, int64_t ldq, float* s, int64_t lds, hipStream_t st) {
  dim3 grid((unsigned)(cols / kColBlockCols), (unsigned)(rows / 128));
  hipLaunchKernelGGL(quant_act_cols_kernel, grid, dim3(256), 0, st, x, ldx, qt, ldq, s, lds);
  return hipGetLastError();
}

hipError_t launch_quant_w(const uint16_t* w, int64_t n, int64_t k, int64_t ldw, uint8_t* q,
                          int64_t ldq, float* s, int64_t lds, uint8_t* qt, int64_t ldqt,
                          hipStream_t st) {
  dim3 grid((unsigned)(k / 128), (unsigned)(n / 128));
  hipLaunchKernelGGL(quant_w_kernel, grid, dim3(256), 0, st, w, ldw, q, ldq, s, lds, qt, ldqt);
  return hipGetLastError();
}

}  // namespace fp8bq
