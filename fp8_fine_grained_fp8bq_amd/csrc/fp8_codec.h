// E4M3 tile codec shared by the quantisers and the GEMM epilogue that
// quantises its own output: the scale of a group from its absmax and the
// encoding of values with that scale. Both users compute exactly the same
// codes and scales from the same bf16 values.
//
// Numerics (DeepSeek-V3 report, Chinese translation, section 3.3.2
// "fine-grained quantization" / "online quantization"; tech note "DeepSeek-V3
// FP8 dynamic quantisation", fine-grained quantization formulas):
// s = fl32(absmax / 448) and q = E4M3(fl32(x / s)), rounded to nearest even,
// sign kept, s = 0 and +-0 codes for an all-zero group; or, with power-of-two
// scales (section 3.3.3), s = 2^k with the smallest k such that
// absmax <= 448 * 2^k.
//
//  * absmax is an integer max over the bf16 magnitude bits (bits & 0x7fff
//    order like the values for finite inputs);
//  * the exact quotient fl32(x / s) is needed only to pick an E4M3 code. With
//    r ~ 1 / s, rlo = fl32(r (1 - 2^-19)), rhi = fl32(r (1 + 2^-19)), the
//    products x*rlo and x*rhi bracket fl32(x / s) strictly (see make_scale for
//    the error budget; for x / s below fp32's normal range all three encode to
//    a signed zero). The conversion is monotone, so when both brackets give
//    the same code it is the code of fl32(x / s). Otherwise (about 6 elements
//    in 10^5) the lane recomputes with the correctly-rounded division. Groups
//    whose scale is below 2^-100 always take the division.
//  * v_cvt_pk_fp8_f32 rounds to nearest even, keeps the sign of zero and handles
//    fp32 denormals like the E4M3 definition on every finite input below 448,
//    and returns 448 for inputs in [448, 464]. No quotient here exceeds 450
//    (|x| <= absmax, and s = fl32(absmax / 448) is within 2^-24 relative unless
//    it is a binary32 subnormal, within 0.4% then), so no clamp is needed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8bq {

constexpr float kFmax = 448.0f;
constexpr float kFastScaleMin = 0x1p-100f;

__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

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
//  * s = fl32(amax / 448) without a division: q = fl32(amax * fl32(1/448)) is
//    corrected once with the exact residual amax - 448 q (an FMA), which gives
//    the correctly rounded quotient for every bf16 amax (checked for all 32639
//    positive finite bf16 values, on the CPU and by the GPU parity tests).
//  * r approximates 1 / s with the hardware reciprocal (documented within 1
//    ulp); the brackets x * r (1 -+ 2^-19) enclose fl32(x / s) strictly as
//    long as r is within 13 ulp: e_r + 2 * 2^-24 < 2^-19 - 2^-24.
__device__ __forceinline__ TileScale make_scale(uint32_t amax_bits16) {
  TileScale t;
  const float amax = __uint_as_float(amax_bits16 << 16);
  const float c = 1.0f / kFmax;                                    // constant-folded
  const float q = amax * c;
  t.s = __builtin_fmaf(__builtin_fmaf(-q, kFmax, amax), c, q);     // fl32(amax / 448)
  if (t.s == 0.0f) {
    t.rlo = t.rhi = 0.0f;                  // +-0 * 0 keeps the sign of zero
    t.fast = true;
  } else {
    t.fast = t.s >= kFastScaleMin;
    const float r = t.fast ? __builtin_amdgcn_rcpf(t.s) : 0.0f;
    t.rlo = r * (1.0f - 0x1p-19f);
    t.rhi = r * (1.0f + 0x1p-19f);
  }
  return t;
}

// Power-of-two scale (the report's integral-power-of-2 scaling factors,
// section 3.3.3): s = 2^k with k the smallest integer such that
// amax <= 448 * 2^k, within [-127, 127] (an E8M0 exponent byte); an all-zero
// group gets 2^-127. With 448 * 2^k = 1.75 * 2^(k+8), a normal bf16
// amax = (1 + m/128) 2^(e-127) needs k = e - 135 when m <= 96 (mantissa
// <= 1.75) and k = e - 134 otherwise; subnormal and tiny amax clamp to -127.
// x * 2^-k is then exact (|x * 2^-k| <= 448; products that fall below the
// fp32 normal range encode to zero either way), so one conversion rounds it.
__device__ __forceinline__ TileScale make_scale_pow2(uint32_t amax_bits16) {
  const int e = (int)((amax_bits16 >> 7) & 0xFF), m = (int)(amax_bits16 & 0x7F);
  const int k = max(-127, min(127, e - 135 + (m > 96 ? 1 : 0)));
  TileScale t;
  t.s = k >= -126 ? __uint_as_float((uint32_t)(k + 127) << 23) : __uint_as_float(0x00400000u);
  t.rlo = t.rhi = __uint_as_float((uint32_t)(127 - k) << 23);      // 2^-k, a normal fp32 for k <= 120
  t.fast = true;
  return t;
}

template <bool POW2>
__device__ __forceinline__ TileScale group_scale(uint32_t amax_bits16) {
  if constexpr (POW2) return make_scale_pow2(amax_bits16);
  else return make_scale(amax_bits16);
}

// Encodes four values (one output dword). Exact scales: the exact codes are
// computed only when the brackets disagree. Power-of-two scales: one exact
// product and one conversion.
template <bool POW2>
__device__ __forceinline__ uint32_t encode4(float f0, float f1, float f2, float f3, const TileScale& t) {
  if constexpr (POW2) return cvt4(f0 * t.rlo, f1 * t.rlo, f2 * t.rlo, f3 * t.rlo);
  const uint32_t lo = cvt4(f0 * t.rlo, f1 * t.rlo, f2 * t.rlo, f3 * t.rlo);
  const uint32_t hi = cvt4(f0 * t.rhi, f1 * t.rhi, f2 * t.rhi, f3 * t.rhi);
  if (__builtin_expect(t.fast && lo == hi, 1)) return lo;
  return cvt4(f0 / t.s, f1 / t.s, f2 / t.s, f3 / t.s);
}

}  // namespace fp8bq
