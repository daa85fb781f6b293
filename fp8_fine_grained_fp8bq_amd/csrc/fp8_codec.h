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
//  * the exact quotient fl32(x / s) comes from one correctly rounded
//    reciprocal per group, y = RN(1 / s), and per element q0 = RN(x y),
//    e = RN(s q0 - x) (exact: the remainder of a quotient within an ulp),
//    q = RN(q0 - e y): Markstein's correction, which gives RN(x / s) whenever
//    nothing underflows. Checked on the CPU for every positive finite bf16
//    absmax with s >= 2^-100 against every bf16 x with |x| <= absmax, both
//    signs (1.04e9 pairs, tests/exact_quotient_check.c): the E4M3 codes are
//    those of RN(x / s) in every case; the quotient bits differ only below
//    2^-11, where both encode to the same signed zero. Branch-free: the
//    earlier bracket test (two reciprocal products, exact division where they
//    disagreed) sent a whole wave through four divisions whenever one lane's
//    quotient lay near an E4M3 rounding midpoint, which bf16 data hits for
//    about 0.5% of elements (ratios of short mantissas). Groups whose scale is
//    below 2^-100 divide.
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
  float s, y;   // the scale and its reciprocal (RN(1 / s); 2^-k for a power of two)
  bool fast;
};

// Scale of a group from the magnitude bits (upper 16 bits of an fp32) of its absmax.
//  * s = fl32(amax / 448) without a division: q = fl32(amax * fl32(1/448)) is
//    corrected once with the exact residual amax - 448 q (an FMA), which gives
//    the correctly rounded quotient for every bf16 amax (checked for all 32639
//    positive finite bf16 values, on the CPU and by the GPU parity tests).
//  * y = RN(1 / s), the IEEE division (once per group).
__device__ __forceinline__ TileScale make_scale(uint32_t amax_bits16) {
  TileScale t;
  const float amax = __uint_as_float(amax_bits16 << 16);
  const float c = 1.0f / kFmax;                                    // constant-folded
  const float q = amax * c;
  t.s = __builtin_fmaf(__builtin_fmaf(-q, kFmax, amax), c, q);     // fl32(amax / 448)
  if (t.s == 0.0f) {
    // all-zero group: y = 0 turns every +-0 into the same-signed zero
    // (q0 = +-0, e = +0, q = +-0), as the method's s = 0, q = +-0 rule asks
    t.y = 0.0f;
    t.fast = true;
  } else {
    t.fast = t.s >= kFastScaleMin;
    t.y = t.fast ? 1.0f / t.s : 0.0f;
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
  t.y = __uint_as_float((uint32_t)(127 - k) << 23);                // 2^-k, a normal fp32 for k <= 120
  t.fast = true;
  return t;
}

template <bool POW2>
__device__ __forceinline__ TileScale group_scale(uint32_t amax_bits16) {
  if constexpr (POW2) return make_scale_pow2(amax_bits16);
  else return make_scale(amax_bits16);
}

// RN(x / s) from the group's reciprocal (Markstein's correction; see above).
// The negations are exact, so x = -0 gives -0 like the division.
__device__ __forceinline__ float exact_quotient(float x, const TileScale& t) {
  const float q0 = x * t.y;
  const float e = __builtin_fmaf(t.s, q0, -x);
  return __builtin_fmaf(-e, t.y, q0);
}

// Encodes four values (one output dword). Exact scales: the correctly rounded
// quotients from the group's reciprocal, or the division itself for groups
// with 0 < s < 2^-100. Power-of-two scales: one exact product.
template <bool POW2>
__device__ __forceinline__ uint32_t encode4(float f0, float f1, float f2, float f3, const TileScale& t) {
  if constexpr (POW2) return cvt4(f0 * t.y, f1 * t.y, f2 * t.y, f3 * t.y);
  if (__builtin_expect(t.fast, 1))
    return cvt4(exact_quotient(f0, t), exact_quotient(f1, t), exact_quotient(f2, t), exact_quotient(f3, t));
  return cvt4(f0 / t.s, f1 / t.s, f2 / t.s, f3 / t.s);
}

}  // namespace fp8bq
