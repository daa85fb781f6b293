"""E4M3 codec of the oracle (test infrastructure; see the package docstring).

Format. The parallelism-summary page (FP8 part, floating-point format table)
gives float8 e4m3 as 1 sign bit, 4 exponent bits and 3 mantissa bits; the
DeepSeek-V3 report (section 3.3.2, "mantissa over exponents") uses E4M3 for
every GEMM operand. The pages do not name the variant or its largest finite
value; this oracle takes the OCP E4M3FN variant:

* exponent bias 7; exponent field 0 holds subnormals m * 2^-9 (m = 1..7);
* no infinities; S.1111.111 (0x7F / 0xFF) is NaN, so the largest finite
  magnitude is 1.75 * 2^8 = 448 (0x7E / 0xFE);
* signed zero: 0x00 is +0, 0x80 is -0.

Encoding. The tech note's quantiser rounds x / s to FP8 ("round"), and the
parallelism-summary page describes casting as taking the nearest representable
number. This oracle rounds to nearest with ties to the even code (the code
whose mantissa LSB is 0), saturates magnitudes beyond 448 to 448 and keeps the
sign (a negative value that rounds to zero gives 0x80).

Pinned by: tests/test_oracle_codec.py -- the closed-form decode table, the
page's count of 7 e4m3 values strictly inside (1, 2), the brute-force nearest
encoder on every bf16 bit pattern times several scales and on every rounding
midpoint +-1 fp32 ulp, and the scalar encoder against the vectorised one.
"""

from __future__ import annotations

import math

import numpy as np

FMAX = 448.0          # largest finite E4M3FN magnitude: (1 + 6/8) * 2^(15 - 7)
EXP_BIAS = 7
MANT_BITS = 3
MIN_NORMAL = 2.0 ** -6   # exponent field 1, mantissa 0
SUBNORMAL_QUANTUM = 2.0 ** -9


# ---------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------

def decode_scalar(code: int) -> float:
    """Value of one E4M3FN code, from its bit fields (NaN for 0x7F / 0xFF)."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        mag = m * SUBNORMAL_QUANTUM
    else:
        mag = (1.0 + m / 8.0) * 2.0 ** (e - EXP_BIAS)
    return sign * mag


DECODE_TABLE = np.array([decode_scalar(c) for c in range(256)], dtype=np.float64)


def decode(codes: np.ndarray) -> np.ndarray:
    """Vectorised decode of uint8 codes to float64 (exact)."""
    return DECODE_TABLE[np.asarray(codes, dtype=np.uint8)]


# ---------------------------------------------------------------------------
# encode (scalar, from the definition)
# ---------------------------------------------------------------------------

def encode_scalar(v: float) -> int:
    """Round one real value to E4M3FN: nearest, ties to even code, saturating.

    `v` is a Python float; callers pass fp32 values. Every step below is exact
    in binary64 (only power-of-two rescaling and Python's round-half-even).
    """
    v = float(v)
    if math.isnan(v):
        return 0x7F
    sign = 0x80 if math.copysign(1.0, v) < 0 else 0x00
    a = abs(v)
    if a >= FMAX:
        # anything at or beyond 448 rounds to 448 or past it; past it saturates
        return sign | 0x7E
    if a < MIN_NORMAL:
        # subnormal binade: multiples of 2^-9; n = 8 is the smallest normal (code 0x08)
        n = round(a / SUBNORMAL_QUANTUM)          # round-half-even on an exact quotient
        return sign | int(n)
    m, e2 = math.frexp(a)                        # a = m * 2^e2, m in [0.5, 1)
    e = e2 - 1                                   # a in [2^e, 2^(e+1))
    n = round(a / 2.0 ** (e - MANT_BITS))        # 8 <= n <= 16
    if n == 16:
        e += 1
        n = 8
    code = ((e + EXP_BIAS) << MANT_BITS) | (n - 8)
    return sign | min(code, 0x7E)


# ---------------------------------------------------------------------------
# encode (vectorised, same definition)
# ---------------------------------------------------------------------------

def encode(v: np.ndarray) -> np.ndarray:
    """Vectorised `encode_scalar` on an fp32 (or fp64-held fp32) array -> uint8."""
    v = np.asarray(v, dtype=np.float64)
    sign = np.where(np.signbit(v), 0x80, 0x00).astype(np.int64)
    a = np.abs(v)
    out = np.zeros(v.shape, dtype=np.int64)

    sub = a < MIN_NORMAL
    out[sub] = np.rint(a[sub] / SUBNORMAL_QUANTUM).astype(np.int64)   # rint = half-even

    nor = (~sub) & (a < FMAX)
    _, e2 = np.frexp(a[nor])
    e = e2.astype(np.int64) - 1
    n = np.rint(a[nor] / np.ldexp(1.0, e - MANT_BITS)).astype(np.int64)
    carry = n == 16
    e = np.where(carry, e + 1, e)
    n = np.where(carry, 8, n)
    out[nor] = np.minimum(((e + EXP_BIAS) << MANT_BITS) | (n - 8), 0x7E)

    out[a >= FMAX] = 0x7E
    res = (out | sign).astype(np.uint8)
    res[np.isnan(v)] = 0x7F
    return res


# ---------------------------------------------------------------------------
# brute force (pin only)
# ---------------------------------------------------------------------------

_FINITE_CODES = np.array([c for c in range(256) if not math.isnan(decode_scalar(c))], dtype=np.int64)
_FINITE_VALS = DECODE_TABLE[_FINITE_CODES]


def encode_bruteforce(v: float) -> int:
    """Nearest finite E4M3FN value by exhaustive search with exact (rational)
    distances; a tie goes to the even code; a zero result keeps the sign of
    `v`. Nearest-among-finite saturates by construction (no finite value lies
    beyond 448)."""
    from fractions import Fraction
    v = float(v)
    fv = Fraction(v)
    d = [abs(Fraction(float(x)) - fv) for x in _FINITE_VALS]
    best = min(d)
    cand = [int(c) for c, di in zip(_FINITE_CODES, d) if di == best]
    if len(cand) > 1:
        # candidates hold at most two distinct values (or +-0); prefer even mantissa
        even = [c for c in cand if (c & 1) == 0]
        cand = even if even else cand
    if all(DECODE_TABLE[c] == 0.0 for c in cand):
        return 0x80 if math.copysign(1.0, v) < 0 else 0x00
    # remaining candidates share one nonzero value and hence one code
    return cand[0]


def encode_bruteforce_vec(v: np.ndarray, chunk: int = 16384) -> np.ndarray:
    """Array form of `encode_bruteforce`: distance to every finite code, nearest
    wins, a tie goes to the even code, a zero result keeps the sign of v."""
    v = np.asarray(v, dtype=np.float64).ravel()
    out = np.empty(v.shape, dtype=np.uint8)
    even = (_FINITE_CODES & 1) == 0
    for i in range(0, v.size, chunk):
        x = v[i:i + chunk]
        # |x - val| is exact in binary64 for fp32 x with |x| < 2^20 (all bits lie
        # between 2^20 and 2^-33 or x is far below every nonzero value); beyond,
        # |x| > 448 >= |val| and |x - val| - |x| = -sign(x) * val orders exactly.
        big = np.abs(x) >= 2.0 ** 20
        d = np.where(big[:, None], -np.sign(x)[:, None] * _FINITE_VALS[None, :],
                     np.abs(_FINITE_VALS[None, :] - x[:, None]))
        near = d == d.min(axis=1, keepdims=True)
        pref = near & even[None, :]
        pick = np.where(pref.any(axis=1), pref.argmax(axis=1), near.argmax(axis=1))
        codes = _FINITE_CODES[pick]
        zero = _FINITE_VALS[pick] == 0.0
        codes = np.where(zero, np.where(np.signbit(x), 0x80, 0x00), codes)
        out[i:i + chunk] = codes.astype(np.uint8)
    return out
