"""E5M6 activation-cache codec of the oracle (test infrastructure: only the
tests, the smoke check and the bench's CPU leg use it; the library never does).

What the pages say. The DeepSeek-V3 report (Chinese translation, section 3.3.3
"low-precision storage and communication", low-precision activations, item 1)
caches the inputs of the Linear that follows the attention operator in a
custom E5M6 format, in 1x128 tiles that the backward pass turns into 128x1
tiles, with every scaling factor an integral power of two so that the
conversion adds no quantisation error of its own. The FP8 notes page (section
9, low-precision storage) adds that E5M6 is 12 bits in all. Nothing more is
given; this oracle takes the plainest reading:

* Format: 1 sign bit, 5 exponent bits with bias 15, 6 mantissa bits, laid out
  like IEEE binary16 with the four lowest mantissa bits removed: exponent
  field 0 holds subnormals m * 2^-20 (m = 1..63), field 31 infinities (mantissa
  0) and NaN. Largest finite magnitude (2 - 2^-6) * 2^15 = 65024; smallest
  normal 2^-14. Signed zeros.
* Rounding: to nearest, ties to the even code; magnitudes above 65024 saturate
  to 65024 (the scale below keeps every scaled value at or below it); a value
  that rounds to zero keeps its sign.
* Tile scale: s = 2^k with k the smallest integer such that the tile's absmax
  is at most 65024 * 2^k, clamped to [-127, 127] (the power-of-two rule of the
  FP8 quantisers with E5M6's largest value); an all-zero tile gets 2^-127.
  Codes are E5M6(x * 2^-k), the product exact, rounded once.
* Storage: 12-bit codes, two per 3 bytes, little-endian within the 24-bit
  group (element 2i in bits 0..11, element 2i+1 in bits 12..23); a row of C
  elements takes 1.5 C bytes. Scales chunk-major, like the FP8 activation
  scales: tile (row r, chunk c) at s[c * lds + r].

Pinned by tests/test_oracle_e5m6.py: the value set against numpy's binary16
(every code's value is the binary16 value of the same bits shifted left by 4),
closed forms (count of values, extremes), the brute-force nearest-value encoder
on every bf16 pattern at several scales and on every rounding midpoint, a
hand-packed example, and the round-trip error bound; the backward conversion
to 128x1 FP8 tiles against the separately pinned 128x1 power-of-two FP8
quantiser applied to the cached values (exact in bf16 there) and against a
hand-worked column.
"""

from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

EXP_BIAS = 15
MANT_BITS = 6
FMAX = (2.0 - 2.0 ** -6) * 2.0 ** 15       # 65024
MIN_NORMAL = 2.0 ** -14
SUBNORMAL_QUANTUM = 2.0 ** -20
K_MIN, K_MAX = -127, 127


def decode_scalar(code: int) -> float:
    """Value of one 12-bit E5M6 code from its bit fields."""
    code = int(code) & 0xFFF
    sign = -1.0 if code & 0x800 else 1.0
    e = (code >> 6) & 0x1F
    m = code & 0x3F
    if e == 0x1F:
        return sign * math.inf if m == 0 else math.nan
    if e == 0:
        return sign * m * SUBNORMAL_QUANTUM
    return sign * (1.0 + m / 64.0) * 2.0 ** (e - EXP_BIAS)


DECODE_TABLE = np.array([decode_scalar(c) for c in range(4096)], dtype=np.float64)
_FINITE_CODES = np.array([c for c in range(4096) if math.isfinite(DECODE_TABLE[c])], dtype=np.int64)
_FINITE_VALS = DECODE_TABLE[_FINITE_CODES]


def decode(codes: np.ndarray) -> np.ndarray:
    """Vectorised decode of 12-bit codes (any integer dtype) to float64 (exact)."""
    return DECODE_TABLE[np.asarray(codes, dtype=np.int64) & 0xFFF]


def encode_scalar(v: float) -> int:
    """E5M6 code of a finite float: round to nearest, ties to even, saturate
    beyond 65024, keep the sign of zero. Works on the exact binary value of v."""
    v = float(v)
    sign = 0x800 if math.copysign(1.0, v) < 0 else 0
    a = abs(v)
    if a == 0.0:
        return sign
    if a >= FMAX:
        return sign | (30 << 6) | 0x3F
    e = math.frexp(a)[1] - 1              # a = f * 2^e, 1 <= f < 2
    e = max(e, 1 - EXP_BIAS)              # below the normal range: subnormal quantum
    quantum = Fraction(2) ** (e - MANT_BITS)
    q = Fraction(a) / quantum             # exact
    n = math.floor(q)
    rem = q - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    # n * quantum, n <= 128: renormalise into fields
    if n == 0:
        return sign
    if e == 1 - EXP_BIAS and n < 64:
        return sign | n                   # subnormal
    if n == 128:                          # rounded up into the next binade
        n, e = 64, e + 1
    if e + EXP_BIAS > 30:
        return sign | (30 << 6) | 0x3F
    return sign | ((e + EXP_BIAS) << 6) | (n - 64)


def encode(v: np.ndarray) -> np.ndarray:
    """Vectorised E5M6 encoder (float64 input, exact): the same rule as
    encode_scalar, by the binary16 bit layout: the value's binary16-range
    exponent picks the quantum, and the mantissa is rounded with ties to even."""
    v = np.asarray(v, dtype=np.float64)
    sign = np.where(np.signbit(v), 0x800, 0).astype(np.int64)
    a = np.abs(v)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0))).astype(np.int64)
    # floor(log2) can be off by one near powers of two: correct exactly
    e = np.where(np.ldexp(1.0, e) > a, e - 1, e)
    e = np.where(np.ldexp(1.0, e + 1) <= a, e + 1, e)
    e = np.maximum(e, 1 - EXP_BIAS)
    q = np.ldexp(a, -(e - MANT_BITS))             # exact: a / quantum
    n = np.floor(q)
    rem = q - n
    n = n + ((rem > 0.5) | ((rem == 0.5) & (np.mod(n, 2) == 1)))
    n = n.astype(np.int64)
    up = n == 128
    n = np.where(up, 64, n)
    e = np.where(up, e + 1, e)
    sub = (e == 1 - EXP_BIAS) & (n < 64)
    code = np.where(sub, n, ((e + EXP_BIAS) << 6) | (n - 64))
    code = np.where(n == 0, 0, code)
    sat = (a >= FMAX) | (e + EXP_BIAS > 30)
    code = np.where(sat, (30 << 6) | 0x3F, code)
    return (code | sign).astype(np.uint16)


def encode_bruteforce(v: float) -> int:
    """Nearest finite E5M6 value by exhaustive search with exact (rational)
    distances; a tie goes to the even code; zero keeps the sign of v."""
    fv = Fraction(float(v))
    d = [abs(Fraction(float(x)) - fv) for x in _FINITE_VALS]
    best = min(d)
    cand = [int(c) for c, di in zip(_FINITE_CODES, d) if di == best]
    if len(cand) > 1:
        even = [c for c in cand if (c & 1) == 0]
        cand = even if even else cand
    if all(DECODE_TABLE[c] == 0.0 for c in cand):
        return 0x800 if math.copysign(1.0, float(v)) < 0 else 0x000
    return cand[0]


# ---------------------------------------------------------------------------
# the 1x128 cache quantiser, packing and its inverse
# ---------------------------------------------------------------------------

def pow2_exponent(amax: np.ndarray) -> np.ndarray:
    """Smallest integer k with amax <= 65024 * 2^k, clamped to [K_MIN, K_MAX];
    K_MIN for amax = 0 (exact comparisons in float64)."""
    a = np.asarray(amax, dtype=np.float64)
    pos = a > 0
    k = np.zeros(a.shape, dtype=np.int64)
    k[pos] = np.ceil(np.log2(a[pos] / FMAX)).astype(np.int64)
    for _ in range(4):
        k = np.where(pos & (a > FMAX * np.ldexp(1.0, k)), k + 1, k)
        k = np.where(pos & (a <= FMAX * np.ldexp(1.0, k - 1)), k - 1, k)
    k = np.where(pos, k, K_MIN)
    return np.clip(k, K_MIN, K_MAX)


def pack(codes: np.ndarray) -> np.ndarray:
    """[rows, C] 12-bit codes (C even) -> [rows, 1.5 C] bytes."""
    c = np.asarray(codes, dtype=np.uint32)
    lo, hi = c[:, 0::2], c[:, 1::2]
    w = lo | (hi << 12)                               # 24 bits per pair
    out = np.empty((c.shape[0], c.shape[1] // 2, 3), dtype=np.uint8)
    out[..., 0] = w & 0xFF
    out[..., 1] = (w >> 8) & 0xFF
    out[..., 2] = (w >> 16) & 0xFF
    return out.reshape(c.shape[0], -1)


def unpack(packed: np.ndarray, cols: int) -> np.ndarray:
    """Inverse of pack: [rows, 1.5 C] bytes -> [rows, C] codes (uint16)."""
    b = np.asarray(packed, dtype=np.uint32)[:, : cols * 3 // 2].reshape(packed.shape[0], cols // 2, 3)
    w = b[..., 0] | (b[..., 1] << 8) | (b[..., 2] << 16)
    out = np.empty((packed.shape[0], cols), dtype=np.uint16)
    out[:, 0::2] = w & 0xFFF
    out[:, 1::2] = w >> 12
    return out


def cache_1x128(x_bits: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """bf16 [rows, C] (C % 128 == 0) -> (packed codes [rows, 1.5 C] uint8,
    power-of-two scales chunk-major [C / 128, rows] float32)."""
    from oracle import quant
    xf = quant.bf16_bits_to_f32(x_bits)
    rows, cols = xf.shape
    assert cols % 128 == 0
    xg = xf.reshape(rows, cols // 128, 128).astype(np.float64)
    k = pow2_exponent(np.max(np.abs(xg), axis=-1))
    codes = encode(xg * np.ldexp(1.0, -k)[..., None])          # exact product
    return pack(codes.reshape(rows, cols)), np.ldexp(np.float32(1.0), k.astype(np.int32)).astype(np.float32).T.copy()


def uncache_1x128(packed: np.ndarray, s: np.ndarray, cols: int) -> np.ndarray:
    """Exact values x_hat = E5M6(code) * s as float64 [rows, C]."""
    codes = unpack(packed, cols)
    rows = codes.shape[0]
    v = decode(codes).reshape(rows, cols // 128, 128)
    return (v * s.T.astype(np.float64)[..., None]).reshape(rows, cols)


def requant_128x1(packed: np.ndarray, s: np.ndarray, cols: int) -> tuple[np.ndarray, np.ndarray]:
    """The backward conversion of the cache (report section 3.3.3: the 1x128
    tiles become 128x1 tiles, and the power-of-two scales keep the conversion
    from adding an error of its own): x_hat = E5M6(code) * s exactly, 128x1
    groups (128 consecutive rows of one column), the group's scale 2^k with k
    the smallest integer such that its absmax is at most 448 * 2^k (within
    [-127, 127]), codes E4M3(fl32(x_hat * 2^-k)) -- the FP8 operand of the
    weight-gradient GEMM, in the layout of the 128x1 FP8 quantiser.

    packed [rows, 1.5 cols] with chunk-major scales s [cols / 128, rows] as
    `cache_1x128` writes them (rows a multiple of 128). Returns qT uint8
    [cols, rows] and sT float32 [rows / 128, cols] (chunk-major, like the
    library's 128x1 quantiser)."""
    from oracle import e4m3, quant
    rows = packed.shape[0]
    assert rows % 128 == 0 and cols % 128 == 0
    xh = uncache_1x128(packed, s, cols)                               # exact
    g = np.ascontiguousarray(xh.T).reshape(cols, rows // 128, 128)
    k = quant.pow2_exponent(np.max(np.abs(g), axis=-1))
    v = (g * np.ldexp(1.0, -k)[..., None]).astype(np.float32)       # exact product, one fp32 rounding
    qt = e4m3.encode(v).reshape(cols, rows)
    st = np.ldexp(np.float32(1.0), k.astype(np.int32)).astype(np.float32).T.copy()
    return qt, st
