"""Online fine-grained quantisation of the oracle (test infrastructure).

What is computed, and where the pages say so:

* Grouping (DeepSeek-V3 report, section 3.3.2 "fine-grained quantization",
  Figure 7a): activations are grouped and scaled per 1x128 tile (one token,
  128 channels); weights per 128x128 block (128 input channels x 128 output
  channels). The scaling factor runs along the GEMM's inner dimension K.
* Online scale (same section, "online quantization"; tech note "DeepSeek-V3 FP8
  dynamic quantisation", fine-grained quantization implementation formula):
  for every tile or block the max-abs value is taken on the fly and
  s = absmax / F_max, with F_max the largest finite FP8 value (448 for E4M3FN);
  then q = FP8(x / s).
* Backward transposition (report section 3.3.3 "low-precision activations"
  and section 3.5.2 "support for transposed GEMM"): for the weight-gradient
  GEMM the tiles run along the token dimension (128x1). The oracle quantises
  the bf16 tensor's transpose with 1x128 tiles, which is that grouping.

Readings where the pages leave a step open:

* s is the IEEE binary32 quotient fl32(absmax / 448.0), rounded to nearest even.
* x / s is the IEEE binary32 quotient fl32(x / s); it is then rounded to E4M3
  (round to nearest even, saturating, sign kept) by `e4m3.encode`.
* A tile whose absmax is zero gets s = 0 and codes +0 / -0 by the sign of x.
* Inputs are bf16 bit patterns (uint16) and must be finite.

Power-of-two scales (scale_mode="pow2"): the report (section 3.3.3,
"low-precision storage and communication") gives some activations scaling
factors that are integral powers of 2 (the inputs of the Linear after
attention, the activations dispatched to the MoE up-projection). Reading: s is
the smallest power of two with absmax / s <= 448, i.e. s = 2^k with
k = ceil(log2(absmax / 448)), so nothing saturates; k is kept within
[-127, 127] (the range of the E8M0 exponent byte a scaled matrix instruction
takes) and an all-zero group gets s = 2^-127. Then q = E4M3(x * 2^-k), where
the product is exact, so there is one rounding instead of two.

Scale layout here is the natural one: s[r, c] for row r and 128-column chunk c.

Pinned by: tests/test_oracle_quant.py -- every tile's absmax element lands on
+-448; the per-element dequantisation error bound; one outlier changes only
its own tile; exact power-of-two rescaling; negation flips only sign bits;
quantising W^T equals the transpose of quantising W; a hand-derived tile.
"""

from __future__ import annotations

import numpy as np

from . import e4m3

TILE = 128
F_MAX = np.float32(448.0)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


K_MIN, K_MAX = -127, 127   # exponent range of a power-of-two scale


def pow2_exponent(amax: np.ndarray) -> np.ndarray:
    """Smallest integer k with amax <= 448 * 2^k, clamped to [K_MIN, K_MAX];
    K_MIN for amax = 0. Found by search from a float estimate and corrected in
    exact arithmetic (448 * 2^k and amax are exact in float64)."""
    a = np.asarray(amax, dtype=np.float64)
    pos = a > 0
    est = np.zeros(a.shape, dtype=np.int64)
    est[pos] = np.ceil(np.log2(a[pos] / 448.0)).astype(np.int64)
    k = est.copy()
    for _ in range(4):   # the estimate is off by at most one either way
        k = np.where(pos & (a > 448.0 * np.ldexp(1.0, k)), k + 1, k)
        k = np.where(pos & (a <= 448.0 * np.ldexp(1.0, k - 1)), k - 1, k)
    k = np.where(pos, k, K_MIN)
    return np.clip(k, K_MIN, K_MAX)


def _quant_groups_pow2(xg: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Power-of-two scales: s = 2^k as above, q = E4M3(x * 2^-k) (exact product)."""
    amax = np.max(np.abs(xg), axis=-1)
    k = pow2_exponent(amax)
    v = xg.astype(np.float64) * np.ldexp(1.0, -k)[..., None]      # exact
    q = e4m3.encode(v)
    return q, np.ldexp(np.float32(1.0), k.astype(np.int32)).astype(np.float32)


def _quant_groups(xg: np.ndarray, scale_mode: str = "exact") -> tuple[np.ndarray, np.ndarray]:
    """Quantise groups laid out along the last axis of `xg` (float32).

    Returns (codes uint8 with the shape of xg, scales float32 of xg.shape[:-1]).
    """
    if scale_mode == "pow2":
        return _quant_groups_pow2(xg)
    assert scale_mode == "exact", scale_mode
    amax = np.max(np.abs(xg), axis=-1)                         # exact
    s = (amax.astype(np.float32) / F_MAX).astype(np.float32)   # fl32(amax / 448)
    zero = s == 0
    s_safe = np.where(zero, np.float32(1.0), s).astype(np.float32)
    with np.errstate(over="ignore", under="ignore"):
        v = (xg / s_safe[..., None]).astype(np.float32)        # fl32(x / s)
    q = e4m3.encode(v)
    # all-zero groups: s = 0 and +-0 codes by the sign of x
    zq = np.where(np.signbit(xg), 0x80, 0x00).astype(np.uint8)
    q = np.where(zero[..., None], zq, q)
    return q, s


def quant_act_1x128(x_bits: np.ndarray, scale_mode: str = "exact") -> tuple[np.ndarray, np.ndarray]:
    """1x128 tiles along the columns of a bf16 matrix x[rows, cols].

    Returns q uint8 [rows, cols] and s float32 [rows, cols // 128].
    """
    x = bf16_bits_to_f32(x_bits)
    rows, cols = x.shape
    assert cols % TILE == 0, "columns must be a multiple of 128"
    q, s = _quant_groups(x.reshape(rows, cols // TILE, TILE), scale_mode)
    return q.reshape(rows, cols), s


def quant_act_128x1(x_bits: np.ndarray, scale_mode: str = "exact") -> tuple[np.ndarray, np.ndarray]:
    """128x1 tiles (128 consecutive rows of one column) of x[rows, cols].

    The result is stored transposed so that the grouped dimension is
    contiguous: qT uint8 [cols, rows] and sT float32 [cols, rows // 128].
    This is exactly 1x128 quantisation of x's transpose.
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    assert x_bits.shape[0] % TILE == 0, "rows must be a multiple of 128"
    return quant_act_1x128(np.ascontiguousarray(x_bits.T), scale_mode)


def quant_w_128x128(w_bits: np.ndarray, scale_mode: str = "exact") -> tuple[np.ndarray, np.ndarray]:
    """128x128 blocks of a bf16 weight w[n, k].

    Returns q uint8 [n, k] and s float32 [n // 128, k // 128].
    """
    w = bf16_bits_to_f32(w_bits)
    n, k = w.shape
    assert n % TILE == 0 and k % TILE == 0, "weight dims must be multiples of 128"
    blocks = w.reshape(n // TILE, TILE, k // TILE, TILE).transpose(0, 2, 1, 3)
    q, s = _quant_groups(blocks.reshape(n // TILE, k // TILE, TILE * TILE), scale_mode)
    q = q.reshape(n // TILE, k // TILE, TILE, TILE).transpose(0, 2, 1, 3).reshape(n, k)
    return np.ascontiguousarray(q), s


def dequant_act(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """x_hat = dec(q) * s per 1x128 tile, in float64 (exact)."""
    rows, cols = q.shape
    return (e4m3.decode(q).reshape(rows, cols // TILE, TILE)
            * s.astype(np.float64)[..., None]).reshape(rows, cols)


def requant_128x1(q: np.ndarray, s: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Transposing re-quantisation of an FP8 activation cache, 1x128 -> 128x1.

    The report (section 3.5.2, "support for transposed GEMM") describes the
    backward step: the forward pass stored activations as 1x128 FP8 tiles; the
    weight-gradient GEMM needs them as 128x1 tiles, so they are read,
    dequantised, transposed, re-quantised and stored again. For exactly these
    activations the report (section 3.3.3, "low-precision storage and
    communication") makes every scale an integral power of two, so that the
    conversion adds no quantisation error of its own.

    Steps: x_hat = dec(q) * s (float64, exact); 128x1 groups (128 consecutive
    rows of one column); the group's scale is the power of two of
    `pow2_exponent` on its exact absmax; codes E4M3(fl32(x_hat * 2^-k)). With
    power-of-two input scales the product is exact in float32 too, and for
    values that fit bf16 this is the 128x1 power-of-two quantisation of x_hat.

    q uint8 [rows, cols] with s float32 [rows, cols // 128] (the natural layout
    of `quant_act_1x128`). Returns qT uint8 [cols, rows] and sT float32
    [cols, rows // 128], like `quant_act_128x1`.
    """
    rows, cols = q.shape
    assert rows % TILE == 0 and cols % TILE == 0, "dimensions must be multiples of 128"
    xh = dequant_act(q, s)                                         # exact
    g = np.ascontiguousarray(xh.T).reshape(cols, rows // TILE, TILE)
    amax = np.max(np.abs(g), axis=-1)
    k = pow2_exponent(amax)
    v = (g * np.ldexp(1.0, -k)[..., None]).astype(np.float32)      # exact product, one fp32 rounding
    qt = e4m3.encode(v)
    st = np.ldexp(np.float32(1.0), k.astype(np.int32)).astype(np.float32)
    return qt.reshape(cols, rows), st


def dequant_w(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """w_hat = dec(q) * s per 128x128 block, in float64 (exact)."""
    return e4m3.decode(q) * np.repeat(np.repeat(s.astype(np.float64), TILE, 0), TILE, 1)
