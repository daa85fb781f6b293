"""Block-scaled FP8 GEMM of the oracle (test infrastructure).

The contraction is C[m, n] = sum_k A[m, k] * B[n, k]; both operands are stored
with the reduction index k contiguous. What is computed, and where the pages
say so:

* The three GEMMs of a Linear layer (Fprop, Dgrad, Wgrad) take FP8 inputs and
  produce BF16 or FP32 outputs (DeepSeek-V3 report, section 3.3.1 and
  Figure 6). Reading: Fprop and Dgrad give BF16, Wgrad gives FP32 (the report
  keeps weight gradients in FP32, section 3.3.3 "low-precision optimizer
  states").
* Promotion (report section 3.3.2 "increasing accumulation precision",
  Figure 7b; tech note "DeepSeek-V3 FP8 dynamic quantisation", accumulation
  steps): the low-precision partial sum over each interval of N_C = 128
  K-elements is promoted into an FP32 accumulator, multiplied there by the
  per-group scales of both operands (out += MMA(FP8 x, FP8 w) * s_x * s_w).
  Reading: the interval is 128 K-elements, the same 128 that a quantisation
  group spans (the report's "N_C = 128 elements"; the tech note's "every 128
  MMAs" is read as the same thing).

How the oracle evaluates it:

* G1. P_c = sum over the 128 k of chunk c of dec(qA) * dec(qB), in float64.
  Every E4M3 value is an integer multiple of 2^-9 below 2^9, so each product
  is a multiple of 2^-18 and |P_c| < 128 * 448^2 < 2^25; counted in units of
  2^-18 every partial sum is an integer below 2^43 < 2^53, hence exact in
  float64 whatever order the BLAS routine sums in.
* G2. y32 <- fl32(y32 + fl32(P_c * (s_A * s_B))) for c ascending; s_A * s_B is
  exact in float64, the product with P_c is rounded once in float64.
* G3. y64 = sum_c P_c * s_A * s_B in float64, and the tolerance scale
  absbound = sum_k |x_hat_k| * |w_hat_k| (= sum_c s_A s_B sum_k |qA||qB|).
* G4. The BF16 epilogue is round-to-nearest-even of y32.
* G5. Producer fusion (report section 3.5.2, "online quantization support":
  activations are read from HBM, quantised, written back and read again for
  the next matrix multiply, which fusing the cast into the producer saves):
  the BF16 output of G4 quantised at once as the next GEMM's activation
  operand, 1x128 tiles along each row (oracle.quant.quant_act_1x128). Reading:
  the tiles are quantised from the BF16 values the GEMM would store.

Pinned by: tests/test_oracle_gemm.py -- P_c against an exact integer dot of
the codes; tiny shapes against a Fraction triple loop; y64 against the plain
product of the dequantised operands; the uniform-scale special case (textbook
per-tensor-scaled FP8 GEMM); K = 128; the bf16 epilogue against torch; G5
against exact fractions and the exhaustive encoder on a tiny GEMM.
"""

from __future__ import annotations

import numpy as np

from . import e4m3, quant

CHUNK = 128


def gemm_rowscaled(qa: np.ndarray, sa: np.ndarray, qb: np.ndarray, sb: np.ndarray,
                   row_block: int = 1024) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Core G1-G3 with one scale per (operand row, K-chunk) on both sides.

    qa uint8 [M, K], sa float32 [M, K/128]; qb uint8 [N, K], sb float32 [N, K/128].
    Returns (y32 float32 [M, N], y64 float64 [M, N], absbound float64 [M, N]).
    """
    M, K = qa.shape
    N, Kb = qb.shape
    assert K == Kb and K % CHUNK == 0
    nc = K // CHUNK
    assert sa.shape == (M, nc) and sb.shape == (N, nc)
    db = e4m3.decode(qb)                      # [N, K] float64, exact
    y32 = np.zeros((M, N), dtype=np.float32)
    y64 = np.zeros((M, N), dtype=np.float64)
    ab = np.zeros((M, N), dtype=np.float64)
    for r0 in range(0, M, row_block):
        r1 = min(M, r0 + row_block)
        da = e4m3.decode(qa[r0:r1])
        for c in range(nc):
            ks = slice(c * CHUNK, (c + 1) * CHUNK)
            a_c, b_c = da[:, ks], db[:, ks]
            p = a_c @ b_c.T                                              # G1, exact
            scale = sa[r0:r1, c].astype(np.float64)[:, None] * sb[:, c].astype(np.float64)[None, :]
            y32[r0:r1] = (y32[r0:r1] + (p * scale).astype(np.float32)).astype(np.float32)   # G2
            y64[r0:r1] += p * scale                                      # G3
            ab[r0:r1] += (np.abs(a_c) @ np.abs(b_c).T) * scale
    return y32, y64, ab


def expand_block_scales(sw: np.ndarray) -> np.ndarray:
    """Per-row view of 128x128 block scales: [N/128, K/128] -> [N, K/128]."""
    return np.repeat(np.asarray(sw, dtype=np.float32), CHUNK, axis=0)


def fprop(qx, sx, qw, sw, row_block: int = 1024):
    """Y[M, N] = X_hat W_hat^T. qx [M, K] with 1x128 scales sx [M, K/128];
    qw [N, K] with 128x128 block scales sw [N/128, K/128]. Output read as BF16."""
    return gemm_rowscaled(qx, sx, qw, expand_block_scales(sw), row_block)


def dgrad(qdy, sdy, qw, sw, row_block: int = 1024):
    """dX[M, K] = dY_hat W_hat. qdy [M, N] with 1x128 scales sdy [M, N/128];
    qw [N, K] with block scales sw [N/128, K/128]. The B operand is W^T, whose
    128x128 blocks are W's blocks transposed (block grouping is symmetric)."""
    qwT = np.ascontiguousarray(np.asarray(qw).T)
    return gemm_rowscaled(qdy, sdy, qwT, expand_block_scales(np.asarray(sw).T), row_block)


def wgrad(qdyT, sdyT, qxT, sxT, row_block: int = 1024):
    """dW[N, K] = dY_hat^T X_hat, reduced over tokens. qdyT [N, T] and qxT [K, T]
    are the token-contiguous (128x1-tile) quantisations with scales [., T/128].
    Output read as FP32."""
    return gemm_rowscaled(qdyT, sdyT, qxT, sxT, row_block)


def grouped_fprop(qx, sx, row_off, qw_groups, sw_groups, row_block: int = 1024):
    """Per-expert Fprop: rows [row_off[e], row_off[e+1]) of X use expert e's weight.

    qw_groups [G, N, K], sw_groups [G, N/128, K/128]. Returns (y32, y64, absbound)
    for all rows stacked."""
    M = qx.shape[0]
    N = qw_groups.shape[1]
    y32 = np.zeros((M, N), np.float32)
    y64 = np.zeros((M, N), np.float64)
    ab = np.zeros((M, N), np.float64)
    for e in range(len(row_off) - 1):
        r0, r1 = int(row_off[e]), int(row_off[e + 1])
        if r1 > r0:
            y32[r0:r1], y64[r0:r1], ab[r0:r1] = fprop(qx[r0:r1], sx[r0:r1], qw_groups[e],
                                                      sw_groups[e], row_block)
    return y32, y64, ab


def bf16_rne_bits(y32: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bit patterns.
    Inputs are finite."""
    u = np.asarray(y32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns."""
    return (np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def quantise_output(y32: np.ndarray, scale_mode: str = "exact") -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """G5: the GEMM's BF16 output (G4) as the next GEMM's FP8 activation operand.

    Returns (bf16 bits [M, N], codes uint8 [M, N], scales float32 [M, N/128])."""
    bits = bf16_rne_bits(y32)
    q, s = quant.quant_act_1x128(bits, scale_mode)
    return bits, q, s
