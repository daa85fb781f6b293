"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws random tensors and rounds them to bf16; it holds none
of the quantisation or GEMM arithmetic, and both the HIP path and the oracle
consume the identical bf16 bytes it returns (uint16 bit patterns).

Recipe (numpy PCG64 `default_rng(seed)`, fp32 draws, rounded to bf16 with
round-to-nearest-even; each tensor of a workload gets its own child generator
from `rng.spawn`, in the order listed):

* tiny fprop (seed 1001): X [256, 1024] ~ N(0, 1) with a Bernoulli(0.01) mask
  of entries multiplied by 100; W [256, 1024] ~ N(0, 0.02) (0.02 is the std).
* dense fprop (1002): X [4096, 7168] ~ N(0, 1), Bernoulli(0.001) entries x 50;
  W [2048, 7168] ~ N(0, 0.02).
* backward pair (1003): dY [4096, 2048] ~ N(0, 1e-3); dgrad reuses the dense
  W, wgrad reuses the dense X.
* MoE grouped fprop (1004): 16384 tokens each pick 8 distinct experts out of
  256 by Gumbel-top-8 on log p with p_i proportional to (i+1)^-1.1 (Zipf,
  s = 1.1); experts 0..7 are this GPU's; their token counts are padded up to
  multiples of 128 with zero rows; real rows ~ N(0, 1); W_e [2048, 7168] ~
  N(0, 0.02).
* large heavy-tail fprop (1005): X [16384, 7168] ~ Student-t(3); W [18432,
  7168] ~ N(0, 0.02).

Nothing here comes from a public dataset: the workloads these pages describe
(DeepSeek-V3 pre-training) are stood in for by these distributions.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 bit patterns (nearest, ties to even). Finite inputs."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def _normal(rng, shape, std=1.0):
    return rng.standard_normal(shape, dtype=np.float32) * np.float32(std)


def _outliers(rng, x, p, mult):
    if p > 0:
        mask = rng.random(x.shape, dtype=np.float32) < np.float32(p)
        x = np.where(mask, x * np.float32(mult), x).astype(np.float32)
    return x


def act(seed: int, rows: int, cols: int, dist: str = "normal", std: float = 1.0,
        outlier_p: float = 0.0, outlier_mult: float = 1.0) -> np.ndarray:
    """A generic seeded activation-like bf16 matrix (uint16 bits)."""
    rng = np.random.default_rng(seed)
    if dist == "normal":
        x = _normal(rng, (rows, cols), std)
    elif dist == "student_t3":
        x = rng.standard_t(3, size=(rows, cols)).astype(np.float32) * np.float32(std)
    elif dist == "uniform":
        x = (rng.random((rows, cols), dtype=np.float32) * 2 - 1) * np.float32(std)
    else:
        raise ValueError(dist)
    return f32_to_bf16_bits(_outliers(rng, x, outlier_p, outlier_mult))


@dataclass
class Fprop:
    name: str
    x: np.ndarray      # bf16 bits [M, K]
    w: np.ndarray      # bf16 bits [N, K]


def tiny_fprop(seed: int = 1001) -> Fprop:
    rx, rw = np.random.default_rng(seed).spawn(2)
    x = _outliers(rx, _normal(rx, (256, 1024)), 0.01, 100.0)
    w = _normal(rw, (256, 1024), 0.02)
    return Fprop("tiny fprop 256x256x1024", f32_to_bf16_bits(x), f32_to_bf16_bits(w))


def dense_fprop(seed: int = 1002, m: int = 4096, n: int = 2048, k: int = 7168) -> Fprop:
    rx, rw = np.random.default_rng(seed).spawn(2)
    x = _outliers(rx, _normal(rx, (m, k)), 0.001, 50.0)
    w = _normal(rw, (n, k), 0.02)
    return Fprop(f"dense fprop {m}x{n}x{k}", f32_to_bf16_bits(x), f32_to_bf16_bits(w))


def backward_dy(seed: int = 1003, m: int = 4096, n: int = 2048) -> np.ndarray:
    (ry,) = np.random.default_rng(seed).spawn(1)
    return f32_to_bf16_bits(_normal(ry, (m, n), 1e-3))


def large_fprop(seed: int = 1005, m: int = 16384, n: int = 18432, k: int = 7168) -> Fprop:
    rx, rw = np.random.default_rng(seed).spawn(2)
    x = rx.standard_t(3, size=(m, k)).astype(np.float32)
    w = _normal(rw, (n, k), 0.02)
    return Fprop(f"large heavy-tail fprop {m}x{n}x{k}", f32_to_bf16_bits(x), f32_to_bf16_bits(w))


@dataclass
class MoE:
    name: str
    x: np.ndarray          # bf16 bits [sum padded rows, K]; padding rows are zero
    w: np.ndarray          # bf16 bits [G, N, K]
    row_off: np.ndarray    # int64 [G + 1], multiples of 128
    real_rows: np.ndarray  # int64 [G], tokens routed to each local expert


def moe_routing_counts(seed: int, tokens: int = 16384, experts: int = 256, topk: int = 8,
                       local: int = 8, zipf_s: float = 1.1) -> np.ndarray:
    """Tokens routed to each of the `local` first experts (Zipf-popular, top-k distinct)."""
    rng = np.random.default_rng(seed)
    logp = -zipf_s * np.log(np.arange(1, experts + 1, dtype=np.float64))
    counts = np.zeros(local, dtype=np.int64)
    for t0 in range(0, tokens, 4096):
        t1 = min(tokens, t0 + 4096)
        g = rng.gumbel(size=(t1 - t0, experts))
        top = np.argpartition(-(logp[None, :] + g), topk - 1, axis=1)[:, :topk]
        counts += np.bincount(top[top < local], minlength=local)
    return counts


def moe_fprop(seed: int = 1004, tokens: int = 16384, n: int = 2048, k: int = 7168,
              local: int = 8) -> MoE:
    rr, rx, rw = np.random.default_rng(seed).spawn(3)
    counts = moe_routing_counts(int(rr.integers(0, 2**31)), tokens=tokens, local=local)
    padded = (counts + 127) // 128 * 128
    row_off = np.concatenate([[0], np.cumsum(padded)]).astype(np.int64)
    x = np.zeros((int(row_off[-1]), k), dtype=np.uint16)
    for e in range(local):
        r0 = int(row_off[e])
        x[r0:r0 + counts[e]] = f32_to_bf16_bits(_normal(rx, (int(counts[e]), k)))
    w = np.stack([f32_to_bf16_bits(_normal(rw, (n, k), 0.02)) for _ in range(local)])
    return MoE(f"MoE grouped fprop {local} experts, {tokens} tokens top-8, N={n} K={k}",
               x, w, row_off, counts)


def moe_decode(seed: int = 1006, tokens: int = 256, n: int = 2048, k: int = 7168, local: int = 8) -> MoE:
    """Decode step of the MoE up-projection: `tokens` tokens routed top-8 over 256 experts
    (Zipf 1.1), the `local` most popular experts' rows stacked without padding (each at
    most `tokens` rows), X ~ N(0, 1), W_e ~ N(0, 0.02)."""
    rr, rx, rw = np.random.default_rng(seed).spawn(3)
    counts = moe_routing_counts(int(rr.integers(0, 2**31)), tokens=tokens, local=local)
    row_off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    x = f32_to_bf16_bits(_normal(rx, (int(row_off[-1]), k)))
    w = np.stack([f32_to_bf16_bits(_normal(rw, (n, k), 0.02)) for _ in range(local)])
    return MoE(f"MoE decode {local} experts, {tokens} tokens top-8, N={n} K={k}", x, w, row_off, counts)


# E4M3 byte patterns of 0, +-0.5, +-1, +-1.5, +-2, +-3, +-4. A product of two of
# these is a multiple of 1/4 below 16 in magnitude, so a block-scaled GEMM over
# such codes with power-of-two scales near 1 is exact in fp32 (every partial
# sum is a short dyadic number): its output, and therefore the bf16 rounding of
# it, has one right answer.
SMALL_CODES = np.array([0x00, 0x30, 0x38, 0x3C, 0x40, 0x44, 0x48, 0xB0, 0xB8, 0xBC, 0xC0, 0xC4, 0xC8], np.uint8)


def small_codes(seed: int, rows: int, cols: int) -> np.ndarray:
    """uint8 [rows, cols] drawn from SMALL_CODES."""
    rng = np.random.default_rng(seed)
    return SMALL_CODES[rng.integers(0, SMALL_CODES.size, (rows, cols))]


def pow2_scales(seed: int, shape, lo: int = -1, hi: int = 1) -> np.ndarray:
    """float32 powers of two 2^e, e uniform in [lo, hi]."""
    rng = np.random.default_rng(seed)
    return np.ldexp(np.float32(1.0), rng.integers(lo, hi + 1, shape).astype(np.int32)).astype(np.float32)
