"""Pins of the oracle's block-scaled GEMM.

The method reaches, up to rounding order, a result with a plain definition:
Y = X_hat W_hat^T of the dequantised operands (x_hat = dec(q) * s). These
tests pin the oracle's chunked evaluation to that definition and to exact
integer / rational arithmetic, and pin the promotion step of the report
(section 3.3.2, Figure 7b) and the tech note (out += MMA * s_x * s_w) through
special cases where the scales are known in closed form.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import e4m3, gemm, quant
from workloads import act, f32_to_bf16_bits


def _q(seed, rows, cols, **kw):
    return quant.quant_act_1x128(act(seed, rows, cols, **kw))


def _codes_to_units(q):
    # every E4M3 value is an integer multiple of 2^-9
    return (e4m3.decode(q) * 512).astype(np.int64)


def test_chunk_sum_is_exact_integer_dot():
    rng = np.random.default_rng(3)
    cases = [rng.integers(0, 256, size=(8, 128)).astype(np.uint8)]
    cases[0][cases[0] == 0x7F] = 0x7E
    cases[0][cases[0] == 0xFF] = 0xFE
    cases.append(np.full((8, 128), 0x7E, np.uint8))                       # all 448
    mixed = np.where(np.arange(128) % 2 == 0, 0x7E, 0x01).astype(np.uint8)  # 448 and 2^-9
    cases.append(np.tile(mixed, (8, 1)))
    for qa in cases:
        qb = qa[::-1].copy() ^ np.uint8(0x80) * (np.arange(8)[:, None] % 2).astype(np.uint8)
        ones = np.ones((8, 1), np.float32)
        _, y64, _ = gemm.gemm_rowscaled(qa, ones, qb, ones)
        exact = _codes_to_units(qa) @ _codes_to_units(qb).T              # int64, exact
        np.testing.assert_array_equal(y64, exact.astype(np.float64) * 2.0 ** -18)


def test_tiny_shapes_against_fraction_triple_loop():
    rng = np.random.default_rng(4)
    for (m, n, k) in [(3, 5, 128), (4, 2, 384), (1, 1, 256)]:
        qa, sa = _q(int(rng.integers(1 << 30)), m, k, outlier_p=0.05, outlier_mult=30)
        qb, sb = _q(int(rng.integers(1 << 30)), n, k, std=0.02)
        _, y64, ab = gemm.gemm_rowscaled(qa, sa, qb, sb)
        for i in range(m):
            for j in range(n):
                exact = Fraction(0)
                for kk in range(k):
                    c = kk // 128
                    xa = Fraction(e4m3.decode_scalar(qa[i, kk])) * Fraction(float(sa[i, c]))
                    xb = Fraction(e4m3.decode_scalar(qb[j, kk])) * Fraction(float(sb[j, c]))
                    exact += xa * xb
                # one fp64 rounding per chunk term and per addition
                tol = (2 * (k // 128) + 1) * 2.0 ** -53 * ab[i, j]
                assert abs(Fraction(y64[i, j]) - exact) <= Fraction(tol)


def test_fprop_equals_plain_product_of_dequantised_operands():
    qx, sx = _q(20, 96, 512, outlier_p=0.01, outlier_mult=100)
    w = act(21, 256, 512, std=0.02)
    qw, sw = quant.quant_w_128x128(w)
    y32, y64, ab = gemm.fprop(qx, sx, qw, sw)
    plain = quant.dequant_act(qx, sx) @ quant.dequant_w(qw, sw).T
    assert np.all(np.abs(y64 - plain) <= 1e-13 * ab)
    # fp32 accumulation over 4 chunks stays within the fp32 summation bound
    assert np.all(np.abs(y32.astype(np.float64) - y64) <= 6 * 2.0 ** -24 * ab)
    # the tolerance scale is sum_k |x_hat| |w_hat|
    ab_plain = np.abs(quant.dequant_act(qx, sx)) @ np.abs(quant.dequant_w(qw, sw)).T
    np.testing.assert_allclose(ab, ab_plain, rtol=1e-14)


def test_uniform_scale_reduces_to_per_tensor_fp8_gemm():
    # plant +-a at the start of every tile so every scale is the same power of two
    m, n, k = 32, 128, 384
    x = quant.bf16_bits_to_f32(act(22, m, k, outlier_p=0)).copy()
    w = quant.bf16_bits_to_f32(act(23, n, k, std=0.02)).copy()
    x = np.clip(x, -3.0, 3.0); x[:, ::128] = 3.5         # amax 3.5 -> s_x = 2^-7
    w = np.clip(w, -0.05, 0.05); w[:, ::128] = -0.4375    # amax 0.4375 -> s_w = 2^-10
    qx, sx = quant.quant_act_1x128(f32_to_bf16_bits(x))
    qw, sw = quant.quant_w_128x128(f32_to_bf16_bits(w))
    assert np.all(sx == 2.0 ** -7) and np.all(sw == 2.0 ** -10)
    y32, y64, _ = gemm.fprop(qx, sx, qw, sw)
    textbook = (_codes_to_units(qx) @ _codes_to_units(qw).T).astype(np.float64) * 2.0 ** -18 * 2.0 ** -17
    np.testing.assert_array_equal(y64, textbook)


def test_single_chunk_is_scaled_dot():
    qx, sx = _q(24, 16, 128)
    qw, sw = quant.quant_w_128x128(act(25, 128, 128, std=0.02))
    y32, y64, _ = gemm.fprop(qx, sx, qw, sw)
    dot = (_codes_to_units(qx) @ _codes_to_units(qw).T).astype(np.float64) * 2.0 ** -18
    want = dot * (sx[:, :1].astype(np.float64) * np.float64(sw[0, 0]))
    np.testing.assert_array_equal(y64, want)
    np.testing.assert_array_equal(y32, want.astype(np.float32))


def test_bf16_epilogue_matches_torch():
    rng = np.random.default_rng(26)
    y = (rng.standard_normal(100000) * 10.0 ** rng.integers(-6, 6, 100000)).astype(np.float32)
    bits = rng.integers(0, 2 ** 16, 1000, dtype=np.uint32)
    y = np.concatenate([y, ((bits << 16) | 0x8000).astype(np.uint32).view(np.float32)])  # exact ties
    y = y[np.isfinite(y)]
    want = torch.from_numpy(y).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(gemm.bf16_rne_bits(y), want)


def test_dgrad_definition():
    w = act(27, 256, 384, std=0.02)                 # W [N=256, K=384]
    qw, sw = quant.quant_w_128x128(w)
    qdy, sdy = _q(28, 64, 256, std=1e-3)           # dY [M=64, N=256]
    _, y64, ab = gemm.dgrad(qdy, sdy, qw, sw)
    plain = quant.dequant_act(qdy, sdy) @ quant.dequant_w(qw, sw)   # dX = dY W
    assert y64.shape == (64, 384)
    assert np.all(np.abs(y64 - plain) <= 1e-13 * ab)


def test_wgrad_definition():
    T, N, K = 256, 128, 256
    dy = act(29, T, N, std=1e-3)
    x = act(30, T, K)
    qdyT, sdyT = quant.quant_act_128x1(dy)          # [N, T]
    qxT, sxT = quant.quant_act_128x1(x)             # [K, T]
    y32, y64, ab = gemm.wgrad(qdyT, sdyT, qxT, sxT)
    plain = quant.dequant_act(qdyT, sdyT) @ quant.dequant_act(qxT, sxT).T   # dW = dY^T X
    assert y64.shape == (N, K)
    assert np.all(np.abs(y64 - plain) <= 1e-13 * ab)
    # and close to the unquantised product (quantisation error only)
    ref = quant.bf16_bits_to_f32(dy).astype(np.float64).T @ quant.bf16_bits_to_f32(x).astype(np.float64)
    assert np.linalg.norm(y64 - ref) <= 0.1 * np.linalg.norm(ref)


def test_grouped_is_per_expert_fprop_and_padding_rows_are_zero():
    rng = np.random.default_rng(31)
    K, N = 256, 128
    row_off = np.array([0, 128, 128, 384], np.int64)    # expert 1 empty
    x = act(32, 384, K)
    x[100:128] = 0                                      # padding rows of expert 0
    qx, sx = quant.quant_act_1x128(x)
    ws = np.stack([act(int(rng.integers(1 << 30)), N, K, std=0.02) for _ in range(3)])
    qws, sws = zip(*[quant.quant_w_128x128(w) for w in ws])
    qws, sws = np.stack(qws), np.stack(sws)
    y32, y64, ab = gemm.grouped_fprop(qx, sx, row_off, qws, sws)
    for e in range(3):
        r0, r1 = row_off[e], row_off[e + 1]
        if r1 > r0:
            _, ye, _ = gemm.fprop(qx[r0:r1], sx[r0:r1], qws[e], sws[e])
            np.testing.assert_array_equal(y64[r0:r1], ye)
    assert np.all(y32[100:128] == 0) and np.all(sx[100:128] == 0)


@pytest.mark.parametrize("seed", [40, 41])
def test_fp32_accumulation_bound(seed):
    qx, sx = _q(seed, 64, 1024, dist="student_t3", outlier_p=0)
    qw, sw = quant.quant_w_128x128(act(seed + 100, 128, 1024, std=0.02))
    y32, y64, ab = gemm.fprop(qx, sx, qw, sw)
    nc = 1024 // 128
    assert np.all(np.abs(y32.astype(np.float64) - y64) <= (2 * nc + 1) * 2.0 ** -24 * ab)


def _fl32(f: Fraction) -> float:
    """Binary32 round-to-nearest-even of an exact rational (normal range)."""
    if f == 0:
        return 0.0
    sign = -1 if f < 0 else 1
    f = abs(f)
    e = f.numerator.bit_length() - f.denominator.bit_length()
    while Fraction(2) ** e > f:
        e -= 1
    while Fraction(2) ** (e + 1) <= f:
        e += 1
    ulp = Fraction(2) ** (e - 23)
    m = f / ulp
    lo = m.numerator // m.denominator
    rem = m - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    return sign * float(lo * ulp)


@pytest.mark.parametrize("mode", ["exact", "pow2"])
def test_quantise_output_against_fractions(mode):
    # G5 on a tiny GEMM whose output is exact (small codes, power-of-two scales):
    # y from a Fraction triple loop, its bf16 rounding from torch, then per
    # 1x128 row tile the scale (fl32(amax / 448) rounded exactly from the
    # fraction, or the smallest power of two 2^k with amax <= 448 * 2^k) and
    # every code from the exhaustive nearest-value encoder
    from workloads import pow2_scales, small_codes
    qa = small_codes(71, 3, 256)
    qa[1] = 0                                            # a zero row: scale 0 / 2^-127, codes +0
    qb = small_codes(72, 256, 256)
    sa = pow2_scales(73, (3, 2))
    sb = pow2_scales(74, (2, 2))
    y32, _, _ = gemm.fprop(qa, sa, qb, sb)
    bits, q, s = gemm.quantise_output(y32, mode)
    da, db = e4m3.decode(qa), e4m3.decode(qb)
    for i in range(3):
        for g in range(2):
            ys = []
            for j in range(128 * g, 128 * g + 128):
                v = sum(Fraction(float(da[i, k])) * Fraction(float(db[j, k])) * Fraction(float(sa[i, k // 128]))
                        * Fraction(float(sb[j // 128, k // 128])) for k in range(256))
                assert float(y32[i, j]) == v                 # the output is exact
                ys.append(v)
            yb = torch.tensor([float(v) for v in ys], dtype=torch.float32).to(torch.bfloat16)
            np.testing.assert_array_equal(bits[i, 128 * g:128 * g + 128],
                                          yb.view(torch.int16).numpy().view(np.uint16))
            yv = [Fraction(float(v)) for v in yb.float().numpy()]
            amax = max(abs(v) for v in yv)
            if mode == "pow2":
                k = -127
                while amax > 448 * Fraction(2) ** k:
                    k += 1
                want_s = 2.0 ** k
                vals = [v / Fraction(2) ** k for v in yv]
            else:
                want_s = _fl32(amax / 448) if amax else 0.0
                vals = [Fraction(_fl32(v / Fraction(want_s))) if want_s else Fraction(0) for v in yv]
            assert float(s[i, g]) == want_s
            want_q = e4m3.encode_bruteforce_vec(np.array([float(v) for v in vals]))
            np.testing.assert_array_equal(q[i, 128 * g:128 * g + 128], want_q)
    # planted mistake: tiles of the fp32 output instead of its bf16 rounding
    # would give other exact scales on this input, which the checks above reject
    if mode == "exact":
        am = np.abs(y32.reshape(3, 2, 128).astype(np.float64)).max(-1)
        s_f32 = (am / 448).astype(np.float32)
        assert not np.array_equal(s_f32[s_f32 > 0], s[s > 0])
