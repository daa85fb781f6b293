"""Pins of the oracle's online quantisers against what the pages fix.

* s = absmax / 448 maps every tile's absmax element onto +-448 exactly (the
  tech note's implementation formula; the report's "scale the max-abs value
  to the FP8 maximum", section 3.3.2).
* The per-element dequantisation error is bounded by E4M3's 3-bit mantissa.
* A tile with an outlier changes nothing outside that tile (the tech note's
  "an outlier only pollutes its own block"; the report's Figure 7a motivation).
* Exact invariants: power-of-two rescaling, negation, transposition of 128x128
  blocks, and a hand-derived tile.
"""

import numpy as np
import pytest

from oracle import e4m3, quant
from workloads import act, f32_to_bf16_bits


def _x(seed=5, rows=64, cols=512, **kw):
    kw.setdefault("outlier_p", 0.01)
    kw.setdefault("outlier_mult", 100.0)
    return act(seed, rows, cols, **kw)


def test_absmax_element_maps_to_448():
    for x in (_x(), _x(6, dist="student_t3", outlier_p=0), _x(7, std=1e-30, outlier_p=0)):
        q, s = quant.quant_act_1x128(x)
        xf = quant.bf16_bits_to_f32(x).reshape(x.shape[0], -1, 128)
        qq = q.reshape(xf.shape)
        am = np.abs(xf).max(-1, keepdims=True)
        hit = (np.abs(xf) == am) & (am > 0)
        assert hit.any()
        assert np.all((qq[hit] & 0x7F) == 0x7E)
        assert np.all((qq[hit] >> 7) == (xf[hit] < 0))


def _f32_of_fraction(fr):
    """Nearest binary32 of an exact rational that is never a binary32 midpoint.
    Rounding to binary64 first cannot land on a binary32 midpoint here: the
    quotients below have an odd factor (7, or the odd part of a 24-bit scale)
    in the denominator, so their binary expansions are not dyadic and do not
    hold 28 zero bits after the 25th significant bit."""
    return np.float32(float(fr))


def test_scale_definition_and_layout():
    # s is the binary32 rounding of the exact rational absmax / 448, computed
    # here with fractions rather than with the oracle's float32 division
    from fractions import Fraction
    x = _x()
    q, s = quant.quant_act_1x128(x)
    xf = quant.bf16_bits_to_f32(x).reshape(x.shape[0], -1, 128)
    assert s.shape == (64, 4) and s.dtype == np.float32
    for r in range(0, 64, 7):
        for t in range(4):
            amax = max(abs(Fraction(float(v))) for v in xf[r, t])
            assert s[r, t] == _f32_of_fraction(amax / 448), (r, t)


def test_dequant_error_bound():
    for x in (_x(), _x(8, dist="student_t3", outlier_p=0), _x(9, std=1e-3)):
        q, s = quant.quant_act_1x128(x)
        xhat = quant.dequant_act(q, s)
        xf = quant.bf16_bits_to_f32(x).astype(np.float64)
        srow = np.repeat(s.astype(np.float64), 128, axis=1)
        bound = np.maximum(2.0 ** -4 * np.abs(xf), 2.0 ** -10 * srow) * (1 + 2.0 ** -19)
        assert np.all(np.abs(xhat - xf) <= bound)
        # the relative 2^-4 bound holds where |x / s| >= 2^-6 (normal E4M3 range)
        big = np.abs(xf) >= 2.0 ** -6 * srow
        assert np.all(np.abs(xhat - xf)[big] <= 2.0 ** -4 * np.abs(xf)[big] * (1 + 2.0 ** -19))


def test_outlier_only_changes_its_own_tile():
    x = _x(10, outlier_p=0)
    q0, s0 = quant.quant_act_1x128(x)
    xf = quant.bf16_bits_to_f32(x).copy()
    r, c = 17, 3 * 128 + 41
    xf[r, c] = np.float32(5000.0)
    q1, s1 = quant.quant_act_1x128(f32_to_bf16_bits(xf))
    tile = np.zeros_like(s0, dtype=bool)
    tile[r, c // 128] = True
    assert s1[r, c // 128] != s0[r, c // 128]
    np.testing.assert_array_equal(s1[~tile], s0[~tile])
    qmask = np.repeat(tile, 128, axis=1)
    np.testing.assert_array_equal(q1[~qmask], q0[~qmask])
    assert (q1[qmask] != q0[qmask]).any()


@pytest.mark.parametrize("j", [-8, 8])
def test_power_of_two_rescaling(j):
    x = _x(11, outlier_p=0)
    q0, s0 = quant.quant_act_1x128(x)
    xs = f32_to_bf16_bits(np.ldexp(quant.bf16_bits_to_f32(x), j).astype(np.float32))
    q1, s1 = quant.quant_act_1x128(xs)
    np.testing.assert_array_equal(q1, q0)
    np.testing.assert_array_equal(s1, np.ldexp(s0, j).astype(np.float32))


def test_negation_flips_sign_bits_only():
    x = _x(12)
    q0, s0 = quant.quant_act_1x128(x)
    q1, s1 = quant.quant_act_1x128(x ^ np.uint16(0x8000))
    np.testing.assert_array_equal(s1, s0)
    np.testing.assert_array_equal(q1, q0 ^ np.uint8(0x80))


def test_weight_block_transpose_invariance():
    w = act(13, 256, 384, std=0.02)
    q, s = quant.quant_w_128x128(w)
    qt, st = quant.quant_w_128x128(np.ascontiguousarray(w.T))
    np.testing.assert_array_equal(qt, q.T)
    np.testing.assert_array_equal(st, s.T)


def test_weight_block_scale_is_block_absmax():
    from fractions import Fraction
    w = act(14, 256, 256, std=0.02)
    q, s = quant.quant_w_128x128(w)
    wf = quant.bf16_bits_to_f32(w)
    for i in range(2):
        for j in range(2):
            blk = wf[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128]
            amax = max(abs(Fraction(float(v))) for v in blk.ravel()[np.argsort(-np.abs(blk.ravel()))[:4]])
            assert s[i, j] == _f32_of_fraction(amax / 448)
            # a 128x128 block is not 128 independent 1x128 tiles: rows share one scale
            qa, sa = quant.quant_act_1x128(f32_to_bf16_bits(blk))
            assert not np.all(sa == s[i, j])


def test_zero_tile_gives_zero_scale_and_signed_zero_codes():
    x = _x(15, rows=4, cols=256)
    x[2, 128:] = 0
    x[2, 130] = 0x8000                       # -0
    q, s = quant.quant_act_1x128(x)
    assert s[2, 1] == 0
    assert q[2, 130] == 0x80 and np.all(np.delete(q[2, 128:], 2) == 0x00)


def test_hand_derived_tile():
    # amax 448 -> s = 1 exactly, so codes are the plain E4M3 encodings of the inputs
    vals = np.zeros(128, np.float32)
    vals[:6] = [448.0, 1.0, -2.0, 0.30078125, 1.0625, -(2.0 ** -10)]
    q, s = quant.quant_act_1x128(f32_to_bf16_bits(vals[None, :]))
    assert s[0, 0] == 1.0
    assert list(q[0, :6]) == [0x7E, 0x38, 0xC0, 0x2A, 0x38, 0x80]
    # amax 3.5 -> s = fl32(3.5 / 448) = 2^-7 exactly; x = 1 -> 128 = 2^7 -> code 0x70
    vals2 = np.zeros(128, np.float32)
    vals2[:3] = [3.5, 1.0, -0.01]
    q2, s2 = quant.quant_act_1x128(f32_to_bf16_bits(vals2[None, :]))
    assert s2[0, 0] == 2.0 ** -7
    assert q2[0, 0] == 0x7E and q2[0, 1] == 0x70
    # -0.01 in bf16 is -0.010009765625; / 2^-7 = -1.28125 -> 1.25 (code 0x3A) with sign
    assert q2[0, 2] == 0xBA


def test_128x1_is_quantisation_along_rows():
    x = _x(16, rows=256, cols=128)
    qT, sT = quant.quant_act_128x1(x)
    assert qT.shape == (128, 256) and sT.shape == (128, 2)
    xf = quant.bf16_bits_to_f32(x)
    # scales from exact rationals, codes from the brute-force nearest-value
    # search on the binary32 quotient (reading 3), neither through the
    # oracle's own arithmetic
    from fractions import Fraction
    for j in (0, 77):
        for c in range(2):
            col = xf[c * 128:(c + 1) * 128, j]
            amax = max(abs(Fraction(float(v))) for v in col)
            assert sT[j, c] == _f32_of_fraction(amax / 448)
            s = Fraction(float(sT[j, c]))
            want = [e4m3.encode_bruteforce(float(_f32_of_fraction(Fraction(float(v)) / s))) if v != 0
                    else (0x80 if np.signbit(v) else 0x00) for v in col]
            np.testing.assert_array_equal(qT[j, c * 128:(c + 1) * 128], np.array(want, np.uint8))
