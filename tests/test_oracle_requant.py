"""Pins of the oracle's transposing re-quantisation (1x128 FP8 cache -> 128x1).

The report (section 3.5.2, "support for transposed GEMM") describes the step
(read, dequantise, transpose, re-quantise into 128x1 tiles); section 3.3.3 gives
these activations power-of-two scales so the conversion adds no error of its
own. The pins check the oracle against things fixed independently of its code:
the already-pinned 128x1 quantiser where the two must agree, exact
reconstruction where the mathematics says it is exact, the error bound of two
successive roundings, and a per-element brute force with exact fractions. Each
planted mistake at the end fails at least one pin.
"""

from fractions import Fraction

import numpy as np
import pytest

from oracle import e4m3, quant
from workloads import act, f32_to_bf16_bits


def _cache(seed, rows=256, cols=384, mode="pow2", **kw):
    kw.setdefault("outlier_p", 0.01)
    kw.setdefault("outlier_mult", 100.0)
    x = act(seed, rows, cols, **kw)
    q, s = quant.quant_act_1x128(x, mode)
    return x, q, s


CASES = [dict(seed=21), dict(seed=22, dist="student_t3", outlier_p=0.0), dict(seed=23, std=1e-30, outlier_p=0.0),
         dict(seed=24, rows=128, cols=128)]


@pytest.mark.parametrize("case", CASES)
def test_equals_128x1_quantiser_of_the_dequantised_values(case):
    # with power-of-two input scales every x_hat = dec(q) * 2^k has four
    # significant bits; where it also fits bf16 the result must be the (pinned)
    # 128x1 power-of-two quantisation of x_hat itself
    _, q, s = _cache(**case)
    xh = quant.dequant_act(q, s)
    b = f32_to_bf16_bits(xh.astype(np.float32))
    assert np.array_equal(quant.bf16_bits_to_f32(b).astype(np.float64), xh), "x_hat not bf16-exact"
    qt, st = quant.requant_128x1(q, s)
    qt2, st2 = quant.quant_act_128x1(b, "pow2")
    np.testing.assert_array_equal(st, st2)
    np.testing.assert_array_equal(qt, qt2)


def _k(s):
    return np.log2(s.astype(np.float64)).astype(np.int64)


@pytest.mark.parametrize("case", CASES[:3])
def test_exact_where_the_row_scale_is_not_below_the_column_scale(case):
    _, q, s = _cache(**case)
    xh = quant.dequant_act(q, s)                                   # [rows, cols]
    qt, st = quant.requant_128x1(q, s)
    rec = e4m3.decode(qt) * np.repeat(st.astype(np.float64), 128, 1)   # [cols, rows]
    k1 = np.repeat(_k(s), 128, 1)                                  # [rows, cols]
    k2 = np.repeat(_k(st), 128, 1).T                               # [rows, cols]
    exact = k1 >= k2
    assert exact.mean() > 0.3
    np.testing.assert_array_equal(rec.T[exact], xh[exact])


@pytest.mark.parametrize("case", CASES[:3])
def test_group_absmax_reconstructs_exactly_in_the_top_binade(case):
    _, q, s = _cache(**case)
    xh = quant.dequant_act(q, s)
    qt, st = quant.requant_128x1(q, s)
    g = np.abs(xh.T).reshape(qt.shape[0], -1, 128)
    am = g.max(-1, keepdims=True)
    hit = (g == am) & (am > 0)
    codes = (qt.reshape(g.shape) & 0x7F)[hit]
    assert codes.min() >= 0x76 and codes.max() <= 0x7E              # (224, 448] after scaling
    rec = e4m3.decode(qt).reshape(g.shape) * st.astype(np.float64)[..., None]
    np.testing.assert_array_equal(np.abs(rec)[hit], g[hit])


@pytest.mark.parametrize("mode", ["pow2", "exact"])
def test_two_roundings_error_bound(mode):
    x, q, s = _cache(25, mode=mode)
    xf = quant.bf16_bits_to_f32(x).astype(np.float64)
    xh = quant.dequant_act(q, s)
    qt, st = quant.requant_128x1(q, s)
    rec = (e4m3.decode(qt) * np.repeat(st.astype(np.float64), 128, 1)).T
    s1 = np.repeat(s.astype(np.float64), 128, 1)
    s2 = np.repeat(st.astype(np.float64), 128, 1).T
    b1 = np.maximum(2.0 ** -4 * np.abs(xf), 2.0 ** -10 * s1)
    b2 = np.maximum(2.0 ** -4 * np.abs(xh), 2.0 ** -10 * s2)
    assert np.all(np.abs(xh - xf) <= b1)
    assert np.all(np.abs(rec - xh) <= b2)
    assert np.all(np.abs(rec - xf) <= b1 + b2)


def test_general_input_scales_against_exact_fractions():
    # exact (absmax / 448) input scales: x_hat has up to 28 significant bits;
    # the code is E4M3 of the binary32 rounding of x_hat * 2^-k, found here
    # element by element with fractions and the exhaustive nearest-value encoder
    _, q, s = _cache(26, rows=128, cols=128, mode="exact")
    qt, st = quant.requant_128x1(q, s)
    dec = e4m3.decode(q)
    for c in range(0, 128, 7):
        col = [Fraction(float(dec[r, c])) * Fraction(float(s[r, 0])) for r in range(128)]
        amax = max(abs(v) for v in col)
        k = 0
        while amax > 448 * Fraction(2) ** k:
            k += 1
        while k > -127 and amax <= 448 * Fraction(2) ** (k - 1):
            k -= 1
        assert float(st[c, 0]) == 2.0 ** k
        v32 = np.array([float(v / Fraction(2) ** k) for v in col], dtype=np.float64).astype(np.float32)
        np.testing.assert_array_equal(qt[c], e4m3.encode_bruteforce_vec(v32.astype(np.float64)))


def test_zero_groups_and_padding_rows():
    _, q, s = _cache(27, rows=256, cols=128)
    q[128:] = 0                      # a padded block of tokens: codes +0
    qt, st = quant.requant_128x1(q, s)
    assert np.all(qt[:, 128:] == 0)
    assert np.all(st[:, 1] == np.float32(2.0 ** -127))


# --- planted mistakes ---------------------------------------------------------

def _mutant(kind):
    good = quant.requant_128x1

    def f(q, s):
        rows, cols = q.shape
        xh = quant.dequant_act(q, s)
        if kind == "no_input_scale":        # codes taken as values
            return good(q, np.ones_like(s))
        if kind == "row_groups":            # 1x128 groups of x_hat, then transposed
            g = xh.reshape(rows, cols // 128, 128)
            k = quant.pow2_exponent(np.abs(g).max(-1))
            qq = e4m3.encode((g * np.ldexp(1.0, -k)[..., None]).astype(np.float32)).reshape(rows, cols)
            st = np.ldexp(np.float32(1.0), k.T[: cols // 128 * 0 + cols // 128].astype(np.int32))
            return np.ascontiguousarray(qq.T), np.resize(st, (cols, rows // 128)).astype(np.float32)
        if kind == "exponent_one_low":      # floor instead of ceiling: saturates
            g = np.ascontiguousarray(xh.T).reshape(cols, rows // 128, 128)
            k = quant.pow2_exponent(np.abs(g).max(-1)) - 1
            v = np.minimum(np.abs(g * np.ldexp(1.0, -k)[..., None]), 448.0) * np.sign(g)
            return e4m3.encode(v.astype(np.float32)).reshape(cols, rows), np.ldexp(np.float32(1.0), k.astype(np.int32))
        if kind == "no_fl32":               # one rounding straight to E4M3
            g = np.ascontiguousarray(xh.T).reshape(cols, rows // 128, 128)
            k = quant.pow2_exponent(np.abs(g).max(-1))
            return e4m3.encode(g * np.ldexp(1.0, -k)[..., None]).reshape(cols, rows), \
                np.ldexp(np.float32(1.0), k.astype(np.int32))
        raise AssertionError(kind)
    return f


@pytest.mark.parametrize("kind", ["no_input_scale", "row_groups", "exponent_one_low", "no_fl32"])
def test_planted_mistakes_fail_a_pin(kind, monkeypatch):
    monkeypatch.setattr(quant, "requant_128x1", _mutant(kind))
    pins = [lambda: test_equals_128x1_quantiser_of_the_dequantised_values(CASES[0]),
            lambda: test_exact_where_the_row_scale_is_not_below_the_column_scale(CASES[0]),
            lambda: test_group_absmax_reconstructs_exactly_in_the_top_binade(CASES[0]),
            lambda: test_two_roundings_error_bound("pow2"),
            test_general_input_scales_against_exact_fractions]
    failed = 0
    for pin in pins:
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed > 0
