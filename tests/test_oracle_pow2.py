"""Pins of the oracle's power-of-two scale mode (scale_mode="pow2").

The report (section 3.3.3, "low-precision storage and communication") gives
some activations scaling factors that are integral powers of 2. Reading: s is
the smallest power of two with absmax / s <= 448, kept within the exponent
range [-127, 127] of an E8M0 scale byte; an all-zero group gets 2^-127. The
pins below check that reading against hand-worked values, against the exact
mode (already pinned on its own) where the two must agree, and against
invariants that a plausible slip (floor instead of ceiling, rounding the
logarithm, no clamp) breaks; each slip is planted at the end of this file.
"""

import numpy as np
import pytest

from oracle import e4m3, quant
from workloads import act, f32_to_bf16_bits

# amax -> k, each worked by hand from "smallest k with amax <= 448 * 2^k":
HAND = [
    (448.0, 0),            # 448 <= 448 * 2^0
    (450.0, 1),            # next bf16 above 448; 450 > 448, 450 <= 896
    (224.0, -1),           # 224 = 448 * 2^-1 exactly
    (225.0, 0),            # 225 > 224 = 448 * 2^-1
    (1.0, -8),             # 448 * 2^-9 = 0.875 < 1 <= 1.75 = 448 * 2^-8
    (0.875, -9),           # 0.875 = 448 * 2^-9 exactly
    (3.0e38, 120),         # 448 * 2^119 = 2.98e38 < 3e38 <= 5.96e38
    (2.0 ** -133, -127),   # the smallest bf16: k would be -141, clamped
    (0.0, -127),           # all-zero group
]


def test_hand_worked_exponents():
    a = np.array([h[0] for h in HAND], np.float32)
    assert quant.pow2_exponent(a).tolist() == [h[1] for h in HAND]


def _all_positive_bf16():
    bits = np.arange(1, 0x7F80, dtype=np.uint32) << 16
    return bits.view(np.float32)


def test_every_bf16_absmax_feasible_and_minimal():
    a = _all_positive_bf16().astype(np.float64)
    k = quant.pow2_exponent(a.astype(np.float32))
    s = np.ldexp(1.0, k)
    assert np.all(a <= 448.0 * s)                           # nothing saturates
    clamped = k == quant.K_MIN
    assert np.all(a[~clamped] > 448.0 * s[~clamped] / 2)    # no smaller power works
    assert np.all(a[clamped] <= 448.0 * 2.0 ** -127)
    assert k.min() >= -127 and k.max() <= 127


def _x(seed=5, rows=64, cols=512, **kw):
    kw.setdefault("outlier_p", 0.01)
    kw.setdefault("outlier_mult", 100.0)
    return act(seed, rows, cols, **kw)


def test_scales_are_e8m0_powers_of_two():
    for x in (_x(), _x(9, std=1e-39, outlier_p=0)):
        _, s = quant.quant_act_1x128(x, "pow2")
        bits = s.view(np.uint32)
        exp_field = (bits >> 23) & 0xFF
        mant = bits & 0x7FFFFF
        normal = exp_field > 0
        # normal powers of two have no mantissa; 2^-127 is the subnormal 0x00400000
        assert np.all(mant[normal] == 0)
        assert np.all(bits[~normal] == 0x00400000)
        k = np.log2(s.astype(np.float64))
        assert np.all(k == np.round(k))
        assert np.all(np.where(normal, exp_field, 0) == (k + 127))


def test_absmax_element_lands_in_the_top_binade():
    # amax / s lies in (224, 448] unless clamped, so the absmax element's code is
    # 0x76 (224, reached by rounding from just above it) .. 0x7E (448)
    for x in (_x(), _x(6, dist="student_t3", outlier_p=0)):
        q, s = quant.quant_act_1x128(x, "pow2")
        xf = quant.bf16_bits_to_f32(x).reshape(x.shape[0], -1, 128)
        qq = q.reshape(xf.shape)
        am = np.abs(xf).max(-1, keepdims=True)
        hit = (np.abs(xf) == am) & (am > 0)
        mag = qq[hit] & 0x7F
        assert mag.min() >= 0x76 and mag.max() <= 0x7E


def test_agrees_with_exact_mode_when_absmax_is_448_times_a_power_of_two():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((32, 256)).astype(np.float32)
    x = x / np.abs(x.reshape(32, 2, 128)).max(-1).repeat(128, 1)        # |x| <= 1, amax = 1
    x = x * (448.0 * np.ldexp(1.0, rng.integers(-20, 20, (32, 2))).repeat(128, 1))
    bits = f32_to_bf16_bits(x.astype(np.float32))
    xb = quant.bf16_bits_to_f32(bits).reshape(32, 2, 128)
    amax = np.abs(xb).max(-1)
    keep = np.log2(amax / 448.0) == np.round(np.log2(amax / 448.0))   # bf16 rounding kept 448*2^j
    assert keep.mean() > 0.9
    qe, se = quant.quant_act_1x128(bits)
    qp, sp = quant.quant_act_1x128(bits, "pow2")
    np.testing.assert_array_equal(sp[keep], se[keep])
    np.testing.assert_array_equal(qp.reshape(32, 2, 128)[keep], qe.reshape(32, 2, 128)[keep])


def test_dequantisation_error_bound():
    # one rounding of an exact quotient: |dec(q) s - x| <= max(2^-4 |x|, 2^-10 s)
    for x in (_x(), _x(8, dist="student_t3", outlier_p=0)):
        q, s = quant.quant_act_1x128(x, "pow2")
        xh = quant.dequant_act(q, s)
        xf = quant.bf16_bits_to_f32(x).astype(np.float64)
        sr = np.repeat(s.astype(np.float64), 128, 1)
        assert np.all(np.abs(xh - xf) <= np.maximum(2.0 ** -4 * np.abs(xf), 2.0 ** -10 * sr))


def test_codes_are_single_roundings_of_the_exact_quotient():
    x = _x(12, rows=16, cols=256)
    q, s = quant.quant_act_1x128(x, "pow2")
    xf = quant.bf16_bits_to_f32(x).astype(np.float64)
    v = xf / np.repeat(s.astype(np.float64), 128, 1)
    np.testing.assert_array_equal(q, e4m3.encode_bruteforce_vec(v).reshape(q.shape))


def test_weight_blocks_and_transposition():
    w = act(13, 256, 384, std=0.02)
    q, s = quant.quant_w_128x128(w, "pow2")
    qt, st = quant.quant_w_128x128(np.ascontiguousarray(w.T), "pow2")
    np.testing.assert_array_equal(qt, q.T)
    np.testing.assert_array_equal(st, s.T)
    assert np.all(np.log2(s.astype(np.float64)) == np.round(np.log2(s.astype(np.float64))))


# --- planted mistakes ---------------------------------------------------------

def _mutant_exponent(kind):
    good = quant.pow2_exponent

    def f(amax):
        a = np.asarray(amax, np.float64)
        pos = a > 0
        r = np.zeros(a.shape, np.int64)
        x = np.log2(np.where(pos, a, 1.0) / 448.0)
        if kind == "floor":
            r = np.floor(x).astype(np.int64)
        elif kind == "round":
            r = np.round(x).astype(np.int64)
        elif kind == "noclamp":
            r = good(amax)
            r = np.where(pos, np.ceil(x).astype(np.int64), -127)
            return r
        return np.where(pos, np.clip(r, -127, 127), -127)
    return f


@pytest.mark.parametrize("kind", ["floor", "round", "noclamp"])
def test_planted_exponent_mistakes_fail_a_pin(kind, monkeypatch):
    monkeypatch.setattr(quant, "pow2_exponent", _mutant_exponent(kind))
    pins = [test_hand_worked_exponents, test_every_bf16_absmax_feasible_and_minimal,
            test_absmax_element_lands_in_the_top_binade]
    failed = 0
    for pin in pins:
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed > 0
