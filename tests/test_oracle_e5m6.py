"""Pins of the oracle's E5M6 activation-cache codec (oracle/e5m6.py) against
what the format's definition and the mathematics fix, by routes other than the
encoder itself: numpy's IEEE binary16 for the value set, closed forms, an
exhaustive nearest-value search with exact rational distances, a hand-packed
example and the round-trip error bound."""

import math

import numpy as np
import pytest

from oracle import e5m6, quant
from workloads import act, f32_to_bf16_bits


def test_value_set_is_binary16_without_its_four_low_mantissa_bits():
    # the same exponent layout as IEEE binary16: code c has the value of the
    # binary16 bit pattern c << 4 (numpy's float16 decodes those)
    codes = np.arange(4096, dtype=np.uint16)
    h = (codes << np.uint16(4)).view(np.float16).astype(np.float64)
    fin = np.isfinite(h)
    np.testing.assert_array_equal(e5m6.DECODE_TABLE[fin], h[fin])
    assert np.array_equal(np.isinf(e5m6.DECODE_TABLE), np.isinf(h))
    assert np.array_equal(np.isnan(e5m6.DECODE_TABLE), np.isnan(h))


def test_closed_forms():
    v = e5m6.DECODE_TABLE
    pos = v[np.isfinite(v) & (v > 0)]
    assert pos.size == 30 * 64 + 63                  # 30 binades of 64 values + 63 subnormals
    assert pos.max() == 65024.0 == (2 - 2.0 ** -6) * 2.0 ** 15
    assert pos.min() == 2.0 ** -20
    assert np.sum((pos >= 1) & (pos < 2)) == 64      # 6 mantissa bits
    assert e5m6.decode_scalar(0x800) == 0.0 and math.copysign(1.0, e5m6.decode_scalar(0x800)) < 0


def _bf16_all_finite_in_range():
    bits = np.arange(65536, dtype=np.uint32)
    with np.errstate(invalid="ignore"):
        f = (bits << 16).view(np.float32).astype(np.float64)
    ok = np.isfinite(f) & (np.abs(f) <= e5m6.FMAX)
    return f[ok]


@pytest.mark.parametrize("j", [0, -20, 15, -133])
def test_vector_encoder_equals_scalar_encoder_on_every_bf16(j):
    # two implementations of the rounding rule (float64 bit arithmetic against
    # exact fractions) on every bf16 value, shifted into the subnormal and top
    # ranges
    v = np.ldexp(_bf16_all_finite_in_range(), j)
    v = v[np.abs(v) <= e5m6.FMAX]
    got = e5m6.encode(v)
    want = np.array([e5m6.encode_scalar(x) for x in v], dtype=np.uint16)
    np.testing.assert_array_equal(got, want)


def test_encoder_against_bruteforce_sample():
    rng = np.random.default_rng(61)
    v = np.concatenate([
        rng.standard_normal(300) * 10.0 ** rng.integers(-7, 5, 300),
        rng.uniform(-65024, 65024, 50),
        np.ldexp(rng.uniform(-1, 1, 50), -18),       # subnormal range
        [0.0, -0.0, 65024.0, -65024.0, 2.0 ** -20, 2.0 ** -21, 3 * 2.0 ** -22, 2.0 ** -14],
    ])
    got = e5m6.encode(v)
    want = np.array([e5m6.encode_bruteforce(x) for x in v], dtype=np.uint16)
    np.testing.assert_array_equal(got, want)


def test_every_midpoint_rounds_to_the_even_neighbour():
    pos = np.sort(e5m6.DECODE_TABLE[np.isfinite(e5m6.DECODE_TABLE) & (e5m6.DECODE_TABLE >= 0)])
    pos = np.unique(pos)
    lo, hi = pos[:-1], pos[1:]
    mid = (lo + hi) / 2                       # exact in float64
    c_lo, c_hi = e5m6.encode(lo), e5m6.encode(hi)
    got = e5m6.encode(mid)
    even = np.where((c_lo & 1) == 0, c_lo, c_hi)
    np.testing.assert_array_equal(got, even)
    np.testing.assert_array_equal(e5m6.encode(np.nextafter(mid, 0)), c_lo)
    np.testing.assert_array_equal(e5m6.encode(np.nextafter(mid, np.inf)), c_hi)
    # and the same on the negative side, sign bit set
    np.testing.assert_array_equal(e5m6.encode(-mid), even | 0x800)


def test_packing_hand_example_and_round_trip():
    codes = np.array([[0x123, 0xABC, 0x000, 0xFFF]], dtype=np.uint16)
    p = e5m6.pack(codes)
    # 0x123 | 0xABC << 12 = 0xABC123 -> 23 C1 AB; 0x000 | 0xFFF << 12 -> 00 F0 FF
    assert p.tolist() == [[0x23, 0xC1, 0xAB, 0x00, 0xF0, 0xFF]]
    rng = np.random.default_rng(62)
    c = rng.integers(0, 4096, (5, 256)).astype(np.uint16)
    np.testing.assert_array_equal(e5m6.unpack(e5m6.pack(c), 256), c)


def test_scale_rule():
    # absmax exactly 65024 * 2^j gives k = j; one ulp above gives j + 1
    for j in (-20, -1, 0, 3):
        a = 65024.0 * 2.0 ** j
        assert e5m6.pow2_exponent(np.array([a]))[0] == j
        assert e5m6.pow2_exponent(np.array([np.nextafter(a, np.inf)]))[0] == j + 1
    assert e5m6.pow2_exponent(np.array([0.0]))[0] == -127
    assert e5m6.pow2_exponent(np.array([1e-45]))[0] == -127      # clamped


def test_cache_round_trip_bound_and_absmax():
    x = act(63, 64, 1024, dist="student_t3", outlier_p=0.01, outlier_mult=100)
    packed, s = e5m6.cache_1x128(x)
    assert packed.shape == (64, 1536) and s.shape == (8, 64)
    xh = e5m6.uncache_1x128(packed, s, 1024)
    xf = quant.bf16_bits_to_f32(x).astype(np.float64)
    srow = np.repeat(s.T.astype(np.float64), 128, axis=1)
    # half a unit in the last place of a 6-bit mantissa, or of the subnormal quantum
    bound = np.maximum(2.0 ** -7 * np.abs(xf), 2.0 ** -21 * srow)
    assert np.all(np.abs(xh - xf) <= bound)
    # every tile's absmax lands in the top binade of the format (scaled value in (32512, 65024])
    xg = np.abs(xf).reshape(64, 8, 128).max(-1)
    scaled = xg / s.T
    assert np.all((scaled > 32512.0) & (scaled <= 65024.0))


def test_cache_of_exact_values_is_lossless():
    # values with at most 7 significant bits are cached exactly (power-of-two
    # scales do not move the mantissa)
    rng = np.random.default_rng(64)
    m = rng.integers(64, 128, (16, 256)) * rng.choice([-1, 1], (16, 256))
    e = rng.integers(-15, 10, (16, 256))
    xf = np.ldexp(m.astype(np.float64), e - 6)
    # 25 binades: every value stays in the normal range below its tile's scaled absmax
    x = f32_to_bf16_bits(xf.astype(np.float32))
    packed, s = e5m6.cache_1x128(x)
    np.testing.assert_array_equal(e5m6.uncache_1x128(packed, s, 256), quant.bf16_bits_to_f32(x).astype(np.float64))


def test_requant_equals_128x1_pow2_quantisation_of_the_cached_values():
    # the cached values have at most 7 significant bits and lie in bf16's normal
    # range here, so they are exact bf16 values; the 128x1 power-of-two FP8
    # quantiser of those (a separately pinned function) must give the same codes
    x = act(65, 256, 384, dist="student_t3", outlier_p=0.01, outlier_mult=50)
    packed, s = e5m6.cache_1x128(x)
    qt, st = e5m6.requant_128x1(packed, s, 384)
    xh = e5m6.uncache_1x128(packed, s, 384)
    xb = f32_to_bf16_bits(xh.astype(np.float32))
    np.testing.assert_array_equal(quant.bf16_bits_to_f32(xb).astype(np.float64), xh)    # exact in bf16
    qt2, st2 = quant.quant_act_128x1(xb, scale_mode="pow2")
    np.testing.assert_array_equal(qt, qt2)
    np.testing.assert_array_equal(st.T, st2)


def test_requant_hand_worked_column():
    # one column whose cached values are 3, -1.5, 0.25 and zeros: absmax 3 needs
    # k = -7 (448 * 2^-8 = 1.75 < 3 <= 3.5), so the codes are E4M3(384) = 0x7C,
    # E4M3(-192) = 0xF4 and E4M3(32) = 0x60 (exponent field 5 + 7 = 12, mantissa 0)
    x = np.zeros((128, 128), np.float32)
    x[0, 5], x[1, 5], x[2, 5] = 3.0, -1.5, 0.25
    x[:, 0] = 1.0                                  # keeps the row tiles' scales ordinary
    packed, s = e5m6.cache_1x128(f32_to_bf16_bits(x))
    qt, st = e5m6.requant_128x1(packed, s, 128)
    assert st[0, 5] == 2.0 ** -7
    assert list(qt[5, :3]) == [0x7C, 0xF4, 0x60] and np.all(qt[5, 3:] == 0)
