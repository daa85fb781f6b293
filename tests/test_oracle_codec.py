"""Pins of the oracle's E4M3 codec against facts the pages and the format fix.

* The decode table is checked against closed forms of the 1/4/3 bit split that
  the parallelism-summary page's format table gives, and against that page's
  count of e4m3 values inside [1, 2] (golden fixture).
* The round-to-nearest-even encoder is checked against an exhaustive nearest-
  value search on every bf16 bit pattern (times powers of two), on every
  rounding midpoint and its fp32 neighbours, and on hand-derived cases.
"""

import json
import math
import os

import numpy as np
import pytest

from oracle import e4m3

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_decode_table_closed_form():
    vals = [e4m3.decode_scalar(c) for c in range(256)]
    nans = [c for c, v in enumerate(vals) if math.isnan(v)]
    assert nans == [0x7F, 0xFF]
    finite = [v for v in vals if not math.isnan(v)]
    assert len(finite) == 254
    assert len(set(finite)) == 253                 # +0 and -0 coincide
    assert max(finite) == 448.0 and vals[0x7E] == 448.0 and vals[0xFE] == -448.0
    assert vals[0x01] == 2.0 ** -9                 # smallest subnormal
    assert vals[0x08] == 2.0 ** -6                 # smallest normal
    assert vals[0x07] == 7 * 2.0 ** -9             # largest subnormal
    assert sorted(v for v in finite if v >= 256) == [256.0 + 32 * i for i in range(7)]
    # positive codes 0..0x7E are strictly increasing, and the negative half mirrors them
    pos = vals[:0x7F]
    assert all(a < b for a, b in zip(pos, pos[1:]))
    assert all(vals[c | 0x80] == -vals[c] for c in range(0x7F))
    # spacing within binade [2^e, 2^(e+1)) is 2^(e-3); subnormal spacing 2^-9
    for c in range(0x08, 0x7E):
        v, w = vals[c], vals[c + 1]
        e = math.floor(math.log2(v))
        assert w - v == 2.0 ** (e - 3)
    for c in range(0, 8):
        assert vals[c + 1] - vals[c] == 2.0 ** -9


def _e5m2_decode(code):
    # test-only decoder of the 1/5/2 format (bias 15), for the page's resolution count
    e = (code >> 2) & 0x1F
    m = code & 0x3
    if e == 0x1F:
        return math.nan
    mag = (m / 4.0) * 2.0 ** -14 if e == 0 else (1 + m / 4.0) * 2.0 ** (e - 15)
    return -mag if code & 0x80 else mag


def test_page_resolution_counts():
    gold = json.load(open(os.path.join(GOLDEN, "format_resolution.json")))
    inside = [v for v in (e4m3.decode_scalar(c) for c in range(256)) if 1.0 < v < 2.0]
    assert len(inside) == gold["e4m3"]["values_strictly_inside_1_2"] == 7
    inside52 = [v for v in (_e5m2_decode(c) for c in range(256)) if 1.0 < v < 2.0]
    assert len(inside52) == gold["e5m2"]["values_strictly_inside_1_2"] == 3
    assert (e4m3.EXP_BIAS, e4m3.MANT_BITS) == (2 ** (gold["e4m3"]["exponent_bits"] - 1) - 1,
                                               gold["e4m3"]["mantissa_bits"])


HAND_CASES = [
    # (value, code, why)
    (0.0, 0x00, "zero"),
    (-0.0, 0x80, "negative zero keeps its sign"),
    (1.0, 0x38, "1 = 2^0: exponent field 7, mantissa 0"),
    (-2.0, 0xC0, "-2: sign, exponent field 8"),
    (1.0625, 0x38, "tie between 1 and 1.125 goes to the even mantissa (1)"),
    (1.1875, 0x3A, "tie between 1.125 and 1.25 goes to 1.25 (mantissa 010)"),
    (1.0625 + 2.0 ** -23, 0x39, "just above the tie rounds up"),
    (2.0 ** -10, 0x00, "half the smallest subnormal ties to zero (even)"),
    (-(2.0 ** -10), 0x80, "... and keeps the sign"),
    (3 * 2.0 ** -10, 0x02, "tie between 2^-9 and 2^-8 goes to 2^-8 (code 2, even)"),
    (7.5 * 2.0 ** -9, 0x08, "tie between the largest subnormal and 2^-6 goes to 2^-6 (even)"),
    (432.0, 0x7E, "tie between 416 and 448 goes to 448 (mantissa 110)"),
    (400.0, 0x7C, "tie between 384 and 416 goes to 384 (mantissa 100)"),
    (448.0, 0x7E, "largest finite"),
    (463.99, 0x7E, "below the 448/480 midpoint"),
    (464.0, 0x7E, "beyond the range saturates"),
    (1e30, 0x7E, "saturates"),
    (-1e30, 0xFE, "saturates with sign"),
    (-1e-30, 0x80, "negative underflow gives -0"),
    (0.30078125, 0x2A, "bf16(0.3): 9.625 quanta of 2^-5 -> 10 -> 1.25 * 2^-2"),
]


@pytest.mark.parametrize("v,code,why", HAND_CASES)
def test_hand_derived_codes(v, code, why):
    assert e4m3.encode_scalar(v) == code, why
    assert e4m3.encode(np.array([v]))[0] == code, why
    assert e4m3.encode_bruteforce(v) == code, why


def _all_finite_bf16_as_f32():
    bits = np.arange(65536, dtype=np.uint32) << np.uint32(16)
    f = bits.view(np.float32)
    return f[np.isfinite(f)]


def test_encode_vs_bruteforce_all_bf16_times_powers_of_two():
    base = _all_finite_bf16_as_f32().astype(np.float64)
    # only the part that lands near the E4M3 range is interesting for scaling
    near = base[(np.abs(base) < 2.0 ** 12) & (np.abs(base) > 2.0 ** -16) | (base == 0)]
    for j in (-3, 0, 1, 5):
        v = np.ldexp(near, j).astype(np.float32)
        np.testing.assert_array_equal(e4m3.encode(v), e4m3.encode_bruteforce_vec(v))
    # whole bf16 set once (covers huge / tiny magnitudes and every sign)
    np.testing.assert_array_equal(e4m3.encode(base), e4m3.encode_bruteforce_vec(base))


def _midpoints():
    vals = sorted(set(v for v in e4m3.DECODE_TABLE if not math.isnan(v) and v >= 0))
    mids = [(a + b) / 2 for a, b in zip(vals, vals[1:])] + [464.0]
    out = []
    for m in mids:
        m32 = np.float32(m)
        assert float(m32) == m            # every midpoint is an fp32 value
        out += [np.nextafter(m32, np.float32(0)), m32, np.nextafter(m32, np.float32(np.inf))]
    out = np.array(out, dtype=np.float32)
    return np.concatenate([out, -out])


def test_encode_midpoints_and_neighbours():
    v = _midpoints()
    np.testing.assert_array_equal(e4m3.encode(v), e4m3.encode_bruteforce_vec(v))


def test_scalar_matches_vectorised():
    rng = np.random.default_rng(11)
    bits = rng.integers(0, 2 ** 32, size=40000, dtype=np.uint64).astype(np.uint32)
    # bias towards the E4M3 range: exponents 100..140
    bits = (bits & np.uint32(0x807FFFFF)) | ((np.uint32(100) + (bits >> np.uint32(23)) % np.uint32(41)) << np.uint32(23))
    v = np.concatenate([bits.view(np.float32), _midpoints(), _all_finite_bf16_as_f32()[::7]])
    vec = e4m3.encode(v)
    sca = np.array([e4m3.encode_scalar(float(x)) for x in v], dtype=np.uint8)
    np.testing.assert_array_equal(vec, sca)


def test_random_fp32_vs_bruteforce():
    rng = np.random.default_rng(12)
    bits = rng.integers(0, 2 ** 32, size=200000, dtype=np.uint64).astype(np.uint32)
    bits = (bits & np.uint32(0x807FFFFF)) | ((np.uint32(110) + (bits >> np.uint32(23)) % np.uint32(28)) << np.uint32(23))
    v = bits.view(np.float32)
    np.testing.assert_array_equal(e4m3.encode(v), e4m3.encode_bruteforce_vec(v))


def test_decode_encode_roundtrip():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    np.testing.assert_array_equal(e4m3.encode(e4m3.decode(codes)), codes)
