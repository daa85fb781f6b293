"""Planted mistakes: each mutant of the oracle must fail at least one pin.

A mutant is a plausible slip (truncating instead of rounding, ties away from
zero, a lost sign, a wrong F_max, a dropped scale, an off-by-one chunk index,
a transposed weight block grid). Each is swapped into the oracle with
monkeypatch, on the CPU, and the pins from the other test modules are run
against it; the test passes only if some pin fails.
"""

import numpy as np
import pytest

import oracle.e4m3 as e4m3
import oracle.gemm as gemm
import oracle.quant as quant
from tests import test_oracle_codec as codec_pins
from tests import test_oracle_gemm as gemm_pins
from tests import test_oracle_quant as quant_pins


def _fails(fn, *args):
    try:
        fn(*args)
    except AssertionError:
        return True
    except (ValueError, IndexError):
        return True
    return False


def _encode_with(rounder, keep_zero_sign=True):
    good = e4m3.encode

    def enc(v):
        v = np.asarray(v, dtype=np.float64)
        a = np.abs(v)
        out = np.zeros(v.shape, np.int64)
        sub = a < 2.0 ** -6
        out[sub] = rounder(a[sub] / 2.0 ** -9).astype(np.int64)
        nor = (~sub) & (a < 448)
        _, e2 = np.frexp(a[nor])
        e = e2.astype(np.int64) - 1
        n = rounder(a[nor] / np.ldexp(1.0, e - 3)).astype(np.int64)
        e = np.where(n == 16, e + 1, e)
        n = np.where(n == 16, 8, n)
        out[nor] = np.minimum(((e + 7) << 3) | (n - 8), 0x7E)
        out[a >= 448] = 0x7E
        sign = np.signbit(v) if keep_zero_sign else (v < 0)
        res = (out | np.where(sign & ((out != 0) | keep_zero_sign), 0x80, 0)).astype(np.uint8)
        return res
    return good, enc


CODEC_PINS = [
    (codec_pins.test_encode_midpoints_and_neighbours, ()),
    (codec_pins.test_encode_vs_bruteforce_all_bf16_times_powers_of_two, ()),
]


@pytest.mark.parametrize("name,rounder,zsign", [
    ("truncate", np.floor, True),
    ("ties away from zero", lambda t: np.floor(t + 0.5), True),
    ("round half up via ceil", lambda t: np.ceil(t - 0.5), True),
    ("loses the sign of zero", np.rint, False),
])
def test_codec_mutants_are_caught(monkeypatch, name, rounder, zsign):
    _, bad = _encode_with(rounder, zsign)
    monkeypatch.setattr(e4m3, "encode", bad)
    caught = any(_fails(f, *a) for f, a in CODEC_PINS)
    caught = caught or any(_fails(codec_pins.test_hand_derived_codes, v, c, w)
                           for v, c, w in codec_pins.HAND_CASES)
    assert caught, name


def test_wrong_fmax_is_caught(monkeypatch):
    monkeypatch.setattr(quant, "F_MAX", np.float32(447.0))
    assert _fails(quant_pins.test_hand_derived_tile)


def test_division_precision_reading_is_observable(monkeypatch):
    # computing x / s in float64 (no binary32 rounding of the quotient) is a different reading
    orig = quant._quant_groups

    def groups64(xg, scale_mode="exact"):
        amax = np.max(np.abs(xg), axis=-1)
        s = (amax.astype(np.float32) / quant.F_MAX).astype(np.float32)
        v = xg.astype(np.float64) / np.where(s == 0, 1, s)[..., None].astype(np.float64)
        q = e4m3.encode(v)
        return q, s
    monkeypatch.setattr(quant, "_quant_groups", groups64)
    # an input built so that x / s in binary64 sits just past a rounding midpoint while
    # the binary32 quotient lands exactly on it (checked against the real oracle)
    x = np.zeros((1, 128), np.float32)
    found = False
    rng = np.random.default_rng(0)
    for _ in range(4000):
        am = np.float32(rng.uniform(1, 2))
        am = np.frombuffer(np.array([am], np.float32).tobytes(), np.uint32)[0] & 0xFFFF0000
        am = np.array([am], np.uint32).view(np.float32)[0]
        s = np.float32(am) / np.float32(448)
        xs = (np.arange(1, 65536, dtype=np.uint32) << 16).view(np.float32)
        xs = xs[(np.abs(xs) < am) & np.isfinite(xs)]
        v32 = e4m3.encode((xs / s).astype(np.float32))
        v64 = e4m3.encode(xs.astype(np.float64) / np.float64(s))
        diff = np.nonzero(v32 != v64)[0]
        if diff.size:
            x[0, 0] = am
            x[0, 1] = xs[diff[0]]
            found = True
            break
    assert found
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    q_bad, _ = quant.quant_act_1x128(bits)
    monkeypatch.setattr(quant, "_quant_groups", orig)
    q_good, _ = quant.quant_act_1x128(bits)
    assert q_bad[0, 1] != q_good[0, 1]


def test_dropped_weight_scale_is_caught(monkeypatch):
    monkeypatch.setattr(gemm, "expand_block_scales",
                        lambda sw: np.ones((np.asarray(sw).shape[0] * 128, np.asarray(sw).shape[1]), np.float32))
    assert _fails(gemm_pins.test_uniform_scale_reduces_to_per_tensor_fp8_gemm)


def test_off_by_one_chunk_scale_is_caught(monkeypatch):
    orig = gemm.gemm_rowscaled

    def shifted(qa, sa, qb, sb, row_block=1024):
        return orig(qa, np.roll(sa, 1, axis=1), qb, sb, row_block)
    monkeypatch.setattr(gemm, "gemm_rowscaled", shifted)
    assert _fails(gemm_pins.test_tiny_shapes_against_fraction_triple_loop)


def test_untransposed_dgrad_weight_is_caught(monkeypatch):
    def bad_dgrad(qdy, sdy, qw, sw, row_block=1024):
        # forgets to transpose the weight's block-scale grid
        qwT = np.ascontiguousarray(np.asarray(qw).T)
        sw = np.asarray(sw)
        grid = np.resize(sw, (sw.shape[1], sw.shape[0]))
        return gemm.gemm_rowscaled(qdy, sdy, qwT, gemm.expand_block_scales(grid), row_block)
    monkeypatch.setattr(gemm, "dgrad", bad_dgrad)
    assert _fails(gemm_pins.test_dgrad_definition)


def test_transposed_block_grid_is_caught(monkeypatch):
    orig = quant.quant_w_128x128

    def bad(w_bits):
        q, s = orig(np.ascontiguousarray(np.asarray(w_bits).T))
        return np.ascontiguousarray(q.T), np.ascontiguousarray(s)   # scale grid left transposed
    monkeypatch.setattr(quant, "quant_w_128x128", bad)
    assert _fails(quant_pins.test_weight_block_scale_is_block_absmax)
