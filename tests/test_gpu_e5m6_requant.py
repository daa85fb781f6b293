"""GPU parity of fp8bq_requant_e5m6_t_128x1 (E5M6 cache -> 128x1 FP8 tiles with
power-of-two scales, written transposed) through the C ABI: codes and scales
bit-exact against `oracle.e5m6.requant_128x1` on the same cache. The inputs are
the oracle's own cache of seeded bf16 matrices (oracle/e5m6.py, uploaded as
packed bytes and chunk-major scales), or crafted caches holding every finite
code under row scales across the whole range the cache writes."""

import numpy as np
import pytest

import fp8_fine_grained_fp8bq_amd as fb
from oracle import e5m6
from tests.gpu_util import dev, host, log
from workloads import act, f32_to_bf16_bits

pytestmark = pytest.mark.gpu

_FINITE = np.array([c for c in range(4096) if (c >> 6) & 31 != 31], np.uint16)


def _gpu(packed, s, cols, ldq=None, lds=None, ldqt=None, ldst=None):
    """packed uint8 [rows, 1.5 cols], s float32 [cols/128, rows] -> GPU (qt [cols, rows], st [rows/128, cols])."""
    import torch
    rows = packed.shape[0]
    nb = cols * 3 // 2
    ldq, lds, ldqt, ldst = ldq or nb, lds or rows, ldqt or rows, ldst or cols
    qd = torch.zeros((rows, ldq), dtype=torch.uint8, device="cuda")
    qd[:, :nb] = dev(np.ascontiguousarray(packed))
    sd = torch.zeros((cols // 128, lds), dtype=torch.float32, device="cuda")
    sd[:, :rows] = dev(np.ascontiguousarray(s))
    qt = torch.full((cols, ldqt), 0xAA, dtype=torch.uint8, device="cuda")
    st = torch.full((rows // 128, ldst), -1.0, dtype=torch.float32, device="cuda")
    fb.fp8bq_requant_e5m6_t_128x1(qd.data_ptr(), rows, cols, ldq, sd.data_ptr(), lds, qt.data_ptr(), ldqt,
                                  st.data_ptr(), ldst, torch.cuda.current_stream().cuda_stream)
    qth, sth = host(qt), host(st)
    assert np.all(qth[:, rows:] == 0xAA) and np.all(sth[:, cols:] == -1.0), "wrote past the outputs"
    return qth[:, :rows], sth[:, :cols]


def _check(packed, s, cols, name, **kw):
    log(f"[requant e5m6] {name}: rows={packed.shape[0]} cols={cols} {kw}")
    qt, st = _gpu(packed, s, cols, **kw)
    eqt, est = e5m6.requant_128x1(packed, s, cols)
    np.testing.assert_array_equal(st.view(np.uint32), est.view(np.uint32), err_msg=f"{name}: scales")
    np.testing.assert_array_equal(qt, eqt, err_msg=f"{name}: codes")


@pytest.mark.parametrize("rows,cols,seed,kw", [
    (128, 128, 81, {}),
    (256, 384, 82, dict(outlier_p=0.01, outlier_mult=100.0)),
    (384, 256, 83, dict(dist="student_t3")),
    (256, 1152, 84, dict(std=1e-30, outlier_p=0.002, outlier_mult=1e4)),
    (512, 128, 85, dict(std=1e30)),
])
def test_cache_of_seeded_activations(rows, cols, seed, kw):
    x = act(seed, rows, cols, **kw)
    packed, s = e5m6.cache_1x128(x)
    _check(packed, s, cols, f"seed {seed}")


def _crafted(seed, rows, cols, klo=-127, khi=113):
    rng = np.random.default_rng(seed)
    codes = _FINITE[rng.integers(0, _FINITE.size, (rows, cols))]
    k = rng.integers(klo, khi + 1, (cols // 128, rows))
    return e5m6.pack(codes), np.ldexp(np.float32(1.0), k.astype(np.int32)).astype(np.float32)


def test_every_code_under_scales_across_the_range():
    # columns mix rows whose values lie up to 240 binades apart: most of a
    # column encodes to signed zeros, the column maxima reach 2^128
    packed, s = _crafted(86, 512, 256)
    _check(packed, s, 256, "all codes, scales 2^-127 .. 2^113")


@pytest.mark.parametrize("klo,khi", [(-127, -100), (100, 113), (-3, 3)])
def test_every_code_under_narrow_scale_bands(klo, khi):
    # clamp at 2^-127 (tiny columns), the top of the range, and ordinary scales
    packed, s = _crafted(87 + abs(klo), 256, 384, klo, khi)
    _check(packed, s, 384, f"all codes, scales 2^{klo} .. 2^{khi}")


def test_edge_rows():
    x = act(90, 256, 256, outlier_p=0).copy()
    x[0] = 0                                                   # all +0: cache scale 2^-127
    x[1] = 0x8000                                              # all -0
    x[2] = 0xFF7F                                              # bf16 -max: cached as -2^128
    x[3, :128] = 0x7F7F                                        # +max
    x[4] = f32_to_bf16_bits(np.ldexp(np.arange(256, dtype=np.float32) - 128, -140))   # bf16 subnormals
    x[5] = f32_to_bf16_bits(-np.ldexp(np.ones(256, np.float32), -130))
    x[128:256] = 0                                             # second row block: all-zero tiles
    x[130, 7] = 0x8001                                         # ... but one tiny negative value
    packed, s = e5m6.cache_1x128(x)
    _check(packed, s, 256, "edge rows")


def test_leading_dimensions():
    x = act(91, 256, 384, dist="student_t3", outlier_p=0.01, outlier_mult=30)
    packed, s = e5m6.cache_1x128(x)
    _check(packed, s, 384, "padded", ldq=640, lds=300, ldqt=272, ldst=400)


def test_large_workload_sampled_blocks():
    # full size (the large activation, 16384 x 7168) in one launch: crafted
    # codes and scales everywhere, with 6 sampled 128-row blocks holding the
    # oracle's cache of the workload's rows; every output tile of the sampled
    # blocks is checked (an output tile depends on one 128-row block of one
    # 128-column chunk)
    from workloads import large_fprop
    cfg = large_fprop()
    rows, cols = cfg.x.shape
    rng = np.random.default_rng(92)
    codes = rng.integers(0, 4096, (rows, cols), dtype=np.uint16)
    codes[(codes >> 6) & 31 == 31] ^= 1 << 6               # exponent field 31 -> 30: finite codes only
    packed = e5m6.pack(codes)
    del codes
    s = np.ldexp(np.float32(1.0), rng.integers(-20, 20, (cols // 128, rows)).astype(np.int32)).astype(np.float32)
    blocks = sorted(set(int(b) for b in rng.integers(0, rows // 128, 6)))
    for rb in blocks:
        pb, sb = e5m6.cache_1x128(cfg.x[rb * 128:(rb + 1) * 128])
        packed[rb * 128:(rb + 1) * 128], s[:, rb * 128:(rb + 1) * 128] = pb, sb
    log(f"[requant e5m6] large {rows}x{cols}, blocks {blocks}")
    qt, st = _gpu(packed, s, cols)
    for rb in blocks + [rows // 128 - 1]:
        sl = slice(rb * 128, (rb + 1) * 128)
        eqt, est = e5m6.requant_128x1(packed[sl], np.ascontiguousarray(s[:, sl]), cols)
        np.testing.assert_array_equal(qt[:, sl], eqt, err_msg=f"block {rb}: codes")
        np.testing.assert_array_equal(st[rb].view(np.uint32), est[0].view(np.uint32), err_msg=f"block {rb}: scales")
