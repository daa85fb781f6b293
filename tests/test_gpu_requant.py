"""GPU parity of the transposing re-quantisation (1x128 FP8 cache -> 128x1 tiles
with power-of-two scales), through the C ABI, with flags 0 and with the
power-of-two hint (both kernels, on every input): codes and scales bit-exact against
`oracle.quant.requant_128x1` on the same inputs. Inputs are the oracle's own
quantisation of seeded bf16 matrices (power-of-two and exact scales), uploaded
in the C ABI's chunk-major scale layout.
"""

import numpy as np
import pytest

import fp8_fine_grained_fp8bq_amd as fb
from oracle import quant
from tests.gpu_util import dev, host, log
from workloads import act

pytestmark = pytest.mark.gpu


def _gpu_requant(q, s_nat, ldq=None, lds=None, flags=0):
    """q uint8 [rows, cols], s_nat float32 [rows, cols/128] (oracle layout) -> GPU (qT, sT_nat)."""
    import torch
    rows, cols = q.shape
    ldq = ldq or cols
    lds = lds or rows
    qd = torch.zeros((rows, ldq), dtype=torch.uint8, device="cuda")
    qd[:, :cols] = dev(q)
    sd = torch.zeros((cols // 128, lds), dtype=torch.float32, device="cuda")
    sd[:, :rows] = dev(np.ascontiguousarray(s_nat.T))
    qt = torch.full((cols, rows), 0xAA, dtype=torch.uint8, device="cuda")
    st = torch.full((rows // 128, cols), -1.0, dtype=torch.float32, device="cuda")
    fb.fp8bq_requant_t_128x1(qd.data_ptr(), rows, cols, ldq, sd.data_ptr(), lds, qt.data_ptr(), rows,
                             st.data_ptr(), cols, flags, torch.cuda.current_stream().cuda_stream)
    return host(qt), np.ascontiguousarray(host(st).T)


def _check(q, s, name, **kw):
    # both kernels: flags 0 and the power-of-two hint, which must give the same
    # result whatever the scales are
    eqt, est = quant.requant_128x1(q, s)
    for flags in (0, fb.SCALE_POW2):
        log(f"[requant] {name}: {q.shape}, flags {flags:#x}")
        qt, st = _gpu_requant(q, s, flags=flags, **kw)
        np.testing.assert_array_equal(st.view(np.uint32), est.view(np.uint32), err_msg=f"{name}, flags {flags}: scales")
        np.testing.assert_array_equal(qt, eqt, err_msg=f"{name}, flags {flags}: codes")


@pytest.mark.parametrize("mode", ["pow2", "exact"])
@pytest.mark.parametrize("rows,cols,seed,kw", [
    (128, 128, 31, {}),
    (256, 384, 32, dict(outlier_p=0.01, outlier_mult=100.0)),
    (384, 256, 33, dict(dist="student_t3")),
    (256, 256, 34, dict(std=1e-30)),
    (512, 128, 35, dict(std=1e30)),
])
def test_requant_matches_oracle(mode, rows, cols, seed, kw):
    x = act(seed, rows, cols, **kw)
    q, s = quant.quant_act_1x128(x, mode)
    _check(q, s, f"{mode} seed {seed}")


def test_binding_with_and_without_hint():
    # the Python binding, with and without the power-of-two hint, on a
    # power-of-two cache (chunk-major scales as the quantiser writes them)
    import torch
    x = act(41, 256, 384)
    q, s = quant.quant_act_1x128(x, "pow2")
    eqt, est = quant.requant_128x1(q, s)
    qd = dev(q)
    sd = dev(np.ascontiguousarray(s.T))
    for hint in (False, True):
        qt, st = fb.requant_t_128x1(qd, sd, pow2_scales=hint)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(qt), eqt, err_msg=f"hint {hint}: codes")
        np.testing.assert_array_equal(np.ascontiguousarray(host(st).T).view(np.uint32), est.view(np.uint32),
                                      err_msg=f"hint {hint}: scales")


def test_leading_dimensions_and_zero_blocks():
    x = act(36, 384, 256, outlier_p=0.005, outlier_mult=1000.0)
    q, s = quant.quant_act_1x128(x, "pow2")
    q[128:256] = 0                               # padded tokens: +0 codes, 2^-127 scales
    _check(q, s, "ld + zero block", ldq=272, lds=400)


def test_every_code_and_extreme_scales():
    # every E4M3 code (NaN excluded) in every column position, with row scales
    # spanning the E8M0 range, so the new scales hit the clamp at both ends
    rng = np.random.default_rng(37)
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    rows, cols = 256, 256
    q = codes[rng.integers(0, codes.size, (rows, cols))]
    k = rng.integers(-127, 128, (rows, cols // 128))
    k[:16] = 127
    k[16:32] = -127
    s = np.ldexp(np.float32(1.0), k.astype(np.int32)).astype(np.float32)
    _check(q, s, "all codes, scales 2^-127 .. 2^127")


def test_fast_path_scale_bounds():
    # the kernel forms x_hat in binary32 when all 128 row scales of a block are
    # 2^e with -117 <= e <= 118, else in float64: blocks at both bounds and just
    # past them, a block mixing the two bounds (its small rows far below the
    # column maxima), and one whose single out-of-range row sends it to float64
    rng = np.random.default_rng(40)
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    exps = [[-117], [-118], [118], [119], [-117, 118], [0] * 127 + [-118]]
    rows, cols = 128 * len(exps), 256
    q = codes[rng.integers(0, codes.size, (rows, cols))]
    q[::7, :] = 0x7E                              # +448 in every column of some rows
    k = np.zeros((rows, cols // 128), np.int32)
    for b, e in enumerate(exps):
        k[b * 128:(b + 1) * 128] = np.resize(np.array(e, np.int32), 128)[:, None]
    s = np.ldexp(np.float32(1.0), k).astype(np.float32)
    _check(q, s, "scales at the binary32 path's bounds")


def test_general_scales_rounding():
    # scales that are not powers of two: x_hat needs up to 28 bits, the new
    # codes come from one binary32 rounding of x_hat * 2^-k
    rng = np.random.default_rng(38)
    rows, cols = 256, 128
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    q = codes[rng.integers(0, codes.size, (rows, cols))]
    s = (rng.uniform(0.5, 2.0, (rows, 1)) * np.ldexp(1.0, rng.integers(-20, 20, (rows, 1)))).astype(np.float32)
    _check(q, s, "general scales")


def test_large_workload_sampled_blocks():
    # full size (16384 x 7168, the large activation) in one launch; 8 sampled
    # 128-row blocks hold the oracle's power-of-two quantisation of the
    # workload's rows, the other rows seeded random codes and scales; every
    # output tile of the sampled blocks is checked (an output tile depends on
    # one 128-row block of one column)
    from workloads import large_fprop
    cfg = large_fprop()
    rows, cols = cfg.x.shape
    rng = np.random.default_rng(39)
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    q = codes[rng.integers(0, codes.size, (rows, cols))]
    s = np.ldexp(np.float32(1.0), rng.integers(-20, 20, (rows, cols // 128)).astype(np.int32)).astype(np.float32)
    blocks = sorted(set(int(b) for b in rng.integers(0, rows // 128, 8)))
    for rb in blocks:
        qb, sb = quant.quant_act_1x128(cfg.x[rb * 128:(rb + 1) * 128], "pow2")
        q[rb * 128:(rb + 1) * 128], s[rb * 128:(rb + 1) * 128] = qb, sb
    expect = {rb: quant.requant_128x1(q[rb * 128:(rb + 1) * 128], s[rb * 128:(rb + 1) * 128]) for rb in blocks}
    for flags in (0, fb.SCALE_POW2):
        log(f"[requant] large {rows}x{cols}, blocks {blocks}, flags {flags:#x}")
        qt, st = _gpu_requant(q, s, flags=flags)
        for rb in blocks:
            eqt, est = expect[rb]
            np.testing.assert_array_equal(qt[:, rb * 128:(rb + 1) * 128], eqt)
            np.testing.assert_array_equal(st[:, rb].view(np.uint32), est[:, 0].view(np.uint32))
