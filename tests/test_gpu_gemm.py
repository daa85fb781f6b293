"""GPU parity of the block-scaled FP8 GEMMs (Fprop, Dgrad, Wgrad, grouped).

Operands are quantised on the GPU and checked bit-exact against the oracle's
quantisation first; the GEMM output is then accepted when the GPU's FP32
accumulation is within 2e-3 * sum_k |x_hat_k| |w_hat_k| of the oracle's, before
the final rounding to bf16 (for bf16 outputs every admissible fp32 value is
rounded to bf16 and the GPU's bf16 must fall inside; see gpu_util). A tighter
canary bracket (gpu_util.TIGHT) is asserted too: it bounds what gfx950's FP8 MFMA
(blocked, limited-precision summation inside each 128-product chunk) plus the
FP32 promotion deliver on these inputs, so a loss of accuracy shows there first.
"""

import numpy as np
import pytest

import fp8_fine_grained_fp8bq_amd as fb
from oracle import gemm as og
from oracle import quant as oq
from tests.gpu_util import (assert_no_poison, check_gemm_bf16, check_gemm_f32, dev_bf16, host,
                            host_bf16_bits, log, poisoned, tile_rows)
from workloads import act, backward_dy, dense_fprop, large_fprop, moe_fprop, tiny_fprop

pytestmark = pytest.mark.gpu

def _quant_pair_fprop(xbits, wbits, with_qt=False):
    xq, xs = fb.quant_act_1x128(dev_bf16(xbits))
    wq, ws, wqt = fb.quant_w_128x128(dev_bf16(wbits), transposed_copy=with_qt)
    return xq, xs, wq, ws, wqt


def _assert_ok(stats, name):
    log(f"  {name}: {stats}")
    assert stats["bad"] == 0, f"{name}: {stats}"
    assert stats["outside_tight"] == 0, f"{name}: {stats}"


def _fprop_case(xbits, wbits, name, rows=None):
    import torch
    log(f"gemm fprop {name} X{xbits.shape} W{wbits.shape}")
    xq, xs, wq, ws, _ = _quant_pair_fprop(xbits, wbits)
    y = poisoned((xbits.shape[0], wbits.shape[0]))
    fb.gemm(fb.FPROP, xq, xs, wq, ws, out=y.view(torch.bfloat16))
    assert_no_poison(y)
    qx0, sx0 = oq.quant_act_1x128(xbits if rows is None else xbits[rows])
    qw0, sw0 = oq.quant_w_128x128(wbits)
    xq_h, xs_h = host(xq), host(xs).T
    if rows is not None:
        xq_h, xs_h = xq_h[rows], xs_h[rows]
    np.testing.assert_array_equal(xq_h, qx0)
    np.testing.assert_array_equal(xs_h, sx0)
    np.testing.assert_array_equal(host(wq), qw0)
    y32, _, ab = og.fprop(qx0, sx0, qw0, sw0)
    yb = host_bf16_bits(y)
    if rows is not None:
        yb = yb[rows]
    _assert_ok(check_gemm_bf16(yb, y32, ab), name)


def test_fprop_tiny_config():
    cfg = tiny_fprop()
    _fprop_case(cfg.x, cfg.w, "tiny 256x256x1024")


@pytest.mark.parametrize("m,n,k,seed", [(1, 128, 128, 31), (300, 384, 640, 32), (513, 256, 256, 33),
                                         (128, 640, 1152, 34),
                                         (1000, 1024, 512, 39)])   # 32 tiles: the grid deals 4-tile chunks to the XCDs
def test_fprop_ragged(m, n, k, seed):
    x = act(seed, m, k, dist="student_t3", outlier_p=0.002, outlier_mult=20)
    w = act(seed + 1000, n, k, std=0.02)
    _fprop_case(x, w, f"ragged {m}x{n}x{k}")


# The library runs GEMMs with at most 128 tiles of 256 x 256 on 256 x 128 tiles
# (the cases above); these have more, so they take the 256 x 256 kernel, with
# ragged last tiles in both dimensions.
@pytest.mark.parametrize("m,n,k,seed", [(2100, 4224, 256, 37), (2049, 4480, 384, 38)])
def test_fprop_ragged_wide_tiles(m, n, k, seed):
    assert -(-m // 256) * -(-n // 256) > 128
    x = act(seed, m, k, dist="student_t3", outlier_p=0.002, outlier_mult=20)
    w = act(seed + 1000, n, k, std=0.02)
    _fprop_case(x, w, f"ragged wide tiles {m}x{n}x{k}")


def test_dgrad_ragged_wide_tiles():
    m, nw, kw = 2100, 256, 4224
    assert -(-m // 256) * -(-kw // 256) > 128
    dy = act(46, m, nw, std=1e-3)
    w = act(47, nw, kw, std=0.02)
    log(f"gemm dgrad dY{dy.shape} W{w.shape}")
    dq, ds = fb.quant_act_1x128(dev_bf16(dy))
    wq, ws, wqt = fb.quant_w_128x128(dev_bf16(w), transposed_copy=True)
    dx = fb.gemm(fb.DGRAD, dq, ds, wqt, ws)
    qd0, sd0 = oq.quant_act_1x128(dy)
    qw0, sw0 = oq.quant_w_128x128(w)
    y32, _, ab = og.dgrad(qd0, sd0, qw0, sw0)
    _assert_ok(check_gemm_bf16(host_bf16_bits(dx), y32, ab), f"dgrad wide tiles {m}x{kw}x{nw}")


def test_dgrad_tiny_scale_products():
    # dY tiles near 2^-116 against ordinary weights: s_dY * s_W is about 2^-135, an
    # fp32 subnormal with 15 significant bits, inside the documented range (>= 2^-140)
    m, nw, kw = 256, 256, 512
    dy = act(48, m, nw, std=2.0 ** -116)
    w = act(49, nw, kw, std=0.02)
    log(f"gemm dgrad tiny scales dY{dy.shape} W{w.shape}")
    dq, ds = fb.quant_act_1x128(dev_bf16(dy))
    wq, ws, wqt = fb.quant_w_128x128(dev_bf16(w), transposed_copy=True)
    qd0, sd0 = oq.quant_act_1x128(dy)
    qw0, sw0 = oq.quant_w_128x128(w)
    np.testing.assert_array_equal(host(dq), qd0)
    prod = sd0.astype(np.float64).min() * sw0.astype(np.float64).min()
    assert 2.0 ** -140 <= prod < 2.0 ** -126, prod
    dx = fb.gemm(fb.DGRAD, dq, ds, wqt, ws)
    y32, _, ab = og.dgrad(qd0, sd0, qw0, sw0)
    _assert_ok(check_gemm_bf16(host_bf16_bits(dx), y32, ab), "dgrad with subnormal scale products")


def test_fprop_zero_and_outlier_rows():
    x = act(35, 256, 512).copy()
    x[:40] = 0                        # zero rows (like MoE padding): s = 0, output exactly 0
    x[100, 7] = 0x4B00                # a large outlier in one tile only
    w = act(36, 256, 512, std=0.02)
    _fprop_case(x, w, "zero and outlier rows")


def test_dgrad():
    m, nw, kw = 200, 256, 384
    dy = act(41, m, nw, std=1e-3)
    w = act(42, nw, kw, std=0.02)
    log(f"gemm dgrad dY{dy.shape} W{w.shape}")
    dq, ds = fb.quant_act_1x128(dev_bf16(dy))
    wq, ws, wqt = fb.quant_w_128x128(dev_bf16(w), transposed_copy=True)
    dx = fb.gemm(fb.DGRAD, dq, ds, wqt, ws)
    assert tuple(dx.shape) == (m, kw)
    qd0, sd0 = oq.quant_act_1x128(dy)
    qw0, sw0 = oq.quant_w_128x128(w)
    np.testing.assert_array_equal(host(wqt), qw0.T)
    y32, _, ab = og.dgrad(qd0, sd0, qw0, sw0)
    _assert_ok(check_gemm_bf16(host_bf16_bits(dx), y32, ab), "dgrad 200x384x256")


@pytest.mark.parametrize("t,n,k,seed", [(256, 128, 384, 43), (384, 256, 256, 44), (128, 384, 128, 45)])
def test_wgrad(t, n, k, seed):
    dy = act(seed, t, n, std=1e-3)
    x = act(seed + 1, t, k, outlier_p=0.001, outlier_mult=50)
    log(f"gemm wgrad T={t} N={n} K={k}")
    dq, ds = fb.quant_act_1x128(dev_bf16(dy), fb.ACT_COLWISE)     # [n, t], [t/128, n]
    xq, xs = fb.quant_act_1x128(dev_bf16(x), fb.ACT_COLWISE)      # [k, t], [t/128, k]
    dw = fb.gemm(fb.WGRAD, dq, ds, xq, xs)
    assert tuple(dw.shape) == (n, k)
    qd0, sd0 = oq.quant_act_128x1(dy)
    qx0, sx0 = oq.quant_act_128x1(x)
    np.testing.assert_array_equal(host(dq), qd0)
    np.testing.assert_array_equal(host(xq), qx0)
    y32, _, ab = og.wgrad(qd0, sd0, qx0, sx0)
    _assert_ok(check_gemm_f32(host(dw), y32, ab), f"wgrad {n}x{k}x{t}")


def _grouped_case(row_off, n, k, seed, name):
    rng = np.random.default_rng(seed)
    G = len(row_off) - 1
    m = int(row_off[-1])
    x = act(seed, m, k)
    for e in range(G):   # zero padding at the end of each group
        r0, r1 = int(row_off[e]), int(row_off[e + 1])
        if r1 > r0:
            pad = int(rng.integers(0, 100))
            x[r1 - pad:r1] = 0
    ws = np.stack([act(int(rng.integers(1 << 30)), n, k, std=0.02) for _ in range(G)])
    log(f"grouped gemm {name} offsets={list(row_off)} n={n} k={k}")
    xq, xs = fb.quant_act_1x128(dev_bf16(x))
    wq_list, ws_list = zip(*[fb.quant_w_128x128(dev_bf16(ws[e]))[:2] for e in range(G)])
    import torch
    wq = torch.stack(wq_list)
    wsd = torch.stack(ws_list)
    y = fb.grouped_gemm(row_off, xq, xs, wq, wsd)
    qx0, sx0 = oq.quant_act_1x128(x)
    q0 = [oq.quant_w_128x128(ws[e]) for e in range(G)]
    qw0 = np.stack([a for a, _ in q0])
    sw0 = np.stack([b for _, b in q0])
    np.testing.assert_array_equal(host(wq), qw0)
    y32, _, ab = og.grouped_fprop(qx0, sx0, row_off, qw0, sw0)
    _assert_ok(check_gemm_bf16(host_bf16_bits(y), y32, ab), name)


def test_grouped_small():
    _grouped_case(np.array([0, 128, 128, 512, 640], np.int64), 256, 384, 51, "4 groups, one empty")


def test_grouped_single_group_equals_fprop_layout():
    _grouped_case(np.array([0, 384], np.int64), 384, 256, 52, "1 group")


# ---------------------------------------------------------------------------
# full sizes: every quantised byte is checked; the GEMM output is poison-filled
# first (no element may stay unwritten) and compared with the oracle on sampled
# rows, at least one in every 256-row tile of the walk
# ---------------------------------------------------------------------------

def test_dense_fprop_full_size():
    cfg = dense_fprop()
    rows = tile_rows(cfg.x.shape[0], 32, 61)
    _fprop_case(cfg.x, cfg.w, "dense 4096x2048x7168 (sampled rows)", rows=rows)


def test_backward_pair_full_size():
    dense = dense_fprop()
    dy = backward_dy()                                   # [4096, 2048]
    log("backward pair full size: dgrad 4096x7168x2048, wgrad 2048x7168x4096")
    import torch
    dq, ds = fb.quant_act_1x128(dev_bf16(dy))
    wq, ws, wqt = fb.quant_w_128x128(dev_bf16(dense.w), transposed_copy=True)
    dx = poisoned((4096, 7168))
    fb.gemm(fb.DGRAD, dq, ds, wqt, ws, out=dx.view(torch.bfloat16))
    assert_no_poison(dx)
    rows = tile_rows(4096, 16, 62)
    qd0, sd0 = oq.quant_act_1x128(dy[rows])
    qw0, sw0 = oq.quant_w_128x128(dense.w)
    np.testing.assert_array_equal(host(wqt), qw0.T)
    y32, _, ab = og.dgrad(qd0, sd0, qw0, sw0)
    _assert_ok(check_gemm_bf16(host_bf16_bits(dx)[rows], y32, ab), "dgrad full (sampled rows)")

    dqt, dst = fb.quant_act_1x128(dev_bf16(dy), fb.ACT_COLWISE)        # [2048, 4096]
    xqt, xst = fb.quant_act_1x128(dev_bf16(dense.x), fb.ACT_COLWISE)   # [7168, 4096]
    dw = poisoned((2048, 7168), fp32=True)
    fb.gemm(fb.WGRAD, dqt, dst, xqt, xst, out=dw.view(torch.float32))
    assert_no_poison(dw, fp32=True)
    qd0, sd0 = oq.quant_act_128x1(dy)
    np.testing.assert_array_equal(host(dqt), qd0)
    np.testing.assert_array_equal(host(dst).T, sd0)
    rows = tile_rows(2048, 8, 63)
    cols = tile_rows(7168, 480, 64)          # every 256-column tile as well
    qx0, sx0 = oq.quant_act_128x1(dense.x[:, cols])
    np.testing.assert_array_equal(host(xqt)[cols], qx0)
    y32, _, ab = og.wgrad(qd0[rows], sd0[rows], qx0, sx0)
    _assert_ok(check_gemm_f32(host(dw).view(np.float32)[np.ix_(rows, cols)], y32, ab), "wgrad full (sampled)")


def test_moe_grouped_full_size():
    cfg = moe_fprop()
    G = len(cfg.row_off) - 1
    log(f"MoE grouped full size: offsets {list(cfg.row_off)}")
    xq, xs = fb.quant_act_1x128(dev_bf16(cfg.x))
    import torch
    wq = torch.empty((G, 2048, 7168), dtype=torch.uint8, device="cuda")
    wsd = torch.empty((G, 16, 56), dtype=torch.float32, device="cuda")
    for e in range(G):
        q, s, _ = fb.quant_w_128x128(dev_bf16(cfg.w[e]))
        wq[e].copy_(q)
        wsd[e].copy_(s)
    y = poisoned((int(cfg.row_off[-1]), 2048))
    fb.grouped_gemm(cfg.row_off, xq, xs, wq, wsd, out=y.view(torch.bfloat16))
    assert_no_poison(y)
    yb = host_bf16_bits(y)
    for e in range(G):
        r0, r1 = int(cfg.row_off[e]), int(cfg.row_off[e + 1])
        real = r0 + int(cfg.real_rows[e])
        # one row in every 256-row tile of the expert that holds routed rows
        rows = tile_rows(real, 2, 65 + e, lo=r0)
        qx0, sx0 = oq.quant_act_1x128(cfg.x[rows])
        qw0, sw0 = oq.quant_w_128x128(cfg.w[e])
        y32, _, ab = og.fprop(qx0, sx0, qw0, sw0)
        _assert_ok(check_gemm_bf16(yb[rows], y32, ab), f"expert {e}")
        assert np.all(yb[real:r1] == 0), f"padding rows of expert {e} must be exactly zero"


def test_large_fprop_full_size_sampled():
    import torch
    cfg = large_fprop()
    rows = tile_rows(cfg.x.shape[0], 8, 66)
    log("large fprop 16384x18432x7168 (sampled rows, one in every row tile)")
    xq, xs, wq, ws, _ = _quant_pair_fprop(cfg.x, cfg.w)
    y = poisoned((16384, 18432))
    fb.gemm(fb.FPROP, xq, xs, wq, ws, out=y.view(torch.bfloat16))
    assert_no_poison(y)
    # a second launch gives the same bytes (the kernel fixes its summation order)
    y2 = fb.gemm(fb.FPROP, xq, xs, wq, ws)
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), "repeated launches differ"
    del y2
    qx0, sx0 = oq.quant_act_1x128(cfg.x[rows])
    np.testing.assert_array_equal(host(xq)[rows], qx0)
    np.testing.assert_array_equal(host(xs).T[rows], sx0)
    # weight: every byte checked, 2048 rows at a time
    wq_h, ws_h = host(wq), host(ws)
    for r0 in range(0, cfg.w.shape[0], 2048):
        q0, s0 = oq.quant_w_128x128(cfg.w[r0:r0 + 2048])
        np.testing.assert_array_equal(wq_h[r0:r0 + 2048], q0)
        np.testing.assert_array_equal(ws_h[r0 // 128:(r0 + 2048) // 128], s0)
    y32, _, ab = og.fprop(qx0, sx0, wq_h, ws_h)
    _assert_ok(check_gemm_bf16(host_bf16_bits(y)[rows], y32, ab), "large fprop (sampled rows)")
