"""GPU parity of the power-of-two scale path (FP8BQ_SCALE_POW2).

The quantisers must reproduce the oracle's power-of-two mode bit for bit (codes
and scales). The GEMMs then apply the scales inside the scaled matrix
instruction and let it accumulate each chunk into FP32 (it adds the chunk in
blocks of 8 products, not in one rounding); they are accepted against the
oracle, which promotes each chunk with one FP32 rounding, within the same
2e-3 * sum_k |x_hat_k| |w_hat_k| bound and canary bracket as the exact-scale
path.
"""

import numpy as np
import pytest

import fp8_fine_grained_fp8bq_amd as fb
from oracle import gemm as og
from oracle import quant as oq
from tests.gpu_util import check_gemm_bf16, check_gemm_f32, dev_bf16, host, host_bf16_bits, log
from workloads import act, backward_dy, dense_fprop, f32_to_bf16_bits, large_fprop, moe_fprop, tiny_fprop

pytestmark = pytest.mark.gpu
P2 = "pow2"


def _assert_ok(stats, name):
    log(f"  {name}: {stats}")
    assert stats["bad"] == 0, f"{name}: {stats}"
    assert stats["outside_tight"] == 0, f"{name}: {stats}"


# ---- quantisers ---------------------------------------------------------------

def _rows(bits, ldx=None, name=""):
    log(f"quant_act rowwise pow2 {name} shape={bits.shape} ldx={ldx}")
    rows, cols = bits.shape
    if ldx is not None and ldx != cols:
        buf = np.zeros((rows, ldx), np.uint16)
        buf[:, :cols] = bits
        t = dev_bf16(buf)[:, :cols]
    else:
        t = dev_bf16(bits)
    q, s = fb.quant_act_1x128(t, fb.ACT_ROWWISE | fb.SCALE_POW2)
    q0, s0 = oq.quant_act_1x128(bits, P2)
    np.testing.assert_array_equal(host(q), q0, err_msg=name)
    np.testing.assert_array_equal(host(s).T.view(np.uint32), s0.view(np.uint32), err_msg=name)


@pytest.mark.parametrize("rows,cols,ldx,seed", [(1, 128, None, 1), (37, 384, None, 2), (257, 1024, 1088, 3),
                                                 (64, 7168, None, 4)])
def test_rowwise_seeded(rows, cols, ldx, seed):
    _rows(act(seed, rows, cols, dist="student_t3", outlier_p=0.003, outlier_mult=40), ldx, f"seed {seed}")


def test_rowwise_every_bf16_absmax():
    # one tile per positive finite bf16 absmax: every exponent rule and the clamp
    amax = np.arange(1, 0x7F80, dtype=np.uint16)
    a = (amax.astype(np.uint32) << 16).view(np.float32)
    fr = np.linspace(-1, 1, 127, dtype=np.float32)
    body = f32_to_bf16_bits(a[:, None] * fr[None, :])
    signs = np.where(np.arange(amax.size) % 2 == 1, 0x8000, 0).astype(np.uint16)
    x = np.concatenate([(amax | signs)[:, None], body], axis=1).astype(np.uint16)
    _rows(x, name="every bf16 absmax")


def test_rowwise_every_bf16_value():
    # every finite bf16 pattern under power-of-two scales from tiny to huge
    bits = np.arange(65536, dtype=np.uint32)
    f = (bits << 16).view(np.float32)
    for amax_bits in (0x43E0, 0x3F80, 0x0080, 0x7F7F, 0x2E9B):
        amax = float(np.array([amax_bits << 16], np.uint32).view(np.float32)[0])
        vals = bits[np.isfinite(f) & (np.abs(f) <= amax)].astype(np.uint16)
        rows = -(-len(vals) // 127)
        x = np.zeros((rows, 128), np.uint16)
        x[:, 0] = amax_bits
        flat = np.zeros(rows * 127, np.uint16)
        flat[:len(vals)] = vals
        x[:, 1:] = flat.reshape(rows, 127)
        _rows(x, name=f"every bf16 up to {amax_bits:#x}")


def test_rowwise_edge_tiles():
    x = act(7, 8, 256, outlier_p=0).copy()
    x[0, :128] = 0
    x[1, :128] = 0x8000
    x[2, :128] = 0x0001
    x[3, :128] = np.arange(128, dtype=np.uint16) | 0x8000
    x[4, :128] = f32_to_bf16_bits(np.full(128, -3.0e38, np.float32))
    x[5, 128:] = f32_to_bf16_bits(np.array([1e-30] * 127 + [1e30], np.float32))
    x[6, :128] = f32_to_bf16_bits(np.array([448.0, -224.0] * 64, np.float32))
    _rows(x, name="edge tiles")


@pytest.mark.parametrize("rows,cols,seed", [(128, 128, 11), (384, 640, 13)])
def test_colwise(rows, cols, seed):
    x = act(seed, rows, cols, std=1e-3, outlier_p=0.002, outlier_mult=30)
    log(f"quant_act colwise pow2 {x.shape}")
    q, s = fb.quant_act_1x128(dev_bf16(x), fb.ACT_COLWISE | fb.SCALE_POW2)
    q0, s0 = oq.quant_act_128x1(x, P2)
    np.testing.assert_array_equal(host(q), q0)
    np.testing.assert_array_equal(host(s).T.view(np.uint32), s0.view(np.uint32))


@pytest.mark.parametrize("n,k,seed", [(256, 384, 22), (2048, 7168, 24)])
def test_quant_w(n, k, seed):
    w = act(seed, n, k, std=0.02)
    log(f"quant_w pow2 {w.shape}")
    q, s, qt = fb.quant_w_128x128(dev_bf16(w), transposed_copy=True, pow2=True)
    q0, s0 = oq.quant_w_128x128(w, P2)
    np.testing.assert_array_equal(host(q), q0)
    np.testing.assert_array_equal(host(s).view(np.uint32), s0.view(np.uint32))
    np.testing.assert_array_equal(host(qt), q0.T)


# ---- GEMMs ----------------------------------------------------------------------

def _fprop_case(xbits, wbits, name, rows=None):
    log(f"gemm fprop pow2 {name} X{xbits.shape} W{wbits.shape}")
    xq, xs = fb.quant_act_1x128(dev_bf16(xbits), fb.ACT_ROWWISE | fb.SCALE_POW2)
    wq, ws, _ = fb.quant_w_128x128(dev_bf16(wbits), pow2=True)
    y = fb.gemm(fb.FPROP | fb.SCALE_POW2, xq, xs, wq, ws)
    qx0, sx0 = oq.quant_act_1x128(xbits if rows is None else xbits[rows], P2)
    qw0, sw0 = oq.quant_w_128x128(wbits, P2)
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
                                         (128, 640, 1152, 34)])
def test_fprop_ragged(m, n, k, seed):
    x = act(seed, m, k, dist="student_t3", outlier_p=0.002, outlier_mult=20)
    w = act(seed + 1000, n, k, std=0.02)
    _fprop_case(x, w, f"ragged {m}x{n}x{k}")


def test_fprop_zero_rows_and_extreme_scales():
    x = act(35, 256, 512).copy()
    x[:40] = 0                                                        # zero tiles: s = 2^-127, output 0
    x[40:48] = f32_to_bf16_bits((np.random.default_rng(5).standard_normal((8, 512)) * 1e-34).astype(np.float32))
    x[100, 7] = 0x4B00
    w = act(37, 256, 512, std=0.02)
    _fprop_case(x, w, "zero rows, tiny rows, an outlier")


def test_dgrad():
    dy = act(41, 200, 256, std=1e-3)
    w = act(42, 256, 384, std=0.02)
    log(f"gemm dgrad pow2 dY{dy.shape} W{w.shape}")
    dq, ds = fb.quant_act_1x128(dev_bf16(dy), fb.ACT_ROWWISE | fb.SCALE_POW2)
    wq, ws, wqt = fb.quant_w_128x128(dev_bf16(w), transposed_copy=True, pow2=True)
    dx = fb.gemm(fb.DGRAD | fb.SCALE_POW2, dq, ds, wqt, ws)
    qd0, sd0 = oq.quant_act_1x128(dy, P2)
    qw0, sw0 = oq.quant_w_128x128(w, P2)
    y32, _, ab = og.dgrad(qd0, sd0, qw0, sw0)
    _assert_ok(check_gemm_bf16(host_bf16_bits(dx), y32, ab), "dgrad 200x384x256")


@pytest.mark.parametrize("t,n,k,seed", [(256, 128, 384, 43), (384, 256, 256, 44)])
def test_wgrad(t, n, k, seed):
    dy = act(seed, t, n, std=1e-3)
    x = act(seed + 1, t, k, outlier_p=0.001, outlier_mult=50)
    log(f"gemm wgrad pow2 T={t} N={n} K={k}")
    dq, ds = fb.quant_act_1x128(dev_bf16(dy), fb.ACT_COLWISE | fb.SCALE_POW2)
    xq, xs = fb.quant_act_1x128(dev_bf16(x), fb.ACT_COLWISE | fb.SCALE_POW2)
    dw = fb.gemm(fb.WGRAD | fb.SCALE_POW2, dq, ds, xq, xs)
    qd0, sd0 = oq.quant_act_128x1(dy, P2)
    qx0, sx0 = oq.quant_act_128x1(x, P2)
    np.testing.assert_array_equal(host(dq), qd0)
    np.testing.assert_array_equal(host(xq), qx0)
    y32, _, ab = og.wgrad(qd0, sd0, qx0, sx0)
    _assert_ok(check_gemm_f32(host(dw), y32, ab), f"wgrad {n}x{k}x{t}")


def test_grouped_small():
    row_off = np.array([0, 128, 128, 512, 640], np.int64)
    n, k, G = 256, 384, 4
    x = act(51, 640, k)
    x[600:640] = 0
    ws = np.stack([act(52 + e, n, k, std=0.02) for e in range(G)])
    log(f"grouped gemm pow2 offsets={list(row_off)}")
    import torch
    xq, xs = fb.quant_act_1x128(dev_bf16(x), fb.ACT_ROWWISE | fb.SCALE_POW2)
    wq = torch.stack([fb.quant_w_128x128(dev_bf16(ws[e]), pow2=True)[0] for e in range(G)])
    wsd = torch.stack([fb.quant_w_128x128(dev_bf16(ws[e]), pow2=True)[1] for e in range(G)])
    y = fb.grouped_gemm(row_off, xq, xs, wq, wsd, pow2=True)
    qx0, sx0 = oq.quant_act_1x128(x, P2)
    q0 = [oq.quant_w_128x128(ws[e], P2) for e in range(G)]
    y32, _, ab = og.grouped_fprop(qx0, sx0, row_off, np.stack([a for a, _ in q0]), np.stack([b for _, b in q0]))
    _assert_ok(check_gemm_bf16(host_bf16_bits(y), y32, ab), "grouped, 4 groups, one empty")


def _sample_rows(m, count, seed):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, m - 1], rng.choice(m, size=count, replace=False)]))


def test_dense_fprop_full_size():
    cfg = dense_fprop()
    _fprop_case(cfg.x, cfg.w, "dense 4096x2048x7168 (sampled rows)", rows=_sample_rows(4096, 48, 61))


def test_backward_pair_full_size():
    dense = dense_fprop()
    dy = backward_dy()
    log("backward pair pow2 full size")
    dq, ds = fb.quant_act_1x128(dev_bf16(dy), fb.ACT_ROWWISE | fb.SCALE_POW2)
    wq, ws, wqt = fb.quant_w_128x128(dev_bf16(dense.w), transposed_copy=True, pow2=True)
    dx = fb.gemm(fb.DGRAD | fb.SCALE_POW2, dq, ds, wqt, ws)
    rows = _sample_rows(4096, 24, 62)
    qd0, sd0 = oq.quant_act_1x128(dy[rows], P2)
    qw0, sw0 = oq.quant_w_128x128(dense.w, P2)
    y32, _, ab = og.dgrad(qd0, sd0, qw0, sw0)
    _assert_ok(check_gemm_bf16(host_bf16_bits(dx)[rows], y32, ab), "dgrad full (sampled rows)")
    dqt, dst = fb.quant_act_1x128(dev_bf16(dy), fb.ACT_COLWISE | fb.SCALE_POW2)
    xqt, xst = fb.quant_act_1x128(dev_bf16(dense.x), fb.ACT_COLWISE | fb.SCALE_POW2)
    dw = fb.gemm(fb.WGRAD | fb.SCALE_POW2, dqt, dst, xqt, xst)
    qd0, sd0 = oq.quant_act_128x1(dy, P2)
    rows = _sample_rows(2048, 16, 63)
    cols = np.sort(np.random.default_rng(64).choice(7168, size=512, replace=False))
    qx0, sx0 = oq.quant_act_128x1(dense.x[:, cols], P2)
    np.testing.assert_array_equal(host(xqt)[cols], qx0)
    y32, _, ab = og.wgrad(qd0[rows], sd0[rows], qx0, sx0)
    _assert_ok(check_gemm_f32(host(dw)[np.ix_(rows, cols)], y32, ab), "wgrad full (sampled)")


def test_moe_grouped_full_size():
    cfg = moe_fprop()
    G = len(cfg.row_off) - 1
    log(f"MoE grouped pow2 full size: offsets {list(cfg.row_off)}")
    import torch
    xq, xs = fb.quant_act_1x128(dev_bf16(cfg.x), fb.ACT_ROWWISE | fb.SCALE_POW2)
    wq = torch.empty((G, 2048, 7168), dtype=torch.uint8, device="cuda")
    wsd = torch.empty((G, 16, 56), dtype=torch.float32, device="cuda")
    for e in range(G):
        q, s, _ = fb.quant_w_128x128(dev_bf16(cfg.w[e]), pow2=True)
        wq[e].copy_(q)
        wsd[e].copy_(s)
    yb = host_bf16_bits(fb.grouped_gemm(cfg.row_off, xq, xs, wq, wsd, pow2=True))
    rng = np.random.default_rng(65)
    for e in range(G):
        r0, r1 = int(cfg.row_off[e]), int(cfg.row_off[e + 1])
        real = r0 + int(cfg.real_rows[e])
        rows = np.unique(np.concatenate([[r0, real - 1], rng.integers(r0, real, 6)]))
        qx0, sx0 = oq.quant_act_1x128(cfg.x[rows], P2)
        qw0, sw0 = oq.quant_w_128x128(cfg.w[e], P2)
        y32, _, ab = og.fprop(qx0, sx0, qw0, sw0)
        _assert_ok(check_gemm_bf16(yb[rows], y32, ab), f"expert {e}")
        assert np.all(yb[real:r1] == 0), f"padding rows of expert {e} must be exactly zero"


def test_large_fprop_full_size_sampled():
    cfg = large_fprop()
    rows = _sample_rows(cfg.x.shape[0], 24, 66)
    log("large fprop pow2 16384x18432x7168 (sampled rows)")
    xq, xs = fb.quant_act_1x128(dev_bf16(cfg.x), fb.ACT_ROWWISE | fb.SCALE_POW2)
    wq, ws, _ = fb.quant_w_128x128(dev_bf16(cfg.w), pow2=True)
    y = fb.gemm(fb.FPROP | fb.SCALE_POW2, xq, xs, wq, ws)
    qx0, sx0 = oq.quant_act_1x128(cfg.x[rows], P2)
    np.testing.assert_array_equal(host(xq)[rows], qx0)
    np.testing.assert_array_equal(host(xs).T[rows], sx0)
    wq_h, ws_h = host(wq), host(ws)
    for r0 in range(0, cfg.w.shape[0], 4096):
        q0, s0 = oq.quant_w_128x128(cfg.w[r0:r0 + 4096], P2)
        np.testing.assert_array_equal(wq_h[r0:r0 + 4096], q0)
        np.testing.assert_array_equal(ws_h[r0 // 128:(r0 + 4096) // 128], s0)
    y32, _, ab = og.fprop(qx0, sx0, wq_h, ws_h)
    _assert_ok(check_gemm_bf16(host_bf16_bits(y)[rows], y32, ab), "large fprop pow2 (sampled rows)")
