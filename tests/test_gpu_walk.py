"""GPU parity of the persistent tile walk, element by element.

The GEMM kernels are persistent: one workgroup per CU walks a sequence of
output tiles, prefetching the next tile's first K-chunk during the current
tile's last one and carrying its lagged promotion folds across the tile
boundary. These tests run shapes with more than twice as many 256 x 256 tiles
as the chip has CUs (every workgroup owns two or three tiles), ragged last
tiles in both output dimensions and four K-chunks, and compare EVERY output
element with the oracle (2e-3 * sum|x_hat||w_hat| before the bf16 rounding,
plus the tighter canary), for the exact-scale and the power-of-two kernels,
Fprop, Dgrad, Wgrad, the grouped (per-expert) Fprop and the GEMM that
quantises its own output. Outputs are filled with a poison pattern first, so a
tile that is never written fails; each GEMM is launched twice and must give
identical bytes (the summation order is fixed by the kernel, not by timing).

Method: DeepSeek-V3 report (Chinese translation), section 3.3.2 "increasing
accumulation precision" and Figure 7b: every 128-element K interval's partial
sum is promoted into FP32 with both operands' scales, in every chunk of every
tile.
"""

import numpy as np
import pytest

import fp8_fine_grained_fp8bq_amd as fb
from oracle import gemm as og
from oracle import quant as oq
from tests.gpu_util import check_gemm_bf16, check_gemm_f32, dev, dev_bf16, host, host_bf16_bits, log
from workloads import act

pytestmark = pytest.mark.gpu

# 4100 x 8064 outputs = 17 x 32 = 544 tiles of 256 x 256 (> 2 x 256 CUs): the last
# row tile has 4 rows, the last column tile 128 columns; K = 512 is 4 chunks.
M, N, K = 4100, 8064, 512
# The exact-scale kernel picks its tile width per shape (256 x 256, or 256 x 224 when
# that takes fewer rounds of the walk, weighted by the tile's work; see
# prefer_224): N = 7552 keeps 256-column tiles (510 tiles, the last 128 columns
# wide), N = 7936 takes 224-column tiles (612 tiles, the last 96 columns wide,
# waves whose 112 columns straddle two weight blocks).
N_BY_WIDTH = {256: 7552, 224: 7936}


def width_for(m, n, cus=256):
    """Tile width the library's launcher picks for an exact-scale GEMM (mirror of prefer_224)."""
    tm = -(-m // 256)
    r256 = -(-(tm * -(-n // 256)) // cus)
    r224 = -(-(tm * -(-n // 224)) // cus)
    return 224 if r224 * 7 < r256 * 8 else 256
POISON16 = -1            # 0xFFFF: a bf16 NaN, never the rounding of a finite sum
POISON32 = -1            # 0xFFFFFFFF: an fp32 NaN


def _tiles(m, n):
    return -(-m // 256) * -(-n // 256)


def _poisoned(shape, fp32=False):
    import torch
    dt = torch.int32 if fp32 else torch.int16
    return torch.full(shape, POISON32 if fp32 else POISON16, dtype=dt, device="cuda")


def _no_poison(t, fp32=False):
    import torch
    bad = int((t.view(torch.int32 if fp32 else torch.int16) == -1).sum())
    assert bad == 0, f"{bad} output elements were never written"


def _assert_ok(stats, name):
    log(f"  {name}: {stats}")
    assert stats["bad"] == 0, f"{name}: {stats}"
    assert stats["outside_tight"] == 0, f"{name}: {stats}"


def _twice(launch, shape, fp32=False):
    """Launches into two poisoned buffers; both fully written and byte-identical."""
    import torch
    out1, out2 = _poisoned(shape, fp32), _poisoned(shape, fp32)
    launch(out1)
    launch(out2)
    torch.cuda.synchronize()
    _no_poison(out1, fp32)
    assert torch.equal(out1, out2), "two launches of the same GEMM gave different bytes"
    return out1


@pytest.mark.parametrize("pow2,N", [(False, N_BY_WIDTH[256]), (False, N_BY_WIDTH[224]), (True, N)])
def test_fprop_every_element(pow2, N):
    assert _tiles(M, N) >= 2 * 256 - 2
    assert pow2 or width_for(M, N) == (256 if N == N_BY_WIDTH[256] else 224)
    x = act(301, M, K, dist="student_t3", outlier_p=0.002, outlier_mult=20)
    w = act(302, N, K, std=0.02)
    mode = "pow2" if pow2 else "exact"
    log(f"[walk] fprop {M}x{N}x{K} ({_tiles(M, N)} tiles of 256x256) scales={mode}")
    xq, xs = fb.quant_act_1x128(dev_bf16(x), fb.SCALE_POW2 if pow2 else fb.ACT_ROWWISE)
    wq, ws, _ = fb.quant_w_128x128(dev_bf16(w), pow2=pow2)
    op = fb.FPROP | (fb.SCALE_POW2 if pow2 else 0)
    import torch
    y = _twice(lambda out: fb.gemm(op, xq, xs, wq, ws, out=out.view(torch.bfloat16)), (M, N))
    qx0, sx0 = oq.quant_act_1x128(x, mode)
    qw0, sw0 = oq.quant_w_128x128(w, mode)
    np.testing.assert_array_equal(host(xq), qx0)
    np.testing.assert_array_equal(host(wq), qw0)
    y32, _, ab = og.fprop(qx0, sx0, qw0, sw0)
    _assert_ok(check_gemm_bf16(host_bf16_bits(y), y32, ab), f"fprop every element ({mode})")


@pytest.mark.parametrize("pow2,N", [(False, N_BY_WIDTH[256]), (False, N_BY_WIDTH[224]), (True, N)])
def test_dgrad_every_element(pow2, N):
    # dX [M, N] = dY [M, K] W [K, N]: the weight's transposed FP8 copy is the B operand
    dy = act(303, M, K, std=1e-3)
    w = act(304, K, N, std=0.02)
    mode = "pow2" if pow2 else "exact"
    log(f"[walk] dgrad dY{dy.shape} W{w.shape} scales={mode}")
    dq, ds = fb.quant_act_1x128(dev_bf16(dy), fb.SCALE_POW2 if pow2 else fb.ACT_ROWWISE)
    _, ws, wqt = fb.quant_w_128x128(dev_bf16(w), transposed_copy=True, pow2=pow2)
    op = fb.DGRAD | (fb.SCALE_POW2 if pow2 else 0)
    import torch
    dx = _twice(lambda out: fb.gemm(op, dq, ds, wqt, ws, out=out.view(torch.bfloat16)), (M, N))
    qd0, sd0 = oq.quant_act_1x128(dy, mode)
    qw0, sw0 = oq.quant_w_128x128(w, mode)
    np.testing.assert_array_equal(host(wqt), qw0.T)
    y32, _, ab = og.dgrad(qd0, sd0, qw0, sw0)
    _assert_ok(check_gemm_bf16(host_bf16_bits(dx), y32, ab), f"dgrad every element ({mode})")


@pytest.mark.parametrize("pow2,k", [(False, N_BY_WIDTH[256]), (False, N_BY_WIDTH[224]), (True, N)])
def test_wgrad_every_element(pow2, k):
    # dW [n, k] = dY^T X over T = 512 tokens (4 chunks), both operands in 128x1 tiles
    n, t = 4224, K
    assert _tiles(n, k) >= 2 * 256 - 32
    dy = act(305, t, n, std=1e-3)
    x = act(306, t, k, outlier_p=0.001, outlier_mult=50)
    mode = "pow2" if pow2 else "exact"
    log(f"[walk] wgrad n={n} k={k} T={t} scales={mode}")
    pf = fb.SCALE_POW2 if pow2 else 0
    dq, ds = fb.quant_act_1x128(dev_bf16(dy), fb.ACT_COLWISE | pf)
    xq, xs = fb.quant_act_1x128(dev_bf16(x), fb.ACT_COLWISE | pf)
    import torch
    dw = _twice(lambda out: fb.gemm(fb.WGRAD | pf, dq, ds, xq, xs, out=out.view(torch.float32)), (n, k), fp32=True)
    qd0, sd0 = oq.quant_act_128x1(dy, mode)
    qx0, sx0 = oq.quant_act_128x1(x, mode)
    np.testing.assert_array_equal(host(dq), qd0)
    np.testing.assert_array_equal(host(xq), qx0)
    y32, _, ab = og.wgrad(qd0, sd0, qx0, sx0)
    stats = check_gemm_f32(host(dw).view(np.float32), y32, ab)
    _assert_ok(stats, f"wgrad every element ({mode})")


@pytest.mark.parametrize("pow2", [False, True])
def test_grouped_every_element(pow2):
    # five experts, one empty, rows padded to 128 with zero rows at each group's end:
    # 5 + 0 + 4 + 6 + 2 = 17 row tiles x 32 column tiles = 544 tiles
    row_off = np.array([0, 1152, 1152, 2176, 3712, 4096], np.int64)
    G = len(row_off) - 1
    m = int(row_off[-1])
    rng = np.random.default_rng(307)
    x = act(308, m, K, dist="student_t3", outlier_p=0.002, outlier_mult=20)
    for e in range(G):
        r0, r1 = int(row_off[e]), int(row_off[e + 1])
        if r1 > r0:
            x[r1 - int(rng.integers(1, 128)):r1] = 0
    w = np.stack([act(309 + e, N, K, std=0.02) for e in range(G)])
    mode = "pow2" if pow2 else "exact"
    log(f"[walk] grouped offsets={list(row_off)} n={N} k={K} scales={mode}")
    import torch
    xq, xs = fb.quant_act_1x128(dev_bf16(x), fb.SCALE_POW2 if pow2 else fb.ACT_ROWWISE)
    pairs = [fb.quant_w_128x128(dev_bf16(w[e]), pow2=pow2)[:2] for e in range(G)]
    wq = torch.stack([p[0] for p in pairs])
    wsd = torch.stack([p[1] for p in pairs])
    y = _twice(lambda out: fb.grouped_gemm(row_off, xq, xs, wq, wsd, out=out.view(torch.bfloat16), pow2=pow2),
               (m, N))
    qx0, sx0 = oq.quant_act_1x128(x, mode)
    q0 = [oq.quant_w_128x128(w[e], mode) for e in range(G)]
    qw0 = np.stack([a for a, _ in q0])
    sw0 = np.stack([b for _, b in q0])
    np.testing.assert_array_equal(host(wq), qw0)
    y32, _, ab = og.grouped_fprop(qx0, sx0, row_off, qw0, sw0)
    _assert_ok(check_gemm_bf16(host_bf16_bits(y), y32, ab), f"grouped every element ({mode})")


@pytest.mark.parametrize("in_pow2", [False, True])
def test_quantised_output_every_element(in_pow2):
    import torch
    x = act(314, M, K, dist="student_t3", outlier_p=0.002, outlier_mult=20)
    w = act(315, N, K, std=0.02)
    mode = "pow2" if in_pow2 else "exact"
    log(f"[walk] gemm_quant {M}x{N}x{K} in_scales={mode}")
    pf = fb.SCALE_POW2 if in_pow2 else 0
    xq, xs = fb.quant_act_1x128(dev_bf16(x), pf)
    wq, ws, _ = fb.quant_w_128x128(dev_bf16(w), pow2=in_pow2)
    outs = []
    for _ in range(2):
        y = _poisoned((M, N))
        q = torch.full((M, N), 0xFF, dtype=torch.uint8, device="cuda")   # 0xFF: an E4M3 NaN code
        s = torch.full((N // 128, M), -1, dtype=torch.int32, device="cuda")
        fb.fp8bq_gemm_quant(fb.FPROP | pf, M, N, K, xq.data_ptr(), K, xs.data_ptr(), xs.stride(0), wq.data_ptr(),
                            K, ws.data_ptr(), ws.stride(0), y.data_ptr(), N, q.data_ptr(), N, s.data_ptr(), M, 0,
                            torch.cuda.current_stream().cuda_stream)
        outs.append((y, q, s))
    torch.cuda.synchronize()
    (y, q, s), (y2, q2, s2) = outs
    _no_poison(y)
    assert int((q == 0xFF).sum()) == 0 and int((s == -1).sum()) == 0, "codes or scales never written"
    assert torch.equal(y, y2) and torch.equal(q, q2) and torch.equal(s, s2), "repeated launches differ"
    # the fused codes and scales are the library quantiser's of the fused bf16 output
    q3, s3 = fb.quant_act_1x128(y.view(torch.bfloat16))
    assert torch.equal(q, q3) and torch.equal(s, s3.view(torch.int32)), "fused quantisation differs"
    qx0, sx0 = oq.quant_act_1x128(x, mode)
    qw0, sw0 = oq.quant_w_128x128(w, mode)
    y32, _, ab = og.fprop(qx0, sx0, qw0, sw0)
    yb = y.cpu().numpy().view(np.uint16)
    _assert_ok(check_gemm_bf16(yb, y32, ab), f"quantised-output GEMM every element ({mode})")
    # and its codes are the oracle quantiser's of that bf16 output, bit for bit
    q0, s0 = oq.quant_act_1x128(yb)
    np.testing.assert_array_equal(host(q), q0)
    np.testing.assert_array_equal(host(s).T, s0.view(np.int32))
