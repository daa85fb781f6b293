"""GPU parity of the decode-shape grouped Fprop (fp8bq_grouped_gemm_decode and
its workspace form fp8bq_grouped_gemm_decode_ws, where experts of more than 32
rows run as 128-column half-K workgroup pairs) through the C ABI: unpadded
experts of at most 256 rows, against the oracle's grouped Fprop
(oracle.gemm.grouped_fprop, which takes any row offsets) on the same quantised
operands, to the GEMM acceptance bound of the other GEMM tests. Operands are
quantised on the GPU and checked bit-exact against the oracle's quantisation
first.
"""

import numpy as np
import pytest

import fp8_fine_grained_fp8bq_amd as fb
from oracle import gemm as og
from oracle import quant as oq
from tests.gpu_util import check_gemm_bf16, dev_bf16, host, host_bf16_bits, log
from workloads import act, moe_decode

pytestmark = pytest.mark.gpu


def _assert_ok(stats, name):
    log(f"  {name}: {stats}")
    assert stats["bad"] == 0, f"{name}: {stats}"
    assert stats["outside_tight"] == 0, f"{name}: {stats}"


def _quant_experts(ws):
    import torch
    G = ws.shape[0]
    wq, wsc = zip(*[fb.quant_w_128x128(dev_bf16(ws[e]))[:2] for e in range(G)])
    return torch.stack(wq), torch.stack(wsc)


def _decode_case(counts, n, k, seed, name, x=None, ws=None, split=True):
    counts = np.asarray(counts, np.int64)
    row_off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    G, m = len(counts), int(row_off[-1])
    rng = np.random.default_rng(seed)
    if x is None:
        x = act(seed, m, k, outlier_p=0.001, outlier_mult=50)
    if ws is None:
        ws = np.stack([act(int(rng.integers(1 << 30)), n, k, std=0.02) for _ in range(G)])
    log(f"[decode] {name}: counts={list(counts)} n={n} k={k} split={split}")
    import torch
    xq, xs = fb.quant_act_1x128(dev_bf16(x))
    wq, wsd = _quant_experts(ws)
    y = torch.full((m, n), -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    fb.grouped_gemm_decode(row_off, xq, xs, wq, wsd, out=y, split=split)
    qx0, sx0 = oq.quant_act_1x128(x)
    q0 = [oq.quant_w_128x128(ws[e]) for e in range(G)]
    qw0 = np.stack([a for a, _ in q0])
    sw0 = np.stack([b for _, b in q0])
    np.testing.assert_array_equal(host(xq), qx0)
    np.testing.assert_array_equal(host(wq), qw0)
    y32, _, ab = og.grouped_fprop(qx0, sx0, row_off, qw0, sw0)
    _assert_ok(check_gemm_bf16(host_bf16_bits(y), y32, ab), name)


@pytest.mark.parametrize("counts,seed", [
    ([5, 0, 37], 101),            # one expert empty, ragged counts (16-row subtiles: 1 and 3)
    ([16, 1, 9], 102),            # largest 16 rows
    ([32, 17], 103),              # up to 32
    ([64, 3, 50, 33], 104),       # up to 64
    ([128, 100, 1], 105),         # up to 128
    ([256, 129, 7, 200], 106),    # up to 256
])
@pytest.mark.parametrize("split", [False, True])
def test_decode_counts(counts, seed, split):
    _decode_case(counts, 256, 640, seed, f"counts {counts}", split=split)


@pytest.mark.parametrize("split", [False, True])
def test_decode_every_subtile_count(split):
    # 1 .. 16 subtiles of 16 rows, each padded to the next compiled count, with
    # an odd chunk count (the K halves differ by one chunk)
    counts = [1, 17, 33, 49, 65, 81, 97, 113, 129, 145, 161, 177, 193, 209, 225, 241, 256, 48]
    _decode_case(counts, 256, 1152, 112, "every subtile count", split=split)


@pytest.mark.parametrize("k", [128, 384, 1152])
@pytest.mark.parametrize("split", [False, True])
def test_decode_short_k(k, split):
    # fewer chunks than the rings hold: the prologue's and the tail's repeated
    # loads; k = 128 has one chunk, which is never split
    _decode_case([40, 3, 90], 128, k, 107, f"k={k}", split=split)


def test_decode_workspace_reuse():
    # one workspace through calls of decreasing size, each checked against the
    # oracle and repeated bit-identically: every call must leave the counters
    # zero and read only the partial sums its own other half wrote
    import torch
    n, k = 256, 896
    for i, counts in enumerate(([200, 90, 40], [120, 35], [33])):
        counts = np.asarray(counts, np.int64)
        row_off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
        G, m = len(counts), int(row_off[-1])
        x = act(113 + i, m, k, outlier_p=0.001, outlier_mult=50)
        ws = np.stack([act(120 + 10 * i + e, n, k, std=0.02) for e in range(G)])
        log(f"[decode] workspace reuse, call {i}: counts={list(counts)}")
        xq, xs = fb.quant_act_1x128(dev_bf16(x))
        wq, wsd = _quant_experts(ws)
        y1 = fb.grouped_gemm_decode(row_off, xq, xs, wq, wsd, split=True)
        y2 = fb.grouped_gemm_decode(row_off, xq, xs, wq, wsd, split=True)
        assert torch.equal(y1, y2), "split result not reproducible"
        qx0, sx0 = oq.quant_act_1x128(x)
        q0 = [oq.quant_w_128x128(ws[e]) for e in range(G)]
        y32, _, ab = og.grouped_fprop(qx0, sx0, row_off, np.stack([a for a, _ in q0]), np.stack([b for _, b in q0]))
        _assert_ok(check_gemm_bf16(host_bf16_bits(y1), y32, ab), f"reuse call {i}")
    wsp = fb.decode_workspace(0, "cuda")
    cnt = host(wsp[:256 * 256 * 4].view(torch.int32))             # the counters lead the workspace
    assert np.all(cnt == 0), "counters left non-zero"


def test_decode_many_experts():
    rng = np.random.default_rng(108)
    counts = rng.integers(0, 12, 256)
    counts[[3, 77]] = 0
    _decode_case(counts, 128, 256, 108, "256 experts")


def test_decode_leading_dimensions():
    import torch
    counts = np.array([20, 70], np.int64)
    row_off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    m, n, k = int(row_off[-1]), 256, 384
    lda, ldo = k + 128, n + 64
    x = act(109, m, k)
    ws = np.stack([act(110 + e, n, k, std=0.02) for e in range(2)])
    log("[decode] leading dimensions")
    xq_full = torch.zeros((m, lda), dtype=torch.uint8, device="cuda")
    xq, xs = fb.quant_act_1x128(dev_bf16(x))
    xq_full[:, :k] = xq
    wq, wsd = _quant_experts(ws)
    y = torch.full((m, ldo), 7, dtype=torch.int16, device="cuda")
    fb.fp8bq_grouped_gemm_decode(2, list(row_off), n, k, xq_full.data_ptr(), lda, xs.data_ptr(), xs.stride(0),
                                 wq.data_ptr(), wq.stride(1), wsd.data_ptr(), wsd.stride(1), y.data_ptr(), ldo, 0,
                                 torch.cuda.current_stream().cuda_stream)
    yb = host(y).view(np.uint16)
    assert np.all(yb[:, n:] == 7), "wrote past n"
    qx0, sx0 = oq.quant_act_1x128(x)
    q0 = [oq.quant_w_128x128(ws[e]) for e in range(2)]
    y32, _, ab = og.grouped_fprop(qx0, sx0, row_off, np.stack([a for a, _ in q0]), np.stack([b for _, b in q0]))
    _assert_ok(check_gemm_bf16(np.ascontiguousarray(yb[:, :n]), y32, ab), "leading dimensions")


@pytest.mark.parametrize("split", [False, True])
def test_decode_workload_full(split):
    # the decode step the bench times: 256 tokens, 8 local experts of [2048, 7168]
    cfg = moe_decode()
    _decode_case(cfg.real_rows, 2048, 7168, 111, "MoE decode 256 tokens", x=cfg.x, ws=cfg.w, split=split)
