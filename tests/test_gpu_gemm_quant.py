"""GPU parity of the GEMM whose epilogue quantises its own bf16 output
(producer fusion, fp8bq_gemm_quant), through the C ABI.

* Exact-output inputs (small E4M3 codes, power-of-two scales near 1): the GEMM
  is exact in fp32, so its bf16 output has one right answer and the oracle's
  G5 (bf16 rounding, then 1x128 tiles) must be met bit for bit: output, codes
  and scales, for both input paths (scales by the VALU promotion or by the
  matrix instruction) and both output scale rules.
* General inputs (the configs' distributions): the fused codes and scales equal
  the library's own quantiser applied to the fused kernel's bf16 output, which
  equals fp8bq_gemm's; and the dequantised codes lie within the GEMM tolerance
  plus the two roundings (bf16, then E4M3) of the oracle's accumulation.
"""

import numpy as np
import pytest

import fp8_fine_grained_fp8bq_amd as fb
from oracle import e4m3
from oracle import gemm as og
from oracle import quant as oq
from tests.gpu_util import check_gemm_bf16, dev, dev_bf16, host, host_bf16_bits, log
from workloads import act, large_fprop, pow2_scales, small_codes

pytestmark = pytest.mark.gpu


def _dev_scales_chunk_major(s_rows):
    """[rows, K/128] (oracle layout) -> device [K/128, rows] (C ABI layout)."""
    # a fresh copy: a transposed view with a length-1 dimension keeps strides
    # that would give the tensor a leading dimension of 1
    return dev(np.asarray(s_rows, np.float32).T.copy())


@pytest.mark.parametrize("in_pow2", [False, True])
@pytest.mark.parametrize("qmode", ["exact", "pow2"])
@pytest.mark.parametrize("m,n,k,seed", [(300, 384, 512, 81), (64, 128, 128, 82), (513, 640, 256, 83)])
def test_exact_output_bit_exact(m, n, k, seed, qmode, in_pow2):
    qa = small_codes(seed, m, k)
    qa[m // 3] = 0                                   # a zero output row
    qb = small_codes(seed + 1, n, k)
    sa = pow2_scales(seed + 2, (m, k // 128))
    sb = pow2_scales(seed + 3, (n // 128, k // 128))
    log(f"[gemm_quant] exact-output {m}x{n}x{k} q={qmode} in_pow2={in_pow2}")
    op = fb.FPROP | (fb.SCALE_POW2 if in_pow2 else 0)
    y, q, s = fb.gemm_quant(op, dev(qa), _dev_scales_chunk_major(sa), dev(qb), dev(sb), qpow2=qmode == "pow2")
    y32, _, _ = og.fprop(qa, sa, qb, sb)
    bits, q0, s0 = og.quantise_output(y32, qmode)
    np.testing.assert_array_equal(host_bf16_bits(y), bits)
    np.testing.assert_array_equal(host(s).T.view(np.uint32), s0.view(np.uint32))
    np.testing.assert_array_equal(host(q), q0)


def _quant_operands(x, w, pow2, dgrad=False):
    xq, xs = fb.quant_act_1x128(dev_bf16(x), fb.SCALE_POW2 if pow2 else fb.ACT_ROWWISE)
    wq, ws, wqt = fb.quant_w_128x128(dev_bf16(w), transposed_copy=dgrad, pow2=pow2)
    return xq, xs, (wqt if dgrad else wq), ws


def _check_general(y, q, s, y_plain, qmode, y32, ab, name):
    """Fused = plain GEMM output, codes = the library quantiser of it, and the
    dequantised codes within the oracle's bound."""
    import torch
    assert torch.equal(y.view(torch.int16), y_plain.view(torch.int16)), f"{name}: bf16 output differs from fp8bq_gemm"
    q2, s2 = fb.quant_act_1x128(y, fb.SCALE_POW2 if qmode == "pow2" else fb.ACT_ROWWISE)
    assert torch.equal(q, q2), f"{name}: codes differ from the quantiser's"
    assert torch.equal(s.view(torch.int32), s2.view(torch.int32)), f"{name}: scales differ from the quantiser's"
    qh, sh = host(q), host(s).T
    rec = e4m3.decode(qh) * np.repeat(sh.astype(np.float64), 128, axis=1)
    ybits = host_bf16_bits(y)
    yb = og.bf16_bits_to_f64(ybits)
    # bf16 output: the GPU's accumulation within the GEMM tolerance (and the
    # canary) of the oracle's before its rounding to bf16; codes within the E4M3
    # rounding of that output
    stats = check_gemm_bf16(ybits, y32, ab)
    assert stats["bad"] == 0 and stats["outside_tight"] == 0, f"{name}: bf16 output {stats}"
    s_full = np.repeat(sh.astype(np.float64), 128, axis=1)
    tol_q = np.maximum(2.0 ** -4 * (1 + 2.0 ** -18) * np.abs(yb), 2.0 ** -10 * s_full)
    assert np.all(np.abs(rec - yb) <= tol_q), f"{name}: codes"


@pytest.mark.parametrize("qmode", ["exact", "pow2"])
@pytest.mark.parametrize("in_pow2", [False, True])
def test_fprop_general_inputs(qmode, in_pow2):
    m, n, k = 520, 512, 640
    x = act(84, m, k, dist="student_t3", outlier_p=0.002, outlier_mult=20)
    w = act(85, n, k, std=0.02)
    log(f"[gemm_quant] fprop general {m}x{n}x{k} q={qmode} in_pow2={in_pow2}")
    xq, xs, wq, ws = _quant_operands(x, w, in_pow2)
    op = fb.FPROP | (fb.SCALE_POW2 if in_pow2 else 0)
    y, q, s = fb.gemm_quant(op, xq, xs, wq, ws, qpow2=qmode == "pow2")
    y_plain = fb.gemm(op, xq, xs, wq, ws)
    mode = "pow2" if in_pow2 else "exact"
    qx0, sx0 = oq.quant_act_1x128(x, mode)
    qw0, sw0 = oq.quant_w_128x128(w, mode)
    np.testing.assert_array_equal(host(xq), qx0)
    np.testing.assert_array_equal(host(wq), qw0)
    y32, _, ab = og.fprop(qx0, sx0, qw0, sw0)
    _check_general(y, q, s, y_plain, qmode, y32, ab, "fprop general")


def test_dgrad_general_inputs():
    m, nw, kw = 200, 256, 384
    dy = act(86, m, nw, std=1e-3)
    w = act(87, nw, kw, std=0.02)
    log(f"[gemm_quant] dgrad dY{dy.shape} W{w.shape}")
    dq, ds, wqt, ws = _quant_operands(dy, w, False, dgrad=True)
    y, q, s = fb.gemm_quant(fb.DGRAD, dq, ds, wqt, ws)
    y_plain = fb.gemm(fb.DGRAD, dq, ds, wqt, ws)
    qd0, sd0 = oq.quant_act_1x128(dy)
    qw0, sw0 = oq.quant_w_128x128(w)
    y32, _, ab = og.dgrad(qd0, sd0, qw0, sw0)
    _check_general(y, q, s, y_plain, "exact", y32, ab, "dgrad general")


def test_without_bf16_output_and_leading_dimensions():
    import torch
    m, n, k = 384, 256, 384
    x = act(88, m, k, outlier_p=0.01, outlier_mult=100)
    w = act(89, n, k, std=0.02)
    log(f"[gemm_quant] no bf16 output, padded ld {m}x{n}x{k}")
    xq, xs, wq, ws = _quant_operands(x, w, False)
    y, q, s = fb.gemm_quant(fb.FPROP, xq, xs, wq, ws)
    ldq, lds = n + 48, m + 20
    qp = torch.full((m, ldq), 0xA5, dtype=torch.uint8, device="cuda")
    sp = torch.full((n // 128, lds), -1.0, dtype=torch.float32, device="cuda")
    fb.fp8bq_gemm_quant(fb.FPROP, m, n, k, xq.data_ptr(), k, xs.data_ptr(), xs.stride(0), wq.data_ptr(), k,
                        ws.data_ptr(), ws.stride(0), None, n, qp.data_ptr(), ldq, sp.data_ptr(), lds, 0,
                        torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert torch.equal(qp[:, :n], q) and torch.equal(sp[:, :m], s)
    assert bool((qp[:, n:] == 0xA5).all()) and bool((sp[:, m:] == -1.0).all()), "wrote past the tiles"


def test_large_workload_sampled_rows():
    # the large fprop (16384 x 18432 x 7168) in the launch configuration the
    # bench times: the whole output against the quantiser on the GPU, sampled
    # rows against the oracle
    import torch
    cfg = large_fprop()
    log("[gemm_quant] large 16384x18432x7168")
    xq, xs, wq, ws = _quant_operands(cfg.x, cfg.w, False)
    y, q, s = fb.gemm_quant(fb.FPROP, xq, xs, wq, ws)
    q2, s2 = fb.quant_act_1x128(y)
    assert torch.equal(q, q2) and torch.equal(s.view(torch.int32), s2.view(torch.int32))
    rows = np.unique(np.concatenate([[0, 16383], np.random.default_rng(90).choice(16384, 6, replace=False)]))
    qx0, sx0 = oq.quant_act_1x128(cfg.x[rows])
    qw0, sw0 = oq.quant_w_128x128(cfg.w)
    y32, _, ab = og.fprop(qx0, sx0, qw0, sw0)
    qh, sh = host(q)[rows], host(s).T[rows]
    ybits = host_bf16_bits(y)[rows]
    yb = og.bf16_bits_to_f64(ybits)
    stats = check_gemm_bf16(ybits, y32, ab)
    assert stats["bad"] == 0 and stats["outside_tight"] == 0, f"large workload: bf16 output {stats}"
    rec = e4m3.decode(qh) * np.repeat(sh.astype(np.float64), 128, axis=1)
    s_full = np.repeat(sh.astype(np.float64), 128, axis=1)
    tol_q = np.maximum(2.0 ** -4 * (1 + 2.0 ** -18) * np.abs(yb), 2.0 ** -10 * s_full)
    assert np.all(np.abs(rec - yb) <= tol_q)
