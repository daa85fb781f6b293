"""The accumulation probe: how gfx950's FP8 matrix instruction sums products,
repeating the experiment of the DeepSeek-V3 report (Chinese translation),
section 3.3.2 "increasing accumulation precision" (two random matrices, K =
4096, accumulated inside the matrix unit: maximum relative error near 2% on
H800, whose tensor cores keep about 14 bits, section 3.5.2), next to the
promotion every 128 K-elements that the GEMM uses.

The exact reference is an integer dot product: every E4M3 value is an integer
multiple of 2^-9, so sum_k a_k b_k is an int64 sum in units of 2^-18.

What these tests pin (and the GEMM tests' canary bound rests on):
* promoted every 128: error at most 2^-14 of sum_k |a_k b_k| (measured about
  1e-6), far inside the acceptance bound 2e-3;
* chained inside the unit over K = 4096: no worse than promoted (measured: the
  same error). Unlike the report's H800 tensor cores, gfx950's unit adds its
  result into the FP32 C operand at full FP32 precision; what it loses is
  inside one instruction;
* one instruction on crafted inputs: products in the same block of 8 k are
  aligned to the block's largest with limited precision (2^16 + 1 -> 2^16),
  products in different blocks are added in FP32 (2^16 + 1 exact), and C is
  added in FP32.
On gfx950 the promotion every 128 K-elements is therefore what applies each
chunk's scales, and it costs no accuracy either way.
"""

import numpy as np
import pytest

from oracle import e4m3
from tests.gpu_util import dev, host, log

pytestmark = pytest.mark.gpu

CODE_256 = 0x78    # E4M3 2^8
CODE_1 = 0x38      # E4M3 1.0


def _int_units(codes):
    """E4M3 codes -> exact integer values in units of 2^-9 (int64)."""
    return np.round(e4m3.decode(codes) * 512.0).astype(np.int64)


def _probe():
    from fp8_fine_grained_fp8bq_amd import probe
    return probe


def _accum(a, b):
    import torch
    probe = _probe()
    k = a.shape[1]
    chained = torch.empty((16, 16), dtype=torch.float32, device="cuda")
    promoted = torch.empty((16, 16), dtype=torch.float32, device="cuda")
    da, db = dev(a), dev(b)
    probe.fp8bq_probe_mfma_accum(da.data_ptr(), db.data_ptr(), k, chained.data_ptr(), promoted.data_ptr(),
                                 torch.cuda.current_stream().cuda_stream)
    return host(chained).astype(np.float64), host(promoted).astype(np.float64)


def _random_codes(seed, rows, k):
    # N(0, 1) values scaled so the largest maps near 448 (per-tensor, as a quantiser would)
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, k))
    return e4m3.encode((x * (448.0 / np.abs(x).max())).astype(np.float32))


def test_accumulation_k4096_against_promotion():
    k = 4096
    a, b = _random_codes(501, 16, k), _random_codes(502, 16, k)
    log(f"[probe] accumulation 16x16x{k}")
    chained, promoted = _accum(a, b)
    ia, ib = _int_units(a), _int_units(b)
    exact = (ia @ ib.T).astype(np.float64) * 2.0 ** -18
    absum = (np.abs(ia) @ np.abs(ib).T).astype(np.float64) * 2.0 ** -18
    nz = exact != 0
    stats = {}
    for name, got in (("chained", chained), ("promoted", promoted)):
        err = np.abs(got - exact)
        stats[name] = {"max_err_over_sum_abs": float((err / absum).max()),
                       "max_rel_err": float((err[nz] / np.abs(exact[nz])).max())}
    log(f"  K={k}: {stats} (report, H800 tensor cores: max relative error ~2%)")
    assert stats["promoted"]["max_err_over_sum_abs"] <= 2.0 ** -14, stats
    assert stats["chained"]["max_err_over_sum_abs"] <= 2 * stats["promoted"]["max_err_over_sum_abs"] + 2.0 ** -24, stats


def _once(a, b, c=None):
    import torch
    probe = _probe()
    c = np.zeros((16, 16), np.float32) if c is None else c.astype(np.float32)
    d = torch.empty((16, 16), dtype=torch.float32, device="cuda")
    da, db, dc = dev(a), dev(b), dev(c)
    probe.fp8bq_probe_mfma_once(da.data_ptr(), db.data_ptr(), dc.data_ptr(), d.data_ptr(),
                                torch.cuda.current_stream().cuda_stream)
    return host(d).astype(np.float64)


def _pair(k0, k1):
    a = np.zeros((16, 128), np.uint8)
    b = np.zeros((16, 128), np.uint8)
    a[0, k0] = b[0, k0] = CODE_256        # product 2^16
    a[0, k1] = b[0, k1] = CODE_1          # product 1
    return a, b


def test_single_instruction_block_alignment():
    log("[probe] one 16x16x128 instruction on crafted products")
    same = _once(*_pair(0, 1))[0, 0]       # both products in the first block of 8 k
    apart = _once(*_pair(0, 64))[0, 0]     # in different blocks (another lane's k group)
    log(f"  2^16 + 1 in one block -> {same}; in different blocks -> {apart}")
    assert apart == 65537.0
    assert same == 65536.0
    # a single product is exact, and C is added in FP32
    a, b = _pair(0, 64)
    b[0, 64] = 0
    c = np.zeros((16, 16), np.float32)
    c[0, 0] = 1.0
    assert _once(a, b, c)[0, 0] == 65537.0


def test_power_stream_runs():
    # the matrix-unit stream with and without promotion FMAs (timed by the bench);
    # here only that it runs and keeps its results finite
    import torch
    probe = _probe()
    codes = dev(_random_codes(503, 4096, 1024).reshape(-1))
    scales = torch.full((64,), 1e-3, dtype=torch.float32, device="cuda")
    sink = torch.empty((256 * 512,), dtype=torch.float32, device="cuda")
    ticks = torch.zeros((512,), dtype=torch.int64, device="cuda")
    for fold in (0, 1):
        log(f"[probe] mfma stream fold={fold}")
        probe.fp8bq_probe_mfma_stream(fold, 16, 256, codes.data_ptr(), scales.data_ptr(), sink.data_ptr(),
                                      ticks.data_ptr(), torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        assert bool(torch.isfinite(sink).all())
        assert bool((ticks > 0).all())


def test_stream_2to1_moves_the_bytes():
    import torch
    probe = _probe()
    n = 1 << 20
    src = torch.randint(-32768, 32767, (n,), dtype=torch.int16, device="cuda")
    dst = torch.empty((n,), dtype=torch.uint8, device="cuda")
    log("[probe] stream 2-to-1")
    probe.fp8bq_probe_stream_2to1(src.data_ptr(), dst.data_ptr(), n, torch.cuda.current_stream().cuda_stream)
    expect = (src.cpu().numpy().view(np.uint16) >> 8).astype(np.uint8)
    np.testing.assert_array_equal(host(dst), expect)
