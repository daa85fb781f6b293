"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, and rejects bad arguments with the documented status before
making any HIP call. Valid arguments on a machine without a GPU give
FP8BQ_E_DEVICE (only run where no device is visible, so nothing is launched)."""

import ctypes
import os
import re

import pytest

import fp8_fine_grained_fp8bq_amd as fb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8bq.h")

A16 = 0x10000          # stand-in "device addresses": 16-byte aligned, never dereferenced
B16 = 0x20000
S4 = 0x30000
O16 = 0x40000


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(fb.LIB_PATH):
        pytest.skip("libfp8bq.so not built (run __graft_entry__.build())")
    return fb.lib()


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(fp8bq_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_four_entry_points():
    d = _declared()
    for name in ("fp8bq_quant_act_1x128", "fp8bq_quant_w_128x128", "fp8bq_requant_t_128x1", "fp8bq_gemm",
                 "fp8bq_gemm_quant", "fp8bq_grouped_gemm", "fp8bq_grouped_gemm_decode", "fp8bq_last_error"):
        assert name in d


def test_every_declared_symbol_is_exported(L):
    for name in _declared():
        assert hasattr(L, name), name
    assert set(_declared()) <= set(fb.EXPORTS)
    assert L.fp8bq_version().decode().startswith("fp8bq")


def _st(L, fn, *args):
    return getattr(L, fn)(*args)


def test_quant_act_validation(L):
    f = "fp8bq_quant_act_1x128"
    ok = [A16, 256, 1024, 1024, 0, B16, 1024, S4, 256, None]
    assert _st(L, f, *[None] + ok[1:]) == fb.E_INVAL
    assert _st(L, f, *ok[:1] + [0] + ok[2:]) == fb.E_INVAL                      # rows
    assert _st(L, f, *ok[:4] + [2] + ok[5:]) == fb.E_INVAL                      # mode
    assert _st(L, f, *ok[:4] + [0x12] + ok[5:]) == fb.E_INVAL                   # mode with the pow2 flag
    assert _st(L, f, *ok[:3] + [1000] + ok[4:]) == fb.E_INVAL                   # ldx < cols
    assert _st(L, f, *ok[:2] + [1000, 1000] + ok[4:6] + [1000] + ok[7:]) == fb.E_SHAPE
    assert _st(L, f, *ok[:8] + [255, None]) == fb.E_INVAL                       # lds < rows
    assert _st(L, f, *[A16 + 2] + ok[1:]) == fb.E_ALIGN
    assert _st(L, f, *ok[:3] + [1028] + ok[4:]) == fb.E_ALIGN                   # ldx % 8
    big = 1 << 30                                                               # 2^31 blocks of 32 rows x 128
    assert _st(L, f, A16, big, 8192, 8192, 0, B16, 8192, S4, big, None) == fb.E_SHAPE
    assert "too large" in L.fp8bq_last_error().decode()
    col = [A16, 200, 1024, 1024, 1, B16, 256, S4, 1024, None]
    assert _st(L, f, *col) == fb.E_SHAPE                                        # rows % 128 (col-wise)
    col[1] = 256
    col[6] = 200
    assert _st(L, f, *col) == fb.E_INVAL                                        # ldq < rows
    assert "ldq" in L.fp8bq_last_error().decode()
    # col-wise grid: rows / 128 blocks along x, cols / 128 along y (at most 65535)
    wide = 128 * 65536
    assert _st(L, f, A16, 128, wide, wide, 1, B16, 128, S4, wide, None) == fb.E_SHAPE
    assert "too large" in L.fp8bq_last_error().decode()
    assert _st(L, f, A16, 128, wide - 128, wide - 128, 1, B16, 128, S4, wide, None) == fb.E_DEVICE


def test_quant_w_validation(L):
    f = "fp8bq_quant_w_128x128"
    ok = [A16, 256, 384, 384, B16, 384, S4, 3, O16, 256, 0, None]
    assert _st(L, f, *[A16, 0] + ok[2:]) == fb.E_INVAL
    assert _st(L, f, *ok[:1] + [200, 384, 384] + ok[4:]) == fb.E_SHAPE
    assert _st(L, f, *ok[:7] + [2] + ok[8:]) == fb.E_INVAL                      # lds < k/128
    assert _st(L, f, *ok[:9] + [128, 0, None]) == fb.E_INVAL                    # ldqt < n
    assert _st(L, f, *ok[:8] + [O16 + 1, 256, 0, None]) == fb.E_ALIGN
    assert _st(L, f, *ok[:4] + [B16 + 8] + ok[5:]) == fb.E_ALIGN
    assert _st(L, f, *ok[:10] + [0x20, None]) == fb.E_INVAL                     # unknown flag
    assert "flags" in L.fp8bq_last_error().decode()


def test_requant_validation(L):
    f = "fp8bq_requant_t_128x1"
    # rows, cols = 256, 384: q [256, 384] ldq 384, s lds 256, qt [384, 256] ldqt 256, st ldst 384
    ok = [A16, 256, 384, 384, S4, 256, B16, 256, S4 + 4096, 384, 0, None]
    def bad(i, v):
        a = list(ok); a[i] = v
        return _st(L, f, *a)
    assert bad(0, None) == fb.E_INVAL
    assert bad(10, 1) == fb.E_INVAL and "flags" in L.fp8bq_last_error().decode()
    assert bad(10, 1 | fb.SCALE_POW2) == fb.E_INVAL
    assert bad(10, fb.SCALE_POW2) == fb.E_DEVICE                                # the power-of-two hint
    assert bad(1, 0) == fb.E_INVAL
    assert bad(1, 200) == fb.E_SHAPE
    assert bad(2, 300) == fb.E_SHAPE
    assert bad(3, 256) == fb.E_INVAL                                            # ldq < cols
    assert bad(5, 128) == fb.E_INVAL                                            # lds < rows
    assert bad(7, 128) == fb.E_INVAL                                            # ldqt < rows
    assert bad(9, 256) == fb.E_INVAL                                            # ldst < cols
    assert bad(6, B16 + 8) == fb.E_ALIGN
    assert bad(3, 392) == fb.E_ALIGN                                            # ldq % 16
    assert bad(8, S4 + 2) == fb.E_ALIGN
    wide = 128 * 65536                                                          # 65536 column blocks: one past the grid
    assert _st(L, f, A16, 128, wide, wide, S4, 128, B16, 128, S4 + 4096, wide, 0, None) == fb.E_SHAPE
    assert "too large" in L.fp8bq_last_error().decode()


def test_requant_e5m6_validation(L):
    f = "fp8bq_requant_e5m6_t_128x1"
    # rows, cols = 256, 384: packed codes 576 bytes per row, s lds 256, qt [384, 256] ldqt 256, st ldst 384
    ok = [A16, 256, 384, 576, S4, 256, B16, 256, S4 + 4096, 384, None]
    def bad(i, v):
        a = list(ok); a[i] = v
        return _st(L, f, *a)
    assert _st(L, f, *ok) == fb.E_DEVICE
    assert bad(0, None) == fb.E_INVAL and bad(8, None) == fb.E_INVAL
    assert bad(1, 0) == fb.E_INVAL
    assert bad(1, 200) == fb.E_SHAPE                                            # rows % 128
    assert bad(2, 300) == fb.E_SHAPE                                            # cols % 128
    assert bad(3, 560) == fb.E_INVAL                                            # ldq < 1.5 cols
    assert bad(5, 255) == fb.E_INVAL                                            # lds < rows
    assert bad(7, 128) == fb.E_INVAL                                            # ldqt < rows
    assert bad(9, 383) == fb.E_INVAL                                            # ldst < cols
    assert bad(0, A16 + 4) == fb.E_ALIGN
    assert bad(6, B16 + 8) == fb.E_ALIGN
    assert bad(3, 584) == fb.E_ALIGN                                            # ldq % 16
    assert bad(7, 264) == fb.E_ALIGN                                            # ldqt % 16
    assert bad(4, S4 + 2) == fb.E_ALIGN
    wide = 128 * 65536                                                          # 65536 column blocks: one past the grid
    assert _st(L, f, A16, 128, wide, 192 * 65536, S4, 128, B16, 128, S4, wide, None) == fb.E_SHAPE
    assert "too large" in L.fp8bq_last_error().decode()


@pytest.mark.parametrize("f", ["fp8bq_cache_e5m6_1x128", "fp8bq_uncache_e5m6_1x128"])
def test_e5m6_validation(L, f):
    # rows, cols = 100, 384: bf16 [100, 384] ld 384; packed codes 576 bytes per row, ldq 576; s lds 100
    cache = f == "fp8bq_cache_e5m6_1x128"
    ok = ([A16, 100, 384, 384, B16, 576, S4, 100, None] if cache
          else [B16, 100, 384, 576, S4, 100, A16, 384, None])
    ld16, ldq, lds, p16, pq = (3, 5, 7, 0, 4) if cache else (7, 3, 5, 6, 0)
    def bad(i, v):
        a = list(ok); a[i] = v
        return _st(L, f, *a)
    assert bad(p16, None) == fb.E_INVAL
    assert bad(1, 0) == fb.E_INVAL
    assert bad(2, 300) == fb.E_SHAPE                                            # cols % 128
    assert bad(ld16, 256) == fb.E_INVAL                                         # bf16 ld < cols
    assert bad(ldq, 560) == fb.E_INVAL                                          # ldq < 1.5 cols
    assert bad(lds, 99) == fb.E_INVAL                                           # lds < rows
    assert bad(p16, A16 + 8) == fb.E_ALIGN
    assert bad(pq, B16 + 4) == fb.E_ALIGN
    assert bad(ldq, 584) == fb.E_ALIGN                                          # ldq % 16
    assert bad(ld16, 388) == fb.E_ALIGN                                         # bf16 ld % 8
    assert bad(6 if cache else 4, S4 + 2) == fb.E_ALIGN
    # 2^20 rows x 32768 tiles per row: 2^30 workgroups of 32 rows but 2^31 of the kernels' 16 rows
    rows, cols = 1 << 20, 128 * 32768
    big = ([A16, rows, cols, cols, B16, cols * 3 // 2, S4, rows, None] if cache
           else [B16, rows, cols, cols * 3 // 2, S4, rows, A16, cols, None])
    assert _st(L, f, *big) == fb.E_SHAPE and "too large" in L.fp8bq_last_error().decode()


def _gemm_ok(op=0):
    # m, n, k = 300, 384, 1024
    ldsb = {0: 8, 1: 3, 2: 384}[op]
    return [op, 300, 384, 1024, A16, 1024, S4, 300, B16, 1024, S4, ldsb, O16, 384, None]


def test_gemm_validation(L):
    f = "fp8bq_gemm"
    for op in (0, 1, 2):
        ok = _gemm_ok(op)
        bad = list(ok); bad[0] = 3
        assert _st(L, f, *bad) == fb.E_INVAL
        bad = list(ok); bad[4] = None
        assert _st(L, f, *bad) == fb.E_INVAL
        bad = list(ok); bad[3] = 1000; bad[5] = 1008; bad[9] = 1008
        assert _st(L, f, *bad) == fb.E_SHAPE                                   # k % 128
        bad = list(ok); bad[2] = 200; bad[13] = 208
        assert _st(L, f, *bad) == fb.E_SHAPE                                   # n % 128
        bad = list(ok); bad[7] = 299
        assert _st(L, f, *bad) == fb.E_INVAL                                   # ldsa < m
        bad = list(ok); bad[11] = ok[11] - 1
        assert _st(L, f, *bad) == fb.E_INVAL                                   # ldsb
        bad = list(ok); bad[5] = 1032
        assert _st(L, f, *bad) == fb.E_ALIGN                                   # lda % 16
        bad = list(ok); bad[12] = O16 + 8
        assert _st(L, f, *bad) == fb.E_ALIGN
        bad = list(ok); bad[13] = 383
        assert _st(L, f, *bad) == fb.E_INVAL                                   # ldo < n
        bad = list(ok); bad[0] = op | 0x20
        assert _st(L, f, *bad) == fb.E_INVAL                                   # unknown flag


Q16 = 0x50000


def _gemm_quant_ok(op=0):
    # m, n, k = 300, 384, 1024; bf16 output, codes [300, 384] (ldq 384), scales [3, 300]
    return _gemm_ok(op)[:14] + [Q16, 384, S4, 300, 0, None]


def test_gemm_quant_validation(L):
    f = "fp8bq_gemm_quant"
    for op in (0, 1):
        ok = _gemm_quant_ok(op)
        bad = list(ok); bad[0] = 2
        assert _st(L, f, *bad) == fb.E_INVAL                                   # WGRAD has no bf16 output
        bad = list(ok); bad[14] = None
        assert _st(L, f, *bad) == fb.E_INVAL                                   # null q
        bad = list(ok); bad[16] = None
        assert _st(L, f, *bad) == fb.E_INVAL                                   # null s
        bad = list(ok); bad[18] = 1
        assert _st(L, f, *bad) == fb.E_INVAL                                   # unknown qflags
        bad = list(ok); bad[15] = 368
        assert _st(L, f, *bad) == fb.E_INVAL                                   # ldq < n
        bad = list(ok); bad[17] = 299
        assert _st(L, f, *bad) == fb.E_INVAL                                   # lds < m
        bad = list(ok); bad[14] = Q16 + 4
        assert _st(L, f, *bad) == fb.E_ALIGN
        bad = list(ok); bad[15] = 392
        assert _st(L, f, *bad) == fb.E_ALIGN                                   # ldq % 16
        bad = list(ok); bad[16] = S4 + 2
        assert _st(L, f, *bad) == fb.E_ALIGN
        bad = list(ok); bad[2] = 200; bad[13] = 208; bad[15] = 208
        assert _st(L, f, *bad) == fb.E_SHAPE                                   # n % 128
        bad = list(ok); bad[7] = 299
        assert _st(L, f, *bad) == fb.E_INVAL                                   # ldsa < m


def test_grouped_validation(L):
    f = "fp8bq_grouped_gemm"
    P = ctypes.POINTER(ctypes.c_int64)

    def off(*v):
        return (ctypes.c_int64 * len(v))(*v)
    base = [None, 2048, 7168, A16, 7168, S4, 512, B16, 7168, S4, 56, O16, 2048, 0, None]
    assert _st(L, f, 0, off(0), *base[1:]) == fb.E_INVAL
    assert _st(L, f, 257, off(*([0] * 258)), *base[1:]) == fb.E_INVAL
    assert _st(L, f, 2, None, *base[1:]) == fb.E_INVAL
    assert _st(L, f, 2, off(128, 256, 512), *base[1:]) == fb.E_SHAPE          # row_off[0] != 0
    assert _st(L, f, 2, off(0, 256, 128), *base[1:]) == fb.E_SHAPE            # decreasing
    assert _st(L, f, 2, off(0, 100, 512), *base[1:]) == fb.E_SHAPE            # not multiple of 128
    bad = list(base); bad[6] = 500
    assert _st(L, f, 2, off(0, 256, 512), *bad[1:]) == fb.E_INVAL             # ldsa < m
    bad = list(base); bad[10] = 55
    assert _st(L, f, 2, off(0, 256, 512), *bad[1:]) == fb.E_INVAL             # ldsb < k/128
    bad = list(base); bad[13] = 1
    assert _st(L, f, 2, off(0, 256, 512), *bad[1:]) == fb.E_INVAL             # unknown flag
    assert isinstance(P, type)


def test_grouped_decode_validation(L):
    f = "fp8bq_grouped_gemm_decode"

    def off(*v):
        return (ctypes.c_int64 * len(v))(*v)
    base = [None, 2048, 7168, A16, 7168, S4, 512, B16, 7168, S4, 56, O16, 2048, 0, None]
    assert _st(L, f, 0, off(0), *base[1:]) == fb.E_INVAL
    assert _st(L, f, 2, None, *base[1:]) == fb.E_INVAL
    assert _st(L, f, 2, off(3, 10, 20), *base[1:]) == fb.E_SHAPE              # row_off[0] != 0
    assert _st(L, f, 2, off(0, 30, 20), *base[1:]) == fb.E_SHAPE              # decreasing
    assert _st(L, f, 2, off(0, 257, 300), *base[1:]) == fb.E_SHAPE            # a group of 257 rows
    bad = list(base); bad[13] = 1
    assert _st(L, f, 2, off(0, 30, 50), *bad[1:]) == fb.E_INVAL               # flags
    bad = list(base); bad[6] = 40
    assert _st(L, f, 2, off(0, 30, 50), *bad[1:]) == fb.E_INVAL               # ldsa < m
    bad = list(base); bad[1] = 2000; bad[12] = 2000
    assert _st(L, f, 2, off(0, 30, 50), *bad[1:]) == fb.E_SHAPE              # n % 128
    bad = list(base); bad[3] = A16 + 8
    assert _st(L, f, 2, off(0, 30, 50), *bad[1:]) == fb.E_ALIGN


def test_grouped_decode_workspace_forms_validation(L):
    def off(*v):
        return (ctypes.c_int64 * len(v))(*v)
    big = off(0, 217, 260)                       # 217 and 43 rows: both split (14 + 3 subtiles of 16 rows)
    need = ctypes.c_int64(-1)
    assert L.fp8bq_grouped_gemm_decode_workspace_size(2, big, 2048, 7168, ctypes.byref(need)) == fb.OK
    assert need.value == 256 * 256 * 4 + 2 * 17 * 16 * 2048 * 4
    assert fb.fp8bq_grouped_gemm_decode_workspace_size(2, [0, 30, 50], 2048, 7168) == 0    # nothing split
    assert fb.fp8bq_grouped_gemm_decode_workspace_size(2, [0, 217, 260], 2048, 128) == 0   # one chunk: no halves
    assert fb.fp8bq_grouped_gemm_decode_workspace_size(2, [0, 217, 260], 128 * 257, 7168) == 0   # n > 32768
    assert L.fp8bq_grouped_gemm_decode_workspace_size(2, big, 2048, 7168, None) == fb.E_INVAL
    assert L.fp8bq_grouped_gemm_decode_workspace_size(2, off(0, 300, 310), 2048, 7168, ctypes.byref(need)) == fb.E_SHAPE
    f = "fp8bq_grouped_gemm_decode_ws"
    args = [2048, 7168, A16, 7168, S4, 512, B16, 7168, S4, 56, O16, 2048]
    w = need.value
    assert _st(L, f, 2, big, *args, Q16, w, 0, None) == fb.E_DEVICE
    assert _st(L, f, 2, big, *args, None, w, 0, None) == fb.E_INVAL                     # workspace missing
    assert "workspace" in L.fp8bq_last_error().decode()
    assert _st(L, f, 2, big, *args, Q16, w - 1, 0, None) == fb.E_INVAL                  # too small
    assert _st(L, f, 2, big, *args, Q16 + 8, w, 0, None) == fb.E_ALIGN
    assert _st(L, f, 2, big, *args, Q16, w, 1, None) == fb.E_INVAL                      # flags
    assert _st(L, f, 2, off(0, 30, 50), *args, None, 0, 0, None) == fb.E_DEVICE         # no workspace needed
    f = "fp8bq_grouped_gemm_decode_noalloc"
    assert _st(L, f, 2, big, *args, 0, None) == fb.E_DEVICE
    assert _st(L, f, 2, big, *args, 1, None) == fb.E_INVAL
    huge = off(*[256 * e for e in range(9)])     # 8 x 256 rows at n = 4096: 64 MiB of partial sums
    assert _st(L, f, 8, huge, 4096, 7168, A16, 7168, S4, 2048, B16, 7168, S4, 56, O16, 4096, 0, None) == fb.E_SHAPE
    assert "scratch" in L.fp8bq_last_error().decode()


def test_binding_raises_with_message(L):
    with pytest.raises(fb.Fp8bqError) as ei:
        fb.fp8bq_gemm(7, 1, 128, 128, A16, 128, S4, 1, B16, 128, S4, 1, O16, 128, 0)
    assert ei.value.status == fb.E_INVAL and "op" in str(ei.value)


def _no_device():
    try:
        import torch
        return torch.cuda.device_count() == 0
    except Exception:
        return True


@pytest.mark.skipif(not _no_device(), reason="a GPU is visible; valid arguments would launch")
def test_valid_arguments_without_device_report_e_device(L):
    assert _st(L, "fp8bq_gemm", *_gemm_ok(0)) == fb.E_DEVICE
    assert _st(L, "fp8bq_quant_act_1x128", A16, 256, 1024, 1024, 0, B16, 1024, S4, 256, None) == fb.E_DEVICE
    assert _st(L, "fp8bq_quant_w_128x128", A16, 256, 384, 384, B16, 384, S4, 3, None, 0, 0, None) == fb.E_DEVICE
    off = (ctypes.c_int64 * 3)(0, 256, 512)
    assert _st(L, "fp8bq_grouped_gemm", 2, off, 2048, 7168, A16, 7168, S4, 512, B16, 7168, S4, 56,
               O16, 2048, 0, None) == fb.E_DEVICE
    # the power-of-two flag is accepted everywhere
    pow2 = fb.SCALE_POW2
    assert _st(L, "fp8bq_gemm", *([_gemm_ok(0)[0] | pow2] + _gemm_ok(0)[1:])) == fb.E_DEVICE
    assert _st(L, "fp8bq_gemm", *([_gemm_ok(2)[0] | pow2] + _gemm_ok(2)[1:])) == fb.E_DEVICE
    assert _st(L, "fp8bq_quant_act_1x128", A16, 256, 1024, 1024, 1 | pow2, B16, 256, S4, 1024, None) == fb.E_DEVICE
    assert _st(L, "fp8bq_quant_w_128x128", A16, 256, 384, 384, B16, 384, S4, 3, None, 0, pow2, None) == fb.E_DEVICE
    assert _st(L, "fp8bq_grouped_gemm", 2, off, 2048, 7168, A16, 7168, S4, 512, B16, 7168, S4, 56,
               O16, 2048, pow2, None) == fb.E_DEVICE
    assert _st(L, "fp8bq_gemm_quant", *_gemm_quant_ok(0)) == fb.E_DEVICE
    no_out = _gemm_quant_ok(1); no_out[12] = None; no_out[18] = pow2
    assert _st(L, "fp8bq_gemm_quant", *no_out) == fb.E_DEVICE               # bf16 output optional
    assert _st(L, "fp8bq_grouped_gemm_decode", 3, (ctypes.c_int64 * 4)(0, 17, 17, 273), 2048, 7168, A16, 7168,
               S4, 512, B16, 7168, S4, 56, O16, 2048, 0, None) == fb.E_DEVICE
    assert "device" in L.fp8bq_last_error().decode()


# ---------------------------------------------------------------------------
# the probe library (include/fp8bq_probe.h): exports and host-side validation
# ---------------------------------------------------------------------------

PROBE_HEADER = os.path.join(ROOT, "include", "fp8bq_probe.h")


@pytest.fixture(scope="module")
def P():
    from fp8_fine_grained_fp8bq_amd import probe
    if not os.path.exists(probe.LIB_PATH):
        pytest.skip("libfp8bq_probe.so not built (run __graft_entry__.build())")
    return probe.lib()


def test_probe_symbols_exported(P):
    from fp8_fine_grained_fp8bq_amd import probe
    text = open(PROBE_HEADER).read()
    declared = sorted(set(re.findall(r"\b(fp8bq_probe_[a-z0-9_]+)\s*\(", text)))
    assert declared and set(declared) == set(probe.EXPORTS)
    for name in declared:
        assert hasattr(P, name), name


def test_probe_validation(P):
    assert P.fp8bq_probe_mfma_accum(None, B16, 4096, S4, S4, None) == fb.E_INVAL
    assert P.fp8bq_probe_mfma_accum(A16, B16, 4000, S4, S4, None) == fb.E_SHAPE
    assert P.fp8bq_probe_mfma_accum(A16, B16, 0, S4, S4, None) == fb.E_SHAPE
    assert P.fp8bq_probe_mfma_accum(A16 + 4, B16, 4096, S4, S4, None) == fb.E_ALIGN
    assert P.fp8bq_probe_mfma_once(A16, None, S4, S4, None) == fb.E_INVAL
    assert P.fp8bq_probe_mfma_once(A16, B16 + 8, S4, S4, None) == fb.E_ALIGN
    assert P.fp8bq_probe_mfma_stream(1, 0, 256, A16, S4, S4, S4, None) == fb.E_INVAL
    assert P.fp8bq_probe_mfma_stream(1, 16, 0, A16, S4, S4, S4, None) == fb.E_INVAL
    assert P.fp8bq_probe_mfma_stream(1, 16, 256, A16 + 1, S4, S4, S4, None) == fb.E_ALIGN
    assert P.fp8bq_probe_stream_2to1(None, B16, 1024, None) == fb.E_INVAL
    assert P.fp8bq_probe_stream_2to1(A16, B16, 1000, None) == fb.E_SHAPE
    assert P.fp8bq_probe_stream_2to1(A16, B16 + 4, 1024, None) == fb.E_ALIGN
    assert "aligned" in P.fp8bq_probe_last_error().decode()
