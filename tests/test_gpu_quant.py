"""GPU parity of the quantisers: FP8 bytes and fp32 scales must equal the
oracle's bit for bit, on seeded workloads, ragged shapes, padded leading
dimensions and the edge cases of the method (all-zero tiles, signed zeros,
tiny scales, every bf16 value at a power-of-two and at arbitrary scales)."""

import numpy as np
import pytest

import fp8_fine_grained_fp8bq_amd as fb
from oracle import quant as oq
from tests.gpu_util import dev_bf16, host, log
from workloads import act, dense_fprop, f32_to_bf16_bits, tiny_fprop

pytestmark = pytest.mark.gpu


def _gpu_act(bits, mode=fb.ACT_ROWWISE, ldx=None):
    rows, cols = bits.shape
    if ldx is not None and ldx != cols:
        buf = np.zeros((rows, ldx), np.uint16)
        buf[:, :cols] = bits
        t = dev_bf16(buf)[:, :cols]
    else:
        t = dev_bf16(bits)
    q, s = fb.quant_act_1x128(t, mode)
    return host(q), host(s)


def _assert_act_rows(bits, ldx=None, name=""):
    log(f"quant_act rowwise {name} shape={bits.shape} ldx={ldx}")
    q, s = _gpu_act(bits, fb.ACT_ROWWISE, ldx)
    q0, s0 = oq.quant_act_1x128(bits)
    np.testing.assert_array_equal(q, q0, err_msg=f"codes differ ({name})")
    np.testing.assert_array_equal(s.T.view(np.uint32), s0.view(np.uint32), err_msg=f"scales differ ({name})")


def test_tiny_config_rowwise():
    cfg = tiny_fprop()
    _assert_act_rows(cfg.x, name="tiny X")


@pytest.mark.parametrize("rows,cols,ldx,seed", [
    (1, 128, None, 1), (37, 384, None, 2), (257, 1024, 1088, 3), (64, 7168, None, 4), (3, 256, 264, 5),
    # 9 and 17 tiles per row: partial last 8-tile segment; 33 and 130 rows: partial last 32-row block
    (33, 1152, 1160, 6), (130, 2176, None, 8)])
def test_ragged_rowwise(rows, cols, ldx, seed):
    x = act(seed, rows, cols, dist="student_t3", outlier_p=0.003, outlier_mult=40)
    _assert_act_rows(x, ldx=ldx, name=f"seed {seed}")


def _all_bf16_upto(amax_bits: int) -> np.ndarray:
    """Rows of 128: element 0 is amax, the rest run through every finite bf16 with |x| <= amax."""
    bits = np.arange(65536, dtype=np.uint32)
    f = (bits << 16).view(np.float32)
    amax = float(np.array([amax_bits << 16], np.uint32).view(np.float32)[0])
    vals = bits[np.isfinite(f) & (np.abs(f) <= amax)].astype(np.uint16)
    per = 127
    rows = -(-len(vals) // per)
    x = np.zeros((rows, 128), np.uint16)
    x[:, 0] = amax_bits
    flat = np.zeros(rows * per, np.uint16)
    flat[:len(vals)] = vals
    x[:, 1:] = flat.reshape(rows, per)
    return x


def test_every_bf16_value_at_unit_scale():
    # amax = 448 gives s = 1 exactly: the codes are the plain E4M3 roundings of every bf16 in range
    _assert_act_rows(_all_bf16_upto(0x43E0), name="all bf16, s=1")


@pytest.mark.parametrize("amax_bits", [0x3F80, 0x3FB7, 0x40A3, 0x3C01, 0x447F, 0x2E9B])
def test_every_bf16_value_at_arbitrary_scale(amax_bits):
    _assert_act_rows(_all_bf16_upto(amax_bits), name=f"all bf16 up to {amax_bits:#x}")


def test_scale_for_every_bf16_absmax():
    # one tile per positive finite bf16 absmax (32639 of them), alternating signs; the
    # other elements are fixed fractions of it, so every scale the method can produce
    # is checked bit for bit, together with its codes
    amax = np.arange(1, 0x7F80, dtype=np.uint16)
    a = (amax.astype(np.uint32) << 16).view(np.float32)
    fr = np.linspace(-1, 1, 127, dtype=np.float32)
    body = f32_to_bf16_bits(a[:, None] * fr[None, :])          # |body| <= amax
    signs = np.where(np.arange(amax.size) % 2 == 1, 0x8000, 0).astype(np.uint16)
    x = np.concatenate([(amax | signs)[:, None], body], axis=1).astype(np.uint16)
    _assert_act_rows(x, name="every bf16 absmax")


def test_edge_tiles():
    x = act(7, 16, 1024, outlier_p=0).copy()
    x[0, 0:128] = 0                                    # all +0
    x[1, 0:128] = 0x8000                               # all -0
    x[2, 0:128] = 0; x[2, 5] = 0x8000; x[2, 6] = 0x0001   # amax = smallest bf16 subnormal
    x[3, 0:128] = np.arange(128, dtype=np.uint16) | 0x8000   # negative subnormals only
    x[4, 0:128] = f32_to_bf16_bits(np.linspace(-1e-36, 1e-36, 128).astype(np.float32))  # s < 2^-100
    x[5, 0:128] = f32_to_bf16_bits(np.full(128, -3.0e38, np.float32))                  # huge equal values
    x[6, 128:256] = f32_to_bf16_bits(np.array([1e-30] * 127 + [1e30], np.float32))      # extreme dynamic range
    x[7, 0:128] = f32_to_bf16_bits(np.array([448.0, -448.0] * 64, np.float32))
    _assert_act_rows(x, name="edge tiles")


def _assert_act_cols(bits, ldx=None, name=""):
    log(f"quant_act colwise {name} shape={bits.shape} ldx={ldx}")
    q, s = _gpu_act(bits, fb.ACT_COLWISE, ldx)
    q0, s0 = oq.quant_act_128x1(bits)
    np.testing.assert_array_equal(q, q0, err_msg=f"codes differ ({name})")
    np.testing.assert_array_equal(s.T.view(np.uint32), s0.view(np.uint32), err_msg=f"scales differ ({name})")


@pytest.mark.parametrize("rows,cols,ldx,seed", [(128, 128, None, 11), (256, 384, None, 12),
                                                 (384, 640, 704, 13), (128, 7168, None, 14)])
def test_colwise(rows, cols, ldx, seed):
    x = act(seed, rows, cols, std=1e-3, outlier_p=0.002, outlier_mult=30)
    _assert_act_cols(x, ldx=ldx, name=f"seed {seed}")


def test_colwise_edge_columns():
    x = act(15, 256, 128, outlier_p=0).copy()
    x[:128, 0] = 0
    x[:128, 1] = 0x8000
    x[128:, 2] = 0x0003
    x[:, 3] = f32_to_bf16_bits(np.linspace(-1e-37, 1e-37, 256).astype(np.float32))
    _assert_act_cols(x, name="edge columns")


def _assert_w(bits, ldw=None, with_qt=True, name=""):
    import torch
    log(f"quant_w {name} shape={bits.shape} ldw={ldw}")
    n, k = bits.shape
    if ldw is not None and ldw != k:
        buf = np.zeros((n, ldw), np.uint16)
        buf[:, :k] = bits
        t = dev_bf16(buf)[:, :k]
    else:
        t = dev_bf16(bits)
    q, s, qt = fb.quant_w_128x128(t, transposed_copy=with_qt)
    q0, s0 = oq.quant_w_128x128(bits)
    np.testing.assert_array_equal(host(q), q0, err_msg=name)
    np.testing.assert_array_equal(host(s).view(np.uint32), s0.view(np.uint32), err_msg=name)
    if with_qt:
        np.testing.assert_array_equal(host(qt), q0.T, err_msg=name)
    del torch


# with the transposed copy and without (one 128x128 block per workgroup, or two
# neighbouring blocks along k; odd block counts leave the last workgroup half empty)
@pytest.mark.parametrize("with_qt", [True, False])
@pytest.mark.parametrize("n,k,ldw,seed", [(128, 128, None, 21), (256, 384, None, 22), (384, 256, 320, 23),
                                           (2048, 7168, None, 24), (640, 1152, 1160, 26)])
def test_quant_w(n, k, ldw, seed, with_qt):
    _assert_w(act(seed, n, k, std=0.02), ldw=ldw, with_qt=with_qt, name=f"seed {seed}")


def test_quant_w_edge_blocks():
    w = act(25, 256, 256, std=0.02).copy()
    w[:128, :128] = 0
    w[128:, :128] = 0x8000
    w[:128, 128:] = f32_to_bf16_bits(np.linspace(-1e-36, 1e-36, 128 * 128).reshape(128, 128).astype(np.float32))
    _assert_w(w, name="edge blocks")
    _assert_w(w, with_qt=False, name="edge blocks, no transposed copy")


def test_dense_config_quantisers_full_size():
    cfg = dense_fprop()
    _assert_act_rows(cfg.x, name="dense X 4096x7168")
    _assert_w(cfg.w, name="dense W 2048x7168")
