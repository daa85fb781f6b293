"""GPU parity of the E5M6 activation cache (fp8bq_cache_e5m6_1x128 and its
inverse) through the C ABI: packed 12-bit codes and power-of-two scales must
equal the oracle's (oracle/e5m6.py) bit for bit, and the bf16 values read back
must be the round-to-nearest-even of the oracle's exact cached values."""

import numpy as np
import pytest

import fp8_fine_grained_fp8bq_amd as fb
from oracle import e5m6
from tests.gpu_util import dev_bf16, host, log
from workloads import act, dense_fprop, f32_to_bf16_bits

pytestmark = pytest.mark.gpu


def _cache(bits, ldx=None, ldq=None):
    import torch
    rows, cols = bits.shape
    if ldx is not None and ldx != cols:
        buf = np.zeros((rows, ldx), np.uint16)
        buf[:, :cols] = bits
        x = dev_bf16(buf)
    else:
        x, ldx = dev_bf16(bits), cols
    nb = cols * 3 // 2
    ldq = ldq or (nb + 15) // 16 * 16
    q = torch.full((rows, ldq), 0xA5, dtype=torch.uint8, device="cuda")
    s = torch.full((cols // 128, rows), -1.0, dtype=torch.float32, device="cuda")
    fb.fp8bq_cache_e5m6_1x128(x.data_ptr(), rows, cols, ldx, q.data_ptr(), ldq, s.data_ptr(), rows,
                              torch.cuda.current_stream().cuda_stream)
    qh = host(q)
    assert np.all(qh[:, nb:] == 0xA5), "wrote past the row's packed codes"
    return q, s, qh[:, :nb], host(s)


def _bf16_rne_of_exact(v):
    # the exact cached values have at most 7 significant bits and lie at or
    # above 2^-147, so float32 holds them exactly; one rounding to bf16 follows
    return f32_to_bf16_bits(np.asarray(v, np.float64).astype(np.float32))


def _assert_cache(bits, ldx=None, ldq=None, name=""):
    import torch
    log(f"e5m6 cache {name} shape={bits.shape} ldx={ldx} ldq={ldq}")
    rows, cols = bits.shape
    q, s, qh, sh = _cache(bits, ldx, ldq)
    q0, s0 = e5m6.cache_1x128(bits)
    np.testing.assert_array_equal(qh, q0, err_msg=f"codes differ ({name})")
    np.testing.assert_array_equal(sh.view(np.uint32), s0.view(np.uint32), err_msg=f"scales differ ({name})")
    y = torch.full((rows, cols), -1, dtype=torch.int16, device="cuda")
    fb.fp8bq_uncache_e5m6_1x128(q.data_ptr(), rows, cols, q.stride(0), s.data_ptr(), rows, y.data_ptr(), cols,
                                torch.cuda.current_stream().cuda_stream)
    want = _bf16_rne_of_exact(e5m6.uncache_1x128(q0, s0, cols))
    np.testing.assert_array_equal(host(y).view(np.uint16), want, err_msg=f"values read back differ ({name})")


@pytest.mark.parametrize("rows,cols,ldx,seed", [
    (1, 128, None, 71), (37, 384, None, 72), (257, 1024, 1088, 73), (64, 7168, None, 74), (33, 1152, 1160, 75)])
def test_cache_seeded(rows, cols, ldx, seed):
    _assert_cache(act(seed, rows, cols, dist="student_t3", outlier_p=0.003, outlier_mult=40), ldx=ldx,
                  name=f"seed {seed}")


def test_cache_padded_code_rows():
    _assert_cache(act(76, 40, 256), ldq=512, name="ldq 512")


def _all_bf16_upto(amax_bits):
    bits = np.arange(65536, dtype=np.uint32)
    with np.errstate(invalid="ignore"):
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


@pytest.mark.parametrize("amax_bits", [0x477E, 0x477F, 0x3F80, 0x40A3, 0x2E9B, 0x7F7F])
def test_every_bf16_value_at_several_scales(amax_bits):
    # 0x477E = 65024 (k = 0: the codes are the plain E5M6 roundings), 0x477F just above (k = 1)
    _assert_cache(_all_bf16_upto(amax_bits), name=f"all bf16 up to {amax_bits:#x}")


def test_scale_for_every_bf16_absmax():
    amax = np.arange(1, 0x7F80, dtype=np.uint16)
    a = (amax.astype(np.uint32) << 16).view(np.float32)
    fr = np.linspace(-1, 1, 127, dtype=np.float32)
    body = f32_to_bf16_bits(a[:, None] * fr[None, :])
    signs = np.where(np.arange(amax.size) % 2 == 1, 0x8000, 0).astype(np.uint16)
    x = np.concatenate([(amax | signs)[:, None], body], axis=1).astype(np.uint16)
    _assert_cache(x, name="every bf16 absmax")


def test_edge_tiles():
    x = act(77, 12, 256, outlier_p=0).copy()
    x[0, 0:128] = 0                                        # all +0: s = 2^-127, codes +0
    x[1, 0:128] = 0x8000                                   # all -0
    x[2, 0:128] = 0; x[2, 5] = 0x8001                      # a negative bf16 subnormal absmax
    x[3, 0:128] = f32_to_bf16_bits(np.full(128, -3.0e38, np.float32))
    x[4, 128:256] = f32_to_bf16_bits(np.array([1e-30] * 127 + [1e30], np.float32))   # beyond the format's range
    x[5, 0:128] = f32_to_bf16_bits(np.array([65024.0, -65024.0] * 64, np.float32))
    x[6, 0:128] = f32_to_bf16_bits(np.ldexp(np.arange(128, dtype=np.float32) - 64, -140))
    _assert_cache(x, name="edge tiles")


def test_dense_activation_full_size():
    cfg = dense_fprop()
    _assert_cache(cfg.x, name="dense X 4096x7168")


def test_fast_path_boundaries():
    # A wave covers 4 rows of one 128-column chunk; it encodes with the packed
    # fast path only if every value is zero or has a bf16 magnitude at least
    # (k + 113) << 7, and k >= -111. Rows 0-3: k = -111 tiles, all qualifying;
    # rows 4-7: the same with one value a step below the threshold (the whole
    # wave takes the general codec); rows 8-11: k = -112 tiles (general codec);
    # rows 12-15: ordinary tiles with values exactly at the threshold, signed
    # zeros and the tile maxima.
    rng = np.random.default_rng(78)
    x = np.zeros((16, 256), np.uint16)

    def tile(amax_bits, lo_bits, n=128):
        v = rng.integers(lo_bits, amax_bits + 1, n).astype(np.uint16)
        v[0] = amax_bits
        v |= (rng.integers(0, 2, n) << 15).astype(np.uint16)          # random signs
        return v
    for r in range(4):
        x[r, :128] = tile(0x0F80, 0x0100)          # k = -111: threshold magnitude 0x0100
        x[r, 128:] = tile(0x0FC0, 0x0100)
    x[4:8] = x[0:4]
    x[5, 17] = 0x00FF                               # one value just below the threshold
    for r in range(8, 12):
        x[r, :128] = tile(0x0F00, 0x0080)          # k = -112
        x[r, 128:] = tile(0x0F7F, 0x0080)
    for r in range(12, 16):
        x[r, :128] = tile(0x3F80, 0x3100)          # amax 1.0: k = -15, threshold 0x3100
        x[r, 128:] = tile(0x477E, 0x3800)          # amax 65024: k = 0, threshold 0x3880 -> values below it too
    x[12, 1:9] = [0x3100, 0xB100, 0x0000, 0x8000, 0x3101, 0xB101, 0x3F80, 0xBF80]   # at the threshold, zeros
    _assert_cache(x, name="fast path boundaries")
