"""fp8bq: fine-grained FP8 (E4M3, 1x128 / 128x128) quantisation and block-scaled
FP8 GEMM for AMD MI355X (gfx950).

Thin ctypes binding over the C ABI in include/fp8bq.h (libfp8bq.so, built in
this package directory by `build.py`). Every step of the computation runs in
the library's HIP kernels; this module only marshals arguments. There is no
fallback: if the library is missing or the device is not gfx950, calls raise.

Two layers with the C names:

* `fp8bq_quant_act_1x128`, `fp8bq_quant_w_128x128`, `fp8bq_requant_t_128x1`,
  `fp8bq_gemm`, `fp8bq_gemm_quant`, `fp8bq_grouped_gemm`,
  `fp8bq_grouped_gemm_decode`, `fp8bq_grouped_gemm_decode_workspace_size`,
  `fp8bq_grouped_gemm_decode_ws`, `fp8bq_grouped_gemm_decode_noalloc`, `fp8bq_cache_e5m6_1x128`,
  `fp8bq_uncache_e5m6_1x128`, `fp8bq_requant_e5m6_t_128x1`: pointer-level, exactly the C signatures (ints
  for pointers and the stream); a non-zero status raises `Fp8bqError`.
* `quant_act_1x128`, `quant_w_128x128`, `requant_t_128x1`, `gemm`,
  `gemm_quant`, `grouped_gemm`, `grouped_gemm_decode`, `cache_e5m6_1x128`,
  `uncache_e5m6_1x128`, `requant_e5m6_t_128x1`: take torch tensors on
  the GPU, allocate the outputs with torch (memory and streams are the only
  things torch provides) and call the same entry points on the current stream.
"""

from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfp8bq.so")

OK, E_INVAL, E_SHAPE, E_ALIGN, E_DEVICE, E_HIP = range(6)
STATUS_NAMES = {0: "OK", 1: "E_INVAL", 2: "E_SHAPE", 3: "E_ALIGN", 4: "E_DEVICE", 5: "E_HIP"}
FPROP, DGRAD, WGRAD = 0, 1, 2
ACT_ROWWISE, ACT_COLWISE = 0, 1
SCALE_POW2 = 0x10   # power-of-two scales (OR into the act mode / gemm op; `flags` elsewhere)

EXPORTS = ("fp8bq_quant_act_1x128", "fp8bq_quant_w_128x128", "fp8bq_requant_t_128x1", "fp8bq_gemm",
           "fp8bq_gemm_quant", "fp8bq_grouped_gemm", "fp8bq_grouped_gemm_decode",
           "fp8bq_grouped_gemm_decode_workspace_size", "fp8bq_grouped_gemm_decode_ws",
           "fp8bq_grouped_gemm_decode_noalloc", "fp8bq_cache_e5m6_1x128",
           "fp8bq_uncache_e5m6_1x128", "fp8bq_requant_e5m6_t_128x1", "fp8bq_last_error", "fp8bq_version")


class Fp8bqError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: {STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libfp8bq.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m fp8_fine_grained_fp8bq_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        i64, vp, fp, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int
        L.fp8bq_quant_act_1x128.argtypes = [vp, i64, i64, i64, i32, vp, i64, fp, i64, vp]
        L.fp8bq_quant_w_128x128.argtypes = [vp, i64, i64, i64, vp, i64, fp, i64, vp, i64, i32, vp]
        L.fp8bq_requant_t_128x1.argtypes = [vp, i64, i64, i64, fp, i64, vp, i64, fp, i64, i32, vp]
        L.fp8bq_cache_e5m6_1x128.argtypes = [vp, i64, i64, i64, vp, i64, fp, i64, vp]
        L.fp8bq_uncache_e5m6_1x128.argtypes = [vp, i64, i64, i64, fp, i64, vp, i64, vp]
        L.fp8bq_requant_e5m6_t_128x1.argtypes = [vp, i64, i64, i64, fp, i64, vp, i64, fp, i64, vp]
        L.fp8bq_gemm.argtypes = [i32, i64, i64, i64, vp, i64, fp, i64, vp, i64, fp, i64, vp, i64, vp]
        L.fp8bq_gemm_quant.argtypes = [i32, i64, i64, i64, vp, i64, fp, i64, vp, i64, fp, i64, vp, i64,
                                       vp, i64, fp, i64, i32, vp]
        L.fp8bq_grouped_gemm.argtypes = [ctypes.c_int32, ctypes.POINTER(ctypes.c_int64), i64, i64,
                                         vp, i64, fp, i64, vp, i64, fp, i64, vp, i64, i32, vp]
        for f in ("fp8bq_quant_act_1x128", "fp8bq_quant_w_128x128", "fp8bq_requant_t_128x1", "fp8bq_gemm",
                  "fp8bq_grouped_gemm", "fp8bq_cache_e5m6_1x128", "fp8bq_uncache_e5m6_1x128",
                  "fp8bq_requant_e5m6_t_128x1"):
            getattr(L, f).restype = ctypes.c_int
        L.fp8bq_last_error.restype = ctypes.c_char_p
        L.fp8bq_grouped_gemm_decode.argtypes = L.fp8bq_grouped_gemm.argtypes
        L.fp8bq_grouped_gemm_decode_workspace_size.argtypes = [ctypes.c_int32, ctypes.POINTER(ctypes.c_int64), i64,
                                                               i64, ctypes.POINTER(ctypes.c_int64)]
        L.fp8bq_grouped_gemm_decode_workspace_size.restype = ctypes.c_int
        L.fp8bq_grouped_gemm_decode_ws.argtypes = [ctypes.c_int32, ctypes.POINTER(ctypes.c_int64), i64, i64,
                                                   vp, i64, fp, i64, vp, i64, fp, i64, vp, i64, vp, i64, i32, vp]
        L.fp8bq_grouped_gemm_decode_ws.restype = ctypes.c_int
        L.fp8bq_grouped_gemm_decode_noalloc.argtypes = L.fp8bq_grouped_gemm.argtypes
        L.fp8bq_grouped_gemm_decode_noalloc.restype = ctypes.c_int
        L.fp8bq_last_error.argtypes = []
        L.fp8bq_version.restype = ctypes.c_char_p
        L.fp8bq_version.argtypes = []
        _lib = L
    return _lib


def _check(fn: str, status: int) -> int:
    if status != OK:
        raise Fp8bqError(fn, status, lib().fp8bq_last_error().decode())
    return status


# ---------------------------------------------------------------------------
# pointer-level entry points (C names)
# ---------------------------------------------------------------------------

def fp8bq_quant_act_1x128(x, rows, cols, ldx, mode, q, ldq, s, lds, stream=0):
    return _check("fp8bq_quant_act_1x128",
                  lib().fp8bq_quant_act_1x128(x, rows, cols, ldx, mode, q, ldq, s, lds, stream))


def fp8bq_quant_w_128x128(w, n, k, ldw, q, ldq, s, lds, qt, ldqt, flags=0, stream=0):
    return _check("fp8bq_quant_w_128x128",
                  lib().fp8bq_quant_w_128x128(w, n, k, ldw, q, ldq, s, lds, qt, ldqt, flags, stream))


def fp8bq_requant_t_128x1(q, rows, cols, ldq, s, lds, qt, ldqt, st, ldst, flags=0, stream=0):
    return _check("fp8bq_requant_t_128x1",
                  lib().fp8bq_requant_t_128x1(q, rows, cols, ldq, s, lds, qt, ldqt, st, ldst, flags, stream))


def fp8bq_gemm(op, m, n, k, a, lda, sa, ldsa, b, ldb, sb, ldsb, out, ldo, stream=0):
    return _check("fp8bq_gemm",
                  lib().fp8bq_gemm(op, m, n, k, a, lda, sa, ldsa, b, ldb, sb, ldsb, out, ldo, stream))


def fp8bq_gemm_quant(op, m, n, k, a, lda, sa, ldsa, b, ldb, sb, ldsb, out, ldo, q, ldq, s, lds, qflags=0,
                     stream=0):
    return _check("fp8bq_gemm_quant",
                  lib().fp8bq_gemm_quant(op, m, n, k, a, lda, sa, ldsa, b, ldb, sb, ldsb, out, ldo, q, ldq, s, lds,
                                         qflags, stream))


def fp8bq_grouped_gemm(groups, row_off, n, k, a, lda, sa, ldsa, b, ldb, sb, ldsb, out, ldo, flags=0,
                       stream=0):
    """`row_off` is a sequence of groups + 1 ints (host memory)."""
    arr = (ctypes.c_int64 * (groups + 1))(*[int(v) for v in row_off]) if row_off is not None else None
    return _check("fp8bq_grouped_gemm",
                  lib().fp8bq_grouped_gemm(groups, arr, n, k, a, lda, sa, ldsa, b, ldb, sb, ldsb,
                                           out, ldo, flags, stream))


def fp8bq_grouped_gemm_decode(groups, row_off, n, k, a, lda, sa, ldsa, b, ldb, sb, ldsb, out, ldo, flags=0,
                              stream=0):
    """`row_off` is a sequence of groups + 1 ints (host memory), any counts up to 256 per group."""
    arr = (ctypes.c_int64 * (groups + 1))(*[int(v) for v in row_off]) if row_off is not None else None
    return _check("fp8bq_grouped_gemm_decode",
                  lib().fp8bq_grouped_gemm_decode(groups, arr, n, k, a, lda, sa, ldsa, b, ldb, sb, ldsb,
                                                  out, ldo, flags, stream))


def version() -> str:
    return lib().fp8bq_version().decode()


# ---------------------------------------------------------------------------
# torch-tensor convenience layer (allocation + marshalling only)
# ---------------------------------------------------------------------------

def _stream(t):
    import torch
    return torch.cuda.current_stream(t.device).cuda_stream


def _bf16_2d(t, name):
    import torch
    if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16) or t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be a 2-D row-major bf16 tensor (got {t.dtype}, {tuple(t.shape)})")
    return t


def quant_act_1x128(x, mode: int = ACT_ROWWISE):
    """x bf16 [rows, cols] -> (q uint8, s float32) as laid out by the C ABI:
    ROWWISE q [rows, cols], s [cols/128, rows]; COLWISE q [cols, rows], s [rows/128, cols].
    `mode` may include SCALE_POW2 (power-of-two scales)."""
    import torch
    _bf16_2d(x, "x")
    rows, cols = x.shape
    if (mode & ~SCALE_POW2) == ACT_ROWWISE:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
        s = torch.empty((cols // 128, rows), dtype=torch.float32, device=x.device)
        ldq, lds = cols, rows
    else:
        q = torch.empty((cols, rows), dtype=torch.uint8, device=x.device)
        s = torch.empty((rows // 128, cols), dtype=torch.float32, device=x.device)
        ldq, lds = rows, cols
    fp8bq_quant_act_1x128(x.data_ptr(), rows, cols, x.stride(0), mode, q.data_ptr(), ldq,
                          s.data_ptr(), lds, _stream(x))
    return q, s


def quant_w_128x128(w, transposed_copy: bool = False, pow2: bool = False):
    """w bf16 [n, k] -> (q uint8 [n, k], s float32 [n/128, k/128], qt uint8 [k, n] or None);
    pow2 selects power-of-two scales."""
    import torch
    _bf16_2d(w, "w")
    n, k = w.shape
    q = torch.empty((n, k), dtype=torch.uint8, device=w.device)
    s = torch.empty((n // 128, k // 128), dtype=torch.float32, device=w.device)
    qt = torch.empty((k, n), dtype=torch.uint8, device=w.device) if transposed_copy else None
    fp8bq_quant_w_128x128(w.data_ptr(), n, k, w.stride(0), q.data_ptr(), k, s.data_ptr(), k // 128,
                          qt.data_ptr() if qt is not None else None, n, SCALE_POW2 if pow2 else 0, _stream(w))
    return q, s, qt


def fp8bq_cache_e5m6_1x128(x, rows, cols, ldx, q, ldq, s, lds, stream=0):
    return _check("fp8bq_cache_e5m6_1x128", lib().fp8bq_cache_e5m6_1x128(x, rows, cols, ldx, q, ldq, s, lds, stream))


def fp8bq_uncache_e5m6_1x128(q, rows, cols, ldq, s, lds, y, ldy, stream=0):
    return _check("fp8bq_uncache_e5m6_1x128",
                  lib().fp8bq_uncache_e5m6_1x128(q, rows, cols, ldq, s, lds, y, ldy, stream))


def fp8bq_requant_e5m6_t_128x1(q, rows, cols, ldq, s, lds, qt, ldqt, st, ldst, stream=0):
    return _check("fp8bq_requant_e5m6_t_128x1",
                  lib().fp8bq_requant_e5m6_t_128x1(q, rows, cols, ldq, s, lds, qt, ldqt, st, ldst, stream))


def cache_e5m6_1x128(x):
    """bf16 [rows, cols] (int16/bfloat16 storage) -> (q uint8 [rows, 1.5 cols]: packed 12-bit E5M6
    codes, s float32 [cols/128, rows]: chunk-major power-of-two 1x128 tile scales)."""
    import torch
    if x.dim() != 2 or x.element_size() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D row-major 16-bit tensor of bf16 patterns")
    rows, cols = x.shape
    ldq = (cols * 3 // 2 + 15) // 16 * 16
    q = torch.empty((rows, ldq), dtype=torch.uint8, device=x.device)
    s = torch.empty((cols // 128, rows), dtype=torch.float32, device=x.device)
    fp8bq_cache_e5m6_1x128(x.data_ptr(), rows, cols, x.stride(0), q.data_ptr(), ldq, s.data_ptr(), rows, _stream(x))
    return q[:, : cols * 3 // 2], s


def uncache_e5m6_1x128(q, s, cols):
    """Packed E5M6 codes q (rows of >= 1.5 cols bytes, row stride q.stride(0)) and their scales s
    [cols/128, >=rows] -> bf16 [rows, cols] (torch.bfloat16)."""
    import torch
    if q.dtype != torch.uint8 or q.dim() != 2 or q.stride(1) != 1:
        raise ValueError("q must be a 2-D row-major uint8 tensor")
    rows = q.shape[0]
    y = torch.empty((rows, cols), dtype=torch.bfloat16, device=q.device)
    fp8bq_uncache_e5m6_1x128(q.data_ptr(), rows, cols, q.stride(0), s.data_ptr(), s.stride(0), y.data_ptr(), cols,
                             _stream(q))
    return y


def requant_e5m6_t_128x1(q, s, cols):
    """E5M6 cache q (rows of >= 1.5 cols bytes, row stride q.stride(0)) with its power-of-two
    scales s [cols/128, >=rows] -> (qt uint8 [cols, rows], st float32 [rows/128, cols]): the cached
    values re-quantised to E4M3 in 128x1 tiles with power-of-two scales, COLWISE layout."""
    import torch
    if q.dtype != torch.uint8 or q.dim() != 2 or q.stride(1) != 1:
        raise ValueError("q must be a 2-D row-major uint8 tensor")
    if s.dtype != torch.float32 or s.dim() != 2 or s.stride(1) != 1:
        raise ValueError("s must be a 2-D row-major float32 tensor")
    rows = q.shape[0]
    qt = torch.empty((cols, rows), dtype=torch.uint8, device=q.device)
    st = torch.empty((rows // 128, cols), dtype=torch.float32, device=q.device)
    fp8bq_requant_e5m6_t_128x1(q.data_ptr(), rows, cols, q.stride(0), s.data_ptr(), s.stride(0), qt.data_ptr(),
                               rows, st.data_ptr(), cols, _stream(q))
    return qt, st


def requant_t_128x1(q, s, pow2_scales=False):
    """FP8 activation cache q uint8 [rows, cols] with chunk-major 1x128 scales s [cols/128, >=rows]
    -> (qt uint8 [cols, rows], st float32 [rows/128, cols]): 128x1 tiles with power-of-two scales,
    the layout of COLWISE quantisation. pow2_scales: s holds powers of two (the kernel for that
    case; the result is the same)."""
    import torch
    if q.dtype != torch.uint8 or q.dim() != 2 or q.stride(1) != 1:
        raise ValueError("q must be a 2-D row-major uint8 tensor")
    if s.dtype != torch.float32 or s.dim() != 2 or s.stride(1) != 1:
        raise ValueError("s must be a 2-D row-major float32 tensor")
    rows, cols = q.shape
    qt = torch.empty((cols, rows), dtype=torch.uint8, device=q.device)
    st = torch.empty((rows // 128, cols), dtype=torch.float32, device=q.device)
    fp8bq_requant_t_128x1(q.data_ptr(), rows, cols, q.stride(0), s.data_ptr(), s.stride(0), qt.data_ptr(), rows,
                          st.data_ptr(), cols, SCALE_POW2 if pow2_scales else 0, _stream(q))
    return qt, st


def gemm(op: int, a, sa, b, sb, out=None):
    """a uint8 [m, k] with chunk-major scales sa [k/128, >=m]; b uint8 [n, k] with
    sb laid out per `op` (see include/fp8bq.h); `op` may include SCALE_POW2. Returns out
    (bf16 or fp32) [m, n]."""
    import torch
    m, k = a.shape
    n = b.shape[0]
    if out is None:
        dt = torch.float32 if (op & ~SCALE_POW2) == WGRAD else torch.bfloat16
        out = torch.empty((m, n), dtype=dt, device=a.device)
    fp8bq_gemm(op, m, n, k, a.data_ptr(), a.stride(0), sa.data_ptr(), sa.stride(0),
               b.data_ptr(), b.stride(0), sb.data_ptr(), sb.stride(0), out.data_ptr(), out.stride(0),
               _stream(a))
    return out


def gemm_quant(op: int, a, sa, b, sb, with_out: bool = True, qpow2: bool = False):
    """fp8bq_gemm (FPROP / DGRAD, `op` may include SCALE_POW2) that also quantises its bf16
    output in 1x128 tiles. Returns (out bf16 [m, n] or None, q uint8 [m, n], s float32
    [n/128, m]); qpow2 selects power-of-two output scales."""
    import torch
    m, k = a.shape
    n = b.shape[0]
    out = torch.empty((m, n), dtype=torch.bfloat16, device=a.device) if with_out else None
    q = torch.empty((m, n), dtype=torch.uint8, device=a.device)
    s = torch.empty((n // 128, m), dtype=torch.float32, device=a.device)
    fp8bq_gemm_quant(op, m, n, k, a.data_ptr(), a.stride(0), sa.data_ptr(), sa.stride(0),
                     b.data_ptr(), b.stride(0), sb.data_ptr(), sb.stride(0),
                     out.data_ptr() if out is not None else None, n, q.data_ptr(), n, s.data_ptr(), m,
                     SCALE_POW2 if qpow2 else 0, _stream(a))
    return out, q, s


def grouped_gemm(row_off, a, sa, b, sb, out=None, pow2: bool = False):
    """row_off: host sequence of G + 1 row offsets (multiples of 128); a uint8 [m, k];
    sa [k/128, >=m]; b uint8 [G, n, k]; sb float32 [G, n/128, k/128]. Returns bf16 [m, n].
    pow2: power-of-two scales applied by the matrix instruction."""
    import torch
    G, n, k = b.shape
    m = a.shape[0]
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=a.device)
    fp8bq_grouped_gemm(G, list(row_off), n, k, a.data_ptr(), a.stride(0), sa.data_ptr(), sa.stride(0),
                       b.data_ptr(), b.stride(1), sb.data_ptr(), sb.stride(1), out.data_ptr(),
                       out.stride(0), SCALE_POW2 if pow2 else 0, _stream(a))
    return out


def _offsets(groups, row_off):
    return (ctypes.c_int64 * (groups + 1))(*[int(v) for v in row_off]) if row_off is not None else None


def fp8bq_grouped_gemm_decode_workspace_size(groups, row_off, n, k):
    """Bytes of workspace fp8bq_grouped_gemm_decode_ws needs (row_off: host sequence)."""
    out = ctypes.c_int64(-1)
    _check("fp8bq_grouped_gemm_decode_workspace_size",
           lib().fp8bq_grouped_gemm_decode_workspace_size(groups, _offsets(groups, row_off), n, k, ctypes.byref(out)))
    return out.value


def fp8bq_grouped_gemm_decode_ws(groups, row_off, n, k, a, lda, sa, ldsa, b, ldb, sb, ldsb, out, ldo, workspace,
                                 workspace_bytes, flags=0, stream=0):
    return _check("fp8bq_grouped_gemm_decode_ws",
                  lib().fp8bq_grouped_gemm_decode_ws(groups, _offsets(groups, row_off), n, k, a, lda, sa, ldsa, b,
                                                     ldb, sb, ldsb, out, ldo, workspace, workspace_bytes, flags,
                                                     stream))


def fp8bq_grouped_gemm_decode_noalloc(groups, row_off, n, k, a, lda, sa, ldsa, b, ldb, sb, ldsb, out, ldo, flags=0,
                                      stream=0):
    return _check("fp8bq_grouped_gemm_decode_noalloc",
                  lib().fp8bq_grouped_gemm_decode_noalloc(groups, _offsets(groups, row_off), n, k, a, lda, sa, ldsa, b,
                                                          ldb, sb, ldsb, out, ldo, flags, stream))


DECODE_NOALLOC_SCRATCH_BYTES = 32 << 20

_workspaces = {}


def decode_workspace(nbytes, device):
    """A zero-filled device workspace of at least nbytes for fp8bq_grouped_gemm_decode_ws, kept
    per device and reused (every call leaves its counters zero). Calls that share it must run
    on one stream."""
    import torch
    key = torch.device(device).index if torch.device(device).index is not None else torch.cuda.current_device()
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def grouped_gemm_decode(row_off, a, sa, b, sb, out=None, split=True):
    """Decode-shape grouped Fprop: row_off host sequence of G + 1 offsets (any counts up to
    256 rows per expert); a uint8 [m, k]; sa [k/128, >=m]; b uint8 [G, n, k];
    sb float32 [G, n/128, k/128]. Returns bf16 [m, n]. split: experts of more than 32 rows
    run as 128-column half-K workgroup pairs through a cached workspace."""
    import torch
    G, n, k = b.shape
    m = a.shape[0]
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=a.device)
    if split:
        need = fp8bq_grouped_gemm_decode_workspace_size(G, list(row_off), n, k)
        ws = decode_workspace(need, a.device) if need > 0 else None
        fp8bq_grouped_gemm_decode_ws(G, list(row_off), n, k, a.data_ptr(), a.stride(0), sa.data_ptr(), sa.stride(0),
                                     b.data_ptr(), b.stride(1), sb.data_ptr(), sb.stride(1), out.data_ptr(),
                                     out.stride(0), ws.data_ptr() if ws is not None else None,
                                     ws.numel() if ws is not None else 0, 0, _stream(a))
        return out
    fp8bq_grouped_gemm_decode(G, list(row_off), n, k, a.data_ptr(), a.stride(0), sa.data_ptr(), sa.stride(0),
                              b.data_ptr(), b.stride(1), sb.data_ptr(), sb.stride(1), out.data_ptr(),
                              out.stride(0), 0, _stream(a))
    return out


