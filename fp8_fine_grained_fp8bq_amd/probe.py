"""ctypes binding of libfp8bq_probe.so (include/fp8bq_probe.h): measurements of
gfx950's FP8 matrix instruction that the GEMM's design rests on. Argument
marshalling only; the probes run in the library's HIP kernels and there is no
fallback (the calls raise if the library is missing)."""

from __future__ import annotations

import ctypes
import os

from . import STATUS_NAMES, Fp8bqError

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfp8bq_probe.so")
EXPORTS = ("fp8bq_probe_mfma_accum", "fp8bq_probe_mfma_once", "fp8bq_probe_mfma_stream", "fp8bq_probe_stream_2to1",
           "fp8bq_probe_last_error")

_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m fp8_fine_grained_fp8bq_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        i64, vp, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        L.fp8bq_probe_mfma_accum.argtypes = [vp, vp, i64, vp, vp, vp]
        L.fp8bq_probe_mfma_once.argtypes = [vp, vp, vp, vp, vp]
        L.fp8bq_probe_mfma_stream.argtypes = [i32, i64, ctypes.c_int32, vp, vp, vp, vp, vp]
        L.fp8bq_probe_stream_2to1.argtypes = [vp, vp, i64, vp]
        for f in EXPORTS[:4]:
            getattr(L, f).restype = ctypes.c_int
        L.fp8bq_probe_last_error.restype = ctypes.c_char_p
        L.fp8bq_probe_last_error.argtypes = []
        _lib = L
    return _lib


def _check(fn: str, status: int) -> int:
    if status != 0:
        raise Fp8bqError(fn, status, lib().fp8bq_probe_last_error().decode())
    return status


def fp8bq_probe_mfma_accum(a, b, k, chained, promoted, stream=0):
    return _check("fp8bq_probe_mfma_accum", lib().fp8bq_probe_mfma_accum(a, b, k, chained, promoted, stream))


def fp8bq_probe_mfma_once(a, b, c, d, stream=0):
    return _check("fp8bq_probe_mfma_once", lib().fp8bq_probe_mfma_once(a, b, c, d, stream))


def fp8bq_probe_mfma_stream(fold, iters, workgroups, codes, scales, sink, ticks, stream=0):
    return _check("fp8bq_probe_mfma_stream",
                  lib().fp8bq_probe_mfma_stream(fold, iters, workgroups, codes, scales, sink, ticks, stream))


def fp8bq_probe_stream_2to1(src, dst, n, stream=0):
    return _check("fp8bq_probe_stream_2to1", lib().fp8bq_probe_stream_2to1(src, dst, n, stream))


__all__ = ["fp8bq_probe_stream_2to1", "EXPORTS", "LIB_PATH", "lib", "fp8bq_probe_mfma_accum", "fp8bq_probe_mfma_once",
           "fp8bq_probe_mfma_stream", "STATUS_NAMES"]
