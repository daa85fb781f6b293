"""Builds libfp8bq.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Usage: python -m fp8_fine_grained_fp8bq_amd.build   (or call build()).
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libfp8bq.so")
PROBE_LIB = os.path.join(PKG, "libfp8bq_probe.so")

SOURCES = ["api.cpp", "quant.hip", "gemm.hip", "gemm_quant.hip", "gemm_grouped.hip", "gemm_decode.hip"]
# measurement probes of the matrix instruction (a library of their own, not the GEMM path)
PROBE_SOURCES = ["probe.hip"]

# -packed-fp32-ops: no packed FP32 VALU instructions (v_pk_*_f32) in any kernel.
# -Wno-inline-asm: the LDS-DMA helpers name M0 (a compiler-reserved register) as
# clobbered on purpose; see gemm_kernels.h.
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-inline-asm",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    """Compile every source into libfp8bq.so and the probes into
    libfp8bq_probe.so (always recompiles). The sources compile in parallel to
    objects, which are then linked."""
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    compile_flags = [f for f in HIPCC_FLAGS if f != "-shared"]
    procs = []
    for f in SOURCES + PROBE_SOURCES:
        obj = os.path.join(objdir, f + ".o")
        cmd = [hipcc(), *compile_flags, "-I", os.path.join(ROOT, "include"), "-c", os.path.join(CSRC, f), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((f, obj, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    failed = []
    for f, _, pr in procs:
        out, _ = pr.communicate()
        if pr.returncode != 0:
            sys.stderr.write(out)
            failed.append(f)
    if failed:
        raise RuntimeError(f"hipcc failed on {', '.join(failed)}")
    objs = {f: obj for f, obj, _ in procs}
    for lib, srcs in ((LIB, SOURCES), (PROBE_LIB, PROBE_SOURCES)):
        tmp = lib + ".tmp"
        cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *[objs[f] for f in srcs], "-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            sys.stderr.write(res.stdout + res.stderr)
            raise RuntimeError(f"hipcc link failed with exit code {res.returncode}")
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
