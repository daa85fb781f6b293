"""The LDS DMA statements (global/buffer loads with the LDS bit, issued from
inline asm in csrc/gemm_kernels.h and csrc/gemm_decode.hip) set M0 themselves.
The compiler reserves M0 and cannot look inside an asm block, so this checks
the gfx950 code objects of the built libraries instead:
* every LDS DMA is preceded by exactly "s_mov_b32 m0, ..." and "s_nop 0" (the
  wait state an SALU write of M0 needs before an LDS DMA reads it);
* every instruction that names M0 is such a write, followed by that pair;
* no instruction family that reads M0 implicitly appears (move-relative,
  message, interpolation, GWS/ordered/append LDS operations), so no other
  reader can see the value the DMA statements leave in M0."""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "fp8_fine_grained_fp8bq_amd")
OBJDUMP = "/opt/rocm/llvm/bin/llvm-objdump"
LIBS = ["libfp8bq.so", "libfp8bq_probe.so"]

IMPLICIT_M0 = re.compile(r"^(v_movrel|s_movrel|s_sendmsg|s_ttracedata|v_interp|ds_gws|ds_ordered|ds_append|"
                         r"ds_consume|ds_param_load|ds_direct_load)")


def _is_lds_dma(mnemonic: str, operands: str) -> bool:
    if mnemonic.startswith("global_load_lds") or mnemonic.startswith("scratch_load_lds"):
        return True
    return mnemonic.startswith("buffer_load") and re.search(r"\blds\b", operands) is not None


def _instructions(lib: str, tmp) -> list:
    """(mnemonic, operands) of every instruction in the lib's gfx950 code objects, per object."""
    work = tmp / os.path.basename(lib)
    work.mkdir()
    shutil.copy(lib, work / "lib.so")
    subprocess.run([OBJDUMP, "--offloading", "lib.so"], cwd=work, check=True, capture_output=True)
    objs = sorted(p for p in os.listdir(work) if p.endswith("gfx950"))
    assert objs, f"no gfx950 code object in {lib}"
    out = []
    for o in objs:
        dis = subprocess.run([OBJDUMP, "-d", "--mcpu=gfx950", o], cwd=work, check=True, capture_output=True,
                             text=True).stdout
        ins = []
        for line in dis.splitlines():
            if not line.startswith("\t"):
                ins.append(("<label>", line.strip()))      # symbol headers break a sequence
                continue
            text = line.split("//")[0].strip()
            if not text:
                continue
            mn, _, ops = text.partition(" ")
            ins.append((mn, ops.strip()))
        out.append((o, ins))
    return out


@pytest.mark.skipif(not os.path.exists(OBJDUMP), reason="needs llvm-objdump")
@pytest.mark.parametrize("name", LIBS)
def test_m0_writes_pair_with_lds_dma(name, tmp_path):
    lib = os.path.join(PKG, name)
    if not os.path.exists(lib):
        pytest.skip(f"{name} not built")
    n_dma = 0
    for obj, ins in _instructions(lib, tmp_path):
        for i, (mn, ops) in enumerate(ins):
            where = f"{name}:{obj} #{i}: {mn} {ops}"
            assert not IMPLICIT_M0.match(mn), f"implicit M0 reader {where}"
            if _is_lds_dma(mn, ops):
                n_dma += 1
                assert i >= 2, where
                assert ins[i - 1] == ("s_nop", "0"), f"LDS DMA without the M0 wait state: {where}"
                pm, po = ins[i - 2]
                assert pm == "s_mov_b32" and po.startswith("m0,"), f"LDS DMA not preceded by its M0 write: {where}"
                continue
            if re.search(r"\bm0\b", ops):
                assert mn == "s_mov_b32" and ops.startswith("m0,"), f"M0 named outside a DMA statement: {where}"
                assert i + 2 < len(ins) and ins[i + 1] == ("s_nop", "0") and _is_lds_dma(*ins[i + 2]), \
                    f"M0 write not followed by the wait state and an LDS DMA: {where}"
    if name == "libfp8bq.so":
        assert n_dma > 0, "no LDS DMA found: the disassembly format changed?"
