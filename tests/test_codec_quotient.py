"""The quantisers' branch-free exact quotient (fp8_codec.h, exact_quotient) checked
on the CPU over its whole input domain: every bf16 absmax x every bf16 |x| <= absmax
(tests/exact_quotient_check.c, built here with gcc). This pins the kernel's
arithmetic rule (Markstein's correction with a correctly rounded reciprocal)
against the correctly rounded division that the method specifies (tech note:
q = round(x / s)); the GPU tests then compare the kernels' codes with the oracle's."""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def _cpu_has_fma() -> bool:
    try:
        return " fma " in open("/proc/cpuinfo").read().replace("\n", " ")
    except OSError:
        return False


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_exact_quotient_every_bf16_pair(tmp_path):
    exe = str(tmp_path / "exact_quotient_check")
    flags = ["-O2", "-ffp-contract=off", "-fopenmp"] + (["-mfma"] if _cpu_has_fma() else [])
    subprocess.run(["gcc", *flags, os.path.join(HERE, "exact_quotient_check.c"), "-o", exe, "-lm"], check=True)
    res = subprocess.run([exe, "1"], capture_output=True, text=True, timeout=900)
    print(res.stdout)
    assert res.returncode == 0, res.stdout
    assert "code mismatches 0" in res.stdout
