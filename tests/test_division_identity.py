"""The reciprocal-and-correction form of x / a that the quantize kernel uses (CPU only).

The kernel replaces one IEEE division per element by fp32(1 / a) once per block and two fmas
(Markstein's correction step).  tests/cpu/division_identity.c checks the claim the kernel rests on:
the result equals fp32(x / a) for a in [2^-60, 2^100] whenever |x / a| >= 2^-40, so no code whose
decision points are at least 2^-39 from zero can change.  gcc with -ffp-contract=off and the C
library's correctly rounded fmaf stand in for the GPU's fp32 multiply and fma (both IEEE, round
to nearest, denormals kept).  The GPU parity tests then compare the kernel's codes with the
oracle's (plain division) bit for bit.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_reciprocal_correction_equals_division(tmp_path):
    exe = str(tmp_path / "division_identity")
    r = subprocess.run(["gcc", "-std=c99", "-O2", "-ffp-contract=off",
                        os.path.join(ROOT, "tests", "cpu", "division_identity.c"), "-o", exe, "-lm"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe, "20000000"], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip().endswith("0 differences"), r.stdout
