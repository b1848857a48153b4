"""Exhaustive CPU proof of the quantizers' division shortcut.

The HIP quantizers form fl32(x / s) as Markstein's FMA-corrected product with a
correctly rounded reciprocal for tile scales in [2^-100, 2^100].  The C program
tests/host/div_check.c compares that sequence against IEEE division for every
BF16 tile maximum and every BF16 x that can meet it (about 8.9e8 quotients)
and reports every difference that could change an E4M3 code.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_markstein_quotient_matches_ieee_division(tmp_path):
    exe = tmp_path / "div_check"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-mfma", "-ffp-contract=off", os.path.join(HERE, "host", "div_check.c"),
                    "-o", str(exe), "-lm"], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-2000:]
    assert " 0 code-relevant mismatches" in r.stdout, r.stdout[-2000:]
