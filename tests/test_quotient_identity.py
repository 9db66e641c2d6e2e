"""The row quantizer's kernel takes each quotient w/s from the reciprocal of s with one FMA
correction instead of a division.  This host check (plain C, gcc, libm fmaf) confirms on
about 20 million cases that the result is the correctly rounded float32 quotient outside
underflow and always yields the same int8 code as the division the oracle performs."""
import os
import shutil
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_fma_corrected_quotient_matches_division():
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "check")
        subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-o", exe,
                        os.path.join(HERE, "cpu", "quotient_fma_check.c"), "-lm"], check=True)
        out = subprocess.run([exe, "400", "40000", "4000000"], check=True, capture_output=True,
                             text=True).stdout.split()
    cases, code_bad, quot_bad = (int(v) for v in out)
    assert cases > 15_000_000
    assert code_bad == 0
    assert quot_bad == 0
