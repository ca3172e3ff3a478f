"""The NVFP4 kernels divide a block amax by 6 with a product and one fused multiply-add
correction instead of an IEEE division. This checks on the host, over every finite fp32 value
from 2^-125 up, that the two give the same bits (below 2^-125 the kernels divide)."""
import os
import shutil
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_div6_matches_correctly_rounded_quotient():
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "div6")
        subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fopenmp", os.path.join(HERE, "host_checks", "div6.c"),
                        "-o", exe, "-lm"], check=True)
        out = subprocess.run([exe], check=True, capture_output=True, text=True, timeout=600)
    assert out.stdout.strip() == "0"
