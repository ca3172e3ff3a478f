"""The C ABI on its own: tests/c_abi/c_abi_check (built with the package, no Python or torch in
it) quantizes per tensor and MX dual on hipMalloc'd memory, de-scales, and compares every byte
with the C oracle."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "c_abi_check")


def test_c_abi_program_matches_oracle():
    assert os.path.exists(EXE), "tests/c_abi/c_abi_check is missing: run __graft_entry__.build() first"
    out = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0 and out.stdout.strip().endswith("ok"), out.stdout + out.stderr
