"""The library from plain C (tests/c_abi/abi_from_c.c, built by the build entry point):
a float32 forward, a decode step continuing it and a backward pass through include/ssd.h
with device memory from the HIP runtime, each against the C oracle at 1e-4."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "abi_from_c")


def test_library_from_c_matches_oracle():
    assert os.path.exists(EXE), "C check not built (run the build entry point)"
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr
