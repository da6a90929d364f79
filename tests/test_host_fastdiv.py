"""Launch-time integer division used by the lowering kernels' index math.

The kernels divide element and item indices by shape-dependent divisors with
a multiply-high, add and shift (Granlund and Montgomery, "Division by
Invariant Integers using Multiplication", section 4).  The same inline
function is compiled for the host here and compared with exact integer
division over every divisor below 70000 and random ones up to 2^31 - 1.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_fastdiv_matches_integer_division(tmp_path):
    exe = str(tmp_path / "fastdiv_check")
    src = os.path.join(HERE, "host", "fastdiv_check.cpp")
    subprocess.run([HIPCC, "-O2", "-x", "hip", "--offload-arch=gfx950", "--cuda-host-only", src, "-o", exe],
                   check=True, capture_output=True, timeout=300)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "mismatches 0" in r.stdout
