"""The kernels' quantiser decisions (code_of, nibble_of in iq_device.h) built
for the host and compared with plain threshold counting, including every float
within 64 ulps of each threshold (exact ties, which random data never hits)
and, for the 3-bit code_of, every float that is not a NaN."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "host", "decision_check.hip")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_decisions_equal_threshold_counting(tmp_path):
    exe = tmp_path / "decision_check"
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-O2", "-std=c++17", SRC, "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    r = subprocess.run([str(exe), "3000000", "all"], capture_output=True, text=True, timeout=300)
    print(r.stdout)
    assert r.returncode == 0, r.stdout
