"""The library's per-launch timing bookkeeping (csrc/timing_ring.h), built with
the host compiler against fake events: pending event pairs stay bounded over
100k launches, every duration reaches its phase's sum once, events are
recycled, and a failure is reported by the next read.  CPU only."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "matrix_optimizers_amd", "csrc")


def test_timing_ring_bounded_and_exact(tmp_path):
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = tmp_path / "timing_ring_test"
    subprocess.run([cxx, "-O1", "-std=c++17", "-Wall", "-Werror", "-I", CSRC,
                    os.path.join(HERE, "host", "timing_ring_test.cpp"), "-o", str(exe)],
                   check=True, capture_output=True, text=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "timing ring OK" in res.stdout
