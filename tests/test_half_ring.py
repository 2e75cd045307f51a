"""The grouped GEMM's half-stage load schedule (csrc/half_ring.h): a host
program simulates the order in which a wave issues its weight and A loads and
checks the wait counts the kernel uses against the exact number of younger
loads, slot reuse against the barriers, and that every load happens once
(tests/native/half_ring_check.cc)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "grouped_top_routing_amd", "csrc")
SRC = os.path.join(ROOT, "tests", "native", "half_ring_check.cc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_half_ring_schedule(tmp_path):
    exe = tmp_path / "half_ring_check"
    subprocess.run(["g++", "-O2", "-std=c++17", "-Wall", "-Werror", "-I", CSRC, "-o", str(exe), SRC],
                   check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok "), r.stdout
