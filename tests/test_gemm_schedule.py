"""Host checks of the grouped GEMM's schedules (tests/native/*.cc, built with
g++ against the kernel's own headers):

* half_ring_check: the bf16 half-stage load schedule (csrc/half_ring.h) -- a
  simulation of the order in which a wave issues its weight and A loads,
  against which the kernel's wait counts, slot reuse and single loading are
  checked;
* item_order_check: the persistent walk's item orders (csrc/item_order.h) on
  random plans -- every item visited once, within its expert, and the blocked
  order's windows of 8 m-tiles x 4 n-tiles."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "grouped_top_routing_amd", "csrc")
NATIVE = os.path.join(ROOT, "tests", "native")


def _run(name, tmp_path):
    exe = tmp_path / name
    subprocess.run(["g++", "-O2", "-std=c++17", "-Wall", "-Werror", "-I", CSRC, "-o", str(exe),
                    os.path.join(NATIVE, name + ".cc")], check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok "), r.stdout


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_half_ring_schedule(tmp_path):
    _run("half_ring_check", tmp_path)


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_item_order(tmp_path):
    _run("item_order_check", tmp_path)
