"""Host logic of the planner, built with the host compiler (no GPU, no HIP).

The windowed kernel's work split (window_split) is checked by a small C++
driver (tests/plan_split_check.cpp) linked against plan.cpp: every unit is
covered once, in contiguous ranges; each XCD run starts and ends on a tile
boundary; no range follows an empty one (the kernel's hand-over waits on the
previous workgroup of its run); and on small sizes the largest range cost is
the optimum found by brute force over every contiguous split.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "modulated_deformable_convolution_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="no host C++ compiler")
def test_window_split(tmp_path):
    exe = tmp_path / "plan_split_check"
    subprocess.run(["g++", "-std=c++17", "-O1", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
                    os.path.join(CSRC, "plan.cpp"),
                    os.path.join(ROOT, "tests", "plan_split_check.cpp"), "-o", str(exe)],
                   check=True, capture_output=True, timeout=300)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True, timeout=300)
    assert out.stdout.startswith("ok"), out.stdout
