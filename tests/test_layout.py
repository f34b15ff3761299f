"""Host check of the kernels' index arithmetic (no GPU).

Compiles tests/native/layout_check.cpp against the header the kernels use for
their tile layouts and per-lane addresses (fa2_layout.h) with the system C++
compiler and runs it: every global address a tile copy or register stage
forms must stay inside its tensor and fetch the chunk its LDS slot is meant
to hold, every slot is written once, every MFMA operand read stays inside its
LDS tile and fetches the elements the lane layout expects.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_tiled_attention_34_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs a host C++ compiler")
def test_layout_indexing(tmp_path):
    exe = tmp_path / "layout_check"
    src = os.path.join(ROOT, "tests", "native", "layout_check.cpp")
    subprocess.run(["g++", "-std=c++17", "-O1", "-Wall", "-Wno-unknown-pragmas", "-I", CSRC, src, "-o",
                    str(exe)], check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout[-2000:]
