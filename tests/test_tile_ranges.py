"""Host-side check of which (query row, key) tiles the prefill and backward
kernels visit: the tile-range arithmetic the kernels compile (csrc/g2_tiles.h)
is built into a small C++ program with g++ and compared with a brute-force
enumeration of the visible pairs over a grid of (T, S, W, local/global),
including chunked layers (T < S) whose oldest key blocks no query sees and
windows up to INT_MAX.  No GPU involved.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "tile_check", "tile_check.cpp")
CSRC = os.path.join(ROOT, "attention_g2attn_prefill_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_tile_ranges_cover_exactly_the_visible_pairs(tmp_path):
    exe = str(tmp_path / "tile_check")
    subprocess.run(["g++", "-std=c++17", "-O2", "-Wall", "-I", CSRC, "-o", exe, SRC], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(r.stdout[-2000:])
    assert r.returncode == 0, r.stdout[-4000:]
    assert "0 failures" in r.stdout
