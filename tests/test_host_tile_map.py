"""Work units of the fused dequant products cover every output tile exactly once.

The fused forward and dX products run TM x TN output tiles (512 x 128; 256 x 256 is
checked too); when the last wave of tiles on an XCD is at most half full, those tail
tiles are cut into pieces along the contraction whose fp32 partials a second kernel
sums.  This test compiles a host program against the same header the kernels use and
checks the map over thousands of launch shapes (coverage, contraction ranges, XCD
placement, partial-slot bounds, the summing kernel's slot -> tile lookup).
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "bit_nf4_quantized_09_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_tile_map_covers_every_tile_once(tmp_path):
    exe = tmp_path / "tile_map_check"
    subprocess.run(["g++", "-O2", "-std=c++17", "-I", CSRC,
                    os.path.join(HERE, "c", "tile_map_check.cpp"), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout
    shapes, bad = map(int, out.split()[-2:])
    assert shapes > 4000
    assert bad == 0, out
