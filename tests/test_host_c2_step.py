"""The kernels' division-free fp32(c2/448) equals the IEEE quotient on its whole range.

Double quantization ("Double quantization", zerotofrontier.app "sft/peft") decodes a
first-level constant as E4M3(q) * fp32(c2/448) + mean.  The gfx950 kernels form the
quotient with one multiply and two fused multiply-adds when 2^-100 <= |c2| <= FLT_MAX
and fall back to a division otherwise; this test compiles a small C program that
compares the two for every fp32 value of that range.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_c2_step_matches_ieee_division_exhaustively(tmp_path):
    exe = tmp_path / "c2_step"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-mfma", "-ffp-contract=off",
                    os.path.join(HERE, "c", "c2_step_exhaustive.c"), "-o", str(exe), "-lm"],
                   check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()
    n, bad = int(out[0]), int(out[1])
    # 0x7F7FFFFF - bits(2^-100) + 1 inputs
    assert n == 0x7F7FFFFF - 0x0D800000 + 1
    assert bad == 0
